// Host-only harness of the C ABI's argument checks, built with host-side
// AddressSanitizer and UndefinedBehaviorSanitizer (device code is compiled as
// usual and never launched): every entry point is called with arguments it
// must refuse before launching anything, and the workspace sizes of the
// supported problems are computed.  Exit status 0 when every status is the
// expected one.  Test infrastructure: built and run by
// tests/test_sanitizers.py.
#include <cstdint>
#include <cstdio>

#include "gdn.h"

static int fails = 0;
static void expect(gdn_status got, gdn_status want, const char *what) {
  if (got != want) {
    std::fprintf(stderr, "FAILED: %s: status %d, expected %d\n", what, (int)got, (int)want);
    ++fails;
  }
}

int main() {
  gdn_shape s{1, 4096, 16, 32, 128, 128, 128, 0, GDN_BF16, GDN_F32};
  expect(gdn_validate(&s), GDN_OK, "8B layer");
  expect(gdn_validate(nullptr), GDN_ERR_NULL, "null shape");
  size_t bytes = 0;
  expect(gdn_workspace_size(&s, &bytes), GDN_OK, "workspace size");
  if (bytes == 0) { std::fprintf(stderr, "FAILED: zero workspace\n"); ++fails; }
  expect(gdn_workspace_size(&s, nullptr), GDN_ERR_NULL, "null size pointer");
  // sizes: every rejected field
  const int32_t bad[][10] = {
      {0, 4096, 16, 32, 128, 128, 128, 0, 1, 0},   {1, -1, 16, 32, 128, 128, 128, 0, 1, 0},
      {1, 4096, 16, 24, 128, 128, 128, 0, 1, 0},   {1, 4096, 16, 32, 64, 128, 128, 0, 1, 0},
      {1, 4096, 16, 32, 128, 256, 128, 0, 1, 0},   {1, 4096, 16, 32, 128, 128, 96, 0, 1, 0},
      {1, 4096, 16, 32, 128, 128, 128, 3, 1, 0},   {1, 4096, 16, 32, 128, 128, 128, -1, 1, 0},
      {1, 128 * 70000, 16, 32, 128, 128, 128, 0, 1, 0}};
  for (const auto &b : bad) {
    gdn_shape t{b[0], b[1], b[2], b[3], b[4], b[5], b[6], b[7], b[8], b[9]};
    expect(gdn_validate(&t), GDN_ERR_SHAPE, "bad shape");
    expect(gdn_workspace_size(&t, &bytes), GDN_ERR_SHAPE, "bad shape workspace");
  }
  gdn_shape d = s;
  d.dtype = 7;
  expect(gdn_validate(&d), GDN_ERR_DTYPE, "bad dtype");
  // entry points refuse before launching: null, misaligned, short workspace
  alignas(16) static char buf[64];
  void *ok = buf, *odd = buf + 4;
  const float *fk = reinterpret_cast<const float *>(buf);
  float *fo = reinterpret_cast<float *>(buf);
  expect(gdn_chunk_fwd(&s, nullptr, ok, ok, fk, fk, nullptr, ok, nullptr, ok, bytes, nullptr), GDN_ERR_NULL, "fwd null q");
  expect(gdn_chunk_fwd(&s, odd, ok, ok, fk, fk, nullptr, ok, nullptr, ok, bytes, nullptr), GDN_ERR_ALIGN, "fwd misaligned");
  expect(gdn_chunk_fwd(&s, ok, ok, ok, fk, fk, nullptr, ok, nullptr, ok, bytes - 1, nullptr), GDN_ERR_WORKSPACE,
         "fwd workspace");
  expect(gdn_chunk_fwd_stages(&s, 64, ok, ok, ok, fk, fk, nullptr, ok, nullptr, ok, bytes, nullptr), GDN_ERR_SHAPE,
         "stage bits");
  expect(gdn_chunk_fold(&s, ok, ok, fk, fk, nullptr, fo, ok, bytes, nullptr), GDN_ERR_NULL, "fold null A");
  expect(gdn_chunk_transform(&s, ok, ok, fk, fk, nullptr, nullptr, fo, fo, nullptr), GDN_ERR_NULL, "transform null G");
  expect(gdn_compose_prefix(4, 8, 128, 128, fk, fk, nullptr, nullptr, nullptr, 0, nullptr), GDN_ERR_NULL, "prefix outs");
  expect(gdn_compose_prefix(4, 8, 64, 128, fk, fk, nullptr, fo, nullptr, 0, nullptr), GDN_ERR_SHAPE, "prefix d_k");
  expect(gdn_compose_prefix(4, 8, 128, 128, fk, fk, nullptr, fo, nullptr, GDN_PREFIX_SEQUENTIAL | GDN_PREFIX_BLOCKED,
                            nullptr),
         GDN_ERR_SHAPE, "prefix forms");
  expect(gdn_compose_prefix(4, 8, 128, 128, reinterpret_cast<const float *>(odd), fk, nullptr, fo, nullptr, 0, nullptr),
         GDN_ERR_ALIGN, "prefix misaligned");
  expect(gdn_chunk_fwd_affine(&s, ok, ok, ok, fk, fk, nullptr, ok, nullptr, nullptr, ok, bytes, nullptr), GDN_ERR_NULL,
         "affine null A");
  gdn_shape grouped = s;
  grouped.n_groups = 4;
  expect(gdn_chunk_fwd_affine(&grouped, ok, ok, ok, fk, fk, nullptr, ok, nullptr, fo, ok, bytes, nullptr), GDN_ERR_SHAPE,
         "affine with groups");
  gdn_shape big = s;
  big.T = 65536;
  expect(gdn_chunk_fwd_noalloc(&big, ok, ok, ok, fk, fk, nullptr, ok, nullptr, nullptr), GDN_ERR_WORKSPACE,
         "no-alloc beyond the scratch");
  gdn_shape vl = s;
  vl.B = 8;
  vl.T = 1000;
  expect(gdn_workspace_size_varlen(&vl, &bytes), GDN_OK, "varlen workspace");
  expect(gdn_chunk_fwd_varlen(&vl, nullptr, ok, ok, ok, fk, fk, nullptr, ok, nullptr, ok, bytes, nullptr),
         GDN_ERR_NULL, "varlen null offsets");
  // the backward: one walk per sequence, required pointers, alignment, workspace
  expect(gdn_workspace_size_bwd_grads(&s, &bytes), GDN_OK, "backward workspace");
  expect(gdn_chunk_bwd(&s, ok, ok, ok, fk, fk, nullptr, fk, nullptr, nullptr, fo, fo, fo, fo, nullptr, ok, bytes,
                       nullptr),
         GDN_ERR_NULL, "backward null dq");
  expect(gdn_chunk_bwd(&s, ok, ok, ok, fk, fk, nullptr, fk, nullptr, fo, fo, fo, fo, fo, nullptr, ok, bytes - 1,
                       nullptr),
         GDN_ERR_WORKSPACE, "backward workspace too small");
  expect(gdn_chunk_bwd(&grouped, ok, ok, ok, fk, fk, nullptr, fk, nullptr, fo, fo, fo, fo, fo, nullptr, ok, bytes,
                       nullptr),
         GDN_ERR_SHAPE, "backward grouped");
  expect(gdn_chunk_bwd(&s, reinterpret_cast<const void *>(odd), ok, ok, fk, fk, nullptr, fk, nullptr, fo, fo, fo, fo,
                       fo, nullptr, ok, bytes, nullptr),
         GDN_ERR_ALIGN, "backward misaligned q");
  for (int c = -7; c <= 1; ++c)
    if (!gdn_status_str((gdn_status)c)) { std::fprintf(stderr, "FAILED: status string %d\n", c); ++fails; }
  if (fails) return 1;
  std::printf("ABI harness: all checks passed\n");
  return 0;
}
