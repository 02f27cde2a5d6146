// gdn_api.hip -- C ABI of the GDN chunked forward (declared in include/gdn.h).
//
// Host side only: argument checks, workspace carving and kernel launches on
// the caller's stream.  No allocation and no synchronisation; the only
// global state is the per-device address of the no-allocation entry point's
// static scratch array (looked up once per device).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <mutex>

#include "gdn.h"
#include "gdn_bwd.h"
#include "gdn_kernels.h"

using namespace gdn;

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  size_t G, W, Kt, U, Hs, Vn, A, Bp, Hin, Ct, Jt, Nt, total;
};

int groups_of(const gdn_shape &s) { return s.n_groups > 1 ? s.n_groups : 1; }

// chunks per sequence; a partial last chunk is padded with identity steps
int chunks_of(const gdn_shape &s) { return (int)(((int64_t)s.T + s.chunk - 1) / s.chunk); }

// Packed variable-length sequences: s.B sequences share one row of T tokens;
// their chunks, at most T / C + s.B of them, are numbered across sequences.
int varlen_nmax(const gdn_shape &s) { return (int)((int64_t)s.T / s.chunk + s.B); }

// The walk that forms the outputs itself (walk_out_kernel) takes every
// padded-batch walk (or replay of chunk-groups) of at least this many walks:
// measured at chunk 128, bf16, 128 to 512 walks of 16 to 64 chunks and the
// 262,144-token replay (8192 walks), it runs 7-14% faster than the walk
// and the separate output stage; at 64 walks (two workgroups per walk cover
// half the compute units) 25% slower.  Fewer walks keep the walk forms that
// spread each walk over more of the chip, and the output stage.
#ifndef GDN_FUSED_MIN_WALKS
#define GDN_FUSED_MIN_WALKS 128
#endif
#ifndef GDN_FUSED_WPG
#define GDN_FUSED_WPG 4
#endif
// From this many walks on, each wave of the walk with outputs holds two state
// slices (one workgroup per walk, which forms the chunk's P^T and copies its
// operands once for all 128 columns) instead of one (two workgroups per walk,
// each forming P^T and copying the chunk).  Measured at chunk 128, bf16: 22-25%
// faster from 256 to 8192 walks (the 262,144-token replay 5.18 -> 3.86 ms),
// 30% slower at 128 walks (one workgroup per walk leaves half the compute
// units idle).
#ifndef GDN_FUSED_WIDE_MIN_WALKS
#define GDN_FUSED_WIDE_MIN_WALKS 256
#endif
constexpr int kFusedWpg = GDN_FUSED_WPG;   // slices (waves) per workgroup of walk_out_kernel
bool fused_walk(const gdn_shape &s) {
  return (int64_t)s.B * s.H_v * groups_of(s) >= GDN_FUSED_MIN_WALKS;
}

// Workspace of `rows` sequence rows of N chunks each (plus, for `nseq` packed
// sequences, their chunk tables); `handoff`: room for the chunk-start states
// and corrected values that the walk hands to a separate output stage.
Layout layout_n(const gdn_shape &s, size_t rows, size_t N, size_t nseq, bool handoff = true) {
  const size_t BH = rows * s.H_v, C = s.chunk;
  const size_t J = groups_of(s);
  const size_t in_bytes = s.dtype == GDN_BF16 ? 2 : 4;
  Layout L{};
  size_t off = 0;
  L.G = off;  off += align_up(BH * N * C * 4);
  L.W = off;  off += align_up(BH * N * C * D * in_bytes);
  L.Kt = off; off += align_up(rows * s.H_qk * N * C * D * in_bytes);   // per key head
  L.U = off;  off += align_up(BH * N * C * D * 4);
  if (handoff) {
    L.Hs = off; off += align_up(BH * N * D * D * 4);   // fp32, or bf16 hi + lo planes
    L.Vn = off; off += align_up(BH * N * C * D * 4);
  }
  if (J > 1) {
    L.A = off;   off += align_up(BH * J * D * D * 4);
    L.Bp = off;  off += align_up(BH * J * D * D * 4);
    L.Hin = off; off += align_up(BH * J * D * D * 4);
  }
  if (nseq) {
    L.Ct = off; off += align_up(N * sizeof(int2));
    L.Jt = off; off += align_up(nseq * sizeof(int2));
    L.Nt = off; off += align_up(sizeof(int));
  }
  L.total = off;
  return L;
}
Layout layout(const gdn_shape &s) { return layout_n(s, s.B, chunks_of(s), 0, !fused_walk(s)); }
Layout layout_varlen(const gdn_shape &s) { return layout_n(s, 1, varlen_nmax(s), s.B); }

bool misaligned(const void *p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u); }

gdn_status check_launch() {
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

#define GDN_TRY(x)                       \
  do {                                   \
    gdn_status st_ = (x);                \
    if (st_ != GDN_OK) return st_;       \
  } while (0)

// copies h0 (or zero) to h_T for an empty sequence
__global__ void copy_state_kernel(const float *src, float *dst, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src ? src[i] : 0.f;
}

// identity matrices [n / (D * D)][D][D] (the map of an empty sequence)
__global__ void identity_kernel(float *dst, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = (i % (D * D)) / D == i % D ? 1.f : 0.f;
}

FwdArgs base_args(const gdn_shape &s) {
  FwdArgs a{};
  a.B = s.B; a.T = s.T; a.Hqk = s.H_qk; a.Hv = s.H_v; a.N = chunks_of(s);
  a.jobs = 1; a.cpj = a.N;
  a.n0 = 0; a.nn = a.N;
  return a;
}

// compute units of the current device (256 on MI355X)
int num_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n < 8)
    return 256;
  return n;
}

// Where a kernel goes: the stream, and optionally two timing events that
// record the kernel's own start and end (hipExtLaunchKernel; no event packets
// between kernels).
struct Lx {
  hipStream_t st;
  hipEvent_t e0 = nullptr, e1 = nullptr;
};
template <typename K, typename... Args>
void launch(K kernel, dim3 grid, dim3 block, const Lx &x, Args... args) {
  if (x.e0 || x.e1)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, x.st, x.e0, x.e1, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, x.st, args...);
}

// rag: some chunk is partial (the last one when T % C != 0, or any chunk of
// packed sequences): the row-masked instantiation
template <int C, typename TI, int MODE, bool FWD = true>
gdn_status launch_prep(const FwdArgs &a, const Lx &x, bool rag = false) {
  const long units = (long)a.nn * a.B * a.Hv;   // one workgroup per (chunk, head)
  if (rag || a.T % C)
    launch(prep_kernel<C, TI, MODE, FWD, true>, dim3((unsigned)units), dim3(PNT), x, a);
  else
    launch(prep_kernel<C, TI, MODE, FWD, false>, dim3((unsigned)units), dim3(PNT), x, a);
  return check_launch();
}


template <int C, typename TI, int MODE, int KIND>
gdn_status launch_walk(const FwdArgs &a, const Lx &x) {
  const int width = KIND == WALK ? D : 2 * D;   // state columns (the augmented state for FOLD and WALK_A)
  // Launch form by the number of walks (units), measured:
  //  * many (walk: 65 or more; fold: 256 or more): the throughput form, one
  //    wave per 16-column slice, the slices of a workgroup sharing each
  //    chunk's operands through LDS -- 4 slices per workgroup for the walk
  //    (10-19% faster than 8 between 96 and 512 walks, and at 8192; 0-9%
  //    faster than the latency form from 65 to 95), 8 for the fold (whose
  //    4-slice form ran 40% slower);
  //  * 33..64 walks: two slices per workgroup, each split over waves by rows;
  //  * fewer: one slice per workgroup of 2 or 4 waves that split its rows,
  //    so that a short walk spreads over the chip.
  const long units = (long)a.B * a.Hv * a.jobs;
  constexpr int NWS = C >= 128 ? 4 : 2;   // waves per slice: whole k-blocks of V' rows each
  // (the walk always hands h and V' to the output stage; the throughput and
  // paired forms count on those stores)
  if (KIND != FOLD && (!a.Hs || !a.Vn)) return GDN_ERR_NULL;
  // (the walk that also yields A takes the latency form at any count)
  if constexpr (KIND == WALK_A) {
    launch(walk_ring_kernel<C, TI, MODE, KIND, NWS>, dim3((unsigned)(units * (width / 16))), dim3(64 * NWS), x, a);
  } else if constexpr (KIND == FOLD) {
    if (units * (width / 128) >= 512) {
      // persistent (one workgroup per compute unit, each taking every
      // num_cus-th item and copying its next item's first chunk during the
      // last chunk of the one before) when every item's chunk count is even
      const long items = units * (width / 128);
      const long grid = a.cpj % 2 == 0 ? std::min(items, (long)num_cus()) : items;
      launch(walk_shared_kernel<C, TI, MODE, KIND, 8>, dim3((unsigned)grid), dim3(512), x, a);
    } else {
      launch(walk_ring_kernel<C, TI, MODE, KIND, NWS>, dim3((unsigned)(units * (width / 16))), dim3(64 * NWS), x, a);
    }
  } else {
    if (units >= 65) {
      launch(walk_shared_kernel<C, TI, MODE, KIND, 4>, dim3((unsigned)(units * (width / 64))), dim3(256), x, a);
    } else if (units > 32) {
      // two latency-form slices per compute unit would each stream the same
      // operands: one workgroup of two slices shares a copy in LDS instead
      launch(walk_pair_kernel<C, TI, MODE, NWS>, dim3((unsigned)(units * (D / 32))), dim3(128 * NWS), x, a);
    } else {
      launch(walk_ring_kernel<C, TI, MODE, KIND, NWS>, dim3((unsigned)(units * (width / 16))), dim3(64 * NWS), x, a);
    }
  }
  return check_launch();
}

template <int C, typename TI, int MODE, typename TO>
gdn_status launch_out(const FwdArgs &a, const Lx &x, bool rag = false) {
  const long units = (long)a.nn * a.B * a.Hv;   // one workgroup per (chunk, head)
  if (rag || a.T % C)
    launch(out_kernel<C, TI, MODE, TO, true>, dim3((unsigned)units), dim3(NT), x, a);
  else
    launch(out_kernel<C, TI, MODE, TO, false>, dim3((unsigned)units), dim3(NT), x, a);
  return check_launch();
}

template <int C, typename TI, int MODE, typename TO, int KIND = WALK>
gdn_status launch_walk_out(const FwdArgs &a, const Lx &x) {
  const long units = (long)a.B * a.Hv * a.jobs;
  auto go = [&](auto spw) {
    constexpr int SPW = decltype(spw)::value;   // state slices per wave
    constexpr int NG = (KIND == WALK_A ? 2 : 1) * (D / 16) / (kFusedWpg * SPW);   // workgroups per walk
    if (a.T % C)
      launch(walk_out_kernel<C, TI, MODE, TO, kFusedWpg, true, KIND, SPW>, dim3((unsigned)(units * NG)), dim3(64 * kFusedWpg), x, a);
    else
      launch(walk_out_kernel<C, TI, MODE, TO, kFusedWpg, false, KIND, SPW>, dim3((unsigned)(units * NG)), dim3(64 * kFusedWpg), x, a);
  };
  if (KIND == WALK && units >= GDN_FUSED_WIDE_MIN_WALKS)
    go(std::integral_constant<int, KIND == WALK ? 2 : 1>{});
  else
    go(std::integral_constant<int, 1>{});
  return check_launch();
}

// Pairs per block of the blocked prefix: the divisor of n nearest sqrt(n)
// (at least 3: a block's slots hold its composed pair and incoming state), if
// the blocked prefix is expected to be faster; 0 = the sequential prefix.
// Both are modelled from their MI355X timings over 1..32 rows and 32..1024
// pairs: the sequential prefix costs the larger of 2.1 us per pair with
// split-bf16 products, 2.55 us with fp32 ones (a chain of dependent steps),
// and its traffic (A and B read, h_in written: 3 * 64 KB per pair) at 2.5
// (2.15) TB/s; the blocked one the larger of its 2 s + n / s steps
// (5.6 us each with split-bf16 products, 9 us with fp32 ones) and its
// traffic (A and B read twice: 5 * 64 KB per pair) at 2.4 TB/s.
// force: the blocked prefix whenever n has such a divisor.
int prefix_block(int n, int BH, bool split, bool force) {
  if (n < 9) return 0;
  int s = 0;
  for (int c = 3; c <= n / 3; ++c)
    if (n % c == 0 && (s == 0 || std::abs(c * c - n) < std::abs(s * s - n))) s = c;
  if (s == 0 || force) return s;
  const double pair_bytes = (double)D * D * 4 * BH;
  const double t_seq = std::max(n * (split ? 2.1e-6 : 2.55e-6), 3 * pair_bytes * n / (split ? 2.5e12 : 2.15e12));
  const double t_blk = std::max((2 * s + n / s) * (split ? 5.6e-6 : 9e-6), 5 * pair_bytes * n / 2.4e12);
  return t_blk < t_seq ? s : 0;
}

// the sequential prefix kernel for the precision and whether h_in is written
void launch_prefix_seq(bool split, bool hin, dim3 grid, dim3 block, const Lx &x, const PrefixArgs &p) {
  if (split && hin) launch(prefix_kernel<P_SPLIT_AB, 4, true>, grid, block, x, p);
  else if (split) launch(prefix_kernel<P_SPLIT_AB, 4, false>, grid, block, x, p);
  else if (hin) launch(prefix_kernel<P_F32, 4, true>, grid, block, x, p);
  else launch(prefix_kernel<P_F32, 4, false>, grid, block, x, p);
}

gdn_status launch_prefix(int BH, int n, const float *A, const float *Bm, const float *h_init, float *h_in,
                         float *h_final, bool split, const Lx &x, int form = 0) {   // form: 0 chosen, 1 sequential, 2 blocked
  constexpr int NWS = 4;                              // waves per slice, 32 state rows each
  const int s = (h_in && form != 1) ? prefix_block(n, BH, split, form == 2) : 0;
  if (s == 0) {
    PrefixArgs p{BH, n, A, Bm, h_init, h_in, h_final};
    const unsigned blocks = (unsigned)(D / 16) * BH;   // one workgroup per 16-column slice
    launch_prefix_seq(split, h_in != nullptr, dim3(blocks), dim3(64 * NWS), x, p);
    return check_launch();
  }
  // blocked: compose each block's pairs, the sequential prefix over the
  // blocks' pairs (kept in the incoming-state slots), replay every block
  // (the stage's timing events bound the three launches)
  const int nb = n / s;
  PairWalkArgs w{BH, n, s, A, Bm, h_in};
  const size_t DD = (size_t)D * D;
  PrefixArgs p{BH, nb, h_in + DD, h_in + 2 * DD, h_init, h_in, h_final, (long long)(s * DD), (long long)(n * DD)};
  const Lx first{x.st, x.e0, nullptr}, mid{x.st}, last{x.st, nullptr, x.e1};
  const unsigned units = (unsigned)((long)BH * nb), slices = (unsigned)(D / 16) * BH;
  if (split) {
    launch(pair_walk_kernel<P_SPLIT_AB, PW_COMPOSE>, dim3(2 * units), dim3(512), first, w);
    launch_prefix_seq(true, true, dim3(slices), dim3(64 * NWS), mid, p);
    launch(pair_walk_kernel<P_SPLIT_AB, PW_REPLAY>, dim3(units), dim3(512), last, w);
  } else {
    launch(pair_walk_kernel<P_F32, PW_COMPOSE>, dim3(2 * units), dim3(512), first, w);
    launch_prefix_seq(false, true, dim3(slices), dim3(64 * NWS), mid, p);
    launch(pair_walk_kernel<P_F32, PW_REPLAY>, dim3(units), dim3(512), last, w);
  }
  return check_launch();
}

template <int C, typename TI, int MODE>
gdn_status run_fwd(const gdn_shape &s, int stages, const void *q, const void *k, const void *v, const float *g,
                   const float *beta, const float *h0, void *o, float *h_T, char *ws, hipStream_t st,
                   void *const *ev0 = nullptr, void *const *ev1 = nullptr, float *A = nullptr) {
  // stage bit b (GDN_STAGE_* = 1 << b) launches with events ev0[b], ev1[b]
  auto lx = [&](int b) {
    Lx x{st};
    if (ev0) x.e0 = reinterpret_cast<hipEvent_t>(ev0[b]);
    if (ev1) x.e1 = reinterpret_cast<hipEvent_t>(ev1[b]);
    return x;
  };
  const Layout L = layout(s);
  const bool fused = fused_walk(s);
  FwdArgs a = base_args(s);
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.o = o;
  a.G = reinterpret_cast<float *>(ws + L.G);
  a.W = ws + L.W;
  a.Kt = ws + L.Kt;
  a.U = reinterpret_cast<float *>(ws + L.U);
  if (!fused) {
    a.Hs = reinterpret_cast<float *>(ws + L.Hs);
    a.Vn = reinterpret_cast<float *>(ws + L.Vn);
  }
  // the walk: with its outputs (fused), or handing h and V' to the output stage
  auto walk = [&](const FwdArgs &w) -> gdn_status {
    if (A) {
      if (!fused) return launch_walk<C, TI, MODE, WALK_A>(w, lx(3));
      if (s.o_dtype == GDN_F32) return launch_walk_out<C, TI, MODE, float, WALK_A>(w, lx(3));
      return launch_walk_out<C, TI, MODE, __bf16, WALK_A>(w, lx(3));
    }
    if (!fused) return launch_walk<C, TI, MODE, WALK>(w, lx(3));
    if (s.o_dtype == GDN_F32) return launch_walk_out<C, TI, MODE, float>(w, lx(3));
    return launch_walk_out<C, TI, MODE, __bf16>(w, lx(3));
  };
  const int J = groups_of(s);
  if (stages & GDN_STAGE_PREP) GDN_TRY((launch_prep<C, TI, MODE>(a, lx(0))));
  if (J == 1) {
    a.init = h0; a.init_per_job = 0; a.fin = h_T; a.pairA = A;
    if (stages & GDN_STAGE_WALK) GDN_TRY(walk(a));
  } else {
    FwdArgs f = a;
    f.jobs = J; f.cpj = a.N / J;
    f.pairA = reinterpret_cast<float *>(ws + L.A);
    f.pairB = reinterpret_cast<float *>(ws + L.Bp);
    if (stages & GDN_STAGE_FOLD) GDN_TRY((launch_walk<C, TI, MODE, FOLD>(f, lx(1))));
    // h_T: the end state of the last group's replay; the prefix's composition
    // of all pairs (the same state up to rounding) when the replay is not
    // among the stages
    float *h_in = reinterpret_cast<float *>(ws + L.Hin);
    if (stages & GDN_STAGE_PREFIX)
      GDN_TRY(launch_prefix(s.B * s.H_v, J, f.pairA, f.pairB, h0, h_in, (stages & GDN_STAGE_WALK) ? nullptr : h_T,
                            MODE == MODE_BF16, lx(2)));
    FwdArgs r = a;
    r.jobs = J; r.cpj = a.N / J;
    r.init = h_in; r.init_per_job = 1; r.fin = h_T;
    if (stages & GDN_STAGE_WALK) GDN_TRY(walk(r));
  }
  if (!(stages & GDN_STAGE_OUT)) return GDN_OK;
  if (fused) {
    // the walk wrote o: the output stage has no kernel (its timing events,
    // if any, bound an empty interval)
    const Lx x = lx(4);
    if (x.e0 && hipEventRecord(x.e0, st) != hipSuccess) return GDN_ERR_HIP;
    if (x.e1 && hipEventRecord(x.e1, st) != hipSuccess) return GDN_ERR_HIP;
    return GDN_OK;
  }
  if (s.o_dtype == GDN_F32) return launch_out<C, TI, MODE, float>(a, lx(4));
  return launch_out<C, TI, MODE, __bf16>(a, lx(4));
}

// Packed variable-length sequences: the chunk tables, then prep and out over
// the numbered chunks (every one possibly partial) and one walk per
// (sequence, value head).
template <int C, typename TI, int MODE>
gdn_status run_fwd_varlen(const gdn_shape &s, const int *cu, const void *q, const void *k, const void *v,
                          const float *g, const float *beta, const float *h0, void *o, float *h_T, char *ws,
                          hipStream_t st) {
  const Layout L = layout_varlen(s);
  const int nmax = varlen_nmax(s);
  int2 *ctab = reinterpret_cast<int2 *>(ws + L.Ct);
  int2 *jtab = reinterpret_cast<int2 *>(ws + L.Jt);
  int *ntot = reinterpret_cast<int *>(ws + L.Nt);
  hipLaunchKernelGGL(varlen_tables_kernel, dim3(1), dim3(256), 0, st, cu, s.B, s.T, C, nmax, ctab, jtab, ntot);
  GDN_TRY(check_launch());
  FwdArgs a{};
  a.B = 1; a.T = s.T; a.Hqk = s.H_qk; a.Hv = s.H_v; a.N = nmax;
  a.jobs = 1; a.cpj = 0; a.n0 = 0; a.nn = nmax;
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.o = o;
  a.G = reinterpret_cast<float *>(ws + L.G);
  a.W = ws + L.W;
  a.Kt = ws + L.Kt;
  a.U = reinterpret_cast<float *>(ws + L.U);
  a.Hs = reinterpret_cast<float *>(ws + L.Hs);
  a.Vn = reinterpret_cast<float *>(ws + L.Vn);
  a.ctab = ctab; a.ntot = ntot;
  GDN_TRY((launch_prep<C, TI, MODE>(a, Lx{st}, true)));
  FwdArgs w = a;
  w.B = s.B; w.jtab = jtab; w.init = h0; w.init_per_job = 0; w.fin = h_T;
  if (s.o_dtype == GDN_F32) {
    GDN_TRY((launch_walk<C, TI, MODE, WALK>(w, Lx{st})));
    return launch_out<C, TI, MODE, float>(a, Lx{st}, true);
  }
  GDN_TRY((launch_walk<C, TI, MODE, WALK>(w, Lx{st})));
  return launch_out<C, TI, MODE, __bf16>(a, Lx{st}, true);
}

template <int C, typename TI, int MODE>
gdn_status run_fold(const gdn_shape &s, const void *k, const void *v, const float *g, const float *beta,
                    float *A, float *Bm, char *ws, hipStream_t st) {
  const Layout L = layout(s);
  FwdArgs a = base_args(s);
  a.k = k; a.v = v; a.g = g; a.beta = beta;
  a.G = reinterpret_cast<float *>(ws + L.G);
  a.W = ws + L.W;
  a.Kt = ws + L.Kt;
  a.U = reinterpret_cast<float *>(ws + L.U);
  GDN_TRY((launch_prep<C, TI, MODE>(a, Lx{st})));
  const int J = groups_of(s);
  a.jobs = J; a.cpj = a.N / J; a.pairA = A; a.pairB = Bm;
  return launch_walk<C, TI, MODE, FOLD>(a, Lx{st});
}

template <int C, typename TI, int MODE>
gdn_status run_transform(const gdn_shape &s, const void *k, const void *v, const float *g, const float *beta,
                         float *G, float *Tm, float *W, float *U, hipStream_t st) {
  FwdArgs a = base_args(s);
  a.k = k; a.v = v; a.g = g; a.beta = beta; a.G = G; a.Tm = Tm; a.W = W; a.U = U;
  return launch_prep<C, TI, MODE, false>(a, Lx{st});
}

struct FwdCall {
  const gdn_shape &s; int stages; const void *q, *k, *v; const float *g, *beta, *h0; void *o; float *h_T;
  char *w; hipStream_t st; void *const *ev0 = nullptr, *const *ev1 = nullptr; float *A = nullptr;
  template <int C, typename TI, int MODE> gdn_status run() {
    return run_fwd<C, TI, MODE>(s, stages, q, k, v, g, beta, h0, o, h_T, w, st, ev0, ev1, A);
  }
};
struct VarlenCall {
  const gdn_shape &s; const int *cu; const void *q, *k, *v; const float *g, *beta, *h0; void *o; float *h_T;
  char *w; hipStream_t st;
  template <int C, typename TI, int MODE> gdn_status run() {
    return run_fwd_varlen<C, TI, MODE>(s, cu, q, k, v, g, beta, h0, o, h_T, w, st);
  }
};
struct FoldCall {
  const gdn_shape &s; const void *k, *v; const float *g, *beta; float *A, *Bm; char *w; hipStream_t st;
  template <int C, typename TI, int MODE> gdn_status run() {
    return run_fold<C, TI, MODE>(s, k, v, g, beta, A, Bm, w, st);
  }
};
struct TransformCall {
  const gdn_shape &s; const void *k, *v; const float *g, *beta; float *G, *Tm, *W, *U; hipStream_t st;
  template <int C, typename TI, int MODE> gdn_status run() {
    return run_transform<C, TI, MODE>(s, k, v, g, beta, G, Tm, W, U, st);
  }
};

// (dtype, chunk) -> instantiation
template <typename F>
gdn_status dispatch(const gdn_shape &s, F &&f) {
  if (s.dtype == GDN_BF16 && s.chunk == 128) return f.template run<128, __bf16, MODE_BF16>();
  if (s.dtype == GDN_BF16 && s.chunk == 64) return f.template run<64, __bf16, MODE_BF16>();
  if (s.dtype == GDN_F32 && s.chunk == 64) return f.template run<64, float, MODE_F32>();
  return GDN_ERR_SHAPE;
}

}  // namespace

extern "C" {

const char *gdn_status_str(gdn_status s) {
  switch (s) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL: return "a required pointer is NULL";
    case GDN_ERR_SHAPE: return "unsupported or inconsistent sizes";
    case GDN_ERR_DTYPE: return "unsupported dtype";
    case GDN_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case GDN_ERR_WORKSPACE: return "workspace too small";
    case GDN_ERR_HIP: return "kernel launch failed";
  }
  return "unknown status";
}

}  // extern "C"

namespace {
// checks shared by the padded-batch and packed-sequence entry points
gdn_status validate_common(const gdn_shape *s) {
  if (!s) return GDN_ERR_NULL;
  if (s->dtype != GDN_F32 && s->dtype != GDN_BF16) return GDN_ERR_DTYPE;
  if (s->o_dtype != GDN_F32 && s->o_dtype != GDN_BF16) return GDN_ERR_DTYPE;
  if (s->B < 1 || s->T < 0 || s->H_qk < 1 || s->H_v < 1 || s->H_v % s->H_qk) return GDN_ERR_SHAPE;
  if (s->d_k != D || s->d_v != D) return GDN_ERR_SHAPE;
  if (s->chunk != 64 && s->chunk != 128) return GDN_ERR_SHAPE;
  if (s->dtype == GDN_F32 && s->chunk != 64) return GDN_ERR_SHAPE;
  if (s->n_groups < 0) return GDN_ERR_SHAPE;
  return GDN_OK;
}
}  // namespace

extern "C" {

gdn_status gdn_validate(const gdn_shape *s) {
  GDN_TRY(validate_common(s));
  const int64_t N64 = ((int64_t)s->T + s->chunk - 1) / s->chunk;
  if (N64 > 65535 || (int64_t)s->B * s->H_v > 65535) return GDN_ERR_SHAPE;
  const int N = (int)N64;
  // one workgroup per (chunk, head) in a 1-D grid; the walk's grid is
  // (batch row, head, group or slice) x 16 at most
  if ((int64_t)N * s->B * s->H_v > (1 << 30)) return GDN_ERR_SHAPE;
  if (s->n_groups > 1 && N > 0) {
    if (N % s->n_groups) return GDN_ERR_SHAPE;
    if ((int64_t)s->B * s->n_groups > 65535) return GDN_ERR_SHAPE;
  }
  return GDN_OK;
}

gdn_status gdn_workspace_size(const gdn_shape *s, size_t *bytes) {
  if (!bytes) return GDN_ERR_NULL;
  GDN_TRY(gdn_validate(s));
  *bytes = layout(*s).total;
  return GDN_OK;
}

gdn_status gdn_chunk_fwd(const gdn_shape *s, const void *q, const void *k, const void *v, const float *g,
                         const float *beta, const float *h0, void *o, float *h_T, void *ws, size_t ws_bytes,
                         void *hip_stream) {
  return gdn_chunk_fwd_stages(s, GDN_STAGE_ALL, q, k, v, g, beta, h0, o, h_T, ws, ws_bytes, hip_stream);
}

gdn_status gdn_chunk_fwd_stages(const gdn_shape *s, int32_t stages, const void *q, const void *k, const void *v,
                                const float *g, const float *beta, const float *h0, void *o, float *h_T,
                                void *ws, size_t ws_bytes, void *hip_stream) {
  return gdn_chunk_fwd_timed(s, stages, q, k, v, g, beta, h0, o, h_T, ws, ws_bytes, hip_stream, nullptr, nullptr);
}

gdn_status gdn_chunk_fwd_timed(const gdn_shape *s, int32_t stages, const void *q, const void *k, const void *v,
                               const float *g, const float *beta, const float *h0, void *o, float *h_T,
                               void *ws, size_t ws_bytes, void *hip_stream, void *const *ev_start,
                               void *const *ev_stop) {
  GDN_TRY(gdn_validate(s));
  if (stages & ~GDN_STAGE_ALL) return GDN_ERR_SHAPE;
  hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  if (s->T == 0) {
    if (misaligned(h0) || misaligned(h_T)) return GDN_ERR_ALIGN;
    if (!h_T || !(stages & (GDN_STAGE_WALK | GDN_STAGE_PREFIX))) return GDN_OK;
    const size_t n = (size_t)s->B * s->H_v * D * D;
    hipLaunchKernelGGL(copy_state_kernel, dim3(256), dim3(256), 0, st, h0, h_T, n);
    return check_launch();
  }
  if (!q || !k || !v || !g || !beta || !o || !ws) return GDN_ERR_NULL;
  for (const void *p : {(const void *)q, (const void *)k, (const void *)v, (const void *)g,
                        (const void *)beta, (const void *)h0, (const void *)o, (const void *)h_T,
                        (const void *)ws})
    if (misaligned(p)) return GDN_ERR_ALIGN;
  if (ws_bytes < layout(*s).total) return GDN_ERR_WORKSPACE;
  char *w = reinterpret_cast<char *>(ws);
  FwdCall f{*s, stages, q, k, v, g, beta, h0, o, h_T, w, st, ev_start, ev_stop};
  return dispatch(*s, f);
}

gdn_status gdn_chunk_fwd_affine(const gdn_shape *s, const void *q, const void *k, const void *v, const float *g,
                                const float *beta, const float *h0, void *o, float *h_T, float *A, void *ws,
                                size_t ws_bytes, void *hip_stream) {
  GDN_TRY(gdn_validate(s));
  if (s->n_groups > 1) return GDN_ERR_SHAPE;
  if (!A) return GDN_ERR_NULL;
  if (misaligned(A)) return GDN_ERR_ALIGN;
  hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  if (s->T == 0) {   // no tokens: A = I, h_T = h0
    if (misaligned(h0) || misaligned(h_T)) return GDN_ERR_ALIGN;
    const size_t n = (size_t)s->B * s->H_v * D * D;
    hipLaunchKernelGGL(identity_kernel, dim3(256), dim3(256), 0, st, A, n);
    GDN_TRY(check_launch());
    if (!h_T) return GDN_OK;
    hipLaunchKernelGGL(copy_state_kernel, dim3(256), dim3(256), 0, st, h0, h_T, n);
    return check_launch();
  }
  if (!q || !k || !v || !g || !beta || !o || !ws) return GDN_ERR_NULL;
  for (const void *p : {(const void *)q, (const void *)k, (const void *)v, (const void *)g,
                        (const void *)beta, (const void *)h0, (const void *)o, (const void *)h_T,
                        (const void *)ws})
    if (misaligned(p)) return GDN_ERR_ALIGN;
  if (ws_bytes < layout(*s).total) return GDN_ERR_WORKSPACE;
  FwdCall f{*s, GDN_STAGE_ALL, q, k, v, g, beta, h0, o, h_T, reinterpret_cast<char *>(ws), st, nullptr, nullptr, A};
  return dispatch(*s, f);
}

}  // extern "C"

namespace {
// host checks of a packed-sequences problem (s->B sequences, s->T tokens):
// the chunk table bounds the (chunk, head) grids, the walk grid has 8
// workgroups per (sequence, value head) at most (16 for a fold, not offered)
gdn_status validate_varlen(const gdn_shape *s) {
  GDN_TRY(validate_common(s));
  if (s->n_groups > 1) return GDN_ERR_SHAPE;
  if ((int64_t)varlen_nmax(*s) * s->H_v > (1 << 30)) return GDN_ERR_SHAPE;
  if ((int64_t)s->B * s->H_v > (1 << 26)) return GDN_ERR_SHAPE;
  return GDN_OK;
}
}  // namespace

extern "C" {

gdn_status gdn_workspace_size_varlen(const gdn_shape *s, size_t *bytes) {
  if (!bytes) return GDN_ERR_NULL;
  GDN_TRY(validate_varlen(s));
  *bytes = layout_varlen(*s).total;
  return GDN_OK;
}

gdn_status gdn_chunk_fwd_varlen(const gdn_shape *s, const int32_t *cu_seqlens, const void *q, const void *k,
                                const void *v, const float *g, const float *beta, const float *h0, void *o,
                                float *h_T, void *ws, size_t ws_bytes, void *hip_stream) {
  GDN_TRY(validate_varlen(s));
  hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  if (misaligned(h0) || misaligned(h_T)) return GDN_ERR_ALIGN;
  if (s->T == 0) {   // every sequence empty: h_T = h0
    if (!h_T) return GDN_OK;
    hipLaunchKernelGGL(copy_state_kernel, dim3(256), dim3(256), 0, st, h0, h_T, (size_t)s->B * s->H_v * D * D);
    return check_launch();
  }
  if (!cu_seqlens || !q || !k || !v || !g || !beta || !o || !ws) return GDN_ERR_NULL;
  for (const void *p : {(const void *)cu_seqlens, (const void *)q, (const void *)k, (const void *)v,
                        (const void *)g, (const void *)beta, (const void *)o, (const void *)ws})
    if (misaligned(p)) return GDN_ERR_ALIGN;
  if (ws_bytes < layout_varlen(*s).total) return GDN_ERR_WORKSPACE;
  VarlenCall f{*s, cu_seqlens, q, k, v, g, beta, h0, o, h_T, reinterpret_cast<char *>(ws), st};
  return dispatch(*s, f);
}

gdn_status gdn_chunk_fold(const gdn_shape *s, const void *k, const void *v, const float *g, const float *beta,
                          float *A, float *Bm, void *ws, size_t ws_bytes, void *hip_stream) {
  GDN_TRY(gdn_validate(s));
  if (s->T == 0) return GDN_ERR_SHAPE;
  if (!k || !v || !g || !beta || !A || !Bm || !ws) return GDN_ERR_NULL;
  for (const void *p : {(const void *)k, (const void *)v, (const void *)g, (const void *)beta, (const void *)A,
                        (const void *)Bm, (const void *)ws})
    if (misaligned(p)) return GDN_ERR_ALIGN;
  if (ws_bytes < layout(*s).total) return GDN_ERR_WORKSPACE;
  char *w = reinterpret_cast<char *>(ws);
  hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  FoldCall f{*s, k, v, g, beta, A, Bm, w, st};
  return dispatch(*s, f);
}

gdn_status gdn_compose_prefix(int32_t batch_heads, int32_t n, int32_t d_k, int32_t d_v, const float *A,
                              const float *Bm, const float *h_init, float *h_in, float *h_final, int32_t flags,
                              void *hip_stream) {
  if (batch_heads < 1 || batch_heads > 65535 || n < 1 || d_k != D || d_v != D) return GDN_ERR_SHAPE;
  if ((int64_t)batch_heads * n > (1 << 30)) return GDN_ERR_SHAPE;
  if (!A || !Bm || (!h_in && !h_final)) return GDN_ERR_NULL;
  for (const void *p : {(const void *)A, (const void *)Bm, (const void *)h_init, (const void *)h_in,
                        (const void *)h_final})
    if (misaligned(p)) return GDN_ERR_ALIGN;
  if ((flags & GDN_PREFIX_SEQUENTIAL) && (flags & GDN_PREFIX_BLOCKED)) return GDN_ERR_SHAPE;
  const int form = (flags & GDN_PREFIX_SEQUENTIAL) ? 1 : (flags & GDN_PREFIX_BLOCKED) ? 2 : 0;
  return launch_prefix(batch_heads, n, A, Bm, h_init, h_in, h_final, (flags & GDN_PREFIX_SPLIT_BF16) != 0,
                       Lx{reinterpret_cast<hipStream_t>(hip_stream)}, form);
}

gdn_status gdn_chunk_transform(const gdn_shape *s, const void *k, const void *v, const float *g,
                               const float *beta, float *G, float *Tm, float *W, float *U, void *hip_stream) {
  GDN_TRY(gdn_validate(s));
  if (s->T == 0) return GDN_OK;
  if (!k || !v || !g || !beta || !G || !W || !U) return GDN_ERR_NULL;
  for (const void *p : {(const void *)k, (const void *)v, (const void *)g, (const void *)beta, (const void *)G,
                        (const void *)Tm, (const void *)W, (const void *)U})
    if (misaligned(p)) return GDN_ERR_ALIGN;
  hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  TransformCall f{*s, k, v, g, beta, G, Tm, W, U, st};
  return dispatch(*s, f);
}

}  // extern "C"

// ----------------------------------------------------------------------------
// The forward for callers that cannot allocate device memory: its workspace
// is `scratch`, a static device array that every GPU the library runs on
// holds until the process ends.  Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the symbol): the device
// address comes from hipGetSymbolAddress, looked up once per device with that
// device current and kept per device.
namespace {

constexpr size_t kScratchBytes = (size_t)GDN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices] = {};

// device address of the current device's copy of `scratch`
gdn_status scratch_of_current_device(void **ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GDN_ERR_HIP;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GDN_ERR_HIP;
    scratch_ptr[dev] = p;
  }
  *ptr = scratch_ptr[dev];
  return GDN_OK;
}

}  // namespace

extern "C" gdn_status gdn_chunk_fwd_noalloc(const gdn_shape *s, const void *q, const void *k, const void *v,
                                            const float *g, const float *beta, const float *h0, void *o,
                                            float *h_T, void *hip_stream) {
  GDN_TRY(gdn_validate(s));
  if (layout(*s).total > kScratchBytes) return GDN_ERR_WORKSPACE;
  if (s->T > 0) {
    if (!q || !k || !v || !g || !beta || !o) return GDN_ERR_NULL;
    for (const void *p : {(const void *)q, (const void *)k, (const void *)v, (const void *)g,
                          (const void *)beta, (const void *)h0, (const void *)o, (const void *)h_T})
      if (misaligned(p)) return GDN_ERR_ALIGN;
  }
  void *ws = nullptr;
  GDN_TRY(scratch_of_current_device(&ws));
  return gdn_chunk_fwd(s, q, k, v, g, beta, h0, o, h_T, ws, kScratchBytes, hip_stream);
}

// ----------------------------------------------------------------------------
// The chunked backward's state cotangents: prep in its transform form (G and
// W in fp32), the chunk-parallel term ddh_n, then the reverse walk.
namespace {

struct BwdLayout {
  size_t G, W, ddh, total;
};
BwdLayout layout_bwd(const gdn_shape &s) {
  const size_t BH = (size_t)s.B * s.H_v, N = chunks_of(s), C = s.chunk;
  BwdLayout L{};
  size_t off = 0;
  L.G = off;   off += align_up(BH * N * C * 4);
  L.W = off;   off += align_up(BH * N * C * D * 4);
  L.ddh = off; off += align_up(BH * N * D * D * 4);
  L.total = off;
  return L;
}

template <int C, typename TI, int MODE>
gdn_status run_bwd_state(const gdn_shape &s, const void *q, const void *k, const float *g, const float *beta,
                         const float *dO, const float *dh_T, float *dh, float *dh0, char *ws, hipStream_t st) {
  const BwdLayout L = layout_bwd(s);
  FwdArgs a = base_args(s);
  a.k = k; a.g = g; a.beta = beta;
  a.G = reinterpret_cast<float *>(ws + L.G);
  a.W = ws + L.W;   // fp32, row-major (the transform form)
  a.U = nullptr; a.Tm = nullptr;
  GDN_TRY((launch_prep<C, TI, MODE, false>(a, Lx{st})));
  BwdArgs b{};
  b.B = s.B; b.T = s.T; b.Hqk = s.H_qk; b.Hv = s.H_v; b.N = chunks_of(s);
  b.q = q; b.k = k; b.dO = dO;
  b.G = a.G; b.W = reinterpret_cast<const float *>(a.W);
  b.ddh = reinterpret_cast<float *>(ws + L.ddh);
  b.dhT = dh_T; b.dh = dh; b.dh0 = dh0;
  const unsigned units = (unsigned)((long)b.N * s.B * s.H_v);
  if (s.T % C)
    hipLaunchKernelGGL((bwd_ddh_kernel<C, TI, MODE, true>), dim3(units), dim3(ddh_threads<C>()), 0, st, a, b);
  else
    hipLaunchKernelGGL((bwd_ddh_kernel<C, TI, MODE, false>), dim3(units), dim3(ddh_threads<C>()), 0, st, a, b);
  GDN_TRY(check_launch());
  if (s.T % C)
    hipLaunchKernelGGL((bwd_walk_kernel<C, TI, MODE, true>), dim3((unsigned)(s.B * s.H_v)), dim3(512), 0, st, b);
  else
    hipLaunchKernelGGL((bwd_walk_kernel<C, TI, MODE, false>), dim3((unsigned)(s.B * s.H_v)), dim3(512), 0, st, b);
  return check_launch();
}

// The full chunked backward: prep's transform form (G, T, W, U), the
// forward's incoming states, the reverse walk's state cotangents, then the
// chunk gradients on a persistent grid of kGradSlots workgroups, each with
// its scratch slot; dq, dk per value head are summed per key head last.
constexpr int kGradSlots = 256;
struct GradLayout {
  size_t G, Tm, W, U, ddh, dh, hs, dqv, dkv, scratch, total;
};
GradLayout layout_grads(const gdn_shape &s) {
  const size_t BH = (size_t)s.B * s.H_v, N = chunks_of(s), C = s.chunk, DD = (size_t)D * D;
  const size_t units = BH * N;
  GradLayout L{};
  size_t off = 0;
  L.G = off;   off += align_up(BH * N * C * 4);
  L.Tm = off;  off += align_up(BH * N * C * C * 4);
  L.W = off;   off += align_up(BH * N * C * D * 4);
  L.U = off;   off += align_up(BH * N * C * D * 4);
  L.ddh = off; off += align_up(BH * N * DD * 4);
  L.dh = off;  off += align_up(BH * N * DD * 4);
  L.hs = off;  off += align_up(BH * N * DD * 4);
  if (s.H_v != s.H_qk) {
    L.dqv = off; off += align_up((size_t)s.B * s.T * s.H_v * D * 4);
    L.dkv = off; off += align_up((size_t)s.B * s.T * s.H_v * D * 4);
  }
  const size_t slots = std::min(units, (size_t)kGradSlots);
  const size_t slot = C == 128 ? grad_slot_floats<128>() : grad_slot_floats<64>();
  L.scratch = off; off += align_up(slots * slot * 4);
  L.total = off;
  return L;
}

template <int C, typename TI, int MODE>
gdn_status run_bwd_grads(const gdn_shape &s, const void *q, const void *k, const void *v, const float *g,
                         const float *beta, const float *h0, const float *dO, const float *dh_T, float *dq, float *dk,
                         float *dv, float *dg, float *dbeta, float *dh0, char *ws, hipStream_t st) {
  const GradLayout L = layout_grads(s);
  const int N = chunks_of(s);
  const bool rag = s.T % C != 0;
  FwdArgs a = base_args(s);
  a.k = k; a.v = v; a.g = g; a.beta = beta;
  a.G = reinterpret_cast<float *>(ws + L.G);
  a.Tm = reinterpret_cast<float *>(ws + L.Tm);
  a.W = ws + L.W;
  a.U = reinterpret_cast<float *>(ws + L.U);
  GDN_TRY((launch_prep<C, TI, MODE, false>(a, Lx{st})));
  const unsigned rowsBH = (unsigned)(s.B * s.H_v);
  StatesArgs sa{s.B, s.T, s.H_qk, s.H_v, N, k, a.G, reinterpret_cast<const float *>(a.W), a.U, h0,
                reinterpret_cast<float *>(ws + L.hs)};
  BwdArgs b{};
  b.B = s.B; b.T = s.T; b.Hqk = s.H_qk; b.Hv = s.H_v; b.N = N;
  b.q = q; b.k = k; b.dO = dO;
  b.G = a.G; b.W = reinterpret_cast<const float *>(a.W);
  b.ddh = reinterpret_cast<float *>(ws + L.ddh);
  b.dhT = dh_T; b.dh = reinterpret_cast<float *>(ws + L.dh); b.dh0 = dh0;
  const unsigned units = (unsigned)((long)N * s.B * s.H_v);
  // the reverse walk's chunk term, then both walks in one launch
  if (rag) {
    hipLaunchKernelGGL((bwd_ddh_kernel<C, TI, MODE, true>), dim3(units), dim3(ddh_threads<C>()), 0, st, a, b);
    hipLaunchKernelGGL((bwd_walks_kernel<C, TI, MODE, true>), dim3(2 * rowsBH), dim3(512), 0, st, sa, b);
  } else {
    hipLaunchKernelGGL((bwd_ddh_kernel<C, TI, MODE, false>), dim3(units), dim3(ddh_threads<C>()), 0, st, a, b);
    hipLaunchKernelGGL((bwd_walks_kernel<C, TI, MODE, false>), dim3(2 * rowsBH), dim3(512), 0, st, sa, b);
  }
  GDN_TRY(check_launch());
  const bool per_v = s.H_v != s.H_qk;
  GradArgs ga{};
  ga.B = s.B; ga.T = s.T; ga.Hqk = s.H_qk; ga.Hv = s.H_v; ga.N = N; ga.units = (int)units;
  ga.q = q; ga.k = k; ga.v = v; ga.beta = beta; ga.dO = dO;
  ga.G = a.G; ga.Tm = a.Tm; ga.W = reinterpret_cast<const float *>(a.W); ga.U = a.U;
  ga.hs = reinterpret_cast<const float *>(ws + L.hs); ga.dh = b.dh; ga.dhT = dh_T;
  ga.dq = per_v ? reinterpret_cast<float *>(ws + L.dqv) : dq;
  ga.dk = per_v ? reinterpret_cast<float *>(ws + L.dkv) : dk;
  ga.per_value_head = per_v;
  ga.dv = dv; ga.dg = dg; ga.dbeta = dbeta;
  ga.scratch = reinterpret_cast<float *>(ws + L.scratch);
  const unsigned grid = std::min(units, (unsigned)kGradSlots);
  if (rag)
    hipLaunchKernelGGL((bwd_chunk_kernel<C, TI, MODE, true>), dim3(grid), dim3(512), 0, st, ga);
  else
    hipLaunchKernelGGL((bwd_chunk_kernel<C, TI, MODE, false>), dim3(grid), dim3(512), 0, st, ga);
  GDN_TRY(check_launch());
  if (per_v) {
    const size_t rows = (size_t)s.B * s.T;
    hipLaunchKernelGGL(sum_value_heads_kernel, dim3(1024), dim3(256), 0, st, ga.dq, dq, rows, s.H_qk, s.H_v / s.H_qk);
    hipLaunchKernelGGL(sum_value_heads_kernel, dim3(1024), dim3(256), 0, st, ga.dk, dk, rows, s.H_qk, s.H_v / s.H_qk);
    GDN_TRY(check_launch());
  }
  return GDN_OK;
}

struct BwdGradCall {
  const gdn_shape &s; const void *q, *k, *v; const float *g, *beta, *h0, *dO, *dh_T;
  float *dq, *dk, *dv, *dg, *dbeta, *dh0; char *w; hipStream_t st;
  template <int C, typename TI, int MODE> gdn_status run() {
    return run_bwd_grads<C, TI, MODE>(s, q, k, v, g, beta, h0, dO, dh_T, dq, dk, dv, dg, dbeta, dh0, w, st);
  }
};

struct BwdStateCall {
  const gdn_shape &s; const void *q, *k; const float *g, *beta, *dO, *dh_T; float *dh, *dh0; char *w; hipStream_t st;
  template <int C, typename TI, int MODE> gdn_status run() {
    return run_bwd_state<C, TI, MODE>(s, q, k, g, beta, dO, dh_T, dh, dh0, w, st);
  }
};

}  // namespace

extern "C" {

gdn_status gdn_workspace_size_bwd(const gdn_shape *s, size_t *bytes) {
  if (!bytes) return GDN_ERR_NULL;
  GDN_TRY(gdn_validate(s));
  if (s->n_groups > 1) return GDN_ERR_SHAPE;
  *bytes = layout_bwd(*s).total;
  return GDN_OK;
}

gdn_status gdn_workspace_size_bwd_grads(const gdn_shape *s, size_t *bytes) {
  if (!bytes) return GDN_ERR_NULL;
  GDN_TRY(gdn_validate(s));
  if (s->n_groups > 1) return GDN_ERR_SHAPE;
  *bytes = layout_grads(*s).total;
  return GDN_OK;
}

gdn_status gdn_chunk_bwd(const gdn_shape *s, const void *q, const void *k, const void *v, const float *g,
                         const float *beta, const float *h0, const float *dO, const float *dh_T, float *dq,
                         float *dk, float *dv, float *dg, float *dbeta, float *dh0, void *ws, size_t ws_bytes,
                         void *hip_stream) {
  GDN_TRY(gdn_validate(s));
  if (s->n_groups > 1) return GDN_ERR_SHAPE;
  hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  for (const void *p : {(const void *)h0, (const void *)dh_T, (const void *)dh0})
    if (misaligned(p)) return GDN_ERR_ALIGN;
  if (s->T == 0) {   // no tokens: the cotangent of h0 is that of h_T
    if (!dh0) return GDN_OK;
    hipLaunchKernelGGL(copy_state_kernel, dim3(256), dim3(256), 0, st, dh_T, dh0, (size_t)s->B * s->H_v * D * D);
    return check_launch();
  }
  if (!q || !k || !v || !g || !beta || !dO || !dq || !dk || !dv || !dg || !dbeta || !ws) return GDN_ERR_NULL;
  for (const void *p : {(const void *)q, (const void *)k, (const void *)v, (const void *)g, (const void *)beta,
                        (const void *)dO, (const void *)dq, (const void *)dk, (const void *)dv, (const void *)dg,
                        (const void *)dbeta, (const void *)ws})
    if (misaligned(p)) return GDN_ERR_ALIGN;
  if (ws_bytes < layout_grads(*s).total) return GDN_ERR_WORKSPACE;
  BwdGradCall f{*s, q, k, v, g, beta, h0, dO, dh_T, dq, dk, dv, dg, dbeta, dh0, reinterpret_cast<char *>(ws), st};
  return dispatch(*s, f);
}

gdn_status gdn_chunk_bwd_state(const gdn_shape *s, const void *q, const void *k, const float *g,
                               const float *beta, const float *dO, const float *dh_T, float *dh_chunks,
                               float *dh0, void *ws, size_t ws_bytes, void *hip_stream) {
  GDN_TRY(gdn_validate(s));
  if (s->n_groups > 1) return GDN_ERR_SHAPE;
  if (!dh_chunks && !dh0) return GDN_ERR_NULL;
  hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  for (const void *p : {(const void *)dh_T, (const void *)dh_chunks, (const void *)dh0})
    if (misaligned(p)) return GDN_ERR_ALIGN;
  if (s->T == 0) {   // no chunks: the cotangent of h0 is that of h_T
    if (!dh0) return GDN_OK;
    hipLaunchKernelGGL(copy_state_kernel, dim3(256), dim3(256), 0, st, dh_T, dh0, (size_t)s->B * s->H_v * D * D);
    return check_launch();
  }
  if (!q || !k || !g || !beta || !dO || !ws) return GDN_ERR_NULL;
  for (const void *p : {(const void *)q, (const void *)k, (const void *)g, (const void *)beta, (const void *)dO,
                        (const void *)ws})
    if (misaligned(p)) return GDN_ERR_ALIGN;
  if (ws_bytes < layout_bwd(*s).total) return GDN_ERR_WORKSPACE;
  BwdStateCall f{*s, q, k, g, beta, dO, dh_T, dh_chunks, dh0, reinterpret_cast<char *>(ws), st};
  return dispatch(*s, f);
}

}  // extern "C"
