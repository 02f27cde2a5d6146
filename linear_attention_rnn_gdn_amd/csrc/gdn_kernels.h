// gdn_kernels.h -- device kernels of the GDN chunked forward (gfx950).
//
// Per value head h (bh = b*H_v + h), chunk n of C tokens, rows r = 0..C-1:
//   G_r = sum_{s<=r} g_s                                 decay cumsum
//   S_ri = beta_r e^{G_r-G_i} k_r.k_i  (i < r)           gated strict-lower beta K K^T
//   T = (I+S)^-1                                        UT transform (doubling ladder)
//   W = T diag(beta e^G) K,  U = T diag(beta) V          WY pair
//   V'_n = U_n - W_n h_n                                 corrected values
//   h_{n+1} = e^{G_last} h_n + K^T diag(e^{G_last-G}) V'_n   (= A h_n + B)
//   O_n = diag(e^G) Q h_n + (Q K^T o Gamma o [i<=r]) V'_n
// The affine step is the one of "Shard the GatedDeltaNet sequence under
// ici_context_parallelism" (PR description); the ladder is that of "Fuse the
// Gated Delta Net inter-chunk scan into a Pallas TPU kernel" (section
// "Changes").  w, u, k_g and S are not defined on those pages; the forms above
// are the reading under which the affine step equals the per-token rule.
//
// Kernels:
//   prep_kernel    one workgroup (8 waves) per (chunk, value head, batch):
//                  G, S, T, W, U, and K^T for the walk
//   walk_ring_kernel / walk_pair_kernel / walk_shared_kernel
//                  the sequential chunk walk over 16-column slices of the
//                  state, which stays in matrix-core result registers and
//                  feeds the next product directly.  The ring form (one slice
//                  per workgroup, its rows split over 2 or 4 waves) streams W
//                  and K^T through registers, for walks too few to fill the
//                  chip; the paired form (two such slices per workgroup)
//                  shares one LDS copy of them; the shared form (4 or 8
//                  slices per workgroup, one wave each) copies them once per
//                  workgroup into LDS.  Modes: WALK (state = h, writes
//                  chunk-start states and V') and FOLD (state = the augmented
//                  [A | B] of a group, started from [I | 0]; writes the
//                  group's pair).
//   prefix_kernel  one workgroup per (column slice, bh): exclusive prefix of
//                  the groups' affine pairs.
//   out_kernel     one 4-wave workgroup per (chunk, bh): the output, with
//                  P^T formed once per chunk into LDS between its products.
//   walk_out_kernel  the walk that also forms the outputs (many walks): four
//                  waves per workgroup, one or two 16-column slices per wave.
//
// Workspace tensors (cb = bh*N + n indexes a chunk of a value head).  The
// tensors that pass from one kernel to the next are stored fragment-major: in
// the order in which the consumer's lanes read them, so that each 16-byte
// per-lane load or store of a wave covers 1 KB of consecutive bytes.
// (Row-major tiles read in matrix-core operand layout put consecutive lanes
// on different rows, and each such instruction breaks into dozens of memory
// requests.)  Lane l = lr + 16 g (lr = l % 16, g = l / 16); a fragment's 8
// k-values for lane group g are kk(g, j) = 4g + j (j < 4), 16 + 4g + j - 4
// (j >= 4) within its block of 32 (the order of two stacked result tiles).
//   G   [cb][C] fp32 decay cumsum
//   Wf  [cb][C/16][D/32][64][8]  W[16m + lr][32kb + kk(g, j)], input dtype
//   Ktf [cq][D/16][C/32][64][8]  K[32kb + kk(g, j)][16m + lr], input dtype,
//       once per query/key head (cq = (b*H_qk + hq)*N + n): the value heads
//       that share a key head share its K^T
//   Uf  [cb][C/16][D/16][64][4]  U[16m + 4g + i][16nd + lr], fp32
//   Hsf [cb][D/16][D/16][64][4]  chunk-start state h[16m + 4g + i][16s + lr]
//   Vnf [cb][D/16][C/16][64][4]  corrected values V'[16m + 4g + i][16s + lr]
// (s = the 16-column slice.)  Hsf and Vnf are fp32 for fp32 inputs.  For bf16
// inputs they hold operand fragments -- element j of lane l from tile 2p + j/4,
// row 4g + j%4 -- as a bf16 high and a bf16 low plane, [cb][D/16][rows/32][2][64][8].  Decays are evaluated as exp2 of log2-scaled
// cumsums (one v_exp_f32 each).
//
// Workgroups are numbered 1-D.  The hardware places workgroup i on XCD i % 8;
// xcd_unit() hands all column slices of one (head, chunk or job) to one XCD
// so they share that XCD's L2 for the operands they all read.
#pragma once
#include <type_traits>

#include "gdn_mfma.h"

namespace gdn {

constexpr int D = 128;        // d_k = d_v
constexpr int NT = 256;       // threads per workgroup
// walk kinds: WALK (the state h from h0; hands h and V' to the output stage),
// FOLD (the augmented state [A | B] of a group from [I | 0]: the group's
// pair), WALK_A (the augmented state [A | h] from [I | h0]: a walk that also
// yields the affine map A of the whole sequence, with h as in WALK)
constexpr int WALK = 0, FOLD = 1, WALK_A = 2;

template <typename TI> struct LdPad { static constexpr int v = 8; };
template <> struct LdPad<float> { static constexpr int v = 4; };

// Forms of a tensor handed from the walk to the output stage.
enum : int { ST_F32 = 0, ST_SPLIT = 1, ST_BF16 = 2 };

// Product precision per input precision: MODE_BF16 (bf16 q/k/v) or MODE_F32.
constexpr int MODE_BF16 = 0, MODE_F32 = 1;
template <int MODE> struct Prec {
  static constexpr int exact = MODE == MODE_F32 ? P_F32 : P_BF16;       // bf16 data x bf16 data
  static constexpr int ladder = MODE == MODE_F32 ? P_F32 : P_SPLIT_AB;  // fp32 x fp32 (bf16 inputs: as hi/lo bf16 pairs)
  static constexpr int wy = MODE == MODE_F32 ? P_F32 : P_SPLIT_A;       // T' (fp32) x K/V (data)
  static constexpr int wh = MODE == MODE_F32 ? P_F32 : P_BF16;          // W x h
  static constexpr int kv = MODE == MODE_F32 ? P_F32 : P_SPLIT_B;       // K^T (data) x V'
  static constexpr int hq = MODE == MODE_F32 ? P_F32 : P_SPLIT_A;       // h^T x Q^T (data)
  static constexpr int pv = MODE == MODE_F32 ? P_F32 : P_SPLIT_AB;      // V'^T x P^T
  // How h and V' are handed to the output stage (the walk keeps its state in
  // fp32; only these copies are rounded).  For bf16 inputs both go as hi/lo
  // bf16 planes: one bf16 rounding of V' (several times larger than the output
  // it feeds: the masked intra-chunk product cancels) costs about 2% of RMS(o)
  // at the max, one of h about 1%.
  static constexpr int h_store = MODE == MODE_F32 ? ST_F32 : ST_SPLIT;
  static constexpr int v_store = MODE == MODE_F32 ? ST_F32 : ST_SPLIT;
};

// 1-D workgroup index -> (unit, part) with the `parts` workgroups of a unit on
// one XCD (falls back to unit-major order when units is not a multiple of 8).
__device__ __forceinline__ void xcd_unit(int L, int parts, int units, int &unit, int &part) {
  if ((units & 7) == 0) {
    const int x = L & 7, i = L >> 3;
    unit = (i / parts) * 8 + x;
    part = i % parts;
  } else {
    unit = L / parts;
    part = L % parts;
  }
}

// Store a wave's column of result tiles (rows 16m + 4g + i, column lr) for the
// output stage, at `dst` (this chunk's and slice's part of the tensor).  bf16
// forms: per pair of tiles (2p, 2p+1) the operand fragment the output stage
// reads -- 8 values per lane in the order {tile 2p rows 4g..4g+3, tile 2p+1
// rows 4g..4g+3} -- rounded to bf16 (1 KB per pair), or as a bf16 high plane
// and a bf16 low plane (the rounding remainder; 1 KB each).  fp32 form: one
// 1 KB block per tile.
template <int ST> struct Store {
  static constexpr int tile_floats = ST == ST_BF16 ? 128 : 256;   // per 16x16 tile
  static constexpr int loads = ST == ST_BF16 ? 1 : 2;             // 16-byte loads per fragment
  static constexpr int frag = ST == ST_F32 ? F_F32 : ST == ST_SPLIT ? F_SPLIT : F_BF16;
};
template <int ST, int NTILE>
__device__ __forceinline__ void store_result_tiles(float *dst, const f32x4 (&t)[NTILE], int lane) {
  if constexpr (ST != ST_F32) {
    char *d = reinterpret_cast<char *>(dst);
#pragma unroll
    for (int p = 0; p < NTILE / 2; ++p) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = t[2 * p + j / 4][j % 4];
      bf16x8 hi, lo;
      if constexpr (ST == ST_BF16) hi = to_bf16x8(x);
      else to_bf16x8_split(x, hi, lo);
      if constexpr (ST == ST_BF16) {
        st16_stream(d + p * 1024 + lane * 16, hi);
      } else {
        st16_stream(d + (2 * p) * 1024 + lane * 16, hi);
        st16_stream(d + (2 * p + 1) * 1024 + lane * 16, lo);
      }
    }
  } else {
#pragma unroll
    for (int m = 0; m < NTILE; ++m)
      st16_stream(dst + (m * 64 + lane) * 4, t[m]);
  }
}

constexpr float LOG2E = 1.4426950408889634f;
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

struct FwdArgs {
  int B, T, Hqk, Hv, N;           // N = ceil(T / C) chunks per sequence row (packed: the table capacity)
  const void *q, *k, *v;
  const float *g, *beta;
  float *G, *U, *Tm;              // prep outputs (Tm optional); U is U^T on the forward path
  void *W;                        // prep output, input dtype (fp32 for the transform hook)
  void *Kt;                       // prep output / walk input: K^T per chunk, input dtype
  float *Hs, *Vn;                 // walk outputs (optional) / out inputs
  const float *init;              // walk: initial states (h0 [BH,D,D] or h_in [BH,J,D,D]) or null
  int init_per_job;               // init indexed by job (replay) instead of bh only
  float *fin;                     // walk: final state per bh (h_T), written by the last job, or null
  float *pairA, *pairB;           // fold outputs [BH,J,D,D]
  int jobs, cpj;                  // walk/fold: jobs per bh, chunks per job
  int n0, nn;                     // chunk range [n0, n0 + nn) of this launch (prep, out, single walk)
  void *o;                        // out output
  // packed variable-length sequences (null otherwise): per chunk (first
  // token, tokens), per sequence (first chunk, chunks), number of chunks
  const int2 *ctab, *jtab;
  const int *ntot;
};

// Offset from a value head's chunk index cb = bh*N + n to the chunk index of
// its query/key head, cq = (b*H_qk + hq)*N + n (K^T is stored per key head).
// A wave-uniform 64-bit value moved to scalar registers (so that address
// arithmetic derived from it stays on the scalar unit).
__device__ __forceinline__ unsigned long long uniform64(unsigned long long x) {
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)x);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(x >> 32));
  return ((unsigned long long)hi << 32) | lo;
}

__device__ __forceinline__ long long kt_offset(const FwdArgs &a, size_t bh) {
  const size_t b = bh / a.Hv, hv = bh % a.Hv, hq = hv / (a.Hv / a.Hqk);
  return ((long long)(b * a.Hqk + hq) - (long long)bh) * a.N;
}

// 1-D workgroup index of the per-chunk kernels (prep, out) -> (chunk n,
// batch row b, value head hv), heads fastest.  The workgroups resident at one
// time then cover every head of a few chunks: together they read whole token
// rows of q, k and v (one head's part of a row is only a few hundred bytes)
// and write whole rows of o.  The value heads that share a qk head land on one
// XCD next to each other and share its L2 for that head's q and k.
__device__ __forceinline__ void chunk_head_unit(int L, const FwdArgs &a, int &n, int &b, int &hv) {
  const int grp = a.Hv / a.Hqk;
  int unit, part;
  xcd_unit(L, grp, a.nn * a.B * a.Hqk, unit, part);
  const int hq = unit % a.Hqk, rest = unit / a.Hqk;
  b = rest % a.B;
  n = a.n0 + rest / a.B;
  hv = hq * grp + part;
}

// 1-D workgroup index of the walks -> (walk bh, its job, the workgroup's
// share grp of it, of NG), with the shares of the value heads that share a qk
// head on one XCD next to each other (as the per-chunk kernels place them):
// chunk by chunk they read the same K^T (and, in the walk with outputs, the
// same q and k rows) and share them in that XCD's L2.
__device__ __forceinline__ void walk_unit(int L, int NG, const FwdArgs &a, size_t &bh, int &job, int &grp) {
  const int R = a.Hv / a.Hqk;
  int unit, part;
  xcd_unit(L, NG * R, a.B * a.Hqk * a.jobs, unit, part);
  grp = part % NG;
  job = unit % a.jobs;
  const int bq = unit / a.jobs;   // b * Hqk + hq
  bh = (size_t)(bq / a.Hqk) * a.Hv + (size_t)(bq % a.Hqk) * R + part / NG;
}

// ----------------------------------------------------------------------------
// prep: decay cumsum, S, T (ladder), W, U for one chunk of one value head.
// FWD: the forward path's layouts (W in the input dtype, fragment-major W,
// K^T and U); otherwise the transform hook's (W and U fp32 row-major).
//
// LDS (about 78 KB at C = 128, so two workgroups share a compute unit):
//   sX  one C x D input tile at a time: K row-major (for S), the ladder's
//       scratch, then K^T and V^T (for W and U)
//   sT  S, then T, in packed lower-triangular form (Tri)
// Each thread loads one 8-row block of K and of V into registers at the
// start; the row-major copy of K feeds S, and the same registers are
// transposed in place for the K^T and V^T copies, so K and V are read from
// memory once.

// Packed lower-triangular C x C matrix: row tile m (16 rows) keeps its first
// len(m) = 32 (m/2 + 1) columns -- its part of the lower triangle rounded up
// to whole k-blocks of 32, zero-filled above the diagonal -- with rows padded
// by 4 floats against bank conflicts.
template <int C> struct Tri {
  static constexpr int size = 512 * ((C / 32) * (C / 32 + 1)) + 64 * (C / 16);
  __device__ static int len(int m) { return 32 * (m / 2 + 1); }
  __device__ static int base(int m) {
    const int h = m >> 1;
    return 512 * ((m & 1) ? (h + 1) * (h + 1) : h * (h + 1)) + 64 * m;
  }
  __device__ static int at(int r, int c) {
    const int m = r >> 4;
    return base(m) + (r & 15) * (len(m) + 4) + c;
  }
  // row rr (0..15) of row tile m, column c; m usually wave-uniform
  __device__ static int at_t(int m, int rr, int c) { return base(m) + rr * (len(m) + 4) + c; }
};

// Transposed input tile X^T [D][C] in LDS, unpadded.  The 16-byte blocks of
// row d are XOR-swizzled by (d ^ d/8): the transposing stores (rows 8 apart)
// and the operand reads (16 consecutive rows) then both spread over all banks.
template <int C, typename TI> struct XT {
  static constexpr int VE = 16 / (int)sizeof(TI);   // elements per 16-byte block
  static constexpr int NB = C / VE;                  // blocks per row
  __device__ static int swz(int d) { return (d ^ (d >> 3)) & (NB - 1); }
  __device__ static int at(int d, int k) {           // k a multiple of VE
    return d * C + (((k / VE) ^ swz(d)) * VE);
  }
  __device__ static int at(int d, int k, int sw) { return d * C + (((k / VE) ^ sw) * VE); }
};

// One thread's block of the input tile: rows 8 rb .. 8 rb + 7, columns
// VE cb .. VE cb + VE - 1, as 8 row vectors of 16 bytes.
template <int C, typename TI, int NTH> struct TileBlock {   // NTH threads share the tile; tix = 0..NTH-1
  static constexpr int VE = 16 / (int)sizeof(TI);
  static constexpr int NCB = D / VE, NBLK = (C / 8) * NCB;
  static constexpr int PER = (NBLK + NTH - 1) / NTH;   // blocks per thread
  uint4 v[PER][8];
  // rows at or past `rows` (the padding of a partial last chunk) are zero
  __device__ void load(int tix, const TI *src, size_t gstride, int rows) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int blk = tix + p * NTH, rb = blk / NCB, cb = blk % NCB;
      if (blk < NBLK) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          v[p][j] = 8 * rb + j < rows ? *reinterpret_cast<const uint4 *>(src + (size_t)(8 * rb + j) * gstride + VE * cb)
                                      : uint4{0u, 0u, 0u, 0u};
      }
    }
  }
  // row-major copy [C][ld]
  __device__ void put_rows(int tix, TI *dst, int ld) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int blk = tix + p * NTH, rb = blk / NCB, cb = blk % NCB;
      if (blk < NBLK) {
#pragma unroll
        for (int j = 0; j < 8; ++j) *reinterpret_cast<uint4 *>(dst + (8 * rb + j) * ld + VE * cb) = v[p][j];
      }
    }
  }
  // transposed copy X^T (XT layout): column VE cb + e becomes row d, and the
  // block's 8 rows its 8 consecutive k-values.  transpose() forms the 16-byte
  // pieces in registers, put_transposed() stores them: a thread that keeps
  // its block for a later copy holds it in one form only.
  using Words = uint4[PER][8];
  __device__ void transpose(Words &w) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      if constexpr (sizeof(TI) == 2) {
        // 8 x 8 transpose of 16-bit values: output dword q of column e packs
        // rows 2q (low half) and 2q + 1 (high half)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          uint32_t x[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t lo = (&v[p][2 * q].x)[e >> 1], hi = (&v[p][2 * q + 1].x)[e >> 1];
            // one byte permute: bytes {0,1} (even e) or {2,3} (odd e) of lo, then of hi
            x[q] = __builtin_amdgcn_perm(hi, lo, (e & 1) ? 0x07060302u : 0x05040100u);
          }
          w[p][e] = uint4{x[0], x[1], x[2], x[3]};
        }
      } else {
        // 8 x 4 of 32-bit values: column e = two 16-byte halves of 4 rows
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
            w[p][2 * e + hh] = uint4{(&v[p][4 * hh].x)[e], (&v[p][4 * hh + 1].x)[e], (&v[p][4 * hh + 2].x)[e],
                                     (&v[p][4 * hh + 3].x)[e]};
      }
    }
  }
  __device__ static void put_transposed(int tix, TI *dst, const Words &w) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int blk = tix + p * NTH, rb = blk / NCB, cb = blk % NCB;
      if (blk >= NBLK) continue;
      if constexpr (sizeof(TI) == 2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) *reinterpret_cast<uint4 *>(dst + XT<C, TI>::at(8 * cb + e, 8 * rb)) = w[p][e];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
            *reinterpret_cast<uint4 *>(dst + XT<C, TI>::at(4 * cb + e, 8 * rb + 4 * hh)) = w[p][2 * e + hh];
      }
    }
  }
};

// operand fragment of X^T: row d, k-values k0 .. k0 + 7
template <int K, int C, typename TI>
__device__ __forceinline__ Frag<K> xt_frag(const TI *sxt, int d, int k0, int sw) {
  if constexpr (sizeof(TI) == 2) {
    const bf16x8 u = *reinterpret_cast<const bf16x8 *>(sxt + XT<C, TI>::at(d, k0, sw));
    if constexpr (K == F_BF16) {
      Frag<K> f;
      f.hi = u;
      return f;
    } else {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = (float)u[j];
      return make_frag<K>(x);
    }
  } else {
    const float4 u0 = *reinterpret_cast<const float4 *>(sxt + XT<C, TI>::at(d, k0, sw));
    const float4 u1 = *reinterpret_cast<const float4 *>(sxt + XT<C, TI>::at(d, k0 + 4, sw));
    float x[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
    return make_frag<K>(x);
  }
}

// One level (block size BS) of the doubling ladder of step (5) below, fully
// unrolled: for each 2BS diagonal block [[P,0],[L,Q]] of the packed T, the
// lower-left block becomes -X_Q L X_P.  Tiles are shared out over the PW
// waves; k-blocks that the triangular factors make zero are skipped, not
// multiplied as zeros.  sM holds M1 = L X_P transposed (nb blocks of
// BS x (BS+4)).
template <int C, int BS, int PL, int PW>
__device__ __forceinline__ void ladder_level(float *sT, float *sM, int wave, int lane) {
  using TRI = Tri<C>;
  constexpr int NB = C / (2 * BS), TB = BS / 16, NTILE = NB * TB * TB, PER = (NTILE + PW - 1) / PW;
  constexpr int LDM = BS + 4, KBM = (BS + 31) / 32;
  const int lr = lane & 15, lk = (lane >> 4) * 8, lq = (lane >> 4) * 4;
  // k-values past a 16-wide block (lane groups 2 and 3) enter as zeros
  const bool kin = BS >= 32 || lk < BS;
  // M1 = L X_P (stored transposed in sM).  X_P is lower triangular: the
  // k-blocks above column tile ni's diagonal are skipped (a uniform branch).
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int tt = wave + PW * u;
    if (tt >= NTILE) break;
    const int blk = tt / (TB * TB), ti = tt % (TB * TB), mi = ti / TB, ni = ti % TB;
    const int s = blk * 2 * BS, kb0 = (16 * ni) / 32;
    f32x4 acc = zero4();
#pragma unroll
    for (int kb = 0; kb < KBM; ++kb) {
      if (kb < kb0) continue;
      const int k0 = 32 * kb + lk;
      float a8[8], b8[8];
      if (kin) {
        ld8(sT + TRI::at_t((s + BS) / 16 + mi, lr, s + k0), a8);
        // column s + 16 ni + lr of X_P, rows s + k0 .. + 7 (one row tile)
        const int mk = (s + 32 * kb) / 16 + (lane >> 5);
        const float *col = sT + TRI::at_t(mk, lk & 15, s + 16 * ni + lr);
        const int str = TRI::len(mk) + 4;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) b8[jj] = col[jj * str];
      } else {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) a8[jj] = b8[jj] = 0.f;
      }
      mma_k32<PL>(acc, a8, b8);
    }
    float *M = sM + blk * BS * LDM;
    *reinterpret_cast<float4 *>(M + (16 * ni + lr) * LDM + 16 * mi + lq) = float4{acc[0], acc[1], acc[2], acc[3]};
  }
  lds_barrier();
  // L <- -X_Q M1.  X_Q is lower triangular: row tile mi needs k < 16(mi+1).
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int tt = wave + PW * u;
    if (tt >= NTILE) break;
    const int blk = tt / (TB * TB), ti = tt % (TB * TB), mi = ti / TB, ni = ti % TB;
    const int s = blk * 2 * BS;
    const float *M = sM + blk * BS * LDM;
    f32x4 acc = zero4();
#pragma unroll
    for (int kb = 0; kb < KBM; ++kb) {
      if (kb * 32 >= 16 * (mi + 1)) continue;
      const int k0 = 32 * kb + lk;
      float a8[8], b8[8];
      if (kin) {
        ld8(sT + TRI::at_t((s + BS) / 16 + mi, lr, s + BS + k0), a8);
        ld8(M + (16 * ni + lr) * LDM + k0, b8);
      } else {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) a8[jj] = b8[jj] = 0.f;
      }
      mma_k32<PL>(acc, a8, b8);
    }
    const int mr = (s + BS) / 16 + mi;
    float *rp = sT + TRI::at_t(mr, lq, s + 16 * ni + lr);
    const int rstr = TRI::len(mr) + 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) rp[i * rstr] = -acc[i];
  }
  lds_barrier();
}

constexpr int PW = 8, PNT = 64 * PW;   // prep: waves, threads per workgroup

// RAG: T is not a multiple of C (the last chunk is partial); otherwise every
// chunk is whole and the row masks below fold away.
template <int C, typename TI, int MODE, bool FWD, bool RAG>
__global__ __launch_bounds__(PNT, 4) void prep_kernel(FwdArgs a) {   // two workgroups per CU
  using WT = typename std::conditional<FWD, TI, float>::type;
  using PR = Prec<MODE>;
  using TRI = Tri<C>;
  constexpr int LDI = D + LdPad<TI>::v;   // row-major input tile leading dim
  constexpr int XBYTES_ROWS = C * LDI * (int)sizeof(TI);
  constexpr int XBYTES_T = D * C * (int)sizeof(TI);
  constexpr int XBYTES_M = (C / 2) * (C / 2 + 4) * 4;   // ladder scratch: nb * b * (b+4) <= C/2*(C/2+4)
  constexpr int XBYTES = XBYTES_ROWS > XBYTES_T ? (XBYTES_ROWS > XBYTES_M ? XBYTES_ROWS : XBYTES_M)
                                                : (XBYTES_T > XBYTES_M ? XBYTES_T : XBYTES_M);
  __shared__ __align__(16) char sXraw[XBYTES];
  __shared__ __align__(16) float sT[TRI::size];
  __shared__ __align__(16) float sG[C], sG2[C], sBeta[C], sScale[C];
  __shared__ float sWt[2];
  TI *sX = reinterpret_cast<TI *>(sXraw);
  float *sM = reinterpret_cast<float *>(sXraw);

  int n, b, hv;
  chunk_head_unit(blockIdx.x, a, n, b, hv);
  const int hq = hv / (a.Hv / a.Hqk);
  // (the wave index as a scalar: tests on a wave's row tiles are uniform branches)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, g = lane >> 4, lk = g * 8, lq = g * 4;
  const size_t bh = (size_t)b * a.Hv + hv;
  // packed sequences (launched with the RAG instantiation only): chunk n of
  // the table (past the last one: nothing to do)
  const bool packed = RAG && a.ctab;
  if (packed && n >= *a.ntot) return;
  const size_t t0 = packed ? (size_t)a.ctab[n].x : (size_t)n * C;
  const size_t cb = bh * a.N + n;  // chunk index into the workspace
  // tokens of this chunk; a partial last chunk is padded with identity steps
  // (k = v = 0, g = 0, beta = 0): their rows of S are zero, their rows of T
  // unit rows, their W, U (and so V') rows exactly zero, and G carries the
  // last real token's cumsum, so the walk and the outputs of the real tokens
  // are those of the unpadded sequence
  const int rows = !RAG ? C : packed ? a.ctab[n].y : (int)(a.T - t0 < (size_t)C ? a.T - t0 : (size_t)C);

  // g and beta first, from the row clamped into the chunk and then selected:
  // read before the tiles, they can be waited for while the tiles are still
  // in flight (behind a branch, or after the tiles, the cumsum waited for
  // everything)
  float g_in, b_in;
  {
    const size_t si = ((size_t)b * a.T + t0 + (tid < rows ? tid : rows - 1)) * a.Hv + hv;
    const float gx = a.g[si], bx = a.beta[si];
    g_in = tid < rows ? gx : 0.f;
    b_in = tid < rows ? bx : 0.f;
  }

  // The first half of the workgroup holds the K tile in registers, the second
  // half the V tile, one 8-row block per thread (kept for the transposed
  // copies, so K and V are read from memory once).
  const bool vhalf = wave >= PW / 2;
  const int tix = tid & (PNT / 2 - 1);
  TileBlock<C, TI, PNT / 2> xt;
  if (!vhalf)
    xt.load(tix, reinterpret_cast<const TI *>(a.k) + (((size_t)b * a.T + t0) * a.Hqk + hq) * D, (size_t)a.Hqk * D, rows);
  else if (FWD || a.U)
    xt.load(tix, reinterpret_cast<const TI *>(a.v) + (((size_t)b * a.T + t0) * a.Hv + hv) * D, (size_t)a.Hv * D, rows);
  else
    xt.load(tix, nullptr, 0, 0);   // (the transform hook without U reads no values: zero rows)

  // (1) decay cumsum over the chunk (inclusive), beta
  {
    float x = g_in;
    const float bx = b_in;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (lane == 63 && wave < 2) sWt[wave] = x;
    lds_barrier();
    if (wave == 1) x += sWt[0];
    if (tid < C) {
      sG[tid] = x;
      sG2[tid] = x * LOG2E;
      sBeta[tid] = bx;
      sScale[tid] = bx * exp2_fast(x * LOG2E);
    }
  }
  // (2) K row-major -> LDS; from here on each thread keeps its block in
  // transposed form only
  if (!vhalf) xt.put_rows(tix, sX, LDI);
  typename TileBlock<C, TI, PNT / 2>::Words xw;
  xt.transpose(xw);
  lds_barrier();

  // Work split for the products of (3), (6), (7): row tiles are taken in
  // pairs {j, TC-1-j} (equal shares of the triangle), group j = wave % NGR,
  // and the WPG waves of a group split the pair's column tiles.
  constexpr int TC = C / 16;
  constexpr int NGR = TC / 2, WPG = PW / NGR;
  static_assert(PW % NGR == 0 && TC % WPG == 0, "whole column shares");
  constexpr int RU = 2;   // row tiles per wave
  const int grp = wave % NGR, sub = wave / NGR;
  const int mrow[RU] = {grp, TC - 1 - grp};

  // (3) S = strict-lower( beta_r e^{G_r - G_i} K K^T ) into packed sT.  A
  //     wave takes the column tiles ni = sub + WPG c of its two row tiles;
  //     each k-block's column fragment feeds both.
  {
    using PK = PolicyKinds<PR::exact>;
    constexpr int NC = TC / WPG;
    f32x4 acc[RU][NC];
#pragma unroll
    for (int u = 0; u < RU; ++u)
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[u][c] = zero4();
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) {
      Frag<PK::a> af[RU];
#pragma unroll
      for (int u = 0; u < RU; ++u) af[u] = lds_frag<PK::a>(sX + (16 * mrow[u] + lr) * LDI + 32 * kb + lk);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int ni = sub + WPG * c;
        if (ni > mrow[1]) continue;
        const auto bf = lds_frag<PK::b>(sX + (16 * ni + lr) * LDI + 32 * kb + lk);
#pragma unroll
        for (int u = 0; u < RU; ++u)
          if (ni <= mrow[u]) mma(acc[u][c], af[u], bf);
      }
    }
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      // per-row terms once (this lane's rows r = 16m + lq + i), then per column
      const int m = mrow[u], L = TRI::len(m);
      const float4 br = *reinterpret_cast<const float4 *>(sBeta + 16 * m + lq);
      const float4 gr = *reinterpret_cast<const float4 *>(sG2 + 16 * m + lq);
      const float brv[4] = {br.x, br.y, br.z, br.w}, grv[4] = {gr.x, gr.y, gr.z, gr.w};
      float *rowp = sT + TRI::at(16 * m + lq, lr);   // row 16m + lq, column lr
      const int rstr = L + 4;                         // row stride of this row tile
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        const int ni = sub + WPG * cc;
        if (16 * ni < L) {   // the row tile's stored columns (zeros past the diagonal)
          const int c = 16 * ni + lr;
          const float gc = sG2[c];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * m + lq + i;
            rowp[i * rstr + 16 * ni] = (c < r) ? brv[i] * exp2_fast(grv[i] - gc) * acc[u][cc][i] : 0.f;
          }
        }
      }
    }
  }
  lds_barrier();

  // (4) exact inverses of the 16x16 diagonal blocks (forward substitution,
  //     one thread per block column)
  {
    float x[16];
    const int blk = tid >> 4, j = tid & 15;
    if (tid < C) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float *Srow = sT + TRI::at(16 * blk + r, 16 * blk);
        float v = (r == j) ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < r; ++i) v -= Srow[i] * x[i];
        x[r] = v;
      }
    }
    lds_barrier();
    if (tid < C) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sT[TRI::at(16 * blk + r, 16 * blk + j)] = x[r];
    }
    lds_barrier();
  }

  // (5) doubling ladder: for each 2b diagonal block [[P,0],[L,Q]] the new
  //     lower-left block is -X_Q L X_P (X_P, X_Q the current inverses).
  //     The row-major K tile is dead; its space holds the scratch sM.
  ladder_level<C, 16, PR::ladder, PW>(sT, sM, wave, lane);
  ladder_level<C, 32, PR::ladder, PW>(sT, sM, wave, lane);
  if constexpr (C > 64) ladder_level<C, 64, PR::ladder, PW>(sT, sM, wave, lane);
  static_assert(C == 64 || C == 128, "ladder levels for C = 64 and 128");

  // K^T -> LDS from the registers
  if (!vhalf) TileBlock<C, TI, PNT / 2>::put_transposed(tix, sX, xw);
  // G (and T in the transform form) stored after the transposition: stored
  // before it, they were waited for together with the K tile's loads, which
  // the compiler counts with them where the two halves' paths join
  if (a.Tm) {
    float *Tg = a.Tm + cb * C * C;
    for (int idx = tid; idx < C * C; idx += PNT) {
      const int r = idx / C, c = idx % C;
      Tg[idx] = c < TRI::len(r >> 4) ? sT[TRI::at(r, c)] : 0.f;
    }
  }
  if (tid < C) a.G[cb * C + tid] = sG[tid];
  lds_barrier();
  // (written by the first value head of each key head only)
  if (FWD && hv % (a.Hv / a.Hqk) == 0) {
    // K^T fragments for the walk, fragment-major: (d tile m, k-block kb, lane)
    // holds K[r][16 m + lr] for the 8 tokens r = 32 kb + {4g..4g+3,
    // 16+4g..16+4g+3} (the k order of the walk's register-chained operand);
    // one contiguous 1 KB per wave store
    // fragment f = wave + PW i (i-th store of this wave): d tile m = f / KBC,
    // k-block kb = f % KBC
    constexpr int KBC = C / 32, NF = D * C / 8 / 64;   // fragments (1 KB each)
    static_assert(NF % PW == 0, "whole fragments per wave");
    const size_t cq = ((size_t)b * a.Hqk + hq) * a.N + n;   // chunk of the key head
    TI *Ktg = reinterpret_cast<TI *>(a.Kt) + cq * D * C + lane * 8;
    constexpr int VE = 16 / sizeof(TI);
#pragma unroll
    for (int i = 0; i < NF / PW; ++i) {
      const int f = wave + PW * i, m = f / KBC, kb = f % KBC;
      const int d = 16 * m + lr;
      const int sw = XT<C, TI>::swz(d);
      TI tmp[8];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int k = 32 * kb + 16 * hh + 4 * g;   // 4 consecutive tokens
        const TI *src = sX + XT<C, TI>::at(d, k - k % VE, sw) + k % VE;
        if constexpr (sizeof(TI) == 2) *reinterpret_cast<uint2 *>(tmp + 4 * hh) = *reinterpret_cast<const uint2 *>(src);
        else *reinterpret_cast<uint4 *>(tmp + 4 * hh) = *reinterpret_cast<const uint4 *>(src);
      }
#pragma unroll
      for (int v = 0; v < 8 / VE; ++v) st16(Ktg + f * 512 + v * VE, *reinterpret_cast<const uint4 *>(tmp + v * VE));
    }
  }

  // (6) W = (T diag(beta e^G)) K, computed transposed (W^T = K^T T'^T) so
  //     that each lane ends with 4 consecutive columns of one row of W.
  // (7) U = (T diag(beta)) V, computed as is, so that each lane ends with 4
  //     consecutive rows of one column of U (= 4 consecutive entries of U^T).
  // A wave takes row tiles of its pair and d tiles md0 .. md0 + TDW - 1 (see
  // below); T is lower triangular, so row tile m needs k < 16(m+1).  The T fragments of
  // k-blocks past the diagonal read T's zero-filled or neighbouring entries
  // and their products are skipped.
  // At C = 128 (two waves per row-tile pair) each wave takes one row tile of
  // the pair, mrow[sub], for all d tiles: every T' fragment is then split
  // once per pass instead of once per wave of the pair (the split is most of
  // this phase's vector-ALU work, which bounds the kernel; the longer matrix
  // chain of the pair's larger tile costs less: 1 us less per launch at the
  // 4096-token layer).  At C = 64 (four waves per pair) the d tiles are split.
  constexpr bool ONE = C == 128;
  constexpr int TD = D / 16, TDW = ONE ? TD : TD / WPG;
  static_assert(TD % WPG == 0 && TDW % 2 == 0, "W fragments pair d tiles");
  static_assert(!ONE || WPG == RU, "one row tile of the pair per wave");
  const int md0 = ONE ? 0 : sub * TDW;
  // swizzle term of this lane's X^T rows 16md + lr
  int xsw[TDW];
#pragma unroll
  for (int mdl = 0; mdl < TDW; ++mdl) xsw[mdl] = XT<C, TI>::swz(16 * (md0 + mdl) + lr);
  constexpr int KT = PolicyKinds<PR::wy>::a;   // T' fragments (split)
  constexpr int KX = PolicyKinds<PR::wy>::b;   // K / V fragments (exact data)
  // (one body per pass, the pass a compile-time constant: a runtime choice of
  // the operand order inside the k loop merges the two MFMA sequences'
  // accumulators through register copies on every iteration)
  auto wu_pass = [&](auto pass_c) {
    constexpr int pass = decltype(pass_c)::value;
    const float *scale = pass == 0 ? sScale : sBeta;
    // one row tile at a time (registers: the other half of the workgroup
    // still holds its V block)
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      if (ONE && u != sub) continue;
      f32x4 acc[TDW];
#pragma unroll
      for (int md = 0; md < TDW; ++md) acc[md] = zero4();
      // (k-blocks not unrolled: unrolled, their operand loads are hoisted
      // ahead and the registers run out)
#pragma unroll 1
      for (int kb = 0; kb < C / 32; ++kb) {
        if (32 * kb >= 16 * (mrow[u] + 1)) break;   // T is zero from here
        const int k0 = 32 * kb + lk;
        Frag<KT> tf;
        {
          float x[8], sc[8];
          ld8(sT + TRI::at(16 * mrow[u] + lr, k0), x);
          ld8(scale + k0, sc);
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] *= sc[j];
          tf = make_frag<KT>(x);
        }
#pragma unroll
        for (int mdl = 0; mdl < TDW; ++mdl) {
          // X^T row 16md+lr = column of K (or V)
          const auto xf = xt_frag<KX, C, TI>(sX, 16 * (md0 + mdl) + lr, k0, xsw[mdl]);
          if constexpr (pass == 0) mma(acc[mdl], xf, tf);   // W^T tile (d, r)
          else mma(acc[mdl], tf, xf);                       // U tile (r, d)
        }
      }
#pragma unroll
      for (int mdl = 0; mdl < TDW; ++mdl) {
        const int md = md0 + mdl;
        if constexpr (pass == 0 && FWD) {
          // lane holds W[r][16md + 4g + i], r = 16 mrow + lr.  The walk's
          // fragment (mrow, kb) gives lane (lr, g) the k-values 32 kb +
          // {4g..4g+3, 16+4g..16+4g+3}: tiles md = 2kb and 2kb+1 of this
          // lane, stored together as one 16-byte vector.
          if (md & 1) continue;
          WT tmp[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            tmp[i] = from_f32<WT>(acc[mdl][i]);
            tmp[4 + i] = from_f32<WT>(acc[mdl + 1][i]);
          }
          WT *dst = reinterpret_cast<WT *>(a.W) + ((cb * (C / 16) + mrow[u]) * (D / 32) + (md >> 1)) * 512 + lane * 8;
          constexpr int VE = 16 / sizeof(WT);
#pragma unroll
          for (int v = 0; v < 8 / VE; ++v) st16(dst + v * VE, *reinterpret_cast<const uint4 *>(tmp + v * VE));
        } else if constexpr (pass == 0) {
          WT *dst = reinterpret_cast<WT *>(a.W) + (cb * C + 16 * mrow[u] + lr) * D + 16 * md + lq;
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[i] = from_f32<WT>(acc[mdl][i]);
        } else if constexpr (FWD) {
          // lane holds U[16 mrow + 4g + i][16md + lr]: the walk's fragment (mrow, md)
          st16(a.U + ((cb * (C / 16) + mrow[u]) * TD + md) * 256 + lane * 4, acc[mdl]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            a.U[(cb * C + 16 * mrow[u] + lq + i) * D + 16 * md + lr] = acc[mdl][i];
        }
      }
    }
  };
  wu_pass(std::integral_constant<int, 0>{});
  if (!FWD && !a.U) return;   // (the transform hook without U: the backward's W and G only)
  lds_barrier();
  if (vhalf) TileBlock<C, TI, PNT / 2>::put_transposed(tix, sX, xw);
  lds_barrier();
  wu_pass(std::integral_constant<int, 1>{});
}

// ----------------------------------------------------------------------------
// walk / fold, throughput form: the sequential chunk loop.  Each wave owns a
// 16-column slice of the state; a workgroup of WPG waves covers WPG adjacent
// slices and shares the chunk's W and K^T operand fragments through LDS.
//
// The wave keeps its D x 16 slice of the fp32 state in matrix-core result
// registers (D/16 tiles of 16 x 16).  Per chunk:
//   V' = U - W h                        B operand: the state tiles
//   h  = e^{G_last} h + K^T (d o V')    B operand: the V' result tiles,
//                                       d_r = e^{G_last - G_r}
// A result tile gives lane group g rows 4g..4g+3 of its 16 rows, so two
// stacked tiles give lane group g the k-values {4g..4g+3, 16+4g..16+4g+3} of
// a block of 32: prep stores W and K^T with the k-values of each fragment in
// that order, and neither h nor V' leaves the registers between products.
//
// W and K^T fragments (the A operands; 64 KB per chunk at C = 128) and the
// decay cumsum G are copied from memory straight into LDS (global_load_lds,
// no registers), one chunk ahead into the other of two buffers, the copies
// split over the waves; one barrier per chunk.  U arrives in registers one
// chunk ahead.
// Modes: WALK (state = h; writes chunk-start states and V') and FOLD
// (state = the augmented [A | B] of a group, started from [I | 0]; writes
// the group's pair).
template <int C, typename TI> struct WalkOps {
  static constexpr int MV = C / 16, MH = D / 16;              // V' and state row tiles
  static constexpr int KBW = D / 32, KBK = C / 32;            // k-blocks of the two products
  static constexpr int FW = MV * KBW, FK = MH * KBK, F = FW + FK;   // fragments per chunk
  static constexpr int BPF = 8 * (int)sizeof(TI) / 16;       // 1 KB blocks per fragment
  static constexpr int NBLK = F * BPF;                        // 1 KB blocks per chunk
  static constexpr int GOFF = NBLK * 1024;                    // G (C floats) after the fragments
  static constexpr int ELEMS = (GOFF + 4 * C) / (int)sizeof(TI); // LDS buffer elements
};

template <int C, typename TI, int MODE, int KIND, int WPG>
__global__ __launch_bounds__(64 * WPG) void walk_shared_kernel(FwdArgs a) {
  using PR = Prec<MODE>;
  using PKw = PolicyKinds<PR::wh>;
  using PKk = PolicyKinds<PR::kv>;
  using OPS = WalkOps<C, TI>;
  constexpr bool F32 = sizeof(TI) == 4;
  static_assert(PKw::a == (F32 ? F_F32 : F_BF16) && PKk::a == PKw::a, "W and K^T fragments are used as stored");
  using AF = Frag<PKw::a>;
  constexpr int NS = (KIND == FOLD ? 2 * D : D) / 16;   // slices per unit
  constexpr int NG = NS / WPG;                           // workgroups per unit
  constexpr int MV = OPS::MV, MH = OPS::MH, KBW = OPS::KBW, KBK = OPS::KBK;
  constexpr int FW = OPS::FW, BPF = OPS::BPF, NBLK = OPS::NBLK;
  static_assert(NS % WPG == 0 && NBLK % WPG == 0, "work split");
  __shared__ __align__(16) TI bufA[OPS::ELEMS];
  __shared__ __align__(16) TI bufB[OPS::ELEMS];

  const int tid = threadIdx.x, wave = tid >> 6;
  int lane = tid & 63, lr = lane & 15, g = lane >> 4;
  // A workgroup item: one workgroup's share (grp) of one walk (unit).  A
  // persistent grid (the fold, fewer workgroups than items) takes items
  // blockIdx.x, blockIdx.x + gridDim.x, ... and copies each next item's first
  // chunk during the last chunk of the one before.
  const int items = a.B * a.Hv * a.jobs * NG;
  struct Item {
    size_t bh, cb0;      // walk; its first chunk in the workspace row of its value head
    long long ktoff;     // K^T chunk offset
    int job, cpj, c0, us;
    bool has_u;
  };
  auto item = [&](int L) {
    Item it;
    int grp;
    walk_unit(L, NG, a, it.bh, it.job, grp);
    const int slice = grp * WPG + wave;
    it.c0 = slice * 16;   // first column (of the augmented [A|B] in FOLD)
    it.has_u = KIND == WALK || it.c0 >= D;
    it.us = KIND == WALK ? slice : slice - D / 16;   // U column tile
    // this walk's chunks: the job's share of the head's, or (packed
    // sequences) the sequence's, in the workspace row of its value head
    if (KIND != FOLD && a.jtab) {   // (packed sequences walk, never fold)
      const int2 jt = a.jtab[it.bh / a.Hv];
      // (wave-uniform: scalar loop bounds)
      it.cb0 = (it.bh % a.Hv) * a.N + __builtin_amdgcn_readfirstlane(jt.x);
      it.cpj = __builtin_amdgcn_readfirstlane(jt.y);
      it.ktoff = kt_offset(a, it.bh % a.Hv);
    } else {
      it.cb0 = it.bh * a.N + a.n0 + (size_t)it.job * a.cpj;
      it.cpj = a.cpj;
      it.ktoff = kt_offset(a, it.bh);
    }
    it.cb0 = uniform64(it.cb0);
    it.ktoff = (long long)uniform64((unsigned long long)it.ktoff);
    return it;
  };
  int L = blockIdx.x, k = 0;
  // A persistent workgroup's slots L = blockIdx.x + k gridDim.x take item L,
  // or in odd slots item L ^ 8 (the unit's other workgroup share): the
  // shares differ in cost (only the B half reads U), and a workgroup that kept
  // one of them would finish half again as late as one that mixes them.
  // (L ^ 8 stays in the same block of gridDim.x slots when that is a multiple
  // of 16 and the items fill whole blocks.)
  const bool mix = KIND == FOLD && gridDim.x % 16 == 0 && items % gridDim.x == 0;
  auto slot_item = [&](int Ls, int ks) { return item(mix && (ks & 1) ? Ls ^ 8 : Ls); };
  Item cur_item = slot_item(L, 0);
  size_t bh = cur_item.bh, cb0 = cur_item.cb0;
  long long ktoff = cur_item.ktoff;
  int job = cur_item.job, cpj = cur_item.cpj, c0 = cur_item.c0, us = cur_item.us;
  bool has_u = cur_item.has_u;
  int slice = c0 / 16;

  // state tiles: h[m] holds rows 16m + 4g + i, column c0 + lr
  f32x4 h[MH];
  auto init_state = [&]() {
#pragma unroll
    for (int m = 0; m < MH; ++m) {
      const int col = c0 + lr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kr = 16 * m + 4 * g + i;
        float x = 0.f;
        if (KIND == FOLD) {
          x = (col < D && kr == col) ? 1.f : 0.f;
        } else if (a.init) {
          const float *src = a.init_per_job ? a.init + (bh * a.jobs + job) * D * D : a.init + bh * D * D;
          x = src[(size_t)kr * D + col];
        }
        h[m][i] = x;
      }
    }
  };
  init_state();

  // final state slice (the pair of a group in FOLD)
  auto store_final = [&]() {
    float *dst = nullptr;
    int dcol = c0;
    if (KIND == FOLD) {
      if (c0 < D) dst = a.pairA + (bh * a.jobs + job) * D * D;
      else { dst = a.pairB + (bh * a.jobs + job) * D * D; dcol = c0 - D; }
    } else if (a.fin && job == a.jobs - 1) {   // (the last group's end state)
      dst = a.fin + bh * D * D;
    }
    if (dst) {
#pragma unroll
      for (int m = 0; m < MH; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(size_t)(16 * m + 4 * g + i) * D + dcol + lr] = h[m][i];
    }
  };
  // an empty sequence (packed sequences): the final state is the initial one,
  // and no chunk operand is touched
  if (KIND != FOLD && cpj == 0) {
    store_final();
    return;
  }

  // copy the chunk's operand fragments into an LDS buffer: block j (1 KB) is
  // half j % BPF of fragment j / BPF; wave w copies blocks w, w + WPG, ...
  // (addresses: a wave-uniform base plus a 32-bit lane offset)
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const unsigned loff = lane * 16 * BPF;
  auto stage = [&](TI *buf, size_t cb, long long kto) {
    const char *wbase = reinterpret_cast<const char *>(a.W) + cb * C * D * sizeof(TI);
    const char *kbase = reinterpret_cast<const char *>(a.Kt) + (cb + kto) * D * C * sizeof(TI);
#pragma unroll
    for (int jj = 0; jj < NBLK / WPG; ++jj) {
      const int j = jj * WPG + wv, p = j / BPF, hh = j % BPF;
      const char *src = (p < FW ? wbase + p * 1024 * BPF : kbase + (p - FW) * 1024 * BPF) + hh * 16;
      __builtin_amdgcn_global_load_lds((const void *)(src + loff),
                                       (__attribute__((address_space(3))) void *)(reinterpret_cast<char *>(buf) + j * 1024),
                                       16, 0, 0);
    }
    if (wv == WPG - 1 && lane < C / 4)
      __builtin_amdgcn_global_load_lds((const void *)(a.G + cb * C + lane * 4),
                                       (__attribute__((address_space(3))) void *)(reinterpret_cast<char *>(buf) + OPS::GOFF),
                                       16, 0, 0);
    // keep the copies ahead of everything that follows in program order
    asm volatile("" ::: "memory");
  };
  auto frag = [&](const TI *buf, int p) -> AF {
    AF f;
    const char *base = reinterpret_cast<const char *>(buf) + p * BPF * 1024 + lane * 16;
    if constexpr (F32) {
      const float4 x0 = *reinterpret_cast<const float4 *>(base);
      const float4 x1 = *reinterpret_cast<const float4 *>(base + 1024);
      f.v[0] = x0.x; f.v[1] = x0.y; f.v[2] = x0.z; f.v[3] = x0.w;
      f.v[4] = x1.x; f.v[5] = x1.y; f.v[6] = x1.z; f.v[7] = x1.w;
    } else {
      f.hi = *reinterpret_cast<const bf16x8 *>(base);
    }
    return f;
  };
  // this wave's copies and loads done, then every wave's
  auto chunk_barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __builtin_amdgcn_s_barrier();
  };

  struct UG {
    float4 u[MV];
  };
  auto fetch_u = [&](size_t cb, UG &x, bool hu, int ust) {
#pragma unroll
    for (int m = 0; m < MV; ++m)
      x.u[m] = hu ? *reinterpret_cast<const float4 *>(a.U + ((cb * MV + m) * (D / 16) + ust) * 256 + lane * 4)
                  : float4{0.f, 0.f, 0.f, 0.f};
  };

  UG ug[2];
  stage(bufA, cb0, ktoff);
  fetch_u(cb0, ug[0], has_u, us);
  chunk_barrier();
  // the item after this one in the workgroup, if any (persistent grids)
  bool has_next = false;
  Item nxt_item = cur_item;

  auto step = [&](const TI *cur, TI *nxt, UG &cu, UG &nu, int cc) {
    const size_t cb = cb0 + cc;
    const bool more = cc + 1 < cpj;
    // everything for the next chunk (of this item, or the next item's first);
    // waited for at the chunk's end only
    const size_t pcb = more ? cb + 1 : has_next ? nxt_item.cb0 : cb;
    fetch_u(pcb, nu, more || !has_next ? has_u : nxt_item.has_u, more ? us : nxt_item.us);
    if (more || has_next) stage(nxt, pcb, more ? ktoff : nxt_item.ktoff);
    const float *Gs = reinterpret_cast<const float *>(reinterpret_cast<const char *>(cur) + OPS::GOFF);
    const float gl2 = Gs[C - 1] * LOG2E;
    float dcy[MV][4];
#pragma unroll
    for (int m = 0; m < MV; ++m) {
      const float4 gq = *reinterpret_cast<const float4 *>(Gs + 16 * m + 4 * g);
      dcy[m][0] = exp2_fast(gl2 - gq.x * LOG2E);
      dcy[m][1] = exp2_fast(gl2 - gq.y * LOG2E);
      dcy[m][2] = exp2_fast(gl2 - gq.z * LOG2E);
      dcy[m][3] = exp2_fast(gl2 - gq.w * LOG2E);
    }
    // V' = U - W h
    Frag<PKw::b> hb[KBW];
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb) {
      const float x[8] = {h[2 * kb][0], h[2 * kb][1], h[2 * kb][2], h[2 * kb][3],
                          h[2 * kb + 1][0], h[2 * kb + 1][1], h[2 * kb + 1][2], h[2 * kb + 1][3]};
      hb[kb] = make_frag<PKw::b>(x);
    }
    f32x4 acc[MV];
#pragma unroll
    for (int m = 0; m < MV; ++m) acc[m] = zero4();
    // fragments are read a group (one output tile's k-blocks) ahead
    AF fa[2][KBW];
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb) fa[0][kb] = frag(cur, kb);
#pragma unroll
    for (int m = 0; m < MV; ++m) {
      if (m + 1 < MV) {
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb) fa[(m + 1) & 1][kb] = frag(cur, (m + 1) * KBW + kb);
      }
#pragma unroll
      for (int kb = 0; kb < KBW; ++kb) mma(acc[m], fa[m & 1][kb], hb[kb]);
    }
    // chunk-start state for the output stage (stores issued after the loads
    // this chunk still waits for)
    if (KIND == WALK && a.Hs)
      store_result_tiles<PR::h_store>(a.Hs + (cb * (D / 16) + slice) * MH * Store<PR::h_store>::tile_floats, h, lane);
    Frag<PKk::b> vb[KBK];
    {
      float s[MV][4];
      f32x4 vps[MV];
#pragma unroll
      for (int m = 0; m < MV; ++m) {
        const float4 uu = cu.u[m];
        vps[m] = f32x4{uu.x - acc[m][0], uu.y - acc[m][1], uu.z - acc[m][2], uu.w - acc[m][3]};
#pragma unroll
        for (int i = 0; i < 4; ++i) s[m][i] = vps[m][i] * dcy[m][i];
      }
      if (KIND == WALK && a.Vn)
        store_result_tiles<PR::v_store>(a.Vn + (cb * (D / 16) + slice) * MV * Store<PR::v_store>::tile_floats, vps, lane);
#pragma unroll
      for (int kb = 0; kb < KBK; ++kb) {
        const float x[8] = {s[2 * kb][0], s[2 * kb][1], s[2 * kb][2], s[2 * kb][3],
                            s[2 * kb + 1][0], s[2 * kb + 1][1], s[2 * kb + 1][2], s[2 * kb + 1][3]};
        vb[kb] = make_frag<PKk::b>(x);
      }
    }
    // h <- e^{G_last} h + K^T (d o V')
    const float gl = exp2_fast(gl2);
    AF fk[2][KBK];
#pragma unroll
    for (int kb = 0; kb < KBK; ++kb) fk[0][kb] = frag(cur, FW + kb);
#pragma unroll
    for (int m = 0; m < MH; ++m) {
      if (m + 1 < MH) {
#pragma unroll
        for (int kb = 0; kb < KBK; ++kb) fk[(m + 1) & 1][kb] = frag(cur, FW + (m + 1) * KBK + kb);
      }
      f32x4 acc2 = zero4();
#pragma unroll
      for (int kb = 0; kb < KBK; ++kb) mma(acc2, fk[m & 1][kb], vb[kb]);
#pragma unroll
      for (int i = 0; i < 4; ++i) h[m][i] = gl * h[m][i] + acc2[i];
    }
    chunk_barrier();
  };
  for (;;) {
    // (a persistent grid runs only where every item has an even chunk count,
    // so that each item starts in bufA)
    const int Ln = L + (int)gridDim.x;
    has_next = KIND == FOLD && Ln < items;   // (the walk's grid is never persistent)
    if (has_next) nxt_item = slot_item(Ln, k + 1);
    // two chunks per trip: the LDS buffers and U/G sets alternate statically
    for (int cc = 0; cc < cpj; cc += 2) {
      step(bufA, bufB, ug[0], ug[1], cc);
      if (cc + 1 < cpj) step(bufB, bufA, ug[1], ug[0], cc + 1);
    }
    store_final();
    if (!has_next) break;
    L = Ln;
    ++k;
    // (the lane indices opaque again for each item: the addresses derived
    // from them are then formed per item, not held across all of them)
    asm volatile("" : "+v"(lane), "+v"(lr), "+v"(g));
    cur_item = nxt_item;
    bh = cur_item.bh; cb0 = cur_item.cb0; ktoff = cur_item.ktoff; job = cur_item.job; cpj = cur_item.cpj;
    c0 = cur_item.c0; us = cur_item.us; has_u = cur_item.has_u; slice = c0 / 16;
    init_state();
  }
}

// ----------------------------------------------------------------------------
// walk / fold, latency form: one workgroup of NWS waves per 16-column slice
// of the state, for walks too few to fill the chip.  The state, V' and their
// register chaining are those of walk_shared_kernel above; here the slice's
// rows are split between the waves: wave w holds state rows 128w/NWS.. and
// corrected-value rows Cw/NWS.., and streams only the W and K^T fragments of
// its own rows (1/NWS of a chunk's, through a ring of register slots,
// refilled as soon as consumed: one or more chunks ahead).  The B operands --
// the bf16 state for V' = U - W h, the split d o V' for the state update --
// pass between the waves through LDS, two barriers per chunk.  U and G arrive
// one chunk ahead.
template <int C, typename TI, int MODE, int KIND, int NWS>
__global__ __launch_bounds__(64 * NWS) void walk_ring_kernel(FwdArgs a) {
  using PR = Prec<MODE>;
  using PKw = PolicyKinds<PR::wh>;
  using PKk = PolicyKinds<PR::kv>;
  constexpr bool F32 = sizeof(TI) == 4;
  static_assert(PKw::a == (F32 ? F_F32 : F_BF16) && PKk::a == PKw::a, "W and K^T fragments are used as stored");
  using AF = Frag<PKw::a>;
  using HF = Frag<PKw::b>;   // state operand (for W h)
  using VF = Frag<PKk::b>;   // d o V' operand (for K^T (d o V'))
  constexpr int NS = (KIND == WALK ? D : 2 * D) / 16;   // slices (the augmented state: A columns first)
  constexpr int MV = C / 16, MH = D / 16;                // V' and state row tiles
  constexpr int KBW = D / 32, KBK = C / 32;              // k-blocks of the two products
  constexpr int MVW = MV / NWS, MHW = MH / NWS;          // row tiles per wave
  constexpr int KBWW = KBW / NWS, KBKW = KBK / NWS;      // k-blocks held by each wave
  static_assert(MVW % 2 == 0 && MHW % 2 == 0, "each wave holds whole k-blocks");
  constexpr int FW = MV * KBW;                           // W fragments per chunk (K^T follow)
  constexpr int FWW = MVW * KBW, FKW = MHW * KBK, FPW = FWW + FKW;   // per wave per chunk
  // ring slots: up to 32 (bf16) / 16 (fp32) fragments, at most one chunk's
  // (a ring of two chunks, slot parity = chunk parity, measured no faster)
  constexpr int SLOTS = F32 ? 16 : 32;
  constexpr int RING = SLOTS < FPW ? SLOTS : FPW;
  static_assert(FPW % RING == 0 && KBKW >= 1, "ring slots must repeat every chunk");
  __shared__ __align__(16) HF xh[NWS][KBWW][64];
  __shared__ __align__(16) VF xv[NWS][KBKW][64];

  int unit, slice;
  xcd_unit(blockIdx.x, NS, a.B * a.Hv * a.jobs, unit, slice);
  const int job = unit % a.jobs;
  const size_t bh = (size_t)(unit / a.jobs);
  const int lane = threadIdx.x & 63, lr = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c0 = slice * 16;   // first column (of the augmented [A|B] in FOLD)
  const bool has_u = KIND == WALK || c0 >= D;
  const int us = KIND == WALK ? slice : slice - D / 16;   // U column tile
  // h columns of the augmented state in WALK_A: as a WALK slice of index us
  const bool hcols = KIND == WALK || (KIND == WALK_A && c0 >= D);
  const int mv0 = w * MVW, mh0 = w * MHW;                 // this wave's first V' / state tile
  // this walk's chunks, as in walk_shared_kernel
  size_t cb0;
  int cpj;
  long long ktoff;
  if (KIND != FOLD && a.jtab) {   // (packed sequences walk, never fold)
    const int2 jt = a.jtab[bh / a.Hv];
    // (wave-uniform: scalar loop bounds)
    cb0 = (bh % a.Hv) * a.N + __builtin_amdgcn_readfirstlane(jt.x);
    cpj = __builtin_amdgcn_readfirstlane(jt.y);
    ktoff = kt_offset(a, bh % a.Hv);
  } else {
    cb0 = bh * a.N + a.n0 + (size_t)job * a.cpj;
    cpj = a.cpj;
    ktoff = kt_offset(a, bh);
  }
  cb0 = uniform64(cb0);
  ktoff = (long long)uniform64((unsigned long long)ktoff);

  // state tiles of this wave: h[t] holds rows 16(mh0+t) + 4g + i, column c0 + lr
  f32x4 h[MHW];
#pragma unroll
  for (int t = 0; t < MHW; ++t) {
    const int col = c0 + lr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kr = 16 * (mh0 + t) + 4 * g + i;
      float x = 0.f;
      if (KIND != WALK && col < D) {
        x = kr == col ? 1.f : 0.f;
      } else if (KIND != FOLD && a.init) {
        const float *src = a.init_per_job ? a.init + (bh * a.jobs + job) * D * D : a.init + bh * D * D;
        x = src[(size_t)kr * D + (KIND == WALK ? col : col - D)];
      }
      h[t][i] = x;
    }
  }

  // final state rows of this wave (the pair of a group in FOLD)
  auto store_final = [&]() {
    float *dst = nullptr;
    int dcol = c0;
    if (KIND != WALK && c0 < D) {
      dst = a.pairA + (bh * a.jobs + job) * D * D;
    } else if (KIND == FOLD) {
      dst = a.pairB + (bh * a.jobs + job) * D * D;
      dcol = c0 - D;
    } else if (a.fin && job == a.jobs - 1) {   // (the last group's end state)
      dst = a.fin + bh * D * D;
      dcol = KIND == WALK ? c0 : c0 - D;
    }
    if (dst) {
#pragma unroll
      for (int t = 0; t < MHW; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(size_t)(16 * (mh0 + t) + 4 * g + i) * D + dcol + lr] = h[t][i];
    }
  };
  // an empty sequence (packed sequences): the final state is the initial one,
  // and no chunk operand is touched
  if (KIND != FOLD && cpj == 0) {
    store_final();
    return;
  }

  // this wave's fragment sequence per chunk: W (its V' row tiles, all
  // k-blocks), then K^T (its state row tiles, all k-blocks)
  const TI *Wb = reinterpret_cast<const TI *>(a.W) + lane * 8;
  const TI *Kb = reinterpret_cast<const TI *>(a.Kt) + lane * 8;
  auto load = [&](size_t cb, int q) -> AF {
    const TI *src = q < FWW ? Wb + cb * C * D + (size_t)(mv0 * KBW + q) * 512
                            : Kb + (cb + ktoff) * D * C + (size_t)(mh0 * KBK + q - FWW) * 512;
    AF f;
    if constexpr (F32) {
      const float4 x0 = *reinterpret_cast<const float4 *>(src);
      const float4 x1 = *reinterpret_cast<const float4 *>(src + 4);
      f.v[0] = x0.x; f.v[1] = x0.y; f.v[2] = x0.z; f.v[3] = x0.w;
      f.v[4] = x1.x; f.v[5] = x1.y; f.v[6] = x1.z; f.v[7] = x1.w;
    } else {
      f.hi = *reinterpret_cast<const bf16x8 *>(src);
    }
    return f;
  };
  struct UG {
    float4 u[MVW], g[MVW];
    float glast;
  };
  auto fetch_ug = [&](size_t cb, UG &x) {
#pragma unroll
    for (int m = 0; m < MVW; ++m) {
      x.u[m] = has_u ? *reinterpret_cast<const float4 *>(a.U + ((cb * MV + mv0 + m) * (D / 16) + us) * 256 + lane * 4)
                     : float4{0.f, 0.f, 0.f, 0.f};
      x.g[m] = *reinterpret_cast<const float4 *>(a.G + cb * C + 16 * (mv0 + m) + 4 * g);
    }
    x.glast = a.G[cb * C + C - 1 + vgpr_zero()];
  };
  auto state_frag = [&](int kbl) -> HF {   // own state k-block kbl (tiles 2kbl, 2kbl+1)
    const float x[8] = {h[2 * kbl][0], h[2 * kbl][1], h[2 * kbl][2], h[2 * kbl][3],
                        h[2 * kbl + 1][0], h[2 * kbl + 1][1], h[2 * kbl + 1][2], h[2 * kbl + 1][3]};
    return make_frag<PKw::b>(x);
  };

  // U and G of the first chunk before the ring's fragments: the loop's
  // memory waits are merged over its entry and its back edge, and on entry
  // the first chunk's operands should not be the newest loads
  UG ug[2];
  fetch_ug(cb0, ug[0]);
  AF ring[RING];
#pragma unroll
  for (int q = 0; q < RING; ++q) {
    const size_t c = cb0 + q / FPW;
    ring[q] = load(c < cb0 + cpj - 1 ? c : cb0 + cpj - 1, q % FPW);
  }
  // the state operand of the first chunk
#pragma unroll
  for (int kbl = 0; kbl < KBWW; ++kbl) xh[w][kbl][lane] = state_frag(kbl);
  lds_barrier();

  const size_t cblast = cb0 + cpj - 1;
  // fragment q of chunk cb sits in slot (P FPW + q) % RING (P = chunk parity);
  // once consumed, the slot takes the fragment RING positions later in the
  // sequence (past the last chunk: the last chunk again, unused)
  auto refill = [&](int P, size_t cb, int q) {
    const int nq = q + RING;
    const size_t c = cb + nq / FPW;
    ring[(P * FPW + q) % RING] = load(c < cblast ? c : cblast, nq % FPW);
  };
  auto step = [&](UG &cur, UG &nxt, int cc, auto Pc) {
    constexpr int P = decltype(Pc)::value;
    const size_t cb = cb0 + cc;
    const size_t cbn = cc + 1 < cpj ? cb + 1 : cb;   // last chunk: repeat loads (unused)
    fetch_ug(cbn, nxt);
    const float gl2 = cur.glast * LOG2E;
    float dcy[MVW][4];
#pragma unroll
    for (int m = 0; m < MVW; ++m) {
      dcy[m][0] = exp2_fast(gl2 - cur.g[m].x * LOG2E);
      dcy[m][1] = exp2_fast(gl2 - cur.g[m].y * LOG2E);
      dcy[m][2] = exp2_fast(gl2 - cur.g[m].z * LOG2E);
      dcy[m][3] = exp2_fast(gl2 - cur.g[m].w * LOG2E);
    }
    // V' = U - W h over all state k-blocks: own from registers, partner's from LDS
    // every k-block from LDS, the wave's own included (static indices)
    HF hb[KBW];
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb) hb[kb] = xh[kb / KBWW][kb % KBWW][lane];
    f32x4 acc[MVW];
#pragma unroll
    for (int m = 0; m < MVW; ++m) acc[m] = zero4();
#pragma unroll
    for (int q = 0; q < FWW; ++q) {
      mma(acc[q / KBW], ring[(P * FPW + q) % RING], hb[q % KBW]);
      refill(P, cb, q);
    }
    VF vb[KBK];
    f32x4 vps[MVW];
    {
      float s[MVW][4];
#pragma unroll
      for (int m = 0; m < MVW; ++m) {
        const float4 uu = cur.u[m];
        vps[m] = f32x4{uu.x - acc[m][0], uu.y - acc[m][1], uu.z - acc[m][2], uu.w - acc[m][3]};
#pragma unroll
        for (int i = 0; i < 4; ++i) s[m][i] = vps[m][i] * dcy[m][i];
      }
#pragma unroll
      for (int kbl = 0; kbl < KBKW; ++kbl) {
        const float x[8] = {s[2 * kbl][0], s[2 * kbl][1], s[2 * kbl][2], s[2 * kbl][3],
                            s[2 * kbl + 1][0], s[2 * kbl + 1][1], s[2 * kbl + 1][2], s[2 * kbl + 1][3]};
        xv[w][kbl][lane] = make_frag<PKk::b>(x);
      }
      lds_barrier();
#pragma unroll
      for (int kb = 0; kb < KBK; ++kb) vb[kb] = xv[kb / KBKW][kb % KBKW][lane];
    }
    // h <- e^{G_last} h + K^T (d o V') for this wave's state rows
    const float gl = exp2_fast(gl2);
    f32x4 acc2[MHW];
#pragma unroll
    for (int t = 0; t < MHW; ++t) {
      acc2[t] = zero4();
#pragma unroll
      for (int kb = 0; kb < KBK; ++kb) {
        const int q = FWW + t * KBK + kb;
        mma(acc2[t], ring[(P * FPW + q) % RING], vb[kb]);
        refill(P, cb, q);
      }
    }
    // The chunk-start state and V' go out after the chunk's last loads: the
    // memory counter drains in issue order, so a store issued ahead of a load
    // would hold up every wait for that load.
    // (the plain walk always has both: no branch in the loop, whose memory
    // waits the compiler would otherwise merge conservatively)
    if (KIND == WALK || (KIND == WALK_A && hcols && a.Hs))
      store_result_tiles<PR::h_store>(a.Hs + ((cb * (D / 16) + us) * MH + mh0) * Store<PR::h_store>::tile_floats, h, lane);
    if (KIND == WALK || (KIND == WALK_A && hcols && a.Vn))
      store_result_tiles<PR::v_store>(a.Vn + ((cb * (D / 16) + us) * MV + mv0) * Store<PR::v_store>::tile_floats, vps, lane);
#pragma unroll
    for (int t = 0; t < MHW; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) h[t][i] = gl * h[t][i] + acc2[t][i];
#pragma unroll
    for (int kbl = 0; kbl < KBWW; ++kbl) xh[w][kbl][lane] = state_frag(kbl);
    lds_barrier();
  };
  // two chunks per trip so the U/G sets alternate without copies, and no
  // branch inside a trip; an odd last chunk after the loop
  int cc = 0;
  for (; cc + 1 < cpj; cc += 2) {
    step(ug[0], ug[1], cc, std::integral_constant<int, 0>{});
    step(ug[1], ug[0], cc + 1, std::integral_constant<int, 1>{});
  }
  if (cc < cpj) step(ug[0], ug[1], cc, std::integral_constant<int, 0>{});

  store_final();
}

// ----------------------------------------------------------------------------
// walk, paired form: two 16-column slices of one head per workgroup, each
// split over NWS waves by rows as in walk_ring_kernel, for walks too many to
// give each slice a compute unit of its own and too few for the throughput
// form (33..64 walks of 8 slices: one workgroup per compute unit).  The two
// slices need the same W and K^T fragments: they are copied into LDS once
// per chunk (global_load_lds, double-buffered, one chunk ahead) instead of
// being streamed by every wave, which halves what each compute unit moves
// per chunk against two latency-form workgroups.  State and d o V' operands
// pass between a slice's waves through LDS, as in the latency form.  WALK
// mode only, with h and V' for the output stage always written.
template <int C, typename TI, int MODE, int NWS>
__global__ __launch_bounds__(128 * NWS) void walk_pair_kernel(FwdArgs a) {
  using PR = Prec<MODE>;
  using PKw = PolicyKinds<PR::wh>;
  using PKk = PolicyKinds<PR::kv>;
  using OPS = WalkOps<C, TI>;
  constexpr bool F32 = sizeof(TI) == 4;
  static_assert(PKw::a == (F32 ? F_F32 : F_BF16) && PKk::a == PKw::a, "W and K^T fragments are used as stored");
  using AF = Frag<PKw::a>;
  using HF = Frag<PKw::b>;   // state operand (for W h)
  using VF = Frag<PKk::b>;   // d o V' operand (for K^T (d o V'))
  constexpr int NSL = 2, WPG = NSL * NWS;               // slices per workgroup, waves
  constexpr int MV = OPS::MV, MH = OPS::MH, KBW = OPS::KBW, KBK = OPS::KBK;
  constexpr int FW = OPS::FW, BPF = OPS::BPF, NBLK = OPS::NBLK;
  constexpr int MVW = MV / NWS, MHW = MH / NWS;         // row tiles per wave
  constexpr int KBWW = KBW / NWS, KBKW = KBK / NWS;     // k-blocks written by each wave
  static_assert(MVW % 2 == 0 && MHW % 2 == 0 && KBWW >= 1 && KBKW >= 1, "each wave holds whole k-blocks");
  static_assert(NBLK % WPG == 0, "copies shared out evenly");
  __shared__ __align__(16) TI bufA[OPS::ELEMS];
  __shared__ __align__(16) TI bufB[OPS::ELEMS];
  __shared__ __align__(16) HF xh[NSL][KBW][64];
  __shared__ __align__(16) VF xv[NSL][KBK][64];

  int unit, pair;
  xcd_unit(blockIdx.x, D / 16 / NSL, a.B * a.Hv * a.jobs, unit, pair);
  const int job = unit % a.jobs;
  const size_t bh = (size_t)(unit / a.jobs);
  const int lane = threadIdx.x & 63, lr = lane & 15, g = lane >> 4;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sl = wid / NWS, w = wid % NWS;              // slice of the pair, row part
  const int slice = pair * NSL + sl, c0 = slice * 16;
  const int mv0 = w * MVW, mh0 = w * MHW;               // this wave's first V' / state tile
  size_t cb0;
  int cpj;
  long long ktoff;
  if (a.jtab) {   // packed sequences
    const int2 jt = a.jtab[bh / a.Hv];
    cb0 = (bh % a.Hv) * a.N + __builtin_amdgcn_readfirstlane(jt.x);
    cpj = __builtin_amdgcn_readfirstlane(jt.y);
    ktoff = kt_offset(a, bh % a.Hv);
  } else {
    cb0 = bh * a.N + a.n0 + (size_t)job * a.cpj;
    cpj = a.cpj;
    ktoff = kt_offset(a, bh);
  }
  cb0 = uniform64(cb0);
  ktoff = (long long)uniform64((unsigned long long)ktoff);

  // state tiles of this wave: h[t] holds rows 16(mh0+t) + 4g + i, column c0 + lr
  f32x4 h[MHW];
#pragma unroll
  for (int t = 0; t < MHW; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kr = 16 * (mh0 + t) + 4 * g + i;
      float x = 0.f;
      if (a.init) {
        const float *src = a.init_per_job ? a.init + (bh * a.jobs + job) * D * D : a.init + bh * D * D;
        x = src[(size_t)kr * D + c0 + lr];
      }
      h[t][i] = x;
    }
  }
  auto store_final = [&]() {
    if (a.fin && job == a.jobs - 1) {   // (the last group's end state)
#pragma unroll
      for (int t = 0; t < MHW; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) a.fin[bh * D * D + (size_t)(16 * (mh0 + t) + 4 * g + i) * D + c0 + lr] = h[t][i];
    }
  };
  if (cpj == 0) {   // an empty packed sequence
    store_final();
    return;
  }

  // the chunk's W and K^T fragments into an LDS buffer (block j: half
  // j % BPF of fragment j / BPF), shared out over the WPG waves.  The copies'
  // LDS addresses are plain numbers to the compiler, which then does not tie
  // the LDS reads that follow to them (it would wait for every copy before
  // the first read of any LDS array); the chunk barrier waits for them.
  const unsigned loff = lane * 16 * BPF;
  auto lds_addr = [](TI *buf) {
    unsigned x = (unsigned)(size_t)(__attribute__((address_space(3))) char *)buf;
    asm volatile("" : "+s"(x));
    return x;
  };
  const unsigned ldsA = lds_addr(bufA), ldsB = lds_addr(bufB);
  auto stage = [&](unsigned lbuf, size_t cb) {
    const char *wbase = reinterpret_cast<const char *>(a.W) + cb * C * D * sizeof(TI);
    const char *kbase = reinterpret_cast<const char *>(a.Kt) + (cb + ktoff) * D * C * sizeof(TI);
#pragma unroll
    for (int jj = 0; jj < NBLK / WPG; ++jj) {
      const int j = jj * WPG + wid, p = j / BPF, hh = j % BPF;
      const char *src = (p < FW ? wbase + p * 1024 * BPF : kbase + (p - FW) * 1024 * BPF) + hh * 16;
      __builtin_amdgcn_global_load_lds((const void *)(src + loff),
                                       (__attribute__((address_space(3))) void *)(size_t)(lbuf + j * 1024),
                                       16, 0, 0);
    }
  };
  auto frag = [&](const TI *buf, int p) -> AF {
    AF f;
    const char *base = reinterpret_cast<const char *>(buf) + p * BPF * 1024 + lane * 16;
    if constexpr (F32) {
      const float4 x0 = *reinterpret_cast<const float4 *>(base);
      const float4 x1 = *reinterpret_cast<const float4 *>(base + 1024);
      f.v[0] = x0.x; f.v[1] = x0.y; f.v[2] = x0.z; f.v[3] = x0.w;
      f.v[4] = x1.x; f.v[5] = x1.y; f.v[6] = x1.z; f.v[7] = x1.w;
    } else {
      f.hi = *reinterpret_cast<const bf16x8 *>(base);
    }
    return f;
  };
  struct UG {
    float4 u[MVW], g[MVW];
    float glast;
  };
  auto fetch_ug = [&](size_t cb, UG &x) {
#pragma unroll
    for (int m = 0; m < MVW; ++m) {
      x.u[m] = *reinterpret_cast<const float4 *>(a.U + ((cb * MV + mv0 + m) * (D / 16) + slice) * 256 + lane * 4);
      x.g[m] = *reinterpret_cast<const float4 *>(a.G + cb * C + 16 * (mv0 + m) + 4 * g);
    }
    x.glast = a.G[cb * C + C - 1 + vgpr_zero()];
  };
  auto put_state = [&]() {
#pragma unroll
    for (int kbl = 0; kbl < KBWW; ++kbl) {   // own k-block kbl (tiles 2kbl, 2kbl+1)
      const float x[8] = {h[2 * kbl][0], h[2 * kbl][1], h[2 * kbl][2], h[2 * kbl][3],
                          h[2 * kbl + 1][0], h[2 * kbl + 1][1], h[2 * kbl + 1][2], h[2 * kbl + 1][3]};
      xh[sl][w * KBWW + kbl][lane] = make_frag<PKw::b>(x);
    }
  };
  // The chunk's end: this wave's copies and loads for the next chunk done, and
  // its LDS writes, then every wave's.  The memory counter drains in issue
  // order and the V' stores are the last NVS operations issued, so waiting
  // down to NVS leaves them in flight.
  constexpr int NVS = PR::v_store == ST_BF16 ? MVW / 2 : MVW;   // 16-byte stores of V'
  static_assert(NVS < 16, "vmcnt field");
  auto chunk_barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(0x0070 | NVS);   // vmcnt(NVS) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
  };

  UG ug[2];
  fetch_ug(cb0, ug[0]);
  stage(ldsA, cb0);
  put_state();
  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();

  auto step = [&](const TI *cur, unsigned nxt, UG &cu, UG &nu, int cc) {
    const size_t cb = cb0 + cc;
    const bool more = cc + 1 < cpj;
    // issue order: the chunk-start state for the output stage, the next
    // chunk's U and G (the last chunk: repeated, unused) and operand copies,
    // then (after the W h product) this chunk's V'
    store_result_tiles<PR::h_store>(a.Hs + ((cb * (D / 16) + slice) * MH + mh0) * Store<PR::h_store>::tile_floats, h, lane);
    fetch_ug(more ? cb + 1 : cb, nu);
    if (more) stage(nxt, cb + 1);
    asm volatile("" ::: "memory");   // nothing below moves above the copies
    const float gl2 = cu.glast * LOG2E;
    float dcy[MVW][4];
#pragma unroll
    for (int m = 0; m < MVW; ++m) {
      dcy[m][0] = exp2_fast(gl2 - cu.g[m].x * LOG2E);
      dcy[m][1] = exp2_fast(gl2 - cu.g[m].y * LOG2E);
      dcy[m][2] = exp2_fast(gl2 - cu.g[m].z * LOG2E);
      dcy[m][3] = exp2_fast(gl2 - cu.g[m].w * LOG2E);
    }
    // V' = U - W h over all state k-blocks (the slice's, from LDS)
    HF hb[KBW];
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb) hb[kb] = xh[sl][kb][lane];
    f32x4 acc[MVW];
#pragma unroll
    for (int m = 0; m < MVW; ++m) {
      acc[m] = zero4();
#pragma unroll
      for (int kb = 0; kb < KBW; ++kb) mma(acc[m], frag(cur, (mv0 + m) * KBW + kb), hb[kb]);
    }
    VF vb[KBK];
    {
      float s[MVW][4];
      f32x4 vps[MVW];
#pragma unroll
      for (int m = 0; m < MVW; ++m) {
        const float4 uu = cu.u[m];
        vps[m] = f32x4{uu.x - acc[m][0], uu.y - acc[m][1], uu.z - acc[m][2], uu.w - acc[m][3]};
#pragma unroll
        for (int i = 0; i < 4; ++i) s[m][i] = vps[m][i] * dcy[m][i];
      }
      store_result_tiles<PR::v_store>(a.Vn + ((cb * (D / 16) + slice) * MV + mv0) * Store<PR::v_store>::tile_floats, vps, lane);
#pragma unroll
      for (int kbl = 0; kbl < KBKW; ++kbl) {
        const float x[8] = {s[2 * kbl][0], s[2 * kbl][1], s[2 * kbl][2], s[2 * kbl][3],
                            s[2 * kbl + 1][0], s[2 * kbl + 1][1], s[2 * kbl + 1][2], s[2 * kbl + 1][3]};
        xv[sl][w * KBKW + kbl][lane] = make_frag<PKk::b>(x);
      }
      lds_barrier();
#pragma unroll
      for (int kb = 0; kb < KBK; ++kb) {
        if constexpr (PKk::b == F_SPLIT) {
          vb[kb].hi = xv[sl][kb][lane].hi;
          vb[kb].lo = xv[sl][kb][lane].lo;
        } else {
          vb[kb] = xv[sl][kb][lane];
        }
      }
    }
    // h <- e^{G_last} h + K^T (d o V') for this wave's state rows
    const float gl = exp2_fast(gl2);
    f32x4 acc2[MHW];
#pragma unroll
    for (int t = 0; t < MHW; ++t) {
      acc2[t] = zero4();
#pragma unroll
      for (int kb = 0; kb < KBK; ++kb) mma(acc2[t], frag(cur, FW + (mh0 + t) * KBK + kb), vb[kb]);
    }
#pragma unroll
    for (int t = 0; t < MHW; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) h[t][i] = gl * h[t][i] + acc2[t][i];
    put_state();
    chunk_barrier();
  };
  // two chunks per trip: the LDS buffers and U/G sets alternate statically
  for (int cc = 0; cc < cpj; cc += 2) {
    step(bufA, ldsB, ug[0], ug[1], cc);
    if (cc + 1 < cpj) step(bufB, ldsA, ug[1], ug[0], cc + 1);
  }
  store_final();
}

// ----------------------------------------------------------------------------
// exclusive prefix of affine pairs: h_in[0] = h_init, h_in[j+1] = A_j h_in[j]
// + B_j, h_final = A_{n-1} h_in[n-1] + B_{n-1}.  One workgroup per 16-column
// slice of the state (the recurrence is column-separable); its NWS waves
// split the slice's rows, each holding its rows in matrix-core result
// registers for all n steps, as in the walk.  A_j (row-major fp32) is the A
// operand: per lane two 16-byte runs of a row, in the k order of two stacked
// result tiles, so a wave's two state tiles are one k-block of the B operand
// as they stand; the waves pass their k-blocks through LDS (double-buffered:
// one barrier per step).
struct PrefixArgs {
  int BH, n;
  const float *A, *Bm, *h_init;
  float *h_in, *h_final;
  // element strides (floats) between consecutive pairs / incoming states of
  // a row and between rows; 0 = contiguous [BH, n, D, D]
  long long js, bs;
};

// s_waitcnt immediate: vmcnt(n) lgkmcnt(0)
__host__ __device__ constexpr int vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4); }

// A_j and B_j are copied straight into LDS (global_load_lds, no registers),
// two steps ahead, into two stages declared as separate LDS arrays, the
// waits for the copies placed by hand.  Each
// wave copies and reads only its own 32 rows (A_j: 16 copies of 1 KB, copy q
// = (row tile t, k-block kb, half) giving lane (lr, g) the 16 bytes at row
// 16(m0+t) + lr, columns 32kb + 16 half + 4g ..; B_j: 2 copies, lane l the 16
// bytes at row 16t + l/4, columns c0 + 4(l%4) ..), so a copy needs no
// barrier, only the wave's own memory counter.  Per step and wave, in order:
// the h_in row stores (8), the exchange barrier, the wait for this step's
// copies (issued two steps before; 26 operations per step follow them, so
// 34 may stay in flight -- 18 without h_in stores, and 26 (18) at the first
// step, after the start's copies), the reads of A_j and B_j, the copies of
// step j+2 into the stage just read, then the products.  (B_j loaded into
// registers, one memory operation per element, would put the two steps in
// flight over the counter's 63.)
template <int PREC, int NWS, bool HIN>   // HIN: h_in is written
__global__ __launch_bounds__(64 * NWS) void prefix_kernel(PrefixArgs a) {
  using PK = PolicyKinds<PREC>;
  using HF = Frag<PK::b>;
  constexpr int MH = D / 16, KB = D / 32;
  constexpr int MHW = MH / NWS;
  static_assert(MHW == 2, "each wave holds one k-block of the state");
  constexpr int F = MHW * KB;                  // A fragments per wave and step
  constexpr int WA = 2 * F * 1024;             // a wave's rows of A_j (16 copies of 1 KB)
  constexpr int WB = MHW * 1024;               // a wave's rows of B_j (2 copies of 1 KB)
  constexpr int NOPS = 2 * F + MHW + (HIN ? 4 * MHW : 0);   // memory operations per step and wave
  __shared__ __align__(16) HF xh[2][KB][64];
  __shared__ __align__(16) char sA0[NWS * WA];
  __shared__ __align__(16) char sA1[NWS * WA];
  __shared__ __align__(16) char sB0[NWS * WB];
  __shared__ __align__(16) char sB1[NWS * WB];
  int unit, slice;
  xcd_unit(blockIdx.x, D / 16, a.BH, unit, slice);
  const size_t bh = (size_t)unit;
  const int lane = threadIdx.x & 63, lr = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c0 = slice * 16, m0 = w * MHW;

  f32x4 h[MHW];
#pragma unroll
  for (int t = 0; t < MHW; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      h[t][i] = a.h_init ? a.h_init[(bh * D + 16 * (m0 + t) + 4 * g + i) * D + c0 + lr] : 0.f;
  const size_t js_ = a.js ? (size_t)a.js : (size_t)D * D, bs_ = a.bs ? (size_t)a.bs : (size_t)a.n * D * D;

  // the stages' LDS addresses as plain numbers (the compiler then does not
  // tie the LDS reads to the copies; the waits below are explicit)
  auto lds_addr = [](const void *p) {
    unsigned x = (unsigned)(size_t)(__attribute__((address_space(3))) const char *)p;
    asm volatile("" : "+s"(x));
    return x;
  };
  const unsigned sa0 = lds_addr(sA0) + w * WA, sa1 = lds_addr(sA1) + w * WA;
  const unsigned sb0 = lds_addr(sB0) + w * WB, sb1 = lds_addr(sB1) + w * WB;
  const unsigned voff_a = lr * D * 4 + 16 * g;                    // this lane's 16 bytes of an A copy
  const unsigned voff_b = (lane >> 2) * D * 4 + 16 * (lane & 3);  // and of a B copy
  auto dma = [](const char *base, unsigned voff, unsigned dst) {
    __builtin_amdgcn_global_load_lds((const void *)(base + voff), (__attribute__((address_space(3))) void *)(size_t)dst,
                                     16, 0, 0);
  };
  auto ubase = [](const float *p, size_t off) {
    return reinterpret_cast<const char *>(uniform64(reinterpret_cast<unsigned long long>(p + off)));
  };
  // step j's copies: B_j first, then A_j
  auto copy = [&](size_t j, unsigned sa, unsigned sb) {
    const size_t pj = bh * bs_ + j * js_ + (size_t)(16 * m0) * D;
#pragma unroll
    for (int t = 0; t < MHW; ++t) dma(ubase(a.Bm, pj + (size_t)(16 * t) * D + c0), voff_b, sb + t * 1024);
#pragma unroll
    for (int q = 0; q < 2 * F; ++q) {
      const int p = q >> 1, t = p / KB, kb = p % KB, half = q & 1;
      dma(ubase(a.A, pj + (size_t)(16 * t) * D + 32 * kb + 16 * half), voff_a, sa + q * 1024);
    }
  };
  copy(0, sa0, sb0);
  copy(a.n > 1 ? 1 : 0, sa1, sb1);

  auto step = [&](int j, auto Pc, auto Wc) {
    constexpr int P = decltype(Pc)::value;      // step parity: exchange buffer and stage
    constexpr int WAIT = decltype(Wc)::value;   // operations that may stay in flight
    const size_t jr = j + 2 < a.n ? j + 2 : (j + 1 < a.n ? j + 1 : j);   // last steps: copies repeat (unused)
    const char *sa = (P == 0 ? sA0 : sA1) + w * WA + lane * 16;
    const char *sb = (P == 0 ? sB0 : sB1) + w * WB;
    {
      const float x[8] = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
      xh[P][w][lane] = make_frag<PK::b>(x);
    }
    if constexpr (HIN) {
      float *dst = a.h_in + (bh * bs_ + j * js_) + c0 + lr;
#pragma unroll
      for (int t = 0; t < MHW; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(size_t)(16 * (m0 + t) + 4 * g + i) * D] = h[t][i];
    }
    lds_barrier();
    HF hb[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) hb[kb] = xh[P][kb][lane];
    // this step's copies landed
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(vm_lgkm0(WAIT));
    asm volatile("" ::: "memory");
    float4 fr[2 * F];
#pragma unroll
    for (int q = 0; q < 2 * F; ++q) fr[q] = *reinterpret_cast<const float4 *>(sa + q * 1024);
    float bc[MHW][4];
#pragma unroll
    for (int t = 0; t < MHW; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) bc[t][i] = *reinterpret_cast<const float *>(sb + t * 1024 + (4 * g + i) * 64 + lr * 4);
    // every read of this stage done before the next copies into it
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(vm_lgkm0(63));   // lgkmcnt(0); the memory counter left as it is
    asm volatile("" ::: "memory");
    copy(jr, P == 0 ? sa0 : sa1, P == 0 ? sb0 : sb1);
#pragma unroll
    for (int t = 0; t < MHW; ++t) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int p = t * KB + kb;
        const float x[8] = {fr[2 * p].x, fr[2 * p].y, fr[2 * p].z, fr[2 * p].w,
                            fr[2 * p + 1].x, fr[2 * p + 1].y, fr[2 * p + 1].z, fr[2 * p + 1].w};
        mma(acc, make_frag<PK::a>(x), hb[kb]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) h[t][i] = acc[i] + bc[t][i];
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  constexpr int W_FIRST = NOPS;                          // the start's second copies + step 0's stores
  constexpr int W_STEADY = NOPS + (HIN ? 4 * MHW : 0);   // step j-1's operations + step j's stores
  step(0, I0{}, std::integral_constant<int, W_FIRST>{});
  // then pairs of steps with no branch inside (so that the counter's state at
  // the loop head is the same on every path), and an odd last step
  int j = 1;
  for (; j + 1 < a.n; j += 2) {
    step(j, I1{}, std::integral_constant<int, W_STEADY>{});
    step(j + 1, I0{}, std::integral_constant<int, W_STEADY>{});
  }
  if (j < a.n) step(j, I1{}, std::integral_constant<int, W_STEADY>{});
  // (every copy done before the workgroup ends)
  __builtin_amdgcn_s_waitcnt(vm_lgkm0(0));
  if (a.h_final) {
#pragma unroll
    for (int t = 0; t < MHW; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) a.h_final[(bh * D + 16 * (m0 + t) + 4 * g + i) * D + c0 + lr] = h[t][i];
  }
}

// ----------------------------------------------------------------------------
// Blocked (two-level, log-depth in the block size) exclusive prefix of affine
// pairs: the pairs of every block of s consecutive groups are composed into
// one pair (COMPOSE), the sequential prefix runs over the blocks' pairs, and
// every block replays its own pairs from its incoming state (REPLAY).  Both
// block passes are walks of a state through the pairs' maps,
//   state <- A_j state + B_j,
// COMPOSE on the augmented state [X | Y] from [I | 0] (X the product of the
// block's A, Y its composed B; the composition law (A2,B2) o (A1,B1) =
// (A2 A1, A2 B1 + B2) of "GatedDeltaNet does not support
// ici_context_parallelism", section "The recurrence is affine, so it can be
// parallelized"), REPLAY on the state h from the block's incoming state,
// writing the state entering every pair (the exclusive prefix).  One
// workgroup of eight waves per (row bh, block) and 128 state columns (two for
// COMPOSE: X and Y); A_j, read once per workgroup and split once into
// matrix-core operand fragments in LDS (two buffers: the next pair's arrive
// during this pair's products), is shared by every wave, each holding 16
// columns of the state.
//
// The blocked prefix keeps its intermediates in the incoming-state array
// itself: for block beta (pairs beta s .. beta s + s - 1 of a row, s >= 3),
// slot beta s + 1 holds the block's composed A, slot beta s + 2 its composed
// B, and slot beta s the block's incoming state (written by the sequential
// prefix, read by REPLAY, which then writes every slot of the block).
constexpr int PW_COMPOSE = 0, PW_REPLAY = 1;
struct PairWalkArgs {
  int BH, J, s;               // rows, pairs per row, pairs per block
  const float *A, *Bm;        // [BH, J, D, D]
  float *h_in;                // [BH, J, D, D]: intermediates and the result
};

template <int PREC, int KIND>
__global__ __launch_bounds__(512) void pair_walk_kernel(PairWalkArgs a) {
  using PK = PolicyKinds<PREC>;
  using AF = Frag<PK::a>;
  using SF = Frag<PK::b>;
  static_assert(PK::a == PK::b && (PK::a == F_SPLIT || PK::a == F_F32), "fp32-accurate pair products");
  constexpr int MH = D / 16, KB = D / 32, NF = MH * KB;   // state row tiles, k-blocks, A fragments
  constexpr int NSL = 1;                                   // 16-column slices per wave
  constexpr int PER = NF * 64 / 512;                       // (fragment, lane) items staged per thread
  __shared__ __align__(16) char buf[2][NF * 2048];
  const int nblk = a.J / a.s;
  int unit, part;   // part: the 128 columns of the state this workgroup holds
  xcd_unit(blockIdx.x, KIND == PW_COMPOSE ? 2 : 1, a.BH * nblk, unit, part);
  const size_t bh = unit / nblk;
  const int blk = unit % nblk, j0 = blk * a.s;
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const size_t DD = (size_t)D * D;
  float *row = a.h_in + bh * a.J * DD;   // this row's slots

  // state tiles st[sl][m]: rows 16m + 4g + i, column c(sl) + lr of the
  // state (COMPOSE: columns 0..255 of [X | Y]; REPLAY: 0..127 of h)
  f32x4 st[NSL][MH];
  auto col0 = [&](int sl) { return D * part + 16 * (NSL * w + sl); };
#pragma unroll
  for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
    for (int m = 0; m < MH; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * m + 4 * g + i, c = col0(sl) + lr;
        st[sl][m][i] = KIND == PW_COMPOSE ? (c == r ? 1.f : 0.f) : row[(size_t)j0 * DD + (size_t)r * D + c];
      }
  // stage A_j: item (fragment f, lane ln) holds A[16m + lr'][32kb + kk(g', jj)]
  float ax[PER][8];
  auto load_a = [&](int j) {
    const float *Aj = a.A + (bh * a.J + j) * DD;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int it = tid + 512 * u, f = it / 64, ln = it % 64, m = f / KB, kb = f % KB;
      const float *p = Aj + (size_t)(16 * m + (ln & 15)) * D + 32 * kb + 4 * (ln >> 4);
      const float4 x0 = *reinterpret_cast<const float4 *>(p), x1 = *reinterpret_cast<const float4 *>(p + 16);
      ax[u][0] = x0.x; ax[u][1] = x0.y; ax[u][2] = x0.z; ax[u][3] = x0.w;
      ax[u][4] = x1.x; ax[u][5] = x1.y; ax[u][6] = x1.z; ax[u][7] = x1.w;
    }
  };
  auto put_a = [&](char *b) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int it = tid + 512 * u, f = it / 64, ln = it % 64;
      char *d = b + f * 2048 + ln * 16;
      if constexpr (PK::a == F_SPLIT) {
        bf16x8 hi, lo;
        to_bf16x8_split(ax[u], hi, lo);
        *reinterpret_cast<bf16x8 *>(d) = hi;
        *reinterpret_cast<bf16x8 *>(d + 1024) = lo;
      } else {
        *reinterpret_cast<float4 *>(d) = float4{ax[u][0], ax[u][1], ax[u][2], ax[u][3]};
        *reinterpret_cast<float4 *>(d + 1024) = float4{ax[u][4], ax[u][5], ax[u][6], ax[u][7]};
      }
    }
  };
  auto afrag = [&](const char *b, int f) -> AF {
    AF x;
    const char *p = b + f * 2048 + lane * 16;
    if constexpr (PK::a == F_SPLIT) {
      x.hi = *reinterpret_cast<const bf16x8 *>(p);
      x.lo = *reinterpret_cast<const bf16x8 *>(p + 1024);
    } else {
      const float4 x0 = *reinterpret_cast<const float4 *>(p), x1 = *reinterpret_cast<const float4 *>(p + 1024);
      x.v[0] = x0.x; x.v[1] = x0.y; x.v[2] = x0.z; x.v[3] = x0.w;
      x.v[4] = x1.x; x.v[5] = x1.y; x.v[6] = x1.z; x.v[7] = x1.w;
    }
    return x;
  };
  // B_j for this wave's columns that take it (COMPOSE: the Y half; REPLAY: all)
  const bool takes_b = KIND == PW_REPLAY || col0(0) >= D;
  f32x4 bq[NSL][MH];
  auto load_b = [&](int j) {
    const float *Bj = a.Bm + (bh * a.J + j) * DD;
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
      for (int m = 0; m < MH; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          bq[sl][m][i] = takes_b ? Bj[(size_t)(16 * m + 4 * g + i) * D + (col0(sl) + lr) % D] : 0.f;
  };

  load_a(j0);
  put_a(buf[0]);
  __syncthreads();
  for (int t = 0; t < a.s; ++t) {
    const int j = j0 + t;
    const bool more = t + 1 < a.s;
    if (more) load_a(j + 1);
    load_b(j);
    if (KIND == PW_REPLAY) {   // the state entering pair j
#pragma unroll
      for (int m = 0; m < MH; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) row[(size_t)j * DD + (size_t)(16 * m + 4 * g + i) * D + col0(0) + lr] = st[0][m][i];
    }
    const char *cur = buf[t & 1];
    SF sb[NSL][KB];
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const float x[8] = {st[sl][2 * kb][0], st[sl][2 * kb][1], st[sl][2 * kb][2], st[sl][2 * kb][3],
                            st[sl][2 * kb + 1][0], st[sl][2 * kb + 1][1], st[sl][2 * kb + 1][2], st[sl][2 * kb + 1][3]};
        sb[sl][kb] = make_frag<PK::b>(x);
      }
#pragma unroll
    for (int m = 0; m < MH; ++m) {
      f32x4 acc[NSL];
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl) acc[sl] = bq[sl][m];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const AF af = afrag(cur, m * KB + kb);
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) mma(acc[sl], af, sb[sl][kb]);
      }
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl) st[sl][m] = acc[sl];
    }
    if (more) put_a(buf[(t + 1) & 1]);
    __syncthreads();
  }
  if (KIND == PW_COMPOSE) {   // X -> slot j0 + 1, Y -> slot j0 + 2
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      const int c = col0(sl) + lr;
      float *dst = row + (size_t)(j0 + (c < D ? 1 : 2)) * DD + c % D;
#pragma unroll
      for (int m = 0; m < MH; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(size_t)(16 * m + 4 * g + i) * D] = st[sl][m][i];
    }
  }
}

// ----------------------------------------------------------------------------
// output, one 4-wave workgroup per (chunk, value head), computed transposed:
//   O^T = h^T (diag(e^G) Q)^T + V'^T P^T,   P^T = (K Q^T) o Gamma^T o [i <= r].
// Phase A forms P^T once per chunk: wave w takes query-row tiles {w, R-1-w}
// (balancing the triangle), reads K from LDS (copied in with
// global_load_lds, row pieces XOR-swizzled against bank conflicts) and its
// queries from memory, masks, decays and splits each tile pair and leaves it
// in LDS as the B-operand fragment of (query tile, key block of 32).
// Phase B: wave w owns state columns 32w .. 32w+31 for every query row; its
// h^T and V'^T fragments (stored by the walk in this order) are loaded once
// into registers, the queries stream from memory one tile ahead, and P^T
// comes from LDS.  All contractions use the k order of two stacked result
// tiles (lane group g holds k = 4g..4g+3 and 16+4g..16+4g+3 of each 32).
template <int C, typename TI> struct OutLds {
  static constexpr int RP = D * (int)sizeof(TI) / 16;   // 16-byte pieces per K row
  static constexpr int KB = C * RP * 16;                // K tile bytes
  static constexpr int R = C / 16;                      // query-row tiles
  // (query tile rt, key block kp <= rt/2) pairs before tile rt
  __host__ __device__ static constexpr int pbase(int rt) {
    return (rt & 1) ? (rt / 2 + 1) * (rt / 2 + 1) : (rt / 2) * (rt / 2 + 1);
  }
  static constexpr int NPAIR = pbase(R);
  static constexpr int POFF = KB, GOFF = POFF + NPAIR * 2048, BYTES = GOFF + 4 * C;
  // K[r][piece c] lives at piece position c ^ (r mod 16) of row r
  __device__ static int kpos(int r, int c) { return r * RP + (c ^ (r & 15)); }
};

template <int C, typename TI, int MODE, typename TO, bool RAG>   // RAG as for prep_kernel
__global__ __launch_bounds__(NT, 2) void out_kernel(FwdArgs a) {
  using PR = Prec<MODE>;
  using PKq = PolicyKinds<PR::exact>;   // K x Q^T
  using PKh = PolicyKinds<PR::hq>;      // h^T x Q^T
  using PKv = PolicyKinds<PR::pv>;      // V'^T x P^T
  static_assert(PKq::b == PKh::b, "one query fragment serves both products");
  using OL = OutLds<C, TI>;
  constexpr bool F32 = sizeof(TI) == 4;
  constexpr int R = C / 16;              // query-row tiles
  constexpr int RU = R >= 8 ? 2 : 1;     // phase-A row tiles per wave
  constexpr int MH = D / 16, MV = C / 16, KBD = D / 32, KBC = C / 32;
  static_assert(R == 4 * RU, "phase A: R/4 row tiles per wave");
  using SH = Store<PR::h_store>;
  using SV = Store<PR::v_store>;
  static_assert(PKh::a == SH::frag && PKv::a == SV::frag, "stored copies are used as stored");
  __shared__ __align__(16) char lds[OL::BYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, g = lane >> 4, lq = g * 4;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  int n, b, hv;
  chunk_head_unit(blockIdx.x, a, n, b, hv);
  const size_t bh = (size_t)b * a.Hv + hv;
  const int hq = hv / (a.Hv / a.Hqk);
  const size_t cb = bh * a.N + n;
  const bool packed = RAG && a.ctab;   // packed sequences (RAG instantiation only)
  if (packed && n >= *a.ntot) return;   // past the last chunk
  const size_t tok0 = packed ? (size_t)a.ctab[n].x : (size_t)b * a.T + (size_t)n * C;   // first token of the chunk
  // real tokens of the chunk (a partial last chunk: rows past it read the
  // last real token's q and k, finite values that meet zero V' rows, and
  // write no output)
  const int rows = !RAG ? C : packed ? a.ctab[n].y : (int)(a.T - (size_t)n * C < (size_t)C ? a.T - (size_t)n * C : (size_t)C);
  const float *Gs = reinterpret_cast<const float *>(lds + OL::GOFF);

  // K tile and G into LDS
  {
    const char *kg = reinterpret_cast<const char *>(a.k) + ((tok0 * a.Hqk + hq) * D) * sizeof(TI);
    const size_t krow = (size_t)a.Hqk * D * sizeof(TI);   // bytes between tokens
    using LDSP = __attribute__((address_space(3))) void *;
#pragma unroll
    for (int jj = 0; jj < OL::KB / 4096; ++jj) {
      const int j = jj * 4 + wv;   // 1 KB block: pieces 64 j + lane of the swizzled tile
      const int p = j * 64 + lane, r = p / OL::RP, c = (p % OL::RP) ^ (r & 15);
      __builtin_amdgcn_global_load_lds((const void *)(kg + (r < rows ? r : rows - 1) * krow + c * 16), (LDSP)(lds + j * 1024), 16, 0, 0);
    }
    if (wv == 3 && lane < C / 4)
      __builtin_amdgcn_global_load_lds((const void *)(a.G + cb * C + lane * 4), (LDSP)(lds + OL::GOFF), 16, 0, 0);
  }
  // query fragments of one row tile, k order kk(g, j)
  using QF = Frag<PKq::b>;
  auto load_q = [&](int rt, QF (&q)[KBD]) {
    const int qr = 16 * rt + lr < rows ? 16 * rt + lr : rows - 1;
    const TI *qrow = reinterpret_cast<const TI *>(a.q) + ((tok0 + qr) * a.Hqk + hq) * D;
#pragma unroll
    for (int kb = 0; kb < KBD; ++kb) {
      TI t[8];
      if constexpr (F32) {
        *reinterpret_cast<float4 *>(t) = *reinterpret_cast<const float4 *>(qrow + 32 * kb + 4 * g);
        *reinterpret_cast<float4 *>(t + 4) = *reinterpret_cast<const float4 *>(qrow + 32 * kb + 16 + 4 * g);
      } else {
        *reinterpret_cast<uint2 *>(t) = *reinterpret_cast<const uint2 *>(qrow + 32 * kb + 4 * g);
        *reinterpret_cast<uint2 *>(t + 4) = *reinterpret_cast<const uint2 *>(qrow + 32 * kb + 16 + 4 * g);
      }
      if constexpr (PKq::b == F_BF16) {
        q[kb].hi = *reinterpret_cast<const bf16x8 *>(t);
      } else {
        float x8[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x8[j] = to_f32(t[j]);
        q[kb] = make_frag<PKq::b>(x8);
      }
    }
  };
  QF qa[RU][KBD];
#pragma unroll
  for (int u = 0; u < RU; ++u) load_q(u == 0 ? wv : R - 1 - wv, qa[u]);
  // phase-B operands of this wave's columns: h^T (2 column tiles x KBD) and
  // V'^T (2 x KBC) fragments, as stored by the walk; issued last, they arrive
  // during phase A (one 16-byte load per bf16 fragment, two per split or fp32 one)
  constexpr int NLATE = SH::loads * 2 * KBD + SV::loads * 2 * KBC;
  static_assert(NLATE <= 63, "memory counter range");
  Frag<PKh::a> hf[2][KBD];
  Frag<PKv::a> vf[2][KBC];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int s = 2 * wv + ct;   // walk slice
    const float *hs = a.Hs + (cb * (D / 16) + s) * MH * SH::tile_floats;
    const float *vs = a.Vn + (cb * (D / 16) + s) * MV * SV::tile_floats;
#pragma unroll
    for (int kb = 0; kb < KBD; ++kb) {
      if constexpr (PR::h_store == ST_BF16) {
        hf[ct][kb].hi = *reinterpret_cast<const bf16x8 *>(hs + (kb * 64 + lane) * 4);
      } else if constexpr (PR::h_store == ST_SPLIT) {
        hf[ct][kb].hi = *reinterpret_cast<const bf16x8 *>(hs + ((2 * kb) * 64 + lane) * 4);
        hf[ct][kb].lo = *reinterpret_cast<const bf16x8 *>(hs + ((2 * kb + 1) * 64 + lane) * 4);
      } else {
        const float4 x0 = *reinterpret_cast<const float4 *>(hs + ((2 * kb) * 64 + lane) * 4);
        const float4 x1 = *reinterpret_cast<const float4 *>(hs + ((2 * kb + 1) * 64 + lane) * 4);
        const float x8[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        hf[ct][kb] = make_frag<PKh::a>(x8);
      }
    }
#pragma unroll
    for (int kp = 0; kp < KBC; ++kp) {
      if constexpr (PR::v_store == ST_BF16) {
        vf[ct][kp].hi = *reinterpret_cast<const bf16x8 *>(vs + (kp * 64 + lane) * 4);
      } else if constexpr (PR::v_store == ST_SPLIT) {
        vf[ct][kp].hi = *reinterpret_cast<const bf16x8 *>(vs + ((2 * kp) * 64 + lane) * 4);
        vf[ct][kp].lo = *reinterpret_cast<const bf16x8 *>(vs + ((2 * kp + 1) * 64 + lane) * 4);
      } else {
        const float4 x0 = *reinterpret_cast<const float4 *>(vs + ((2 * kp) * 64 + lane) * 4);
        const float4 x1 = *reinterpret_cast<const float4 *>(vs + ((2 * kp + 1) * 64 + lane) * 4);
        const float x8[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        vf[ct][kp] = make_frag<PKv::a>(x8);
      }
    }
  }
  // the K tile and G copies (issued first) done in every wave; the phase-B
  // loads may still be in flight
  __builtin_amdgcn_s_waitcnt((NLATE & 15) | ((NLATE >> 4) << 14) | (0x7 << 4) | (0xF << 8));   // vmcnt(NLATE)
  __builtin_amdgcn_s_barrier();

  // this lane's byte offsets of its K fragment halves within a 16-row key
  // tile: row lr, piece c = (32kb + 16hh + 4g) * size / 16 stored at c ^ lr
  int koff[KBD][2];
#pragma unroll
  for (int kb = 0; kb < KBD; ++kb)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int k = 32 * kb + 16 * hh + 4 * g;
      const int c = k * (int)sizeof(TI) / 16, off = (k * (int)sizeof(TI)) % 16;
      koff[kb][hh] = lr * OL::RP * 16 + ((c ^ lr) * 16) + off;
    }

  // ---- phase A: P^T fragments into LDS ----
#pragma unroll
  for (int u = 0; u < RU; ++u) {
    const int rt = u == 0 ? wv : R - 1 - wv;
    const int r = 16 * rt + lr;   // this lane's query row (result column)
    const float Gr = Gs[r] * LOG2E;
#pragma unroll
    for (int kp = 0; kp < R / 2; ++kp) {
      if (2 * kp > rt) continue;
      const bool two = 2 * kp + 1 <= rt;
      Frag<PKq::a> kf[2][KBD];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const char *tile = lds + (32 * kp + 16 * t) * OL::RP * 16;   // key rows 32kp + 16t ..
#pragma unroll
        for (int kb = 0; kb < KBD; ++kb) {
          if constexpr (!F32 && PKq::a == F_BF16) {
            const uint2 w0 = *reinterpret_cast<const uint2 *>(tile + koff[kb][0]);
            const uint2 w1 = *reinterpret_cast<const uint2 *>(tile + koff[kb][1]);
            kf[t][kb].hi = __builtin_bit_cast(bf16x8, uint4{w0.x, w0.y, w1.x, w1.y});
          } else {
            float x8[8];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              if constexpr (F32) {
                const float4 v4 = *reinterpret_cast<const float4 *>(tile + koff[kb][hh]);
                x8[4 * hh] = v4.x; x8[4 * hh + 1] = v4.y; x8[4 * hh + 2] = v4.z; x8[4 * hh + 3] = v4.w;
              } else {
                const uint2 v2 = *reinterpret_cast<const uint2 *>(tile + koff[kb][hh]);
                const __bf16 *e = reinterpret_cast<const __bf16 *>(&v2);
#pragma unroll
                for (int j = 0; j < 4; ++j) x8[4 * hh + j] = (float)e[j];
              }
            }
            kf[t][kb] = make_frag<PKq::a>(x8);
          }
        }
      }
      const float4 gk0 = *reinterpret_cast<const float4 *>(Gs + 32 * kp + lq);
      const float4 gk1 = *reinterpret_cast<const float4 *>(Gs + 32 * kp + 16 + lq);
      __builtin_amdgcn_sched_barrier(0);
      f32x4 p0 = zero4(), p1 = zero4();
#pragma unroll
      for (int kb = 0; kb < KBD; ++kb) {
        mma(p0, kf[0][kb], qa[u][kb]);
        if (two) mma(p1, kf[1][kb], qa[u][kb]);
      }
      const float g0[4] = {gk0.x, gk0.y, gk0.z, gk0.w}, g1[4] = {gk1.x, gk1.y, gk1.z, gk1.w};
      float b8[8];
      if (2 * kp + 1 < rt) {
        // both key tiles wholly before this query tile: no mask
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          b8[i] = p0[i] * exp2_fast(Gr - g0[i] * LOG2E);
          b8[4 + i] = p1[i] * exp2_fast(Gr - g1[i] * LOG2E);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int k0i = 32 * kp + lq + i, k1i = k0i + 16;
          b8[i] = k0i <= r ? p0[i] * exp2_fast(Gr - g0[i] * LOG2E) : 0.f;
          b8[4 + i] = (two && k1i <= r) ? p1[i] * exp2_fast(Gr - g1[i] * LOG2E) : 0.f;
        }
      }
      // the B-operand fragment (hi, lo planes; or 8 fp32 in two halves)
      char *pf = lds + OL::POFF + (OL::pbase(rt) + kp) * 2048 + lane * 16;
      const auto bf = make_frag<PKv::b>(b8);
      if constexpr (PKv::b == F_SPLIT) {
        *reinterpret_cast<bf16x8 *>(pf) = bf.hi;
        *reinterpret_cast<bf16x8 *>(pf + 1024) = bf.lo;
      } else {
        *reinterpret_cast<float4 *>(pf) = float4{bf.v[0], bf.v[1], bf.v[2], bf.v[3]};
        *reinterpret_cast<float4 *>(pf + 1024) = float4{bf.v[4], bf.v[5], bf.v[6], bf.v[7]};
      }
    }
  }
  lds_barrier();
  // the query fragments, over the K tile (read by no one from here on): the
  // waves' phase-A tiles cover every query tile once, and phase B reads them
  // back from LDS instead of fetching each tile again in every wave
  static_assert(R * KBD * 64 * sizeof(QF) <= (size_t)OL::KB, "query fragments fit the K tile");
  QF *qs = reinterpret_cast<QF *>(lds);   // [R][KBD][64]
#pragma unroll
  for (int u = 0; u < RU; ++u) {
    const int rt = u == 0 ? wv : R - 1 - wv;
#pragma unroll
    for (int kb = 0; kb < KBD; ++kb) qs[(rt * KBD + kb) * 64 + lane] = qa[u][kb];
  }
  lds_barrier();

  // ---- phase B: this wave's 32 columns for every query tile ----
  TO *og = reinterpret_cast<TO *>(a.o);
  auto tile_out = [&](int rt) {
    const int r = 16 * rt + lr;
    QF q[KBD];
#pragma unroll
    for (int kb = 0; kb < KBD; ++kb) q[kb] = qs[(rt * KBD + kb) * 64 + lane];
    f32x4 acc1[2], acc2[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) acc1[ct] = acc2[ct] = zero4();
#pragma unroll
    for (int kb = 0; kb < KBD; ++kb)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) mma(acc1[ct], hf[ct][kb], q[kb]);
#pragma unroll
    for (int kp = 0; kp < KBC; ++kp) {
      if (2 * kp > rt) continue;
      const char *pf = lds + OL::POFF + (OL::pbase(rt) + kp) * 2048 + lane * 16;
      Frag<PKv::b> bf;
      if constexpr (PKv::b == F_SPLIT) {
        bf.hi = *reinterpret_cast<const bf16x8 *>(pf);
        bf.lo = *reinterpret_cast<const bf16x8 *>(pf + 1024);
      } else {
        const float4 x0 = *reinterpret_cast<const float4 *>(pf), x1 = *reinterpret_cast<const float4 *>(pf + 1024);
        bf.v[0] = x0.x; bf.v[1] = x0.y; bf.v[2] = x0.z; bf.v[3] = x0.w;
        bf.v[4] = x1.x; bf.v[5] = x1.y; bf.v[6] = x1.z; bf.v[7] = x1.w;
      }
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) mma(acc2[ct], vf[ct][kp], bf);
    }
    const float er = exp2_fast(Gs[r] * LOG2E);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      // lane holds O^T[c = 32w + 16ct + 4g + i][r]
      TO *dst = og + ((tok0 + r) * a.Hv + hv) * D + 32 * wv + 16 * ct + lq;
      TO ov[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ov[i] = from_f32<TO>(er * acc1[ct][i] + acc2[ct][i]);
      if (r < rows) {
        if constexpr (sizeof(TO) == 4) st16_stream(dst, ov);
        else st8_stream(dst, ov);
      }
    }
  };
#pragma unroll
  for (int rt = 0; rt < R; ++rt) tile_out(rt);
}

// ----------------------------------------------------------------------------
// walk with outputs (rows a5, a6 and a9 in one kernel): the sequential chunk
// walk of walk_shared_kernel that also forms each chunk's outputs from the
// chunk-start state and corrected values it holds in registers, so neither
// goes to memory.  Per chunk, each wave (SPW 16-column slices c0.. of the
// state; SPW = 2: one workgroup of four waves holds all 128 columns of a
// walk, so that P^T and the chunk's copies serve every column once):
//   P^T = (K Q^T) o Gamma^T o [i <= r]              (shared: the workgroup's
//                                                    waves split its tiles)
//   V' = U - W h                                   (W from LDS, h as B operand)
//   O^T[c][r] = e^{G_r} (h^T Q^T)[c][r] + (V'^T P^T)[c][r]   for c in a slice
//   h <- e^{G_last} h + K^T (d o V')
// U is loaded at the chunk's start and lands while P^T is formed.
// The chunk-start state and V' are A operands of the output products as they
// stand in registers: two stacked result tiles give lane group g the
// k-values kk(g, j) of a block of 32, the k order in which the query and key
// rows are read (and in which P^T's tiles are formed).
//
// LDS holds one chunk's operands in four slots -- W fragments (then the P^T
// fragments: they wait in registers while V' reads W), K^T fragments, the Q
// tile and the K tile -- plus G; each slot is refilled for the next chunk
// (global_load_lds, no registers) as soon as every wave is past its last
// read of it:
//   K after V' (P^T was formed before it),  Q after h^T Q^T,
//   G and W after V'^T P^T,  K^T after the state update.
// The next chunk's P^T, which needs K and Q first, thus finds them copied
// most of a chunk earlier.  The waits before the barriers count the copies,
// U loads and o stores each wave issued after the ones waited for (the
// memory counter completes in issue order).
template <int C, typename TI> struct WalkOutLds {
  using OL = OutLds<C, TI>;
  static constexpr int BPF = 8 * (int)sizeof(TI) / 16;            // 1 KB blocks per fragment
  static constexpr int FW = (C / 16) * (D / 32), FK = (D / 16) * (C / 32);
  static constexpr int WB = FW * BPF * 1024, KTB = FK * BPF * 1024;  // W, K^T fragment bytes
  static constexpr int QB = OL::KB;                                 // Q (or K) tile bytes
  static constexpr int PB = OL::NPAIR * 2048;                       // P^T fragment bytes
  static constexpr int WPB = PB > WB ? PB : WB;                     // W, then P^T
};

// wait (s_waitcnt IMM), then the workgroup barrier; no memory access moves
// across it
template <int IMM>
__device__ __forceinline__ void wait_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(IMM);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The A columns of the augmented state [A | h] (WALK_A): A <- e^{G_last} A -
// K^T (d o (W A)) from A = I, written to a.pairA at the end.  Workgroups of
// walk_out_kernel that hold A columns run this instead of the output-forming
// loop: only W, K^T and G are needed, copied into the same LDS slots.
template <int C, typename TI, int MODE, int WPG>
__device__ __forceinline__ void walk_a_columns(const FwdArgs &a, size_t bh, int slice, char *sW, char *sKt, float *sG) {
  using PR = Prec<MODE>;
  using PKw = PolicyKinds<PR::wh>;
  using PKk = PolicyKinds<PR::kv>;
  using L = WalkOutLds<C, TI>;
  constexpr bool F32 = sizeof(TI) == 4;
  constexpr int MV = C / 16, MH = D / 16, KBW = D / 32, KBK = C / 32, BPF = L::BPF;
  constexpr int NCW = L::WB / 1024 / WPG, NCK = L::KTB / 1024 / WPG, GL = C / 4 / WPG;
  static_assert(KBK >= 1 && NCW >= 1 && NCK >= 1, "whole copies");
  const int lane = threadIdx.x & 63, g = lane >> 4, lr = lane & 15, lq = 4 * g;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c0 = 16 * slice;   // column of A
  const int cpj = a.cpj;
  const size_t cb0 = uniform64(bh * a.N + a.n0);
  const long long ktoff = (long long)uniform64((unsigned long long)kt_offset(a, bh));
  f32x4 h[MH];
#pragma unroll
  for (int m = 0; m < MH; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) h[m][i] = 16 * m + 4 * g + i == c0 + lr ? 1.f : 0.f;
  auto lds_addr = [](const void *p) {
    unsigned x = (unsigned)(size_t)(__attribute__((address_space(3))) const char *)p;
    asm volatile("" : "+s"(x));
    return x;
  };
  auto dma = [&](const char *ubase, unsigned voff, unsigned ldst) {
    __builtin_amdgcn_global_load_lds((const void *)(ubase + voff), (__attribute__((address_space(3))) void *)(size_t)ldst,
                                     16, 0, 0);
  };
  auto ubase = [](const void *p, size_t off) -> const char * {
    return reinterpret_cast<const char *>(uniform64(reinterpret_cast<unsigned long long>(p) + off));
  };
  const unsigned fl = lane * 16 * BPF;
  auto copy_frags = [&](const char *src, char *slot, int ncopies) {
    const unsigned ls = lds_addr(slot);
    for (int jj = 0; jj < ncopies; ++jj) {
      const int j = jj * WPG + wv;
      dma(ubase(src, (size_t)(j / BPF) * 1024 * BPF + (j % BPF) * 16), fl, ls + j * 1024);
    }
  };
  auto copy_w = [&](size_t cb) { copy_frags(reinterpret_cast<const char *>(a.W) + cb * C * D * sizeof(TI), sW, NCW); };
  auto copy_ktg = [&](size_t cb) {
    copy_frags(reinterpret_cast<const char *>(a.Kt) + (cb + ktoff) * D * C * sizeof(TI), sKt, NCK);
    if (lane < GL) dma(ubase(a.G, (cb * C + wv * GL * 4) * sizeof(float)), lane * 16, lds_addr(sG) + wv * GL * 16);
  };
  auto frag = [&](const char *slot, int p) -> Frag<PKw::a> {
    Frag<PKw::a> f;
    const char *base = slot + p * BPF * 1024 + lane * 16;
    if constexpr (F32) {
      const float4 x0 = *reinterpret_cast<const float4 *>(base);
      const float4 x1 = *reinterpret_cast<const float4 *>(base + 1024);
      f.v[0] = x0.x; f.v[1] = x0.y; f.v[2] = x0.z; f.v[3] = x0.w;
      f.v[4] = x1.x; f.v[5] = x1.y; f.v[6] = x1.z; f.v[7] = x1.w;
    } else {
      f.hi = *reinterpret_cast<const bf16x8 *>(base);
    }
    return f;
  };
  copy_w(cb0);
  copy_ktg(cb0);
  wait_barrier<vm_lgkm0(0)>();
  for (int cc = 0; cc < cpj; ++cc) {
    const size_t cb = cb0 + cc;
    const bool more = cc + 1 < cpj;
    // V'_A = -W A
    Frag<PKw::b> hb[KBW];
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb) {
      const float x[8] = {h[2 * kb][0], h[2 * kb][1], h[2 * kb][2], h[2 * kb][3],
                          h[2 * kb + 1][0], h[2 * kb + 1][1], h[2 * kb + 1][2], h[2 * kb + 1][3]};
      hb[kb] = make_frag<PKw::b>(x);
    }
    f32x4 vps[MV];
    {
      Frag<PKw::a> fa[2][KBW];
#pragma unroll
      for (int kb = 0; kb < KBW; ++kb) fa[0][kb] = frag(sW, kb);
#pragma unroll
      for (int m = 0; m < MV; ++m) {
        if (m + 1 < MV) {
#pragma unroll
          for (int kb = 0; kb < KBW; ++kb) fa[(m + 1) & 1][kb] = frag(sW, (m + 1) * KBW + kb);
        }
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb) mma(acc, fa[m & 1][kb], hb[kb]);
        vps[m] = f32x4{-acc[0], -acc[1], -acc[2], -acc[3]};
      }
    }
    // every wave past W; this chunk's K^T and G landed
    wait_barrier<vm_lgkm0(0)>();
    if (more) copy_w(cb + 1);
    // A <- e^{G_last} A + K^T (d o V'_A)
    const float gl2 = sG[C - 1] * LOG2E;
    const float gl = exp2_fast(gl2);
    Frag<PKk::b> vb[KBK];
#pragma unroll
    for (int kb = 0; kb < KBK; ++kb) {
      float y[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int m = 2 * kb + j / 4, i = j % 4;
        y[j] = vps[m][i] * exp2_fast(gl2 - sG[16 * m + lq + i] * LOG2E);
      }
      vb[kb] = make_frag<PKk::b>(y);
    }
    {
      Frag<PKw::a> fk[2][KBK];
#pragma unroll
      for (int kb = 0; kb < KBK; ++kb) fk[0][kb] = frag(sKt, kb);
#pragma unroll
      for (int m = 0; m < MH; ++m) {
        if (m + 1 < MH) {
#pragma unroll
          for (int kb = 0; kb < KBK; ++kb) fk[(m + 1) & 1][kb] = frag(sKt, (m + 1) * KBK + kb);
        }
        f32x4 acc2 = zero4();
#pragma unroll
        for (int kb = 0; kb < KBK; ++kb) mma(acc2, fk[m & 1][kb], vb[kb]);
#pragma unroll
        for (int i = 0; i < 4; ++i) h[m][i] = gl * h[m][i] + acc2[i];
      }
    }
    if (more) {
      wait_barrier<vm_lgkm0(0)>();   // every wave past K^T and G; the next chunk's W landed
      copy_ktg(cb + 1);
    }
  }
#pragma unroll
  for (int m = 0; m < MH; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) a.pairA[bh * D * D + (size_t)(16 * m + 4 * g + i) * D + c0 + lr] = h[m][i];
}

template <int C, typename TI, int MODE, typename TO, int WPG, bool RAG, int KIND, int SPW>
__global__ __launch_bounds__(64 * WPG) void walk_out_kernel(FwdArgs a) {
  using PR = Prec<MODE>;
  using PKw = PolicyKinds<PR::wh>;      // W x h
  using PKk = PolicyKinds<PR::kv>;      // K^T x (d o V')
  using PKq = PolicyKinds<PR::exact>;   // K x Q^T
  using PKh = PolicyKinds<PR::hq>;      // h^T x Q^T
  using PKv = PolicyKinds<PR::pv>;      // V'^T x P^T
  using L = WalkOutLds<C, TI>;
  using OL = OutLds<C, TI>;
  constexpr bool F32 = sizeof(TI) == 4;
  static_assert(PKw::a == (F32 ? F_F32 : F_BF16) && PKk::a == PKw::a, "W and K^T fragments are used as stored");
  static_assert(PKq::a == PKq::b && PKq::b == PKh::b, "one query fragment serves both products");
  static_assert(PKw::b == PKh::a || (PKw::b == F_BF16 && PKh::a == F_SPLIT), "W h takes the state split for h^T Q^T");
  constexpr int MV = C / 16, MH = D / 16, KBW = D / 32, KBK = C / 32, R = C / 16;
  static_assert(KIND == WALK || KIND == WALK_A, "walk kinds with outputs");
  static_assert(SPW == 1 || (SPW == 2 && KIND == WALK), "two slices per wave: walks without A columns");
  constexpr int NGH = (D / 16) / (WPG * SPW);              // workgroups of h columns per walk
  constexpr int NG = (KIND == WALK_A ? 2 : 1) * NGH;        // workgroups per walk (A columns first)
  constexpr int BPF = L::BPF;
  // per wave and chunk: 1 KB copies of W, K^T, Q (and K); U loads; o stores
  constexpr int NCW = L::WB / 1024 / WPG, NCK = L::KTB / 1024 / WPG, NCQ = L::QB / 1024 / WPG;
  static_assert(L::WB % (1024 * WPG) == 0 && L::KTB % (1024 * WPG) == 0 && L::QB % (1024 * WPG) == 0,
                "copies shared out evenly");
  constexpr int GL = C / 4 / WPG;   // lanes of each wave copying 16 bytes of G
  static_assert(GL >= 1 && GL * 4 * WPG == C, "G copies shared out evenly");
  constexpr int NU = MV * SPW;
  // o stores counted as issued: none in the partial-chunk instantiation,
  // where a store may be skipped
  constexpr int NST = RAG ? 0 : R * SPW;
  constexpr int RU = R / (2 * WPG) > 0 ? 2 : 1;   // query tiles per wave in forming P^T
  static_assert(WPG == 4 && R == 4 * RU, "P^T: query tiles {w, R-1-w} (R = 8) or {w} (R = 4) per wave");
  // one array per slot (the compiler then tells the LDS reads of one slot
  // from the copies into another, and waits for neither at the reads)
  __shared__ __align__(16) char sW[L::WPB];   // W, then P^T
  __shared__ __align__(16) char sKt[L::KTB];
  __shared__ __align__(16) char sQ[L::QB];
  __shared__ __align__(16) char sPK[L::QB];   // K
  __shared__ __align__(16) float sG[C];

  size_t bh;
  int job, grp;
  walk_unit(blockIdx.x, NG, a, bh, job, grp);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (KIND == WALK_A) {
    if (grp < NGH) {   // (uniform per workgroup) columns of A
      walk_a_columns<C, TI, MODE, WPG>(a, bh, grp * WPG + wv, sW, sKt, sG);
      return;
    }
    grp -= NGH;
  }
  const int b = (int)(bh / a.Hv), hv = (int)(bh % a.Hv), hq = hv / (a.Hv / a.Hqk);
  const int lane = threadIdx.x & 63, lr = lane & 15, g = lane >> 4, lq = 4 * g;
  // this wave's state slices: slice0 .. slice0 + SPW - 1, columns c0 + 16 s ..
  const int slice0 = (grp * WPG + wv) * SPW, c0 = 16 * slice0;
  const int nfirst = a.n0 + job * a.cpj;   // first chunk of this walk in its sequence row
  const int cpj = a.cpj;
  const size_t cb0 = uniform64(bh * a.N + nfirst);
  const long long ktoff = (long long)uniform64((unsigned long long)kt_offset(a, bh));

  // state tiles: h[s][m] holds rows 16m + 4g + i, column c0 + 16s + lr
  f32x4 h[SPW][MH];
#pragma unroll
  for (int s = 0; s < SPW; ++s)
#pragma unroll
    for (int m = 0; m < MH; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kr = 16 * m + 4 * g + i;
        float x = 0.f;
        if (a.init) {
          const float *src = a.init_per_job ? a.init + (bh * a.jobs + job) * D * D : a.init + bh * D * D;
          x = src[(size_t)kr * D + c0 + 16 * s + lr];
        }
        h[s][m][i] = x;
      }
  auto store_final = [&]() {
    if (a.fin && job == a.jobs - 1) {   // (the last group's end state)
#pragma unroll
      for (int s = 0; s < SPW; ++s)
#pragma unroll
        for (int m = 0; m < MH; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) a.fin[bh * D * D + (size_t)(16 * m + 4 * g + i) * D + c0 + 16 * s + lr] = h[s][m][i];
    }
  };
  if (cpj == 0) {
    store_final();
    return;
  }

  // LDS destinations of the copies as plain numbers (so that the compiler
  // does not tie the LDS reads to the copies and wait for all of them), and
  // re-derived at each use through an empty asm statement: hoisted out of the
  // chunk loop, the 33 copy destinations and their global bases would hold as
  // many scalar registers for the whole walk
  auto lds_addr = [](const void *p) {
    unsigned x = (unsigned)(size_t)(__attribute__((address_space(3))) const char *)p;
    asm volatile("" : "+s"(x));
    return x;
  };
  // copies: a wave-uniform 64-bit base (scalar registers) plus a 32-bit
  // per-lane offset
  auto dma = [&](const char *ubase, unsigned voff, unsigned ldst) {
    __builtin_amdgcn_global_load_lds((const void *)(ubase + voff), (__attribute__((address_space(3))) void *)(size_t)ldst,
                                     16, 0, 0);
  };
  auto ubase = [](const void *p, size_t off) -> const char * {
    return reinterpret_cast<const char *>(uniform64(reinterpret_cast<unsigned long long>(p) + off));
  };
  const unsigned fl = lane * 16 * BPF;   // this lane's bytes within a fragment
  // fragment-major tensors: LDS block j = half j % BPF of fragment j / BPF
  auto copy_frags = [&](const char *src, char *slot, int ncopies) {
    const unsigned ls = lds_addr(slot);
    for (int jj = 0; jj < ncopies; ++jj) {   // (not unrolled: one base at a time)
      const int j = jj * WPG + wv;
      dma(ubase(src, (size_t)(j / BPF) * 1024 * BPF + (j % BPF) * 16), fl, ls + j * 1024);
    }
  };
  auto copy_w = [&](size_t cb) { copy_frags(reinterpret_cast<const char *>(a.W) + cb * C * D * sizeof(TI), sW, NCW); };
  auto copy_kt = [&](size_t cb) {
    copy_frags(reinterpret_cast<const char *>(a.Kt) + (cb + ktoff) * D * C * sizeof(TI), sKt, NCK);
  };
  // a C x D tile of q or k (query/key head hq) in the swizzled row-major
  // layout of OutLds: piece c of row r at piece position c ^ (r mod 16).  Rows
  // past the chunk's real tokens repeat its last one (finite values that meet
  // zero rows of V' and write no output).  LDS block j holds pieces 64j ..
  // 64j + 63: rows RB j .. RB j + RB - 1 (RB = 64 / RP).
  constexpr int RB = 64 / OL::RP;
  const size_t rowb = (size_t)a.Hqk * D * sizeof(TI);   // bytes between tokens
  auto copy_rows = [&](const void *src, size_t tok0, int rows, char *slot) {
    const unsigned ls = lds_addr(slot);
    const char *base = reinterpret_cast<const char *>(src) + (tok0 * a.Hqk + hq) * D * sizeof(TI);
    for (int jj = 0; jj < NCQ; ++jj) {
      const int j = jj * WPG + wv, r = RB * j + lane / OL::RP, c = (lane % OL::RP) ^ (r & 15);
      const int rr = !RAG ? r : (r < rows ? r : rows - 1);
      dma(ubase(base, 0), (unsigned)(rr * rowb + c * 16), ls + j * 1024);
    }
  };
  auto copy_g = [&](size_t cb) {
    if (lane < GL) dma(ubase(a.G, (cb * C + wv * GL * 4) * sizeof(float)), lane * 16, lds_addr(sG) + wv * GL * 16);
  };
  auto chunk_tokens = [&](int cc, size_t &tok0, int &rows) {
    const size_t n = (size_t)nfirst + cc;
    tok0 = (size_t)b * a.T + n * C;
    rows = !RAG ? C : (int)((size_t)a.T - n * C < (size_t)C ? (size_t)a.T - n * C : (size_t)C);
  };
  auto copy_q = [&](int cc) {
    size_t tok0;
    int rows;
    chunk_tokens(cc, tok0, rows);
    copy_rows(a.q, tok0, rows, sQ);
  };
  auto copy_k = [&](int cc) {
    size_t tok0;
    int rows;
    chunk_tokens(cc, tok0, rows);
    copy_rows(a.k, tok0, rows, sPK);
  };
  float4 u[SPW][MV];
  auto fetch_u = [&](size_t cb) {
#pragma unroll
    for (int s = 0; s < SPW; ++s)
#pragma unroll
      for (int m = 0; m < MV; ++m)
        u[s][m] = *reinterpret_cast<const float4 *>(a.U + ((cb * MV + m) * (D / 16) + slice0 + s) * 256 + lane * 4);
  };
  // operand fragment p of the W or K^T slot
  auto frag = [&](const char *slot, int p) -> Frag<PKw::a> {
    Frag<PKw::a> f;
    const char *base = slot + p * BPF * 1024 + lane * 16;
    if constexpr (F32) {
      const float4 x0 = *reinterpret_cast<const float4 *>(base);
      const float4 x1 = *reinterpret_cast<const float4 *>(base + 1024);
      f.v[0] = x0.x; f.v[1] = x0.y; f.v[2] = x0.z; f.v[3] = x0.w;
      f.v[4] = x1.x; f.v[5] = x1.y; f.v[6] = x1.z; f.v[7] = x1.w;
    } else {
      f.hi = *reinterpret_cast<const bf16x8 *>(base);
    }
    return f;
  };
  // this lane's byte offsets of its row fragment halves within a 16-row tile
  // of Q or K: row lr, k-values 32kb + 16hh + 4g .. +3 (piece c at c ^ lr)
  int koff[KBW][2];
#pragma unroll
  for (int kb = 0; kb < KBW; ++kb)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int k = 32 * kb + 16 * hh + 4 * g;
      const int c = k * (int)sizeof(TI) / 16, off = (k * (int)sizeof(TI)) % 16;
      koff[kb][hh] = lr * OL::RP * 16 + ((c ^ lr) * 16) + off;
    }
  using QF = Frag<PKq::b>;
  auto row_frag = [&](const char *slot, int tile, int kb) -> QF {
    const char *t = slot + tile * 16 * OL::RP * 16;
    QF f;
    if constexpr (!F32 && PKq::b == F_BF16) {
      const uint2 w0 = *reinterpret_cast<const uint2 *>(t + koff[kb][0]);
      const uint2 w1 = *reinterpret_cast<const uint2 *>(t + koff[kb][1]);
      f.hi = __builtin_bit_cast(bf16x8, uint4{w0.x, w0.y, w1.x, w1.y});
    } else {
      static_assert(F32 && PKq::b == F_F32, "fp32 rows feed the fp32 matrix cores");
      const float4 x0 = *reinterpret_cast<const float4 *>(t + koff[kb][0]);
      const float4 x1 = *reinterpret_cast<const float4 *>(t + koff[kb][1]);
      f.v[0] = x0.x; f.v[1] = x0.y; f.v[2] = x0.z; f.v[3] = x0.w;
      f.v[4] = x1.x; f.v[5] = x1.y; f.v[6] = x1.z; f.v[7] = x1.w;
    }
    return f;
  };
  const float *Gs = sG;
  TO *og = reinterpret_cast<TO *>(a.o);

  // the first chunk's copies, in the order of the chunk loop's (K, Q, G, W,
  // then K^T)
  copy_k(0);
  copy_q(0);
  copy_g(cb0);
  copy_w(cb0);
  copy_kt(cb0);

  // one chunk; more: a next chunk follows, whose operands are copied during
  // this one (the last chunk is a separate copy of the body, so that the
  // loop holds no branch around a memory operation: the compiler merges its
  // memory waits over every path through the loop)
  auto chunk = [&](int cc, auto MoreC) {
    constexpr bool more = decltype(MoreC)::value;
    const size_t cb = cb0 + cc;

    size_t tok0;
    int rows;
    chunk_tokens(cc, tok0, rows);

    // U of this chunk, issued first: it lands while P^T is formed
    fetch_u(cb);
    // this chunk's K, Q and G landed (its W and K^T copies and U, issued
    // after them, may be in flight)
    wait_barrier<vm_lgkm0(NCW + NCK + NU)>();

    // ---- V' = U - W h, formed while the P^T fragments wait in registers
    //      (their LDS slot is W's)
    f32x4 vps[SPW][MV];
    auto form_vprime = [&]() {
      Frag<PKw::b> hb[SPW][KBW];
#pragma unroll
      for (int s = 0; s < SPW; ++s)
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb) {
          const float x[8] = {h[s][2 * kb][0], h[s][2 * kb][1], h[s][2 * kb][2], h[s][2 * kb][3],
                              h[s][2 * kb + 1][0], h[s][2 * kb + 1][1], h[s][2 * kb + 1][2], h[s][2 * kb + 1][3]};
          hb[s][kb] = make_frag<PKw::b>(x);
        }
      {
        Frag<PKw::a> fa[2][KBW];
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb) fa[0][kb] = frag(sW, kb);
#pragma unroll
        for (int m = 0; m < MV; ++m) {
          if (m + 1 < MV) {
#pragma unroll
            for (int kb = 0; kb < KBW; ++kb) fa[(m + 1) & 1][kb] = frag(sW, (m + 1) * KBW + kb);
          }
#pragma unroll
          for (int s = 0; s < SPW; ++s) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kb = 0; kb < KBW; ++kb) mma(acc, fa[m & 1][kb], hb[s][kb]);
            vps[s][m] = f32x4{u[s][m].x - acc[0], u[s][m].y - acc[1], u[s][m].z - acc[2], u[s][m].w - acc[3]};
          }
        }
      }
      // (V' complete here: sunk below the next chunk's K copies, its
      // subtractions would wait for those copies as well as for U)
#pragma unroll
      for (int s = 0; s < SPW; ++s)
#pragma unroll
        for (int m = 0; m < MV; ++m) asm volatile("" : "+v"(vps[s][m]));
    };

    // ---- P^T = (K Q^T) o Gamma^T o [i <= r]: wave w forms the pairs (query
    //      tile rt, key tiles 2kp and 2kp + 1) of its query tiles {w, R-1-w}
    //      (equal shares of the triangle).  Every pair is masked (outside the
    //      diagonal the mask keeps all), so that no branch stands between the
    //      pairs and the LDS reads of one overlap the products of the last.
    auto form_pair = [&](const QF *qf, int rt, int kp) -> Frag<PKv::b> {
      QF k0[KBW], k1[KBW];
#pragma unroll
      for (int kb = 0; kb < KBW; ++kb) {
        k0[kb] = row_frag(sPK, 2 * kp, kb);
        k1[kb] = row_frag(sPK, 2 * kp + 1, kb);   // (past the diagonal: read, multiplied, masked)
      }
      f32x4 p0 = zero4(), p1 = zero4();
#pragma unroll
      for (int kb = 0; kb < KBW; ++kb) {
        mma(p0, k0[kb], qf[kb]);
        mma(p1, k1[kb], qf[kb]);
      }
      const int r = 16 * rt + lr;
      const float Gr = Gs[r] * LOG2E;
      const float4 gk0 = *reinterpret_cast<const float4 *>(Gs + 32 * kp + lq);
      const float4 gk1 = *reinterpret_cast<const float4 *>(Gs + 32 * kp + 16 + lq);
      const float g0[4] = {gk0.x, gk0.y, gk0.z, gk0.w}, g1[4] = {gk1.x, gk1.y, gk1.z, gk1.w};
      float b8[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k0i = 32 * kp + lq + i, k1i = k0i + 16;
        b8[i] = k0i <= r ? p0[i] * exp2_fast(Gr - g0[i] * LOG2E) : 0.f;
        b8[4 + i] = k1i <= r ? p1[i] * exp2_fast(Gr - g1[i] * LOG2E) : 0.f;
      }
      return make_frag<PKv::b>(b8);
    };
    auto store_pair = [&](int rt, int kp, const Frag<PKv::b> &f) {
      char *pf = sW + (OL::pbase(rt) + kp) * 2048 + lane * 16;
      if constexpr (PKv::b == F_SPLIT) {
        *reinterpret_cast<bf16x8 *>(pf) = f.hi;
        *reinterpret_cast<bf16x8 *>(pf + 1024) = f.lo;
      } else {
        *reinterpret_cast<float4 *>(pf) = float4{f.v[0], f.v[1], f.v[2], f.v[3]};
        *reinterpret_cast<float4 *>(pf + 1024) = float4{f.v[4], f.v[5], f.v[6], f.v[7]};
      }
    };
    if constexpr (RU == 2) {
      // R = 8: the pairs (w, 0) and (7-w, 0..2) of every wave, and a fifth,
      // (w, 1) for w >= 2 and (7-w, 3) below.  (Query tiles opaque each chunk:
      // the masks and decays derived from them are formed where used instead
      // of being hoisted out of the chunk loop, where they would hold scalar
      // registers for the whole walk.)
      int rt0 = wv, rt1 = R - 1 - wv, rtx = wv >= 2 ? wv : R - 1 - wv, kpx = wv >= 2 ? 1 : 3;
      asm volatile("" : "+s"(rt0), "+s"(rt1), "+s"(rtx), "+s"(kpx));
      QF q0[KBW], qx[KBW], q1[KBW];
#pragma unroll
      for (int kb = 0; kb < KBW; ++kb) {
        q0[kb] = row_frag(sQ, rt0, kb);
        qx[kb] = row_frag(sQ, rtx, kb);
      }
      Frag<PKv::b> pt[5];
      pt[0] = form_pair(q0, rt0, 0);
      pt[1] = form_pair(qx, rtx, kpx);
#pragma unroll
      for (int kb = 0; kb < KBW; ++kb) q1[kb] = row_frag(sQ, rt1, kb);
#pragma unroll
      for (int kp = 0; kp < 3; ++kp) pt[2 + kp] = form_pair(q1, rt1, kp);
      form_vprime();
      wait_barrier<vm_lgkm0(63)>();   // every wave past the K tile and W
      if constexpr (more) copy_k(cc + 1);
      store_pair(rt0, 0, pt[0]);
      store_pair(rtx, kpx, pt[1]);
#pragma unroll
      for (int kp = 0; kp < 3; ++kp) store_pair(rt1, kp, pt[2 + kp]);
    } else {
      // R = 4: query tile w; its pairs (w, 0) and, for w >= 2, (w, 1)
      int rt = wv;
      asm volatile("" : "+s"(rt));
      QF qf[KBW];
#pragma unroll
      for (int kb = 0; kb < KBW; ++kb) qf[kb] = row_frag(sQ, rt, kb);
      Frag<PKv::b> pt[2];
#pragma unroll
      for (int kp = 0; kp < 2; ++kp)
        if (2 * kp <= rt) pt[kp] = form_pair(qf, rt, kp);
      form_vprime();
      wait_barrier<vm_lgkm0(63)>();   // every wave past the K tile and W
      if constexpr (more) copy_k(cc + 1);
#pragma unroll
      for (int kp = 0; kp < 2; ++kp)
        if (2 * kp <= rt) store_pair(rt, kp, pt[kp]);
    }
    wait_barrier<vm_lgkm0(63)>();   // P^T in place


    // ---- outputs O^T = e^{G_r} h^T Q^T + V'^T P^T for each slice's columns,
    //      one slice after the other: first h^T Q^T for every query tile
    //      (query fragments one tile ahead), then V'^T P^T pair by pair (P^T
    //      fragments one pair ahead)
    const float gl2 = Gs[C - 1] * LOG2E;
    const float gl = exp2_fast(gl2);
    Frag<PKk::b> vb[SPW][KBK];   // d o V' for the state update (G is recopied before it)
    auto pfrag = [&](int p) -> Frag<PKv::b> {
      const char *pf = sW + p * 2048 + lane * 16;
      Frag<PKv::b> bf;
      if constexpr (PKv::b == F_SPLIT) {
        bf.hi = *reinterpret_cast<const bf16x8 *>(pf);
        bf.lo = *reinterpret_cast<const bf16x8 *>(pf + 1024);
      } else {
        const float4 x0 = *reinterpret_cast<const float4 *>(pf), x1 = *reinterpret_cast<const float4 *>(pf + 1024);
        bf.v[0] = x0.x; bf.v[1] = x0.y; bf.v[2] = x0.z; bf.v[3] = x0.w;
        bf.v[4] = x1.x; bf.v[5] = x1.y; bf.v[6] = x1.z; bf.v[7] = x1.w;
      }
      return bf;
    };
    // h^T Q^T for each slice first, so that the next chunk's Q can be copied
    // while V'^T P^T runs (one slice after the other in each part: the
    // scheduler would otherwise interleave both slices' products and hold
    // both sets of operands)
    f32x4 a1[SPW][R];
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      Frag<PKh::a> hT[KBW];   // the chunk-start state, split for this product
#pragma unroll
      for (int kb = 0; kb < KBW; ++kb) {
        const float x[8] = {h[s][2 * kb][0], h[s][2 * kb][1], h[s][2 * kb][2], h[s][2 * kb][3],
                            h[s][2 * kb + 1][0], h[s][2 * kb + 1][1], h[s][2 * kb + 1][2], h[s][2 * kb + 1][3]};
        hT[kb] = make_frag<PKh::a>(x);
      }
      QF qf[2][KBW];
#pragma unroll
      for (int kb = 0; kb < KBW; ++kb) qf[0][kb] = row_frag(sQ, 0, kb);
#pragma unroll
      for (int rt = 0; rt < R; ++rt) {
        if (rt + 1 < R) {
#pragma unroll
          for (int kb = 0; kb < KBW; ++kb) qf[(rt + 1) & 1][kb] = row_frag(sQ, rt + 1, kb);
        }
        a1[s][rt] = zero4();
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb) mma(a1[s][rt], hT[kb], qf[rt & 1][kb]);
      }
    }
    if constexpr (more) {
      wait_barrier<vm_lgkm0(63)>();   // every wave past Q
      copy_q(cc + 1);
    }
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      Frag<PKv::a> vT[KBK];
#pragma unroll
      for (int kb = 0; kb < KBK; ++kb) {
        float x[8], y[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int m = 2 * kb + j / 4, i = j % 4;
          x[j] = vps[s][m][i];
          y[j] = vps[s][m][i] * exp2_fast(gl2 - Gs[16 * m + lq + i] * LOG2E);
        }
        vT[kb] = make_frag<PKv::a>(x);
        vb[s][kb] = make_frag<PKk::b>(y);
      }
      // pairs in storage order: (rt, kp), kp <= rt / 2, p = pbase(rt) + kp
      Frag<PKv::b> pf[2];
      pf[0] = pfrag(0);
#pragma unroll
      for (int rt = 0; rt < R; ++rt) {
        f32x4 a2 = zero4();
#pragma unroll
        for (int kp = 0; kp <= rt / 2; ++kp) {
          const int p = OL::pbase(rt) + kp;
          if (p + 1 < OL::NPAIR) pf[(p + 1) & 1] = pfrag(p + 1);
          mma(a2, vT[kp], pf[p & 1]);
        }
        const int r = 16 * rt + lr;
        const float er = exp2_fast(Gs[r] * LOG2E);
        TO ov[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[i] = from_f32<TO>(er * a1[s][rt][i] + a2[i]);
        TO *dst = og + ((tok0 + r) * a.Hv + hv) * D + c0 + 16 * s + lq;
        if (!RAG || r < rows) {
          if constexpr (sizeof(TO) == 4) st16_stream(dst, ov);
          else st8_stream(dst, ov);
        }
      }
    }
    // every wave past P^T (W's slot) and G; this chunk's K^T landed (U, the
    // next chunk's K and Q copies and this chunk's o stores, issued after it,
    // may be in flight)
    if constexpr (more) wait_barrier<vm_lgkm0(NU + 2 * NCQ + NST)>();
    else wait_barrier<vm_lgkm0(NST)>();
    if constexpr (more) {
      copy_g(cb + 1);
      copy_w(cb + 1);
    }

    // ---- h <- e^{G_last} h + K^T (d o V'), K^T fragments one state tile
    //      ahead (and serving every slice of the wave)
    {
      Frag<PKw::a> fk[2][KBK];
#pragma unroll
      for (int kb = 0; kb < KBK; ++kb) fk[0][kb] = frag(sKt, kb);
#pragma unroll
      for (int m = 0; m < MH; ++m) {
        if (m + 1 < MH) {
#pragma unroll
          for (int kb = 0; kb < KBK; ++kb) fk[(m + 1) & 1][kb] = frag(sKt, (m + 1) * KBK + kb);
        }
#pragma unroll
        for (int s = 0; s < SPW; ++s) {
          f32x4 acc2 = zero4();
#pragma unroll
          for (int kb = 0; kb < KBK; ++kb) mma(acc2, fk[m & 1][kb], vb[s][kb]);
#pragma unroll
          for (int i = 0; i < 4; ++i) h[s][m][i] = gl * h[s][m][i] + acc2[i];
        }
      }
    }
    if constexpr (more) {
      wait_barrier<vm_lgkm0(63)>();   // every wave past K^T
      copy_kt(cb + 1);
    }
  };
  for (int cc = 0; cc + 1 < cpj; ++cc) chunk(cc, std::true_type{});
  chunk(cpj - 1, std::false_type{});
  store_final();
}

// ----------------------------------------------------------------------------
// packed variable-length sequences: the chunk tables.  Sequence s covers
// tokens [cu[s], cu[s+1]) of the packed tensors (offsets clamped into
// [0, T], a sequence ending no earlier than it starts) and is cut into
// ceil(len / C) chunks, the last one partial.  One workgroup of 256 threads;
// thread t takes a contiguous block of sequences.  Writes, with nmax the
// table capacity (T / C + nseq, enough for any valid cu):
//   jtab[s] = (first chunk, chunks)      ctab[c] = (first token, tokens)
//   *ntot   = number of chunks
// Entries that would pass nmax (only for offsets that are not a valid
// partition of [0, T]) are dropped, so no access leaves the tables.
__global__ __launch_bounds__(256) void varlen_tables_kernel(const int *cu, int nseq, int T, int C, int nmax,
                                                            int2 *ctab, int2 *jtab, int *ntot) {
  __shared__ int part[256];
  const int t = threadIdx.x, per = (nseq + 255) / 256;
  const int s0 = t * per < nseq ? t * per : nseq, s1 = s0 + per < nseq ? s0 + per : nseq;
  auto seg = [&](int s, int &st, int &en) {
    st = cu[s] < 0 ? 0 : cu[s] > T ? T : cu[s];
    en = cu[s + 1] < st ? st : cu[s + 1] > T ? T : cu[s + 1];
  };
  int mine = 0;
  for (int s = s0; s < s1; ++s) {
    int st, en;
    seg(s, st, en);
    mine += (en - st + C - 1) / C;
  }
  part[t] = mine;
  __syncthreads();
  if (t == 0) {
    int run = 0;
    for (int i = 0; i < 256; ++i) {
      const int x = part[i];
      part[i] = run;
      run += x;
    }
    *ntot = run < nmax ? run : nmax;
  }
  __syncthreads();
  int c = part[t];
  for (int s = s0; s < s1; ++s) {
    int st, en;
    seg(s, st, en);
    const int nch = (en - st + C - 1) / C;
    const int first = c < nmax ? c : nmax;
    const int room = nmax - first;
    jtab[s] = int2{first, nch < room ? nch : room};
    for (int j = 0; j < nch && c + j < nmax; ++j) {
      const int a0 = st + j * C;
      ctab[c + j] = int2{a0, en - a0 < C ? en - a0 : C};
    }
    c += nch;
  }
}

}  // namespace gdn
