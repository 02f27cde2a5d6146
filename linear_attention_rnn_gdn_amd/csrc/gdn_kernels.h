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
// Kernels (all 256 threads = 4 waves of 64):
//   prep_kernel    one workgroup per (chunk, value head, batch): G, S, T, W, U,
//                  and K^T for the walk
//   walk_kernel    one workgroup per (column slice, value head, batch, job):
//                  the sequential chunk walk.  Each wave keeps its part of the
//                  fp32 state in registers; W and K^T operand fragments come
//                  straight from global memory one chunk ahead; only a bf16
//                  copy of the state and the corrected values V' pass through
//                  LDS.  Modes: WALK (state = h, writes chunk-start states and
//                  V') and FOLD (state = the augmented [A | B] of a group,
//                  started from [I | 0]; writes the group's pair).
//   prefix_kernel  one workgroup per (column slice, bh): exclusive prefix of
//                  the groups' affine pairs.
//   out_kernel     one workgroup per (column slice, chunk, bh): the output,
//                  with P^T kept in registers between its two products.
//
// Workspace tensors (cb = bh*N + n indexes a chunk of a value head).  The
// tensors that pass from one kernel to the next are stored fragment-major: in
// the order in which the consumer's lanes read them, so that each 16-byte
// per-lane load or store of a wave covers 1 KB of consecutive bytes.
// (Row-major tiles read in matrix-core operand layout put consecutive lanes
// on different rows, and each such instruction breaks into dozens of memory
// requests.)  Lane l = lr + 16 g (lr = l % 16, g = l / 16).
//   G   [cb][C] fp32 decay cumsum
//   Wf  [cb][C/16][D/32][64][8]  W[16m + lr][32kb + 8g + j], input dtype
//   Ktf [cb][D/16][C/32][64][8]  K[32kb + 8g + j][16m + lr], input dtype
//   Uf  [cb][C/16][D/16][64][4]  U[16m + 4g + i][16nd + lr], fp32
//   Hsf [cb][D/S][D/16][S/16][64][4]  chunk-start state h[16m + 4g + i][c0 + 16ni + lr]
//   Vnf [cb][D/S][C/16][S/16][64][4]  corrected values V'[16m + 4g + i][c0 + 16ni + lr]
// (S = column-slice width, c0 = S * slice.)  Decays are evaluated as exp2 of
// log2-scaled cumsums (one v_exp_f32 each).
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
constexpr int WALK = 0, FOLD = 1;

template <typename TI> struct LdPad { static constexpr int v = 8; };
template <> struct LdPad<float> { static constexpr int v = 4; };

// Product precision per input precision: MODE_BF16 (bf16 q/k/v) or MODE_F32.
constexpr int MODE_BF16 = 0, MODE_F32 = 1;
template <int MODE> struct Prec {
  static constexpr int exact = MODE == MODE_F32 ? P_F32 : P_BF16;       // bf16 data x bf16 data
  static constexpr int ladder = MODE == MODE_F32 ? P_F32 : P_SPLIT_AB;
  static constexpr int wy = MODE == MODE_F32 ? P_F32 : P_SPLIT_A;       // T' (fp32) x K/V (data)
  static constexpr int wh = MODE == MODE_F32 ? P_F32 : P_BF16;          // W x h
  static constexpr int kv = MODE == MODE_F32 ? P_F32 : P_SPLIT_B;       // K^T (data) x V'
  static constexpr int hq = MODE == MODE_F32 ? P_F32 : P_SPLIT_A;       // h^T x Q^T (data)
  static constexpr int pv = MODE == MODE_F32 ? P_F32 : P_SPLIT_AB;      // V'^T x P^T
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

constexpr float LOG2E = 1.4426950408889634f;
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

struct FwdArgs {
  int B, T, Hqk, Hv, N;           // N = T / C chunks per sequence
  const void *q, *k, *v;
  const float *g, *beta;
  float *G, *U, *Tm;              // prep outputs (Tm optional); U is U^T on the forward path
  void *W;                        // prep output, input dtype (fp32 for the transform hook)
  void *Kt;                       // prep output / walk input: K^T per chunk, input dtype
  float *Hs, *Vn;                 // walk outputs (optional) / out inputs
  const float *init;              // walk: initial states (h0 [BH,D,D] or h_in [BH,J,D,D]) or null
  int init_per_job;               // init indexed by job (replay) instead of bh only
  float *fin;                     // walk: final state per bh (h_T) when jobs == 1, or null
  float *pairA, *pairB;           // fold outputs [BH,J,D,D]
  int jobs, cpj;                  // walk/fold: jobs per bh, chunks per job
  void *o;                        // out output
};

// Copy C rows of D elements (row stride `gstride` elements in global memory)
// into LDS rows of leading dimension `ld`, 16 bytes per thread access.
// All loads are issued before the first LDS store so their latencies overlap.
template <typename TI, int ROWS>
__device__ __forceinline__ void load_rows(TI *dst, int ld, const TI *src, size_t gstride) {
  constexpr int VE = 16 / sizeof(TI);
  constexpr int PER_ROW = D / VE;
  constexpr int NV = ROWS * PER_ROW / NT;
  static_assert(ROWS * PER_ROW % NT == 0, "tile must split evenly over the workgroup");
  uint4 v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int idx = threadIdx.x + i * NT, r = idx / PER_ROW, cv = idx % PER_ROW;
    v[i] = *reinterpret_cast<const uint4 *>(src + (size_t)r * gstride + cv * VE);
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int idx = threadIdx.x + i * NT, r = idx / PER_ROW, cv = idx % PER_ROW;
    *reinterpret_cast<uint4 *>(dst + r * ld + cv * VE) = v[i];
  }
}

// Copy ROWS rows of COLS floats (global row stride gld) into LDS (row stride ld).
template <int ROWS, int COLS>
__device__ __forceinline__ void load_rows_f32(float *dst, int ld, const float *src, int gld) {
  constexpr int PER_ROW = COLS / 4;
  constexpr int NV = ROWS * PER_ROW / NT;
  static_assert(ROWS * PER_ROW % NT == 0, "tile must split evenly over the workgroup");
  float4 v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int idx = threadIdx.x + i * NT, r = idx / PER_ROW, c4 = (idx % PER_ROW) * 4;
    v[i] = *reinterpret_cast<const float4 *>(src + (size_t)r * gld + c4);
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int idx = threadIdx.x + i * NT, r = idx / PER_ROW, c4 = (idx % PER_ROW) * 4;
    *reinterpret_cast<float4 *>(dst + r * ld + c4) = v[i];
  }
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
// Each thread loads one 8-row block of K (and later of V) into registers
// once; the row-major copy feeds S, and the same registers are transposed in
// place for the K^T copy, so K is read from memory once.

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
};

// Transposed input tile X^T [D][C] in LDS, unpadded.  The 16-byte blocks of
// row d are XOR-swizzled by (d ^ d/8): the transposing stores (rows 8 apart)
// and the operand reads (16 consecutive rows) then both spread over all banks.
template <int C, typename TI> struct XT {
  static constexpr int VE = 16 / (int)sizeof(TI);   // elements per 16-byte block
  static constexpr int NB = C / VE;                  // blocks per row
  __device__ static int at(int d, int k) {           // k a multiple of VE
    return d * C + (((k / VE) ^ ((d ^ (d >> 3)) & (NB - 1))) * VE);
  }
};

// One thread's block of the input tile: rows 8 rb .. 8 rb + 7, columns
// VE cb .. VE cb + VE - 1, as 8 row vectors of 16 bytes.
template <int C, typename TI> struct TileBlock {
  static constexpr int VE = 16 / (int)sizeof(TI);
  static constexpr int NCB = D / VE, NBLK = (C / 8) * NCB;
  static constexpr int PER = (NBLK + NT - 1) / NT;   // blocks per thread
  uint4 v[PER][8];
  __device__ void load(const TI *src, size_t gstride) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int blk = threadIdx.x + p * NT, rb = blk / NCB, cb = blk % NCB;
      if (blk < NBLK) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          v[p][j] = *reinterpret_cast<const uint4 *>(src + (size_t)(8 * rb + j) * gstride + VE * cb);
      }
    }
  }
  // row-major copy [C][ld]
  __device__ void put_rows(TI *dst, int ld) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int blk = threadIdx.x + p * NT, rb = blk / NCB, cb = blk % NCB;
      if (blk < NBLK) {
#pragma unroll
        for (int j = 0; j < 8; ++j) *reinterpret_cast<uint4 *>(dst + (8 * rb + j) * ld + VE * cb) = v[p][j];
      }
    }
  }
  // transposed copy X^T (XT layout): column VE cb + e becomes row d, and the
  // block's 8 rows its 8 consecutive k-values
  __device__ void put_transposed(TI *dst) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int blk = threadIdx.x + p * NT, rb = blk / NCB, cb = blk % NCB;
      if (blk >= NBLK) continue;
      if constexpr (sizeof(TI) == 2) {
        // 8 x 8 transpose of 16-bit values: output dword q of column e packs
        // rows 2q (low half) and 2q + 1 (high half)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          uint32_t w[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t lo = (&v[p][2 * q].x)[e >> 1], hi = (&v[p][2 * q + 1].x)[e >> 1];
            w[q] = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
          }
          *reinterpret_cast<uint4 *>(dst + XT<C, TI>::at(8 * cb + e, 8 * rb)) = uint4{w[0], w[1], w[2], w[3]};
        }
      } else {
        // 8 x 4 of 32-bit values: column e = two 16-byte halves of 4 rows
#pragma unroll
        for (int e = 0; e < 4; ++e) {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const uint4 x = {(&v[p][4 * hh].x)[e], (&v[p][4 * hh + 1].x)[e], (&v[p][4 * hh + 2].x)[e],
                             (&v[p][4 * hh + 3].x)[e]};
            *reinterpret_cast<uint4 *>(dst + XT<C, TI>::at(4 * cb + e, 8 * rb + 4 * hh)) = x;
          }
        }
      }
    }
  }
};

// operand fragment of X^T: row d, k-values k0 .. k0 + 7
template <int K, int C, typename TI>
__device__ __forceinline__ Frag<K> xt_frag(const TI *sxt, int d, int k0) {
  if constexpr (sizeof(TI) == 2) {
    const bf16x8 u = *reinterpret_cast<const bf16x8 *>(sxt + XT<C, TI>::at(d, k0));
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
    const float4 u0 = *reinterpret_cast<const float4 *>(sxt + XT<C, TI>::at(d, k0));
    const float4 u1 = *reinterpret_cast<const float4 *>(sxt + XT<C, TI>::at(d, k0 + 4));
    float x[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
    return make_frag<K>(x);
  }
}

template <int C, typename TI, int MODE, bool FWD>
__global__ __launch_bounds__(NT, 2) void prep_kernel(FwdArgs a) {
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

  const int n = blockIdx.x, hv = blockIdx.y, b = blockIdx.z;
  const int hq = hv / (a.Hv / a.Hqk);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, g = lane >> 4, lk = g * 8, lq = g * 4;
  const size_t bh = (size_t)b * a.Hv + hv;
  const size_t t0 = (size_t)n * C;
  const size_t cb = bh * a.N + n;  // chunk index into the workspace

  // K block of this thread -> registers (kept for the transposed copy)
  TileBlock<C, TI> kt, vt;
  kt.load(reinterpret_cast<const TI *>(a.k) + (((size_t)b * a.T + t0) * a.Hqk + hq) * D, (size_t)a.Hqk * D);

  // (1) decay cumsum over the chunk (inclusive), beta
  {
    float x = 0.f, bx = 0.f;
    if (tid < C) {
      const size_t si = ((size_t)b * a.T + t0 + tid) * a.Hv + hv;
      x = a.g[si];
      bx = a.beta[si];
    }
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
  // (2) K row-major -> LDS
  kt.put_rows(sX, LDI);
  lds_barrier();

  // (3) S = strict-lower( beta_r e^{G_r - G_i} K K^T ) into packed sT.
  //     Wave w owns row tiles {w, TC-1-w} (balanced triangle); each k-block's
  //     column fragment feeds both of them.
  constexpr int TC = C / 16;
  constexpr int RU = TC / 4;   // row tiles per wave
  int mrow[RU];
#pragma unroll
  for (int u = 0; u < RU; ++u) mrow[u] = u == 0 ? wave : TC - 1 - wave;
  {
    using PK = PolicyKinds<PR::exact>;
    f32x4 acc[RU][TC];
#pragma unroll
    for (int u = 0; u < RU; ++u)
#pragma unroll
      for (int ni = 0; ni < TC; ++ni) acc[u][ni] = zero4();
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) {
      Frag<PK::a> af[RU];
#pragma unroll
      for (int u = 0; u < RU; ++u) af[u] = lds_frag<PK::a>(sX + (16 * mrow[u] + lr) * LDI + 32 * kb + lk);
#pragma unroll
      for (int ni = 0; ni < TC; ++ni) {
        const auto bf = lds_frag<PK::b>(sX + (16 * ni + lr) * LDI + 32 * kb + lk);
#pragma unroll
        for (int u = 0; u < RU; ++u)
          if (ni <= mrow[u]) mma(acc[u][ni], af[u], bf);
      }
    }
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      const int m = mrow[u], L = TRI::len(m);
#pragma unroll
      for (int ni = 0; ni < TC; ++ni) {
        const int c = 16 * ni + lr;
        if (16 * ni < L) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * m + lq + i;
            sT[TRI::at(r, c)] = (c < r) ? sBeta[r] * exp2_fast(sG2[r] - sG2[c]) * acc[u][ni][i] : 0.f;
          }
        }
      }
    }
  }
  // V block -> registers; its latency hides behind the inversion
  vt.load(reinterpret_cast<const TI *>(a.v) + (((size_t)b * a.T + t0) * a.Hv + hv) * D, (size_t)a.Hv * D);
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
  for (int bs = 16; bs < C; bs *= 2) {
    const int nb = C / (2 * bs), tb = bs / 16, ldm = bs + 4;
    // M1 = L X_P  (stored transposed in sM)
    for (int tt = wave; tt < nb * tb * tb; tt += 4) {
      const int blk = tt / (tb * tb), ti = tt % (tb * tb), mi = ti / tb, ni = ti % tb;
      const int s = blk * 2 * bs;
      f32x4 acc = zero4();
      for (int kb = (16 * ni) / 32; kb * 32 < bs; ++kb) {
        float a8[8], b8[8];
        const int k0 = 32 * kb + lk;
        if (k0 < bs) {
          ld8(sT + TRI::at(s + bs + 16 * mi + lr, s + k0), a8);
#pragma unroll
          for (int j = 0; j < 8; ++j) b8[j] = sT[TRI::at(s + k0 + j, s + 16 * ni + lr)];
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) a8[j] = b8[j] = 0.f;
        }
        mma_k32<PR::ladder>(acc, a8, b8);
      }
      float *M = sM + blk * bs * ldm;
      *reinterpret_cast<float4 *>(M + (16 * ni + lr) * ldm + 16 * mi + lq) =
          float4{acc[0], acc[1], acc[2], acc[3]};
    }
    lds_barrier();
    // L <- -X_Q M1
    for (int tt = wave; tt < nb * tb * tb; tt += 4) {
      const int blk = tt / (tb * tb), ti = tt % (tb * tb), mi = ti / tb, ni = ti % tb;
      const int s = blk * 2 * bs;
      const float *M = sM + blk * bs * ldm;
      f32x4 acc = zero4();
      for (int kb = 0; kb * 32 < 16 * (mi + 1); ++kb) {
        float a8[8], b8[8];
        const int k0 = 32 * kb + lk;
        if (k0 < bs) {
          ld8(sT + TRI::at(s + bs + 16 * mi + lr, s + bs + k0), a8);
          ld8(M + (16 * ni + lr) * ldm + k0, b8);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) a8[j] = b8[j] = 0.f;
        }
        mma_k32<PR::ladder>(acc, a8, b8);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sT[TRI::at(s + bs + 16 * mi + lq + i, s + 16 * ni + lr)] = -acc[i];
    }
    lds_barrier();
  }

  if (a.Tm) {
    float *Tg = a.Tm + cb * C * C;
    for (int idx = tid; idx < C * C; idx += NT) {
      const int r = idx / C, c = idx % C;
      Tg[idx] = c < TRI::len(r >> 4) ? sT[TRI::at(r, c)] : 0.f;
    }
  }
  if (tid < C) a.G[cb * C + tid] = sG[tid];

  // K^T -> LDS from the registers
  kt.put_transposed(sX);
  lds_barrier();
  if constexpr (FWD) {
    // K^T fragments for the walk, fragment-major: (d tile m, k-block kb, lane)
    // holds K[32 kb + 8 g + j][16 m + lr]; one contiguous 1 KB per wave store
    TI *Ktg = reinterpret_cast<TI *>(a.Kt) + cb * D * C;
#pragma unroll
    for (int i = 0; i < D * C / 8 / NT; ++i) {
      const int f = tid + i * NT;
      const int l = f & 63, mk = f >> 6, m = mk / (C / 32), kb = mk % (C / 32);
      const int d = 16 * m + (l & 15), r0 = 32 * kb + 8 * (l >> 4);
      constexpr int VE = 16 / sizeof(TI);
#pragma unroll
      for (int v = 0; v < 8 / VE; ++v)
        *reinterpret_cast<uint4 *>(Ktg + (size_t)f * 8 + v * VE) =
            *reinterpret_cast<const uint4 *>(sX + XT<C, TI>::at(d, r0 + v * VE));
    }
  }

  // (6) W = (T diag(beta e^G)) K, computed transposed (W^T = K^T T'^T) so
  //     that each lane ends with 4 consecutive columns of one row of W.
  // (7) U = (T diag(beta)) V, computed as is, so that each lane ends with 4
  //     consecutive rows of one column of U (= 4 consecutive entries of U^T).
  // Wave w owns row tiles {w, TC-1-w}; T is lower triangular, so row tile m
  // needs k < 16(m+1).  The T fragments of k-blocks past the diagonal read
  // T's zero-filled or neighbouring entries and their products are skipped.
  constexpr int TD = D / 16;
  constexpr int KT = PolicyKinds<PR::wy>::a;   // T' fragments (split)
  constexpr int KX = PolicyKinds<PR::wy>::b;   // K / V fragments (exact data)
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) {
      lds_barrier();
      vt.put_transposed(sX);
      lds_barrier();
    }
    const float *scale = pass == 0 ? sScale : sBeta;
    f32x4 acc[RU][TD];
#pragma unroll
    for (int u = 0; u < RU; ++u)
#pragma unroll
      for (int md = 0; md < TD; ++md) acc[u][md] = zero4();
#pragma unroll
    for (int kb = 0; kb < C / 32; ++kb) {
      const int k0 = 32 * kb + lk;
      Frag<KT> tf[RU];
      bool live[RU];
#pragma unroll
      for (int u = 0; u < RU; ++u) {
        live[u] = 32 * kb < 16 * (mrow[u] + 1);
        float x[8], sc[8];
        ld8(sT + TRI::at(16 * mrow[u] + lr, k0), x);
        ld8(scale + k0, sc);
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] *= sc[j];
        tf[u] = make_frag<KT>(x);
      }
#pragma unroll
      for (int md = 0; md < TD; ++md) {
        const auto xf = xt_frag<KX, C, TI>(sX, 16 * md + lr, k0);   // X^T row 16md+lr = column of K (or V)
#pragma unroll
        for (int u = 0; u < RU; ++u) {
          if (!live[u]) continue;
          if (pass == 0) mma(acc[u][md], xf, tf[u]);   // W^T tile (d, r)
          else mma(acc[u][md], tf[u], xf);             // U tile (r, d)
        }
      }
    }
#pragma unroll
    for (int u = 0; u < RU; ++u) {
#pragma unroll
      for (int md = 0; md < TD; ++md) {
        if (pass == 0 && FWD) {
          // lane holds W[r][16md + 4g + i], r = 16 mrow + lr: in the walk's
          // fragment (mrow, kb = md/2) these are lane lr + 16 (2 (md%2) + g/2),
          // elements 4 (g%2) + i
          const int kb = md >> 1, gg = 2 * (md & 1) + (g >> 1);
          WT *dst = reinterpret_cast<WT *>(a.W) +
                    ((cb * (C / 16) + mrow[u]) * (D / 32) + kb) * 512 + (lr + 16 * gg) * 8 + 4 * (g & 1);
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[i] = from_f32<WT>(acc[u][md][i]);
        } else if (pass == 0) {
          WT *dst = reinterpret_cast<WT *>(a.W) + (cb * C + 16 * mrow[u] + lr) * D + 16 * md + lq;
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[i] = from_f32<WT>(acc[u][md][i]);
        } else if constexpr (FWD) {
          // lane holds U[16 mrow + 4g + i][16md + lr]: the walk's fragment (mrow, md)
          *reinterpret_cast<float4 *>(a.U + ((cb * (C / 16) + mrow[u]) * TD + md) * 256 + lane * 4) =
              float4{acc[u][md][0], acc[u][md][1], acc[u][md][2], acc[u][md][3]};
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            a.U[(cb * C + 16 * mrow[u] + lq + i) * D + 16 * md + lr] = acc[u][md][i];
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------
// walk / fold: the sequential chunk loop for one column slice of the state.
//
// 8 waves (512 threads; two per SIMD so one can issue while the other waits).
// Wave w owns one row tile of V' (C x S) and one row tile of the state
// (D x S), with the column tiles shared out as below.  Its share of the fp32
// state stays in registers for the whole walk.  Per chunk:
//   V' = U - W h        A = W rows (fragments loaded from global, one chunk
//                       ahead), B = bf16 copy of h in LDS
//   h  = e^{G_last} h + K^T (d o V')   A = K^T rows (global, one chunk
//                       ahead), B = d o V' in LDS, already split into the
//                       operand form (hi/lo bf16) by its producer;
//                       d_r = e^{G_last - G_r}
// with two barriers per chunk.
constexpr int WALK_NT = 512;

template <int C, typename TI, int MODE, int S, int KIND>
__global__ __launch_bounds__(WALK_NT) void walk_kernel(FwdArgs a) {
  using PR = Prec<MODE>;
  using PKw = PolicyKinds<PR::wh>;
  using PKk = PolicyKinds<PR::kv>;
  static_assert(PKw::a == (sizeof(TI) == 2 ? F_BF16 : F_F32) && PKk::a == PKw::a,
                "W and K^T fragments are read as stored");
  constexpr bool F32 = PKk::b == F_F32;
  using HB = typename std::conditional<PKw::b == F_F32, float, __bf16>::type;   // state copy for W h
  constexpr int NW = WALK_NT / 64;
  constexpr int NS = (KIND == FOLD ? 2 * D : D) / S;
  constexpr int TN = S / 16;          // column tiles of the slice
  constexpr int TRV = C / 16;         // V' row tiles
  constexpr int CPW = TN * TRV / NW;  // V' column tiles per wave
  constexpr int CPH = TN * (D / 16) / NW;   // state column tiles per wave
  constexpr int KBW = D / 32, KBK = C / 32;
  constexpr int LDHB = D + (sizeof(HB) == 2 ? 8 : 4);   // sHb [S][LDHB]
  constexpr int LDV = C + (F32 ? 4 : 8);                 // sV  [S][LDV] (x2 when split)
  static_assert(CPW >= 1 && CPH >= 1 && TN % CPW == 0 && TN % CPH == 0, "tiling");
  __shared__ __align__(16) HB sHb[S * LDHB];
  __shared__ __align__(16) typename std::conditional<F32, float, __bf16>::type sV[(F32 ? 1 : 2) * S * LDV];

  int unit, slice;
  xcd_unit(blockIdx.x, NS, a.B * a.Hv * a.jobs, unit, slice);
  const int job = unit % a.jobs;
  const size_t bh = (size_t)(unit / a.jobs);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lk = (lane >> 4) * 8, lq = (lane >> 4) * 4;
  const int c0 = slice * S;   // first column of the slice (augmented [A|B] in FOLD)
  const bool has_u = KIND == WALK || c0 >= D;
  const int uc0 = KIND == WALK ? c0 : c0 - D;
  // this wave's tiles
  const int mv = wave % TRV, nv0 = (wave / TRV) * CPW;             // V' row tile, first column tile
  const int mh = wave % (D / 16), nh0 = (wave / (D / 16)) * CPH;   // state row tile, first column tile

  // state: tiles (mh, nh0 + t): rows 16 mh + lq + i, column 16 (nh0 + t) + lr
  f32x4 h[CPH];
#pragma unroll
  for (int t = 0; t < CPH; ++t) {
    const int col = c0 + 16 * (nh0 + t) + lr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kr = 16 * mh + lq + i;
      float x = 0.f;
      if (KIND == FOLD) {
        x = (col < D && kr == col) ? 1.f : 0.f;
      } else if (a.init) {
        const float *src = a.init_per_job ? a.init + (bh * a.jobs + job) * D * D : a.init + bh * D * D;
        x = src[(size_t)kr * D + col];
      }
      h[t][i] = x;
    }
  }
  auto put_state_copy = [&]() {
#pragma unroll
    for (int t = 0; t < CPH; ++t) {
      HB *dst = sHb + (16 * (nh0 + t) + lr) * LDHB + 16 * mh + lq;
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = from_f32<HB>(h[t][i]);
    }
  };

  struct Ops {
    Frag<PKw::a> wf[KBW];
    Frag<PKk::a> kf[KBK];
    float4 u[CPW];
    float4 g;
    float glast;
  };
  auto fetch = [&](Ops &op, int n) {
    const size_t cb = bh * a.N + n;
    const TI *Wg = reinterpret_cast<const TI *>(a.W) + cb * C * D + (size_t)mv * KBW * 512 + lane * 8;
    const TI *Kg = reinterpret_cast<const TI *>(a.Kt) + cb * D * C + (size_t)mh * KBK * 512 + lane * 8;
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb) {
      if constexpr (sizeof(TI) == 2) {
        op.wf[kb].hi = *reinterpret_cast<const bf16x8 *>(Wg + kb * 512);
      } else {
        const float4 x0 = *reinterpret_cast<const float4 *>(Wg + kb * 512);
        const float4 x1 = *reinterpret_cast<const float4 *>(Wg + kb * 512 + 4);
        float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        op.wf[kb] = make_frag<PKw::a>(x);
      }
    }
#pragma unroll
    for (int kb = 0; kb < KBK; ++kb) {
      if constexpr (sizeof(TI) == 2) {
        op.kf[kb].hi = *reinterpret_cast<const bf16x8 *>(Kg + kb * 512);
      } else {
        const float4 x0 = *reinterpret_cast<const float4 *>(Kg + kb * 512);
        const float4 x1 = *reinterpret_cast<const float4 *>(Kg + kb * 512 + 4);
        float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        op.kf[kb] = make_frag<PKk::a>(x);
      }
    }
#pragma unroll
    for (int t = 0; t < CPW; ++t)
      op.u[t] = has_u ? *reinterpret_cast<const float4 *>(
                            a.U + ((cb * TRV + mv) * (D / 16) + uc0 / 16 + nv0 + t) * 256 + lane * 4)
                      : float4{0.f, 0.f, 0.f, 0.f};
    op.g = *reinterpret_cast<const float4 *>(a.G + cb * C + 16 * mv + lq);
    op.glast = a.G[cb * C + C - 1 + vgpr_zero()];
  };

  Ops ops[2];
  fetch(ops[0], job * a.cpj);
  put_state_copy();
  lds_barrier();

  auto step = [&](Ops &cur, Ops &nxt, int cc) {
    const int n = job * a.cpj + cc;
    const size_t cb = bh * a.N + n;
    if (cc + 1 < a.cpj) fetch(nxt, n + 1);

    // chunk-start state for the output stage, fragment-major
    if (KIND == WALK && a.Hs) {
#pragma unroll
      for (int t = 0; t < CPH; ++t)
        *reinterpret_cast<float4 *>(a.Hs + (((cb * NS + slice) * (D / 16) + mh) * TN + nh0 + t) * 256 + lane * 4) =
            float4{h[t][0], h[t][1], h[t][2], h[t][3]};
    }
    // V' = U - W h, then d o V' into LDS in the update's operand form
    const float gl2 = cur.glast * LOG2E;
    {
      f32x4 acc[CPW];
#pragma unroll
      for (int t = 0; t < CPW; ++t) acc[t] = zero4();
#pragma unroll
      for (int kb = 0; kb < KBW; ++kb) {
#pragma unroll
        for (int t = 0; t < CPW; ++t)
          mma(acc[t], cur.wf[kb], lds_frag<PKw::b>(sHb + (16 * (nv0 + t) + lr) * LDHB + 32 * kb + lk));
      }
      const int r0 = 16 * mv + lq;
      const float d0 = exp2_fast(gl2 - cur.g.x * LOG2E), d1 = exp2_fast(gl2 - cur.g.y * LOG2E);
      const float d2 = exp2_fast(gl2 - cur.g.z * LOG2E), d3 = exp2_fast(gl2 - cur.g.w * LOG2E);
#pragma unroll
      for (int t = 0; t < CPW; ++t) {
        const int c = 16 * (nv0 + t) + lr;
        const float4 uu = cur.u[t];
        const float4 vp = {uu.x - acc[t][0], uu.y - acc[t][1], uu.z - acc[t][2], uu.w - acc[t][3]};
        if (KIND == WALK && a.Vn)
          *reinterpret_cast<float4 *>(a.Vn + (((cb * NS + slice) * TRV + mv) * TN + nv0 + t) * 256 + lane * 4) = vp;
        const float s4[4] = {vp.x * d0, vp.y * d1, vp.z * d2, vp.w * d3};
        if constexpr (F32) {
          *reinterpret_cast<float4 *>(sV + c * LDV + r0) = float4{s4[0], s4[1], s4[2], s4[3]};
        } else {
          __bf16 hi[4], lo[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            hi[i] = (__bf16)s4[i];
            lo[i] = (__bf16)(s4[i] - (float)hi[i]);
          }
          *reinterpret_cast<uint2 *>(sV + c * LDV + r0) = *reinterpret_cast<const uint2 *>(hi);
          *reinterpret_cast<uint2 *>(sV + S * LDV + c * LDV + r0) = *reinterpret_cast<const uint2 *>(lo);
        }
      }
    }
    lds_barrier();
    // h <- e^{G_last} h + K^T (d o V')
    {
      const float gl = exp2_fast(gl2);
      f32x4 acc[CPH];
#pragma unroll
      for (int t = 0; t < CPH; ++t) acc[t] = zero4();
#pragma unroll
      for (int kb = 0; kb < KBK; ++kb) {
#pragma unroll
        for (int t = 0; t < CPH; ++t) {
          const int off = (16 * (nh0 + t) + lr) * LDV + 32 * kb + lk;
          Frag<PKk::b> bf;
          if constexpr (F32) {
            bf = lds_frag<PKk::b>(sV + off);
          } else {
            bf.hi = *reinterpret_cast<const bf16x8 *>(sV + off);
            bf.lo = *reinterpret_cast<const bf16x8 *>(sV + S * LDV + off);
          }
          mma(acc[t], cur.kf[kb], bf);
        }
      }
#pragma unroll
      for (int t = 0; t < CPH; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) h[t][i] = gl * h[t][i] + acc[t][i];
    }
    put_state_copy();
    lds_barrier();
  };
  // two chunks per trip so the operand sets alternate without copies
  for (int cc = 0; cc < a.cpj; cc += 2) {
    step(ops[0], ops[1], cc);
    if (cc + 1 < a.cpj) step(ops[1], ops[0], cc + 1);
  }

  // final state slice
  float *dst = nullptr;
  int dcol = c0;
  if (KIND == FOLD) {
    if (c0 < D) dst = a.pairA + (bh * a.jobs + job) * D * D;
    else { dst = a.pairB + (bh * a.jobs + job) * D * D; dcol = c0 - D; }
  } else if (a.fin) {
    dst = a.fin + bh * D * D;
  }
  if (dst) {
#pragma unroll
    for (int t = 0; t < CPH; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dst[(size_t)(16 * mh + lq + i) * D + dcol + 16 * (nh0 + t) + lr] = h[t][i];
  }
}

// ----------------------------------------------------------------------------
// exclusive prefix of affine pairs, one column slice of the state.
struct PrefixArgs {
  int BH, n;
  const float *A, *Bm, *h_init;
  float *h_in, *h_final;
};

template <int S, int PREC>
__global__ __launch_bounds__(NT) void prefix_kernel(PrefixArgs a) {
  constexpr int LDA = D + 4, LDH = D + 4;
  __shared__ __align__(16) float sA[D * LDA];
  __shared__ __align__(16) float sH[S * LDH];
  int unit, slice;
  xcd_unit(blockIdx.x, D / S, a.BH, unit, slice);
  const size_t bh = (size_t)unit;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lk = (lane >> 4) * 8, lq = (lane >> 4) * 4;
  const int c0 = slice * S;
  for (int idx = tid; idx < D * S; idx += NT) {
    const int kr = idx / S, c = idx % S;
    sH[c * LDH + kr] = a.h_init ? a.h_init[(bh * D + kr) * D + c0 + c] : 0.f;
  }
  for (int j = 0; j < a.n; ++j) {
    const size_t pj = bh * a.n + j;
    const float *Ag = a.A + pj * D * D;
    for (int idx = tid; idx < D * D / 4; idx += NT) {
      const int r = idx / (D / 4), c4 = (idx % (D / 4)) * 4;
      *reinterpret_cast<float4 *>(sA + r * LDA + c4) = *reinterpret_cast<const float4 *>(Ag + (size_t)r * D + c4);
    }
    lds_barrier();
    if (a.h_in) {
      float *Hg = a.h_in + pj * D * D;
      for (int idx = tid; idx < D * S; idx += NT) {
        const int kr = idx / S, c = idx % S;
        Hg[(size_t)kr * D + c0 + c] = sH[c * LDH + kr];
      }
    }
    // all of this wave's tiles share column tile wave % (S/16)
    constexpr int NTU = (D / 16) * (S / 16) / 4;
    static_assert(4 % (S / 16) == 0, "tiling");
    using PK = PolicyKinds<PREC>;
    f32x4 acc[NTU];
#pragma unroll
    for (int u = 0; u < NTU; ++u) acc[u] = zero4();
    {
      const int ni = wave % (S / 16);
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb) {
        const auto bf = lds_frag<PK::b>(sH + (16 * ni + lr) * LDH + 32 * kb + lk);
#pragma unroll
        for (int u = 0; u < NTU; ++u) {
          const int mi = (wave + 4 * u) / (S / 16);
          mma(acc[u], lds_frag<PK::a>(sA + (16 * mi + lr) * LDA + 32 * kb + lk), bf);
        }
      }
    }
    lds_barrier();
    const float *Bg = a.Bm + pj * D * D;
#pragma unroll
    for (int u = 0; u < (D / 16) * (S / 16) / 4; ++u) {
      const int tt = wave + 4 * u;
      const int mi = tt / (S / 16), ni = tt % (S / 16);
      const int c = 16 * ni + lr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * mi + lq + i;
        sH[c * LDH + m] = acc[u][i] + Bg[(size_t)m * D + c0 + c];
      }
    }
    lds_barrier();
  }
  if (a.h_final) {
    for (int idx = tid; idx < D * S; idx += NT) {
      const int kr = idx / S, c = idx % S;
      a.h_final[(bh * D + kr) * D + c0 + c] = sH[c * LDH + kr];
    }
  }
}

// ----------------------------------------------------------------------------
// output for one column slice of one chunk, computed transposed:
//   O^T = h^T (diag(e^G) Q)^T + V'^T P^T,   P^T = (K Q^T) o Gamma^T o [i <= r].
// Each wave owns query-row tiles (w and R-1-w, balancing the triangle).  P^T
// tiles stay in the matrix-core result registers and feed V'^T P^T directly
// as B operands: a result tile holds rows 4g..4g+3 of 16 for lane group g, so
// two stacked tiles give lane group g the k-values {4g..4g+3, 16+4g..16+4g+3},
// and the A operand is fetched with the same k order.
template <int C, typename TI, int MODE, int S, typename TO>
__global__ __launch_bounds__(NT, 2) void out_kernel(FwdArgs a) {
  using PR = Prec<MODE>;
  using PKq = PolicyKinds<PR::exact>;   // K x Q^T
  using PKh = PolicyKinds<PR::hq>;      // h^T x Q^T
  using PKv = PolicyKinds<PR::pv>;      // V'^T x P^T
  static_assert(PKq::b == PKh::b, "one query fragment serves both products");
  constexpr int VE = 16 / sizeof(TI);
  constexpr int LDK = D + LdPad<TI>::v;   // K tile [C][LDK]
  constexpr int LDH = D + 4;              // h^T slice [S][LDH]
  constexpr int LDV = C + 4;              // V'^T slice [S][LDV]
  constexpr int R = C / 16;               // query-row tiles
  constexpr int RU = R / 4;               // row tiles per wave
  constexpr int NS = D / S;
  constexpr int CT = S / 16;              // column tiles of the slice
  static_assert(R % 4 == 0, "row tiles must split over 4 waves");
  __shared__ __align__(16) TI sK[C * LDK];
  __shared__ __align__(16) float sH[S * LDH];
  __shared__ __align__(16) float sV[S * LDV];
  __shared__ float sG[C];

  int unit, slice;
  xcd_unit(blockIdx.x, NS, a.N * a.B * a.Hv, unit, slice);
  const size_t bh = (size_t)(unit / a.N);
  const int n = unit % a.N;
  const int b = (int)(bh / a.Hv), hv = (int)(bh % a.Hv);
  const int hq = hv / (a.Hv / a.Hqk);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lk = (lane >> 4) * 8, lq = (lane >> 4) * 4;
  const size_t cb = bh * a.N + n;
  const size_t t0 = (size_t)n * C;
  const int c0 = slice * S;

  const size_t koff = (((size_t)b * a.T + t0) * a.Hqk + hq) * D;
  load_rows<TI, C>(sK, LDK, reinterpret_cast<const TI *>(a.k) + koff, (size_t)a.Hqk * D);
  // chunk-start state and V' of this slice (fragment-major, contiguous),
  // scattered into transposed LDS tiles sH[c][d], sV[c][r]
  {
    constexpr int NH = (D / 16) * CT * 64 / NT, NV = (C / 16) * CT * 64 / NT;
    const float *Hg = a.Hs + (cb * NS + slice) * (size_t)(D * S);
    const float *Vg = a.Vn + (cb * NS + slice) * (size_t)(C * S);
    float4 hv4[NH], vv4[NV];
#pragma unroll
    for (int i = 0; i < NH; ++i) hv4[i] = *reinterpret_cast<const float4 *>(Hg + (size_t)(tid + i * NT) * 4);
#pragma unroll
    for (int i = 0; i < NV; ++i) vv4[i] = *reinterpret_cast<const float4 *>(Vg + (size_t)(tid + i * NT) * 4);
#pragma unroll
    for (int i = 0; i < NH; ++i) {
      const int f = tid + i * NT, l = f & 63, t = f >> 6, m = t / CT, ni = t % CT;
      *reinterpret_cast<float4 *>(sH + (16 * ni + (l & 15)) * LDH + 16 * m + 4 * (l >> 4)) = hv4[i];
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int f = tid + i * NT, l = f & 63, t = f >> 6, m = t / CT, ni = t % CT;
      *reinterpret_cast<float4 *>(sV + (16 * ni + (l & 15)) * LDV + 16 * m + 4 * (l >> 4)) = vv4[i];
    }
  }
  if (tid < C) sG[tid] = a.G[cb * C + tid] * LOG2E;   // log2-scaled
  lds_barrier();

  TO *og = reinterpret_cast<TO *>(a.o);
#pragma unroll 1
  for (int u = 0; u < RU; ++u) {
    const int rt = u == 0 ? wave : R - 1 - wave;
    const int r = 16 * rt + lr;   // this lane's query row (result column)
    // query fragments of this row tile (B operand: n = row, k = feature)
    Frag<PKq::b> qf[D / 32];
    {
      const TI *qrow = reinterpret_cast<const TI *>(a.q) + (((size_t)b * a.T + t0 + r) * a.Hqk + hq) * D;
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb) {
        TI tmp[8];
#pragma unroll
        for (int v = 0; v < 8 / VE; ++v)
          *reinterpret_cast<uint4 *>(tmp + v * VE) = *reinterpret_cast<const uint4 *>(qrow + 32 * kb + lk + v * VE);
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = to_f32(tmp[j]);
        qf[kb] = make_frag<PKq::b>(x);
      }
    }
    const float Gr = sG[r];
    f32x4 acc1[CT], acc2[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc1[ct] = acc2[ct] = zero4();
    // h^T Q^T for every column tile of the slice
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        mma(acc1[ct], lds_frag<PKh::a>(sH + (16 * ct + lr) * LDH + 32 * kb + lk), qf[kb]);
    }
    // key blocks of 32: P^T tiles (2kp, 2kp+1) are formed and consumed at
    // once.  A result tile gives lane group g keys {4g..4g+3} (first tile)
    // and {16+4g..16+4g+3} (second tile) of the block; the V'^T fragment is
    // read with the same key order.
#pragma unroll
    for (int kp = 0; kp < R / 2; ++kp) {
      if (2 * kp <= rt) {
        f32x4 p0 = zero4(), p1 = zero4();
        const bool two = 2 * kp + 1 <= rt;
#pragma unroll
        for (int kb = 0; kb < D / 32; ++kb) {
          mma(p0, lds_frag<PKq::a>(sK + (32 * kp + lr) * LDK + 32 * kb + lk), qf[kb]);
          if (two) mma(p1, lds_frag<PKq::a>(sK + (32 * kp + 16 + lr) * LDK + 32 * kb + lk), qf[kb]);
        }
        float b8[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int k0 = 32 * kp + lq + i, k1 = k0 + 16;
          b8[i] = k0 <= r ? p0[i] * exp2_fast(Gr - sG[k0]) : 0.f;
          b8[4 + i] = (two && k1 <= r) ? p1[i] * exp2_fast(Gr - sG[k1]) : 0.f;
        }
        const auto bf = make_frag<PKv::b>(b8);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          float a8[8];
          const float *vrow = sV + (16 * ct + lr) * LDV + 32 * kp + lq;
          const float4 v0 = *reinterpret_cast<const float4 *>(vrow);
          const float4 v1 = *reinterpret_cast<const float4 *>(vrow + 16);
          a8[0] = v0.x; a8[1] = v0.y; a8[2] = v0.z; a8[3] = v0.w;
          a8[4] = v1.x; a8[5] = v1.y; a8[6] = v1.z; a8[7] = v1.w;
          mma(acc2[ct], make_frag<PKv::a>(a8), bf);
        }
      }
    }
    const float er = exp2_fast(Gr);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      // lane holds O^T[c = 16ct + 4g + i][r]
      TO *dst = og + (((size_t)b * a.T + t0 + r) * a.Hv + hv) * D + c0 + 16 * ct + lq;
      if constexpr (sizeof(TO) == 4) {
        *reinterpret_cast<float4 *>(dst) = float4{er * acc1[ct][0] + acc2[ct][0], er * acc1[ct][1] + acc2[ct][1],
                                                  er * acc1[ct][2] + acc2[ct][2], er * acc1[ct][3] + acc2[ct][3]};
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = from_f32<TO>(er * acc1[ct][i] + acc2[ct][i]);
      }
    }
  }
}

}  // namespace gdn
