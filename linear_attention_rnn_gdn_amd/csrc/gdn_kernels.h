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
//   prep_kernel    one workgroup per (chunk, value head, batch): G, S, T, W, U
//   walk_kernel    one workgroup per (column slice, value head, batch*job):
//                  the sequential chunk walk with the state slice resident in
//                  LDS.  Modes: WALK (state = h, writes chunk-start states and
//                  V') and FOLD (state = the augmented [A | B] of a group,
//                  started from [I | 0]; writes the group's pair).
//   prefix_kernel  one workgroup per (column slice, bh): exclusive prefix of
//                  the groups' affine pairs.
//   out_kernel     one workgroup per (column slice, chunk, bh): the output.
//
// Workspace tensors (fp32):  G [BH,N,C]  W [BH,N,C,D]  U [BH,N,C,D]
//   Hs [BH,N,D,D] chunk-start states   Vn [BH,N,C,D] corrected values V'.
#pragma once
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
  static constexpr int kv = MODE == MODE_F32 ? P_F32 : P_SPLIT_B;       // K^T x V'
  static constexpr int qh = MODE == MODE_F32 ? P_F32 : P_SPLIT_B;       // Q x h
  static constexpr int pv = MODE == MODE_F32 ? P_F32 : P_SPLIT_AB;      // P x V'
};

struct FwdArgs {
  int B, T, Hqk, Hv, N;           // N = T / C chunks per sequence
  const void *q, *k, *v;
  const float *g, *beta;
  float *G, *W, *U, *Tm;          // prep outputs (Tm optional)
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
template <typename TI, int ROWS>
__device__ __forceinline__ void load_rows(TI *dst, int ld, const TI *src, size_t gstride) {
  constexpr int VE = 16 / sizeof(TI);
  constexpr int PER_ROW = D / VE;
  for (int idx = threadIdx.x; idx < ROWS * PER_ROW; idx += NT) {
    const int r = idx / PER_ROW, cv = idx % PER_ROW;
    const uint4 val = *reinterpret_cast<const uint4 *>(src + (size_t)r * gstride + cv * VE);
    *reinterpret_cast<uint4 *>(dst + r * ld + cv * VE) = val;
  }
}

// ----------------------------------------------------------------------------
// prep: decay cumsum, S, T (ladder), W, U for one chunk of one value head.
template <int C, typename TI, int MODE>
__global__ __launch_bounds__(NT) void prep_kernel(FwdArgs a) {
  using PR = Prec<MODE>;
  constexpr int LDI = D + LdPad<TI>::v;   // input tile leading dim
  constexpr int LDS_ = C + 4;             // S / T leading dim
  constexpr int LDM_MAX = C / 2 + 4;
  __shared__ __align__(16) TI sIn[C * LDI];
  __shared__ __align__(16) float sS[C * LDS_];
  __shared__ __align__(16) float sM[(C / 2) * LDM_MAX];   // ladder scratch: nb * b * (b+4) <= C/2*(C/2+4)
  __shared__ float sG[C], sBeta[C], sScale[C];
  __shared__ float sWt[2];

  const int n = blockIdx.x, hv = blockIdx.y, b = blockIdx.z;
  const int hq = hv / (a.Hv / a.Hqk);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lk = (lane >> 4) * 8, lq = (lane >> 4) * 4;
  const size_t bh = (size_t)b * a.Hv + hv;
  const size_t t0 = (size_t)n * C;

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
    __syncthreads();
    if (wave == 1) x += sWt[0];
    if (tid < C) {
      sG[tid] = x;
      sBeta[tid] = bx;
      sScale[tid] = bx * expf(x);
    }
  }
  // (2) K chunk -> LDS
  const TI *kin = reinterpret_cast<const TI *>(a.k) + (((size_t)b * a.T + t0) * a.Hqk + hq) * D;
  load_rows<TI, C>(sIn, LDI, kin, (size_t)a.Hqk * D);
  __syncthreads();

  // (3) S = strict-lower( beta_r e^{G_r - G_i} K K^T ); upper tiles zero
  constexpr int TC = C / 16;
  for (int tt = wave; tt < TC * TC; tt += 4) {
    const int mi = tt / TC, ni = tt % TC;
    f32x4 acc = zero4();
    if (ni <= mi) {
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb) {
        float a8[8], b8[8];
        ld8(sIn + (16 * mi + lr) * LDI + 32 * kb + lk, a8);
        ld8(sIn + (16 * ni + lr) * LDI + 32 * kb + lk, b8);
        mma_k32<PR::exact>(acc, a8, b8);
      }
    }
    const int c = 16 * ni + lr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * mi + lq + i;
      sS[r * LDS_ + c] = (c < r) ? sBeta[r] * expf(sG[r] - sG[c]) * acc[i] : 0.f;
    }
  }
  __syncthreads();

  // (4) exact inverses of the 16x16 diagonal blocks (forward substitution,
  //     one thread per block column)
  {
    float x[16];
    const int blk = tid >> 4, j = tid & 15;
    if (tid < C) {
      const float *Sb = sS + (16 * blk) * LDS_ + 16 * blk;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = (r == j) ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < r; ++i) v -= Sb[r * LDS_ + i] * x[i];
        x[r] = v;
      }
    }
    __syncthreads();
    if (tid < C) {
      float *Sb = sS + (16 * blk) * LDS_ + 16 * blk;
#pragma unroll
      for (int r = 0; r < 16; ++r) Sb[r * LDS_ + j] = x[r];
    }
    __syncthreads();
  }

  // (5) doubling ladder: for each 2b diagonal block [[P,0],[L,Q]] the new
  //     lower-left block is -X_Q L X_P (X_P, X_Q the current inverses).
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
          ld8(sS + (s + bs + 16 * mi + lr) * LDS_ + s + k0, a8);
          ld8s(sS + (s + k0) * LDS_ + s + 16 * ni + lr, LDS_, b8);
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
    __syncthreads();
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
          ld8(sS + (s + bs + 16 * mi + lr) * LDS_ + s + bs + k0, a8);
          ld8(M + (16 * ni + lr) * ldm + k0, b8);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) a8[j] = b8[j] = 0.f;
        }
        mma_k32<PR::ladder>(acc, a8, b8);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sS[(s + bs + 16 * mi + lq + i) * LDS_ + s + 16 * ni + lr] = -acc[i];
    }
    __syncthreads();
  }

  const size_t cb = bh * a.N + n;  // chunk index into the workspace
  if (a.Tm) {
    float *Tg = a.Tm + cb * C * C;
    for (int idx = tid; idx < C * C; idx += NT) Tg[idx] = sS[(idx / C) * LDS_ + idx % C];
  }
  if (tid < C) a.G[cb * C + tid] = sG[tid];

  // (6) W = (T diag(beta e^G)) K ;  (7) U = (T diag(beta)) V
  constexpr int TD = D / 16;
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) {
      __syncthreads();
      const TI *vin = reinterpret_cast<const TI *>(a.v) + (((size_t)b * a.T + t0) * a.Hv + hv) * D;
      load_rows<TI, C>(sIn, LDI, vin, (size_t)a.Hv * D);
      __syncthreads();
    }
    const float *scale = pass == 0 ? sScale : sBeta;
    float *out = (pass == 0 ? a.W : a.U) + cb * C * D;
    for (int tt = wave; tt < TC * TD; tt += 4) {
      const int mi = tt / TD, ni = tt % TD;
      f32x4 acc = zero4();
      for (int kb = 0; kb * 32 < 16 * (mi + 1); ++kb) {
        float a8[8], b8[8];
        const int k0 = 32 * kb + lk;
        ld8(sS + (16 * mi + lr) * LDS_ + k0, a8);
#pragma unroll
        for (int j = 0; j < 8; ++j) a8[j] *= scale[k0 + j];
        ld8s(sIn + k0 * LDI + 16 * ni + lr, LDI, b8);
        mma_k32<PR::wy>(acc, a8, b8);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) out[(size_t)(16 * mi + lq + i) * D + 16 * ni + lr] = acc[i];
    }
  }
}

// ----------------------------------------------------------------------------
// walk / fold: the sequential chunk loop for one column slice of the state.
template <int C, typename TI, int MODE, int S, int KIND>
__global__ __launch_bounds__(NT) void walk_kernel(FwdArgs a) {
  using PR = Prec<MODE>;
  constexpr int LDW = D + LdPad<TI>::v;   // W tile [C][LDW]
  constexpr int LDK = C + LdPad<TI>::v;   // K^T tile [D][LDK]
  constexpr int RSZ = (C * LDW > D * LDK) ? C * LDW : D * LDK;
  constexpr int LDH = D + 4;              // state slice, transposed [S][LDH]
  constexpr int LDV = C + 4;              // scaled V' slice, transposed [S][LDV]
  __shared__ __align__(16) TI sR[RSZ];
  __shared__ __align__(16) float sH[S * LDH];
  __shared__ __align__(16) float sV[S * LDV];
  __shared__ float sD[C];

  const int slice = blockIdx.x, hv = blockIdx.y;
  const int b = blockIdx.z / a.jobs, job = blockIdx.z % a.jobs;
  const int hq = hv / (a.Hv / a.Hqk);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lk = (lane >> 4) * 8, lq = (lane >> 4) * 4;
  const size_t bh = (size_t)b * a.Hv + hv;
  const int c0 = slice * S;   // first column of the slice (augmented [A|B] in FOLD)

  // initial state slice
  for (int idx = tid; idx < D * S; idx += NT) {
    const int kr = idx / S, c = idx % S, col = c0 + c;
    float x = 0.f;
    if (KIND == FOLD) {
      x = (col < D && kr == col) ? 1.f : 0.f;
    } else if (a.init) {
      const float *src = a.init_per_job ? a.init + (bh * a.jobs + job) * D * D : a.init + bh * D * D;
      x = src[(size_t)kr * D + col];
    }
    sH[c * LDH + kr] = x;
  }

  for (int cc = 0; cc < a.cpj; ++cc) {
    const int n = job * a.cpj + cc;
    const size_t cb = bh * a.N + n;
    const float glog = a.G[cb * C + C - 1];
    if (tid < C) sD[tid] = expf(glog - a.G[cb * C + tid]);
    // W_n -> sR (as TI)
    {
      const float *Wg = a.W + cb * C * D;
      for (int idx = tid; idx < C * D / 4; idx += NT) {
        const int r = idx / (D / 4), c4 = (idx % (D / 4)) * 4;
        const float4 w = *reinterpret_cast<const float4 *>(Wg + (size_t)r * D + c4);
        TI *dst = sR + r * LDW + c4;
        dst[0] = from_f32<TI>(w.x); dst[1] = from_f32<TI>(w.y);
        dst[2] = from_f32<TI>(w.z); dst[3] = from_f32<TI>(w.w);
      }
    }
    __syncthreads();   // sH (previous update / init) and sR visible
    if (KIND == WALK && a.Hs) {
      float *Hg = a.Hs + cb * D * D;
      for (int idx = tid; idx < D * S; idx += NT) {
        const int kr = idx / S, c = idx % S;
        Hg[(size_t)kr * D + c0 + c] = sH[c * LDH + kr];
      }
    }
    // V' = U - W h  (tiles of C x S)
    for (int tt = wave; tt < (C / 16) * (S / 16); tt += 4) {
      const int mi = tt / (S / 16), ni = tt % (S / 16);
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb) {
        float a8[8], b8[8];
        ld8(sR + (16 * mi + lr) * LDW + 32 * kb + lk, a8);
        ld8(sH + (16 * ni + lr) * LDH + 32 * kb + lk, b8);
        mma_k32<PR::wh>(acc, a8, b8);
      }
      const int c = 16 * ni + lr, col = c0 + c;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * mi + lq + i;
        float u = 0.f;
        if (KIND == WALK) u = a.U[(cb * C + r) * D + col];
        else if (col >= D) u = a.U[(cb * C + r) * D + col - D];
        const float vp = u - acc[i];
        if (KIND == WALK && a.Vn) a.Vn[(cb * C + r) * D + col] = vp;
        sV[c * LDV + r] = vp * sD[r];
      }
    }
    __syncthreads();   // done with W; sV complete
    // K_n^T -> sR  ([D][LDK])
    {
      const TI *kin = reinterpret_cast<const TI *>(a.k) + (((size_t)b * a.T + (size_t)n * C) * a.Hqk + hq) * D;
      constexpr int VE = 16 / sizeof(TI);
      for (int idx = tid; idx < C * D / VE; idx += NT) {
        const int r = idx / (D / VE), cv = (idx % (D / VE)) * VE;
        TI tmp[VE];
        *reinterpret_cast<uint4 *>(tmp) = *reinterpret_cast<const uint4 *>(kin + (size_t)r * a.Hqk * D + cv);
#pragma unroll
        for (int j = 0; j < VE; ++j) sR[(cv + j) * LDK + r] = tmp[j];
      }
    }
    __syncthreads();
    // h <- e^{G_last} h + K^T (diag(e^{G_last-G}) V')   (tiles of D x S)
    const float gl = expf(glog);
    for (int tt = wave; tt < (D / 16) * (S / 16); tt += 4) {
      const int mi = tt / (S / 16), ni = tt % (S / 16);
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < C / 32; ++kb) {
        float a8[8], b8[8];
        ld8(sR + (16 * mi + lr) * LDK + 32 * kb + lk, a8);
        ld8(sV + (16 * ni + lr) * LDV + 32 * kb + lk, b8);
        mma_k32<PR::kv>(acc, a8, b8);
      }
      const int c = 16 * ni + lr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float *h = sH + c * LDH + 16 * mi + lq + i;
        *h = gl * *h + acc[i];
      }
    }
    __syncthreads();
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
    for (int idx = tid; idx < D * S; idx += NT) {
      const int kr = idx / S, c = idx % S;
      dst[(size_t)kr * D + dcol + c] = sH[c * LDH + kr];
    }
  }
}

// ----------------------------------------------------------------------------
// exclusive prefix of affine pairs, one column slice of the state.
struct PrefixArgs {
  int n;
  const float *A, *Bm, *h_init;
  float *h_in, *h_final;
};

template <int S, int PREC>
__global__ __launch_bounds__(NT) void prefix_kernel(PrefixArgs a) {
  constexpr int LDA = D + 4, LDH = D + 4;
  __shared__ __align__(16) float sA[D * LDA];
  __shared__ __align__(16) float sH[S * LDH];
  const int slice = blockIdx.x;
  const size_t bh = blockIdx.y;
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
    __syncthreads();
    if (a.h_in) {
      float *Hg = a.h_in + pj * D * D;
      for (int idx = tid; idx < D * S; idx += NT) {
        const int kr = idx / S, c = idx % S;
        Hg[(size_t)kr * D + c0 + c] = sH[c * LDH + kr];
      }
    }
    f32x4 acc[(D / 16) * (S / 16) / 4];
#pragma unroll
    for (int u = 0; u < (D / 16) * (S / 16) / 4; ++u) {
      const int tt = wave + 4 * u;
      const int mi = tt / (S / 16), ni = tt % (S / 16);
      acc[u] = zero4();
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb) {
        float a8[8], b8[8];
        ld8(sA + (16 * mi + lr) * LDA + 32 * kb + lk, a8);
        ld8(sH + (16 * ni + lr) * LDH + 32 * kb + lk, b8);
        mma_k32<PREC>(acc[u], a8, b8);
      }
    }
    __syncthreads();
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
    __syncthreads();
  }
  if (a.h_final) {
    for (int idx = tid; idx < D * S; idx += NT) {
      const int kr = idx / S, c = idx % S;
      a.h_final[(bh * D + kr) * D + c0 + c] = sH[c * LDH + kr];
    }
  }
}

// ----------------------------------------------------------------------------
// output for one column slice of one chunk.
template <int C, typename TI, int MODE, int S, typename TO>
__global__ __launch_bounds__(NT) void out_kernel(FwdArgs a) {
  using PR = Prec<MODE>;
  constexpr int LDI = D + LdPad<TI>::v;
  constexpr int LDP = C + 4;
  constexpr int LDH = D + 4;
  constexpr int LDV = C + 4;
  constexpr int KB = C * LDI * (int)sizeof(TI), HVB = S * (LDH + LDV) * 4;
  __shared__ __align__(16) TI sQ[C * LDI];
  __shared__ __align__(16) char sKraw[KB > HVB ? KB : HVB];   // K tile, then the h / V' slices
  __shared__ __align__(16) float sP[C * LDP];
  __shared__ float sG[C], sE[C];
  TI *sK = reinterpret_cast<TI *>(sKraw);
  float *sH = reinterpret_cast<float *>(sKraw);   // reused after P is formed
  float *sV = sH + S * LDH;

  const int slice = blockIdx.x, n = blockIdx.y;
  const size_t bh = blockIdx.z;
  const int b = (int)(bh / a.Hv), hv = (int)(bh % a.Hv);
  const int hq = hv / (a.Hv / a.Hqk);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lk = (lane >> 4) * 8, lq = (lane >> 4) * 4;
  const size_t cb = bh * a.N + n;
  const size_t t0 = (size_t)n * C;
  const int c0 = slice * S;

  if (tid < C) {
    const float x = a.G[cb * C + tid];
    sG[tid] = x;
    sE[tid] = expf(x);
  }
  const size_t qoff = (((size_t)b * a.T + t0) * a.Hqk + hq) * D;
  load_rows<TI, C>(sQ, LDI, reinterpret_cast<const TI *>(a.q) + qoff, (size_t)a.Hqk * D);
  load_rows<TI, C>(sK, LDI, reinterpret_cast<const TI *>(a.k) + qoff, (size_t)a.Hqk * D);
  __syncthreads();

  // P = (Q K^T) o Gamma o [i <= r]
  constexpr int TC = C / 16;
  for (int tt = wave; tt < TC * TC; tt += 4) {
    const int mi = tt / TC, ni = tt % TC;
    f32x4 acc = zero4();
    if (ni <= mi) {
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb) {
        float a8[8], b8[8];
        ld8(sQ + (16 * mi + lr) * LDI + 32 * kb + lk, a8);
        ld8(sK + (16 * ni + lr) * LDI + 32 * kb + lk, b8);
        mma_k32<PR::exact>(acc, a8, b8);
      }
    }
    const int c = 16 * ni + lr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * mi + lq + i;
      sP[r * LDP + c] = (c <= r) ? acc[i] * expf(sG[r] - sG[c]) : 0.f;
    }
  }
  __syncthreads();
  // chunk-start state slice and V' slice, both transposed
  {
    const float *Hg = a.Hs + cb * D * D;
    const float *Vg = a.Vn + cb * C * D;
    for (int idx = tid; idx < D * S; idx += NT) {
      const int kr = idx / S, c = idx % S;
      sH[c * LDH + kr] = Hg[(size_t)kr * D + c0 + c];
    }
    for (int idx = tid; idx < C * S; idx += NT) {
      const int r = idx / S, c = idx % S;
      sV[c * LDV + r] = Vg[(size_t)r * D + c0 + c];
    }
  }
  __syncthreads();
  TO *og = reinterpret_cast<TO *>(a.o);
  for (int tt = wave; tt < TC * (S / 16); tt += 4) {
    const int mi = tt / (S / 16), ni = tt % (S / 16);
    f32x4 acc1 = zero4(), acc2 = zero4();
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) {
      float a8[8], b8[8];
      ld8(sQ + (16 * mi + lr) * LDI + 32 * kb + lk, a8);
      ld8(sH + (16 * ni + lr) * LDH + 32 * kb + lk, b8);
      mma_k32<PR::qh>(acc1, a8, b8);
    }
    for (int kb = 0; kb * 32 < 16 * (mi + 1); ++kb) {
      float a8[8], b8[8];
      ld8(sP + (16 * mi + lr) * LDP + 32 * kb + lk, a8);
      ld8(sV + (16 * ni + lr) * LDV + 32 * kb + lk, b8);
      mma_k32<PR::pv>(acc2, a8, b8);
    }
    const int c = 16 * ni + lr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * mi + lq + i;
      og[(((size_t)b * a.T + t0 + r) * a.Hv + hv) * D + c0 + c] = from_f32<TO>(sE[r] * acc1[i] + acc2[i]);
    }
  }
}

}  // namespace gdn
