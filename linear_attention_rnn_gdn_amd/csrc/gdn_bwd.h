// gdn_bwd.h -- device kernels of the chunked backward's state cotangents
// (gfx950): the reverse chunk walk and its chunk-parallel term.
//
// The scan's backward walks the chunks in reverse ("Fuse the Gated Delta Net
// inter-chunk scan into a Pallas TPU kernel", section "Changes").  With the
// forward's chunk quantities (oracle reading of w, u, k_g: W = T diag(beta
// e^G) K, K_g = diag(e^{G_last - G}) K), the cotangent of chunk n's incoming
// state is
//   dh_n = e^{G_last} dh_{n+1} - W^T (K_g dh_{n+1}) + ddh_n,    dh_N = dh_T,
// the transposed affine step A_n^T dh_{n+1} plus the part that reaches h_n
// through the chunk's own outputs.  The outputs are
//   O = diag(e^G) Q h + P V',  V' = U - W h,  P = (Q K^T) o Gamma o [i <= r],
// so O depends on h through Qeff = diag(e^G) Q - P W, and
//   ddh_n = Qeff^T dO_n,
// which needs no state: it is formed for every chunk in parallel
// (bwd_ddh_kernel), and the walk (bwd_walk_kernel) only adds it.
//
// Products take the forward's precision policy: data x data in one bf16
// pass (K Q^T), data x fp32 with the fp32 side as hi/lo bf16 halves
// (K dh), fp32 x fp32 with both split (P W, Qeff^T dO, W^T X); fp32 inputs
// use the fp32 matrix cores throughout.
#pragma once
#include "gdn_kernels.h"

namespace gdn {

struct BwdArgs {
  int B, T, Hqk, Hv, N;
  const void *q, *k;          // [B, T, H_qk, D] input dtype
  const float *dO;            // [B, T, H_v, D] fp32 output cotangent
  const float *G, *W;         // prep (transform form): G [cb][C], W [cb][C][D] fp32
  float *ddh;                 // [cb][D/16 slices][D/16 tiles][64][4]: ddh_n in the walk's tile order
  const float *dhT;           // [B, H_v, D, D] or null (zero)
  float *dh;                  // [B, H_v, N, D, D] incoming-state cotangent of every chunk, or null
  float *dh0;                 // [B, H_v, D, D], or null
};

// the chunk-parallel term ddh_n = Qeff^T dO, one workgroup of four waves per
// (chunk, value head); Qeff = diag(e^G) Q - P W is formed per query tile
// (wave w takes query tiles {w, R-1-w}, or {w} at C = 64), P^T's tiles in
// registers, then written to LDS transposed next to dO^T for the product.
template <int C, typename TI> struct BwdLds {
  static constexpr int QK = C * D * (int)sizeof(TI);       // one row-major Q or K tile
  static constexpr int LDT = C + 4;                        // row stride of the [D][C] transposed tiles
  static constexpr int LDW = D + 4;                        // row stride of W [C][D]
  static constexpr int TB = D * LDT * 4;                   // a transposed fp32 tile
  static constexpr int RA = 2 * QK > TB ? 2 * QK : TB;     // region A: Q, K; then dO^T
  static constexpr int RB = C * LDW * 4 > TB ? C * LDW * 4 : TB;   // region B: W; then Qeff^T
};

template <int C, typename TI, int MODE, bool RAG>
__global__ __launch_bounds__(256) void bwd_ddh_kernel(FwdArgs fa, BwdArgs a) {
  using L = BwdLds<C, TI>;
  constexpr int PX = MODE == MODE_F32 ? P_F32 : P_BF16;       // K Q^T
  constexpr int PS = MODE == MODE_F32 ? P_F32 : P_SPLIT_AB;   // fp32 x fp32
  constexpr int R = C / 16, RU = R >= 8 ? 2 : 1, KBD = D / 32, TD = D / 16;
  static_assert(R == 4 * RU, "query tiles {w, R-1-w} per wave");
  __shared__ __align__(16) char rA[L::RA];
  __shared__ __align__(16) char rB[L::RB];
  __shared__ __align__(16) float sG[C];
  TI *sQ = reinterpret_cast<TI *>(rA);
  TI *sK = reinterpret_cast<TI *>(rA + L::QK);
  float *sW = reinterpret_cast<float *>(rB);
  float *sQt = reinterpret_cast<float *>(rB);   // Qeff^T [D][LDT], after W
  float *sOt = reinterpret_cast<float *>(rA);   // dO^T [D][LDT], after Q and K

  int n, b, hv;
  chunk_head_unit(blockIdx.x, fa, n, b, hv);
  const int hq = hv / (a.Hv / a.Hqk);
  const size_t bh = (size_t)b * a.Hv + hv, cb = bh * a.N + n;
  const size_t t0 = (size_t)b * a.T + (size_t)n * C;   // first token (row of the token-major tensors)
  const int rows = !RAG ? C : (a.T - n * C < C ? a.T - n * C : C);
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, g = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Q, K rows (zero past the chunk's tokens), W (row stride D + 4) and G
  constexpr int VE = 16 / (int)sizeof(TI);
  for (int e = tid; e < C * D / VE; e += 256) {
    const int r = e / (D / VE), c = (e % (D / VE)) * VE;
    uint4 xq{0u, 0u, 0u, 0u}, xk{0u, 0u, 0u, 0u};
    if (r < rows) {
      xq = *reinterpret_cast<const uint4 *>(reinterpret_cast<const TI *>(a.q) + ((t0 + r) * a.Hqk + hq) * D + c);
      xk = *reinterpret_cast<const uint4 *>(reinterpret_cast<const TI *>(a.k) + ((t0 + r) * a.Hqk + hq) * D + c);
    }
    *reinterpret_cast<uint4 *>(sQ + r * D + c) = xq;
    *reinterpret_cast<uint4 *>(sK + r * D + c) = xk;
  }
  for (int e = tid; e < C * D / 4; e += 256) {
    const int r = e / (D / 4), c = (e % (D / 4)) * 4;
    *reinterpret_cast<float4 *>(sW + r * L::LDW + c) = *reinterpret_cast<const float4 *>(a.W + (cb * C + r) * D + c);
  }
  if (tid < C) sG[tid] = a.G[cb * C + tid];
  __syncthreads();

  // P^T tiles (key tile kt, query tile rt), kt <= rt, masked and decayed:
  // lane (lr, g) holds P^T[16kt + 4g + i][16rt + lr]; two key tiles stacked
  // are the A operand of P W with the keys in the order kk(g, j)
  auto row8 = [&](const TI *t, int r, int k0, float (&x)[8]) {   // 8 consecutive elements of row r
    ld8(t + r * D + k0, x);
  };
  f32x4 pt[RU][R];
  float qeff[RU][TD][4];
#pragma unroll
  for (int u = 0; u < RU; ++u) {
    const int rt = u == 0 ? wv : R - 1 - wv;
    const int r = 16 * rt + lr;
    const float Gr = sG[r] * LOG2E;
#pragma unroll
    for (int kt = 0; kt < R; ++kt) {
      pt[u][kt] = zero4();
      if (kt > rt) continue;
#pragma unroll
      for (int kb = 0; kb < KBD; ++kb) {
        float ka[8], qb[8];
        row8(sK, 16 * kt + lr, 32 * kb + 8 * g, ka);
        row8(sQ, 16 * rt + lr, 32 * kb + 8 * g, qb);
        mma_k32<PX>(pt[u][kt], ka, qb);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 16 * kt + 4 * g + i;
        pt[u][kt][i] = key <= r ? pt[u][kt][i] * exp2_fast(Gr - sG[key] * LOG2E) : 0.f;
      }
    }
    // Qeff rows of query tile rt: e^{G_r} Q[r][d] - (P W)[r][d]; result lane
    // (lr, g) holds rows 16rt + 4g + i, column 16dt + lr
#pragma unroll
    for (int dt = 0; dt < TD; ++dt) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < C / 32; ++kb) {
        if (32 * kb > 16 * rt + 15) continue;   // keys past the query tile: P is zero
        const float pa[8] = {pt[u][2 * kb][0], pt[u][2 * kb][1], pt[u][2 * kb][2], pt[u][2 * kb][3],
                             pt[u][2 * kb + 1][0], pt[u][2 * kb + 1][1], pt[u][2 * kb + 1][2], pt[u][2 * kb + 1][3]};
        float wb[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) wb[j] = sW[(32 * kb + (j < 4 ? 4 * g + j : 16 + 4 * g + j - 4)) * L::LDW + 16 * dt + lr];
        mma_k32<PS>(acc, pa, wb);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 16 * rt + 4 * g + i;
        qeff[u][dt][i] = exp2_fast(sG[rr] * LOG2E) * to_f32(sQ[rr * D + 16 * dt + lr]) - acc[i];
      }
    }
  }
  __syncthreads();   // every wave past W, Q and K
  // Qeff^T [d][r] and dO^T [c][r] (zero past the chunk's tokens)
#pragma unroll
  for (int u = 0; u < RU; ++u) {
    const int rt = u == 0 ? wv : R - 1 - wv;
#pragma unroll
    for (int dt = 0; dt < TD; ++dt)
      *reinterpret_cast<float4 *>(sQt + (16 * dt + lr) * L::LDT + 16 * rt + 4 * g) =
          float4{qeff[u][dt][0], qeff[u][dt][1], qeff[u][dt][2], qeff[u][dt][3]};
  }
  for (int e = tid; e < C * D / 4; e += 256) {
    const int r = e / (D / 4), c = (e % (D / 4)) * 4;
    float4 x{0.f, 0.f, 0.f, 0.f};
    if (r < rows) x = *reinterpret_cast<const float4 *>(a.dO + ((t0 + r) * a.Hv + hv) * D + c);
    sOt[(c + 0) * L::LDT + r] = x.x;
    sOt[(c + 1) * L::LDT + r] = x.y;
    sOt[(c + 2) * L::LDT + r] = x.z;
    sOt[(c + 3) * L::LDT + r] = x.w;
  }
  __syncthreads();
  // ddh tiles (d tile dt, column tile ct): wave w takes tiles w, w + 4, ...
  for (int t = wv; t < TD * TD; t += 4) {
    const int dt = t % TD, ct = t / TD;
    f32x4 acc = zero4();
#pragma unroll
    for (int kb = 0; kb < C / 32; ++kb) {
      float xa[8], xb[8];
      ld8(sQt + (16 * dt + lr) * L::LDT + 32 * kb + 8 * g, xa);
      ld8(sOt + (16 * ct + lr) * L::LDT + 32 * kb + 8 * g, xb);
      mma_k32<PS>(acc, xa, xb);
    }
    st16(a.ddh + ((cb * TD + ct) * TD + dt) * 256 + lane * 4, acc);
  }
}

// the reverse walk: one workgroup of eight waves per (batch, value head),
// wave s holding the 16 columns 16s.. of dh in matrix-core result registers;
// per chunk, from the last to the first, K (row-major, the input rows), W
// (fp32, row stride D + 4) and G go to LDS, then
//   Y = K dh,  X = diag(e^{G_last - G}) Y,  dh <- e^{G_last} dh - W^T X + ddh_n
template <int C, typename TI, int MODE, bool RAG>
__global__ __launch_bounds__(512) void bwd_walk_kernel(BwdArgs a) {
  constexpr int PKD = MODE == MODE_F32 ? P_F32 : P_SPLIT_B;    // K (data) x dh
  constexpr int PS = MODE == MODE_F32 ? P_F32 : P_SPLIT_AB;    // W^T x X
  constexpr int MV = C / 16, MH = D / 16, KBW = D / 32, KBK = C / 32;
  constexpr int LDW = D + 4;
  __shared__ __align__(16) TI sK[C * D];
  __shared__ __align__(16) float sW[C * LDW];
  __shared__ __align__(16) float sG[C];
  const size_t bh = blockIdx.x;
  const int b = (int)(bh / a.Hv), hv = (int)(bh % a.Hv), hq = hv / (a.Hv / a.Hqk);
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, g = lane >> 4;
  const int s = __builtin_amdgcn_readfirstlane(tid >> 6), c0 = 16 * s;
  // dh tiles: dh[m] holds rows 16m + 4g + i, column c0 + lr
  f32x4 dh[MH];
#pragma unroll
  for (int m = 0; m < MH; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) dh[m][i] = a.dhT ? a.dhT[(bh * D + 16 * m + 4 * g + i) * D + c0 + lr] : 0.f;
  // the k order of a k-block: two stacked result tiles give lane group g the
  // rows kk(g, j) = 4g + j (j < 4), 16 + 4g + j - 4 (j >= 4)
  auto kk = [&](int j) { return j < 4 ? 4 * g + j : 16 + 4 * g + j - 4; };
  for (int n = a.N - 1; n >= 0; --n) {
    const size_t cb = bh * a.N + n, t0 = (size_t)b * a.T + (size_t)n * C;
    const int rows = !RAG ? C : (a.T - n * C < C ? a.T - n * C : C);
    __syncthreads();   // every wave past the previous chunk's tiles
    constexpr int VE = 16 / (int)sizeof(TI);
    for (int e = tid; e < C * D / VE; e += 512) {
      const int r = e / (D / VE), c = (e % (D / VE)) * VE;
      uint4 x{0u, 0u, 0u, 0u};
      if (r < rows) x = *reinterpret_cast<const uint4 *>(reinterpret_cast<const TI *>(a.k) + ((t0 + r) * a.Hqk + hq) * D + c);
      *reinterpret_cast<uint4 *>(sK + r * D + c) = x;
    }
    for (int e = tid; e < C * D / 4; e += 512) {
      const int r = e / (D / 4), c = (e % (D / 4)) * 4;
      *reinterpret_cast<float4 *>(sW + r * LDW + c) = *reinterpret_cast<const float4 *>(a.W + (cb * C + r) * D + c);
    }
    if (tid < C) sG[tid] = a.G[cb * C + tid];
    // the incoming-state cotangent of chunk n + 1 (the state after chunk n)
    if (a.dh && n + 1 < a.N) {
#pragma unroll
      for (int m = 0; m < MH; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) a.dh[((bh * a.N + n + 1) * D + 16 * m + 4 * g + i) * D + c0 + lr] = dh[m][i];
    }
    __syncthreads();
    const float gl2 = sG[C - 1] * LOG2E;
    // Y = K dh: rows of the chunk (tiles mv), dh as the B operand
    float db[KBW][8];
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) db[kb][j] = dh[2 * kb + j / 4][j % 4];
    f32x4 y[MV];
#pragma unroll
    for (int mv = 0; mv < MV; ++mv) {
      y[mv] = zero4();
#pragma unroll
      for (int kb = 0; kb < KBW; ++kb) {
        float ka[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) ka[j] = to_f32(sK[(16 * mv + lr) * D + 32 * kb + kk(j)]);
        mma_k32<PKD>(y[mv], ka, db[kb]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) y[mv][i] *= exp2_fast(gl2 - sG[16 * mv + 4 * g + i] * LOG2E);
    }
    // dh <- e^{G_last} dh - W^T X + ddh_n
    float xb[KBK][8];
#pragma unroll
    for (int kb = 0; kb < KBK; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) xb[kb][j] = y[2 * kb + j / 4][j % 4];
    const float gl = exp2_fast(gl2);
#pragma unroll
    for (int m = 0; m < MH; ++m) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < KBK; ++kb) {
        float wa[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) wa[j] = sW[(32 * kb + kk(j)) * LDW + 16 * m + lr];
        mma_k32<PS>(acc, wa, xb[kb]);
      }
      const float4 dd = *reinterpret_cast<const float4 *>(a.ddh + ((cb * MH + s) * MH + m) * 256 + lane * 4);
      const float ddv[4] = {dd.x, dd.y, dd.z, dd.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) dh[m][i] = gl * dh[m][i] - acc[i] + ddv[i];
    }
  }
  // chunk 0's incoming-state cotangent: that of h0
#pragma unroll
  for (int m = 0; m < MH; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t e = (size_t)(16 * m + 4 * g + i) * D + c0 + lr;
      if (a.dh) a.dh[(bh * a.N) * D * D + e] = dh[m][i];
      if (a.dh0) a.dh0[bh * D * D + e] = dh[m][i];
    }
}

// ----------------------------------------------------------------------------
// The forward's incoming state of every chunk, fp32 row-major, for the
// chunk gradients: h_0 = h0 and
//   h_{n+1} = e^{G_last} h_n + K_g^T (U - W h_n),   K_g = diag(e^{G_last - G}) K,
// with W and U of the transform form (fp32).  One workgroup of eight waves
// per (batch, value head), wave s holding the 16 columns 16s.. of h in
// matrix-core result registers, as in the reverse walk.
struct StatesArgs {
  int B, T, Hqk, Hv, N;
  const void *k;              // [B, T, H_qk, D] input dtype
  const float *G, *W, *U;     // transform form: [cb][C], [cb][C][D], [cb][C][D]
  const float *h0;            // [B, H_v, D, D] or null (zero)
  float *hs;                  // [B, H_v, N, D, D]
};

template <int C, typename TI, int MODE, bool RAG>
__global__ __launch_bounds__(512) void fwd_states_kernel(StatesArgs a) {
  constexpr int PW = MODE == MODE_F32 ? P_F32 : P_SPLIT_AB;   // W (fp32) x h
  constexpr int PK = MODE == MODE_F32 ? P_F32 : P_SPLIT_B;    // K^T (data) x X
  constexpr int MV = C / 16, MH = D / 16, KBW = D / 32, KBK = C / 32;
  constexpr int LDW = D + 4;
  __shared__ __align__(16) TI sK[C * D];
  __shared__ __align__(16) float sW[C * LDW];
  __shared__ __align__(16) float sG[C];
  const size_t bh = blockIdx.x;
  const int b = (int)(bh / a.Hv), hv = (int)(bh % a.Hv), hq = hv / (a.Hv / a.Hqk);
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, g = lane >> 4;
  const int s = __builtin_amdgcn_readfirstlane(tid >> 6), c0 = 16 * s;
  f32x4 h[MH];   // rows 16m + 4g + i, column c0 + lr
#pragma unroll
  for (int m = 0; m < MH; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) h[m][i] = a.h0 ? a.h0[(bh * D + 16 * m + 4 * g + i) * D + c0 + lr] : 0.f;
  auto kk = [&](int j) { return j < 4 ? 4 * g + j : 16 + 4 * g + j - 4; };
  for (int n = 0; n < a.N; ++n) {
    const size_t cb = bh * a.N + n, t0 = (size_t)b * a.T + (size_t)n * C;
    const int rows = !RAG ? C : (a.T - n * C < C ? a.T - n * C : C);
    __syncthreads();
    constexpr int VE = 16 / (int)sizeof(TI);
    for (int e = tid; e < C * D / VE; e += 512) {
      const int r = e / (D / VE), c = (e % (D / VE)) * VE;
      uint4 x{0u, 0u, 0u, 0u};
      if (r < rows) x = *reinterpret_cast<const uint4 *>(reinterpret_cast<const TI *>(a.k) + ((t0 + r) * a.Hqk + hq) * D + c);
      *reinterpret_cast<uint4 *>(sK + r * D + c) = x;
    }
    for (int e = tid; e < C * D / 4; e += 512) {
      const int r = e / (D / 4), c = (e % (D / 4)) * 4;
      *reinterpret_cast<float4 *>(sW + r * LDW + c) = *reinterpret_cast<const float4 *>(a.W + (cb * C + r) * D + c);
    }
    if (tid < C) sG[tid] = a.G[cb * C + tid];
#pragma unroll
    for (int m = 0; m < MH; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) a.hs[(cb * D + 16 * m + 4 * g + i) * D + c0 + lr] = h[m][i];
    __syncthreads();
    const float gl2 = sG[C - 1] * LOG2E;
    // X = diag(e^{G_last - G}) (U - W h)
    float hb[KBW][8];
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) hb[kb][j] = h[2 * kb + j / 4][j % 4];
    f32x4 x[MV];
#pragma unroll
    for (int mv = 0; mv < MV; ++mv) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < KBW; ++kb) {
        float wa[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) wa[j] = sW[(16 * mv + lr) * LDW + 32 * kb + kk(j)];
        mma_k32<PW>(acc, wa, hb[kb]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * mv + 4 * g + i;
        x[mv][i] = (a.U[(cb * C + r) * D + c0 + lr] - acc[i]) * exp2_fast(gl2 - sG[r] * LOG2E);
      }
    }
    // h <- e^{G_last} h + K^T X
    float xb[KBK][8];
#pragma unroll
    for (int kb = 0; kb < KBK; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) xb[kb][j] = x[2 * kb + j / 4][j % 4];
    const float gl = exp2_fast(gl2);
#pragma unroll
    for (int m = 0; m < MH; ++m) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < KBK; ++kb) {
        float ka[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) ka[j] = to_f32(sK[(32 * kb + kk(j)) * D + 16 * m + lr]);
        mma_k32<PK>(acc, ka, xb[kb]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) h[m][i] = gl * h[m][i] + acc[i];
    }
  }
}

// ----------------------------------------------------------------------------
// The gradients of one chunk (the adjoint of each line of the chunk's forward,
// in reverse order; the chunk backward that the scan kernel of "Fuse the Gated
// Delta Net inter-chunk scan into a Pallas TPU kernel", section "Changes",
// walks, with the triangular inverse's analytic backward
// dS = -(T^T dT T^T) on the strict lower triangle).  Given the chunk's
// inputs, its incoming state h (fwd_states_kernel) and the cotangent dh' of
// its outgoing state (the reverse walk's dh of the next chunk, or dh_T):
//   V'  = U - W h                          P  = (Q K^T) o Gam o [i <= r]
//   dP  = (dO V'^T) o [i <= r]             dR = dP o Gam
//   dq  = diag(E) dO h^T + dR K
//   dV  = P^T dO + diag(s) K dh'           (dV' over both paths; s = e^{G_last - G})
//   dW  = -dV h^T                          dU~ = T^T dV,  dW~ = T^T dW
//   dv  = diag(beta) dU~
//   dT  = (dW K^T) diag(beta E) + (dV V^T) diag(beta)
//   dS  = -strict-lower(T^T dT T^T)        dKk = diag(beta) dS o Gam
//   dk  = diag(s) V' dh'^T + diag(beta E) dW~ + dR^T Q + (dKk + dKk^T) K
//   dbeta_r = <dU~_r, v_r> + E_r <dW~_r, k_r> + sum_i dS_ri Gam_ri (K K^T)_ri
//   dG_r = E_r <q_r, (dO h^T)_r> + beta_r E_r <dW~_r, k_r> - s_r <(V' dh'^T)_r, k_r>
//          + (row r - column r sums of (dP o R + diag(beta) dS o K K^T) o Gam)
//          + [r = last] (e^{G_last} <h, dh'> + sum_r s_r <(V' dh'^T)_r, k_r>)
//   dg  = reverse cumulative sum of dG over the chunk
// E = e^G, Gam_ri = e^{G_r - G_i} (i <= r).  One workgroup of eight waves
// per (chunk, value head) at a time (a persistent grid); every product is a
// set of 16 x 16 result tiles shared out over the waves, each tile formed
// from operands read straight from memory (L2) in whichever orientation the
// product takes them, into the workgroup's scratch slot in between.  The
// chunk's Q, K, V and dO are first copied there as fp32 with zero rows past
// the sequence's end (the identity padding of a partial last chunk).
__device__ float g_zero_state[D * D];   // dh' of the last chunk without dh_T

struct GradArgs {
  int B, T, Hqk, Hv, N, units;
  const void *q, *k, *v;      // [B, T, H, D] input dtype
  const float *beta;          // [B, T, H_v]
  const float *dO;            // [B, T, H_v, D]
  const float *G, *Tm, *W, *U;   // transform form: [cb][C], [cb][C][C], [cb][C][D], [cb][C][D]
  const float *hs, *dh;       // [B, H_v, N, D, D]: incoming states, their cotangents
  const float *dhT;           // [B, H_v, D, D] or null (zero)
  float *dq, *dk;             // [B, T, qk_heads, D]
  int per_value_head;         // dq, dk per value head (H_v heads) instead of per key head
  float *dv;                  // [B, T, H_v, D]
  float *dg, *dbeta;          // [B, T, H_v]
  float *scratch;             // [gridDim.x][grad_slot_floats(C)]
};

template <int C> constexpr size_t grad_slot_floats() { return (size_t)9 * C * D + (size_t)7 * C * C; }

// A (rows i0.., k) times B (k, columns j0..) over k < K into acc: element
// (i, k) of A at A[i * lda + k] (TA = false) or A[k * lda + i] (TA = true),
// element (k, j) of B at B[k * ldb + j] (TB = false) or B[j * ldb + k]
// (TB = true).  Lane (lr, g) takes k = k0 + 8g + j, j = 0..7, of each block.
template <int P, bool TA, bool TB>
__device__ __forceinline__ void tile_mm(f32x4 &acc, const float *A, int lda, int i0, const float *B, int ldb, int j0,
                                        int K, int lane) {
  const int lr = lane & 15, g = lane >> 4;
#pragma unroll 2
  for (int k0 = 0; k0 < K; k0 += 32) {
    const int kb = k0 + 8 * g;
    float a8[8], b8[8];
    if constexpr (!TA) {
      ld8(A + (size_t)(i0 + lr) * lda + kb, a8);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) a8[j] = A[(size_t)(kb + j) * lda + i0 + lr];
    }
    if constexpr (TB) {
      ld8(B + (size_t)(j0 + lr) * ldb + kb, b8);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) b8[j] = B[(size_t)(kb + j) * ldb + j0 + lr];
    }
    mma_k32<P>(acc, a8, b8);
  }
}

// sums over the 16 lanes of a lane group (the columns of a result tile), and
// over the four lane groups
__device__ __forceinline__ float sum_cols(float x) {
  x += __shfl_xor(x, 1, 64);
  x += __shfl_xor(x, 2, 64);
  x += __shfl_xor(x, 4, 64);
  x += __shfl_xor(x, 8, 64);
  return x;
}
__device__ __forceinline__ float sum_groups(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}
// acc[r] += w * (row sums of a result tile v, rows i0 + 4g + i)
__device__ __forceinline__ void add_row_sums(float *acc, int i0, const float (&v)[4], float w, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x = sum_cols(v[i]);
    if ((lane & 15) == 0) atomicAdd(acc + i0 + 4 * (lane >> 4) + i, w * x);
  }
}
// acc[c] += w * (column sums of a result tile v, columns j0 + lr)
__device__ __forceinline__ void add_col_sums(float *acc, int j0, const float (&v)[4], float w, int lane) {
  const float x = sum_groups(v[0] + v[1] + v[2] + v[3]);
  if ((lane >> 4) == 0) atomicAdd(acc + j0 + lane, w * x);
}

template <int C, typename TI, int MODE, bool RAG>
__global__ __launch_bounds__(512) void bwd_chunk_kernel(GradArgs a) {
  constexpr int P = MODE == MODE_F32 ? P_F32 : P_SPLIT_AB;
  constexpr int CD = C * D, CC = C * C, DD = D * D, TC = C / 16, TD = D / 16;
  constexpr int NW = 8;   // waves
  __shared__ float sG[C], sE[C], sS[C], sB[C], sdG[C], sdB[C];
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, g = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  float *slot = a.scratch + (size_t)blockIdx.x * grad_slot_floats<C>();
  float *Qs = slot, *Ks = Qs + CD, *Vs = Ks + CD, *dOs = Vs + CD, *Vp = dOs + CD, *dV = Vp + CD, *dW = dV + CD,
        *dQp = dW + CD, *dKp = dQp + CD;
  float *R = dKp + CD, *Pm = R + CC, *dR = Pm + CC, *dT = dR + CC, *X = dT + CC, *dKk = X + CC, *Kk = dKk + CC;
  const int grp = a.Hv / a.Hqk;
  const int oheads = a.per_value_head ? a.Hv : a.Hqk;

  for (int unit = blockIdx.x; unit < a.units; unit += gridDim.x) {
    const size_t cb = unit, bh = cb / a.N;
    const int n = (int)(cb % a.N), b = (int)(bh / a.Hv), hv = (int)(bh % a.Hv), hq = hv / grp;
    const int oh = a.per_value_head ? hv : hq;
    const size_t t0 = (size_t)b * a.T + (size_t)n * C;
    const int rows = !RAG ? C : (a.T - n * C < C ? a.T - n * C : C);
    const float *Tm = a.Tm + cb * CC, *Wm = a.W + cb * CD, *Um = a.U + cb * CD, *h = a.hs + cb * DD;
    const float *dhn = n + 1 < a.N ? a.dh + (cb + 1) * DD : a.dhT ? a.dhT + bh * DD : g_zero_state;
    __syncthreads();   // the previous unit is done with the slot and the LDS sums

    // inputs as fp32, zero past the sequence's end
    constexpr int VE = 16 / (int)sizeof(TI);
    for (int e = tid; e < CD / VE; e += 64 * NW) {
      const int r = e / (D / VE), c = (e % (D / VE)) * VE;
      float xq[VE], xk[VE], xv[VE];
#pragma unroll
      for (int j = 0; j < VE; ++j) xq[j] = xk[j] = xv[j] = 0.f;
      if (r < rows) {
        const TI *pq = reinterpret_cast<const TI *>(a.q) + ((t0 + r) * a.Hqk + hq) * D + c;
        const TI *pk = reinterpret_cast<const TI *>(a.k) + ((t0 + r) * a.Hqk + hq) * D + c;
        const TI *pv = reinterpret_cast<const TI *>(a.v) + ((t0 + r) * a.Hv + hv) * D + c;
#pragma unroll
        for (int j = 0; j < VE; ++j) {
          xq[j] = to_f32(pq[j]);
          xk[j] = to_f32(pk[j]);
          xv[j] = to_f32(pv[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < VE; j += 4) {
        *reinterpret_cast<float4 *>(Qs + r * D + c + j) = float4{xq[j], xq[j + 1], xq[j + 2], xq[j + 3]};
        *reinterpret_cast<float4 *>(Ks + r * D + c + j) = float4{xk[j], xk[j + 1], xk[j + 2], xk[j + 3]};
        *reinterpret_cast<float4 *>(Vs + r * D + c + j) = float4{xv[j], xv[j + 1], xv[j + 2], xv[j + 3]};
      }
    }
    for (int e = tid; e < CD / 4; e += 64 * NW) {
      const int r = e / (D / 4), c = (e % (D / 4)) * 4;
      float4 x{0.f, 0.f, 0.f, 0.f};
      if (r < rows) x = *reinterpret_cast<const float4 *>(a.dO + ((t0 + r) * a.Hv + hv) * D + c);
      *reinterpret_cast<float4 *>(dOs + r * D + c) = x;
    }
    if (tid < C) {
      const float Gr = a.G[cb * C + tid], Gl = a.G[cb * C + C - 1];
      sG[tid] = Gr * LOG2E;
      sE[tid] = exp2_fast(Gr * LOG2E);
      sS[tid] = exp2_fast((Gl - Gr) * LOG2E);
      sB[tid] = tid < rows ? a.beta[(t0 + tid) * a.Hv + hv] : 0.f;
      sdG[tid] = 0.f;
      sdB[tid] = 0.f;
    }
    __syncthreads();
    auto gam = [&](int r, int c) { return exp2_fast(sG[r] - sG[c]); };   // Gam_rc, c <= r

    // (1) V' = U - W h;  dq's first term E o (dO h^T) and its dG term;
    //     R = Q K^T, P, K K^T
    for (int t = wv; t < TC * TD; t += NW) {
      const int i0 = 16 * (t / TD), j0 = 16 * (t % TD), c = j0 + lr;
      f32x4 acc = zero4();
      tile_mm<P, false, false>(acc, Wm, D, i0, h, D, j0, D, lane);
      f32x4 oh_ = zero4();
      tile_mm<P, false, true>(oh_, dOs, D, i0, h, D, j0, D, lane);
      float rs[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = i0 + 4 * g + i;
        Vp[r * D + c] = Um[r * D + c] - acc[i];
        dQp[r * D + c] = sE[r] * oh_[i];
        rs[i] = sE[r] * Qs[r * D + c] * oh_[i];
      }
      add_row_sums(sdG, i0, rs, 1.f, lane);
    }
    for (int t = wv; t < TC * TC; t += NW) {
      const int i0 = 16 * (t / TC), j0 = 16 * (t % TC), c = j0 + lr;
      f32x4 acc = zero4(), kk_ = zero4();
      tile_mm<P, false, true>(acc, Qs, D, i0, Ks, D, j0, D, lane);
      tile_mm<P, false, true>(kk_, Ks, D, i0, Ks, D, j0, D, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = i0 + 4 * g + i;
        R[r * C + c] = acc[i];
        Pm[r * C + c] = c <= r ? acc[i] * gam(r, c) : 0.f;
        Kk[r * C + c] = kk_[i];
      }
    }
    __syncthreads();

    // (2) dP, dR and dP o R's dG terms;  dV = P^T dO + diag(s) K dh';
    //     V' dh'^T: dk's first term and its dG terms;  <h, dh'>
    for (int t = wv; t < TC * TC; t += NW) {
      const int i0 = 16 * (t / TC), j0 = 16 * (t % TC), c = j0 + lr;
      f32x4 acc = zero4();
      tile_mm<P, false, true>(acc, dOs, D, i0, Vp, D, j0, D, lane);
      float tv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = i0 + 4 * g + i;
        const float gm = c <= r ? gam(r, c) : 0.f;
        dR[r * C + c] = acc[i] * gm;
        tv[i] = acc[i] * R[r * C + c] * gm;
      }
      add_row_sums(sdG, i0, tv, 1.f, lane);
      add_col_sums(sdG, j0, tv, -1.f, lane);
    }
    for (int t = wv; t < TC * TD; t += NW) {
      const int i0 = 16 * (t / TD), j0 = 16 * (t % TD), c = j0 + lr;
      f32x4 pd = zero4(), kd = zero4(), vd = zero4();
      tile_mm<P, true, false>(pd, Pm, C, i0, dOs, D, j0, C, lane);
      tile_mm<P, false, false>(kd, Ks, D, i0, dhn, D, j0, D, lane);
      tile_mm<P, false, true>(vd, Vp, D, i0, dhn, D, j0, D, lane);
      float dd[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = i0 + 4 * g + i;
        dV[r * D + c] = pd[i] + sS[r] * kd[i];
        const float x = sS[r] * vd[i];
        dKp[r * D + c] = x;
        dd[i] = x * Ks[r * D + c];
      }
      // dG_r -= dd_r, dG_last += sum_r dd_r
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = sum_cols(dd[i]);
        if (lr == 0) {
          atomicAdd(sdG + i0 + 4 * g + i, -x);
          atomicAdd(sdG + C - 1, x);
        }
      }
    }
    {
      float hsum = 0.f;
      for (int e = tid; e < DD / 4; e += 64 * NW) {
        const float4 x = reinterpret_cast<const float4 *>(h)[e], y = reinterpret_cast<const float4 *>(dhn)[e];
        hsum += x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
      }
      hsum = sum_groups(sum_cols(hsum));
      if (lane == 0) atomicAdd(sdG + C - 1, exp2_fast(sG[C - 1]) * hsum);
    }
    __syncthreads();

    // (3) dW = -dV h^T;  dq = E o (dO h^T) + dR K;  dU~ = T^T dV: dv, dbeta
    for (int t = wv; t < TC * TD; t += NW) {
      const int i0 = 16 * (t / TD), j0 = 16 * (t % TD), c = j0 + lr;
      f32x4 wd = zero4(), rq = zero4(), ut = zero4();
      tile_mm<P, false, true>(wd, dV, D, i0, h, D, j0, D, lane);
      tile_mm<P, false, false>(rq, dR, C, i0, Ks, D, j0, C, lane);
      tile_mm<P, true, false>(ut, Tm, C, i0, dV, D, j0, C, lane);
      float bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = i0 + 4 * g + i;
        dW[r * D + c] = -wd[i];
        if (r < rows) {
          a.dq[((t0 + r) * oheads + oh) * D + c] = dQp[r * D + c] + rq[i];
          a.dv[((t0 + r) * a.Hv + hv) * D + c] = sB[r] * ut[i];
        }
        bv[i] = ut[i] * Vs[r * D + c];
      }
      add_row_sums(sdB, i0, bv, 1.f, lane);
    }
    __syncthreads();

    // (4) dW~ = T^T dW: dk's second term, dbeta and dG terms;
    //     dT = (dW K^T) diag(beta E) + (dV V^T) diag(beta)
    for (int t = wv; t < TC * TD; t += NW) {
      const int i0 = 16 * (t / TD), j0 = 16 * (t % TD), c = j0 + lr;
      f32x4 acc = zero4();
      tile_mm<P, true, false>(acc, Tm, C, i0, dW, D, j0, C, lane);
      float rw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = i0 + 4 * g + i;
        dKp[r * D + c] += sB[r] * sE[r] * acc[i];
        rw[i] = acc[i] * Ks[r * D + c];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = sum_cols(rw[i]);
        const int r = i0 + 4 * g + i;
        if (lr == 0) {
          atomicAdd(sdB + r, sE[r] * x);
          atomicAdd(sdG + r, sB[r] * sE[r] * x);
        }
      }
    }
    for (int t = wv; t < TC * TC; t += NW) {
      const int i0 = 16 * (t / TC), j0 = 16 * (t % TC), c = j0 + lr;
      f32x4 wk = zero4(), vv = zero4();
      tile_mm<P, false, true>(wk, dW, D, i0, Ks, D, j0, D, lane);
      tile_mm<P, false, true>(vv, dV, D, i0, Vs, D, j0, D, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = i0 + 4 * g + i;
        dT[r * C + c] = (wk[i] * sE[c] + vv[i]) * sB[c];
      }
    }
    __syncthreads();

    // (5) X = dT T^T
    for (int t = wv; t < TC * TC; t += NW) {
      const int i0 = 16 * (t / TC), j0 = 16 * (t % TC), c = j0 + lr;
      f32x4 acc = zero4();
      tile_mm<P, false, true>(acc, dT, C, i0, Tm, C, j0, C, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) X[(i0 + 4 * g + i) * C + c] = acc[i];
    }
    __syncthreads();

    // (6) dS = -strict-lower(T^T X): dbeta, dG terms, dKk
    for (int t = wv; t < TC * TC; t += NW) {
      const int i0 = 16 * (t / TC), j0 = 16 * (t % TC), c = j0 + lr;
      f32x4 acc = zero4();
      tile_mm<P, true, false>(acc, Tm, C, i0, X, C, j0, C, lane);
      float bs[4], tv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = i0 + 4 * g + i;
        const float ds = c < r ? -acc[i] : 0.f;
        const float gm = c < r ? gam(r, c) : 0.f;
        const float kkv = Kk[r * C + c];
        bs[i] = ds * gm * kkv;
        tv[i] = sB[r] * bs[i];
        dKk[r * C + c] = sB[r] * ds * gm;
      }
      add_row_sums(sdB, i0, bs, 1.f, lane);
      add_row_sums(sdG, i0, tv, 1.f, lane);
      add_col_sums(sdG, j0, tv, -1.f, lane);
    }
    __syncthreads();

    // (7) dk = diag(s) V' dh'^T + diag(beta E) dW~ + dR^T Q + (dKk + dKk^T) K;
    //     dg = reverse cumulative sum of dG, dbeta
    for (int t = wv; t < TC * TD; t += NW) {
      const int i0 = 16 * (t / TD), j0 = 16 * (t % TD), c = j0 + lr;
      f32x4 acc;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = dKp[(i0 + 4 * g + i) * D + c];
      tile_mm<P, true, false>(acc, dR, C, i0, Qs, D, j0, C, lane);
      tile_mm<P, false, false>(acc, dKk, C, i0, Ks, D, j0, C, lane);
      tile_mm<P, true, false>(acc, dKk, C, i0, Ks, D, j0, C, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = i0 + 4 * g + i;
        if (r < rows) a.dk[((t0 + r) * oheads + oh) * D + c] = acc[i];
      }
    }
    if (tid < rows) {
      float sdg = 0.f;
      for (int j = tid; j < C; ++j) sdg += sdG[j];
      a.dg[(t0 + tid) * a.Hv + hv] = sdg;
      a.dbeta[(t0 + tid) * a.Hv + hv] = sdB[tid];
    }
  }
}

// dq, dk of a key head: the sum over the value heads that read it, from the
// per-value-head rows [rows][H_v][D] into [rows][H_qk][D]
__global__ void sum_value_heads_kernel(const float *src, float *dst, size_t rows, int Hqk, int grp) {
  const size_t n4 = rows * Hqk * (D / 4);
  for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n4; e += (size_t)gridDim.x * blockDim.x) {
    const size_t c4 = e % (D / 4), rh = e / (D / 4), hq = rh % Hqk, row = rh / Hqk;
    float4 s{0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < grp; ++p) {
      const float4 x = reinterpret_cast<const float4 *>(src)[((row * Hqk + hq) * grp + p) * (D / 4) + c4];
      s.x += x.x; s.y += x.y; s.z += x.z; s.w += x.w;
    }
    reinterpret_cast<float4 *>(dst)[e] = s;
  }
}

}  // namespace gdn
