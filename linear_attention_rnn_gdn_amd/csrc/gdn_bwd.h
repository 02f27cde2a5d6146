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

}  // namespace gdn
