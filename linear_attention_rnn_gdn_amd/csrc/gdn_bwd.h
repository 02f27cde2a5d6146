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

// the chunk-parallel term ddh_n = Qeff^T dO, one workgroup per (chunk, value
// head) of eight waves at C = 128 (four at C = 64); Qeff = diag(e^G) Q - P W
// is formed per query tile: wave w takes query tiles {w', R-1-w'} (w' = w mod
// 4; {w'} at C = 64), forms their P^T tiles in registers and, with the other
// wave of the same w' at C = 128, half of the Qeff columns each; Qeff is then
// written to LDS transposed next to dO^T for the product.
template <int C> constexpr int ddh_threads() { return C >= 128 ? 512 : 256; }
template <int C, typename TI> struct BwdLds {
  static constexpr int LDQ = D + 16 / (int)sizeof(TI);     // Q, K row stride: 16 bytes of padding put
                                                           // the 16 rows a fragment read touches on distinct banks
  static constexpr int QK = C * LDQ * (int)sizeof(TI);     // one row-major Q or K tile
  static constexpr int LDT = C + 4;                        // row stride of the [D][C] transposed tiles
  static constexpr int LDW = D + 4;                        // row stride of W [C][D]
  static constexpr int TB = D * LDT * 4;                   // a transposed fp32 tile
  static constexpr int RA = 2 * QK > TB ? 2 * QK : TB;     // region A: Q, K; then dO^T
  static constexpr int RB = C * LDW * 4 > TB ? C * LDW * 4 : TB;   // region B: W; then Qeff^T
};

// 16 bytes at base + off_bytes, or zero where the row is not one of the
// chunk's tokens (real = false; the offset then names the chunk's last row,
// so the read stays in bounds).  The read is issued either way and the value
// selected: a read behind a branch is waited for where the branches join.
__device__ __forceinline__ uint4 row_or_zero(const void *base, size_t off_bytes, bool real) {
  const uint4 x = *reinterpret_cast<const uint4 *>(reinterpret_cast<const char *>(base) + off_bytes);
  return real ? x : uint4{0u, 0u, 0u, 0u};
}

template <int C, typename TI, int MODE, bool RAG>
__global__ __launch_bounds__(ddh_threads<C>()) void bwd_ddh_kernel(FwdArgs fa, BwdArgs a) {
  using L = BwdLds<C, TI>;
  constexpr int PX = MODE == MODE_F32 ? P_F32 : P_BF16;       // K Q^T
  constexpr int PS = MODE == MODE_F32 ? P_F32 : P_SPLIT_AB;   // fp32 x fp32
  constexpr int R = C / 16, RU = R >= 8 ? 2 : 1, KBD = D / 32, TD = D / 16;
  constexpr int NTH = ddh_threads<C>(), NW = NTH / 64;        // threads, waves
  constexpr int DS = NW / 4, TDW = TD / DS;                   // waves per query-tile pair, Qeff column tiles each
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
  const int wq = wv % 4, dt0 = (wv / 4) * TDW;   // query-tile pair, first Qeff column tile

  // Q, K rows (zero past the chunk's tokens), W (row stride D + 4) and G
  constexpr int VE = 16 / (int)sizeof(TI);
  // (rows past the chunk's tokens read from its last row, then zeroed: a
  // read behind a branch is waited for at once)
  static_assert((C * D / VE) % NTH == 0, "whole vectors per thread");
#pragma unroll 4
  for (int u = 0; u < C * D / VE / NTH; ++u) {
    const int e = tid + NTH * u, r = e / (D / VE), c = (e % (D / VE)) * VE;
    const size_t row = ((t0 + (r < rows ? r : rows - 1)) * a.Hqk + hq) * D + c;
    const uint4 xq = row_or_zero(a.q, row * sizeof(TI), r < rows), xk = row_or_zero(a.k, row * sizeof(TI), r < rows);
    *reinterpret_cast<uint4 *>(sQ + r * L::LDQ + c) = xq;
    *reinterpret_cast<uint4 *>(sK + r * L::LDQ + c) = xk;
  }
  for (int e = tid; e < C * D / 4; e += NTH) {
    const int r = e / (D / 4), c = (e % (D / 4)) * 4;
    *reinterpret_cast<float4 *>(sW + r * L::LDW + c) = *reinterpret_cast<const float4 *>(a.W + (cb * C + r) * D + c);
  }
  if (tid < C) sG[tid] = a.G[cb * C + tid];
  __syncthreads();

  // P^T tiles (key tile kt, query tile rt), kt <= rt, masked and decayed:
  // lane (lr, g) holds P^T[16kt + 4g + i][16rt + lr]; two key tiles stacked
  // are the A operand of P W with the keys in the order kk(g, j)
  auto row8 = [&](const TI *t, int r, int k0, float (&x)[8]) {   // 8 consecutive elements of row r
    ld8(t + r * L::LDQ + k0, x);
  };
  f32x4 pt[RU][R];
  float qeff[RU][TDW][4];
#pragma unroll
  for (int u = 0; u < RU; ++u) {
    const int rt = u == 0 ? wq : R - 1 - wq;
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
    for (int jt = 0; jt < TDW; ++jt) {
      const int dt = dt0 + jt;
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
        qeff[u][jt][i] = exp2_fast(sG[rr] * LOG2E) * to_f32(sQ[rr * L::LDQ + 16 * dt + lr]) - acc[i];
      }
    }
  }
  __syncthreads();   // every wave past W, Q and K
  // Qeff^T [d][r] and dO^T [c][r] (zero past the chunk's tokens)
#pragma unroll
  for (int u = 0; u < RU; ++u) {
    const int rt = u == 0 ? wq : R - 1 - wq;
#pragma unroll
    for (int jt = 0; jt < TDW; ++jt)
      *reinterpret_cast<float4 *>(sQt + (16 * (dt0 + jt) + lr) * L::LDT + 16 * rt + 4 * g) =
          float4{qeff[u][jt][0], qeff[u][jt][1], qeff[u][jt][2], qeff[u][jt][3]};
  }
  static_assert((C * D / 4) % NTH == 0, "whole vectors per thread");
#pragma unroll 4
  for (int u = 0; u < C * D / 4 / NTH; ++u) {
    const int e = tid + NTH * u, r = e / (D / 4), c = (e % (D / 4)) * 4;
    const float4 x = __builtin_bit_cast(
        float4, row_or_zero(a.dO, (((t0 + (r < rows ? r : rows - 1)) * a.Hv + hv) * D + c) * sizeof(float), r < rows));
    sOt[(c + 0) * L::LDT + r] = x.x;
    sOt[(c + 1) * L::LDT + r] = x.y;
    sOt[(c + 2) * L::LDT + r] = x.z;
    sOt[(c + 3) * L::LDT + r] = x.w;
  }
  __syncthreads();
  // ddh tiles (d tile dt, column tile ct): wave w takes tiles w, w + NW, ...
  for (int t = wv; t < TD * TD; t += NW) {
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

__device__ __forceinline__ uint4 uint4_pair(uint2 a, uint2 b) { return uint4{a.x, a.y, b.x, b.y}; }

// 8 k-values of an input-dtype row in the order kk(g, j) (p points at the
// block's first k-value): bf16 data as one exact bf16 fragment, fp32 as fp32
template <typename TI>
__device__ __forceinline__ Frag<sizeof(TI) == 2 ? F_BF16 : F_F32> kk_frag(const TI *p, int g) {
  if constexpr (sizeof(TI) == 2) {
    Frag<F_BF16> f;
    f.hi = __builtin_bit_cast(bf16x8, uint4_pair(*reinterpret_cast<const uint2 *>(p + 4 * g),
                                                 *reinterpret_cast<const uint2 *>(p + 16 + 4 * g)));
    return f;
  } else {
    Frag<F_F32> f;
    const float4 u = *reinterpret_cast<const float4 *>(p + 4 * g), w = *reinterpret_cast<const float4 *>(p + 16 + 4 * g);
    f.v[0] = u.x; f.v[1] = u.y; f.v[2] = u.z; f.v[3] = u.w;
    f.v[4] = w.x; f.v[5] = w.y; f.v[6] = w.z; f.v[7] = w.w;
    return f;
  }
}

// A staged operand in LDS: up to 128 rows (the rows of A, or the columns of
// B, of a product) of up to 128 k-values each, k contiguous.  With bf16
// inputs every value is split once, when staged, into hi and lo bf16 planes
// (the products' hi/lo policy), so that a fragment is two 16-byte reads; with
// fp32 inputs the values stay fp32.  A source matrix is staged as is or
// transposed, whichever puts its contraction index along the rows.
constexpr int GLDH = 136;   // bf16 plane row stride (elements; 272 bytes)
constexpr int GLDX = 132;   // fp32 row stride
template <int MODE> struct GStage {
  static constexpr bool SPLIT = MODE != MODE_F32;
  static constexpr int KIND = SPLIT ? F_SPLIT : F_F32;
  static constexpr int BYTES = SPLIT ? 2 * 128 * GLDH * 2 : 128 * GLDX * 4;
  // source row r, columns c .. c+3 to (r, c..c+3), or transposed to (c..c+3, r)
  template <bool TR>
  __device__ static void put4(char *buf, int r, int c, float4 x) {
    if constexpr (SPLIT) {
      unsigned short *hi = reinterpret_cast<unsigned short *>(buf), *lo = hi + 128 * GLDH;
      const unsigned h01 = pk_bf16(x.x, x.y), h23 = pk_bf16(x.z, x.w);
      const unsigned l01 = pk_bf16(x.x - __builtin_bit_cast(float, h01 << 16),
                                   x.y - __builtin_bit_cast(float, h01 & 0xffff0000u));
      const unsigned l23 = pk_bf16(x.z - __builtin_bit_cast(float, h23 << 16),
                                   x.w - __builtin_bit_cast(float, h23 & 0xffff0000u));
      if constexpr (!TR) {
        *reinterpret_cast<uint2 *>(hi + r * GLDH + c) = uint2{h01, h23};
        *reinterpret_cast<uint2 *>(lo + r * GLDH + c) = uint2{l01, l23};
      } else {
        hi[(c + 0) * GLDH + r] = (unsigned short)h01;
        hi[(c + 1) * GLDH + r] = (unsigned short)(h01 >> 16);
        hi[(c + 2) * GLDH + r] = (unsigned short)h23;
        hi[(c + 3) * GLDH + r] = (unsigned short)(h23 >> 16);
        lo[(c + 0) * GLDH + r] = (unsigned short)l01;
        lo[(c + 1) * GLDH + r] = (unsigned short)(l01 >> 16);
        lo[(c + 2) * GLDH + r] = (unsigned short)l23;
        lo[(c + 3) * GLDH + r] = (unsigned short)(l23 >> 16);
      }
    } else {
      float *f = reinterpret_cast<float *>(buf);
      if constexpr (!TR) {
        *reinterpret_cast<float4 *>(f + r * GLDX + c) = x;
      } else {
        f[(c + 0) * GLDX + r] = x.x;
        f[(c + 1) * GLDX + r] = x.y;
        f[(c + 2) * GLDX + r] = x.z;
        f[(c + 3) * GLDX + r] = x.w;
      }
    }
  }
  // a 4 x 4 block of the source, rows r0 .. r0+3 and columns c0 .. c0+3
  // (v[row][column]), transposed: column c0 + e becomes row c0 + e with the
  // four values at r0 .. r0+3 (one 8-byte write per plane and row)
  __device__ static void put4x4t(char *buf, int r0, int c0, const float (&v)[4][4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (SPLIT) {
        unsigned short *hi = reinterpret_cast<unsigned short *>(buf), *lo = hi + 128 * GLDH;
        const unsigned h01 = pk_bf16(v[0][e], v[1][e]), h23 = pk_bf16(v[2][e], v[3][e]);
        const unsigned l01 = pk_bf16(v[0][e] - __builtin_bit_cast(float, h01 << 16),
                                     v[1][e] - __builtin_bit_cast(float, h01 & 0xffff0000u));
        const unsigned l23 = pk_bf16(v[2][e] - __builtin_bit_cast(float, h23 << 16),
                                     v[3][e] - __builtin_bit_cast(float, h23 & 0xffff0000u));
        *reinterpret_cast<uint2 *>(hi + (c0 + e) * GLDH + r0) = uint2{h01, h23};
        *reinterpret_cast<uint2 *>(lo + (c0 + e) * GLDH + r0) = uint2{l01, l23};
      } else {
        *reinterpret_cast<float4 *>(reinterpret_cast<float *>(buf) + (c0 + e) * GLDX + r0) =
            float4{v[0][e], v[1][e], v[2][e], v[3][e]};
      }
    }
  }
  // row i, the k-values k0 + kk(g, j) of a block of 32 (k0 a multiple of
  // 32): 4g .. 4g+3 and 16+4g .. 16+4g+3, the rows two stacked result tiles
  // give lane group g
  __device__ static Frag<KIND> frag_kk(const char *buf, int i, int k0, int g) {
    Frag<KIND> f;
    if constexpr (SPLIT) {
      const __bf16 *hi = reinterpret_cast<const __bf16 *>(buf), *lo = hi + 128 * GLDH;
      const int o = i * GLDH + k0 + 4 * g;
      f.hi = __builtin_bit_cast(bf16x8, uint4_pair(*reinterpret_cast<const uint2 *>(hi + o),
                                                   *reinterpret_cast<const uint2 *>(hi + o + 16)));
      f.lo = __builtin_bit_cast(bf16x8, uint4_pair(*reinterpret_cast<const uint2 *>(lo + o),
                                                   *reinterpret_cast<const uint2 *>(lo + o + 16)));
    } else {
      const float *x = reinterpret_cast<const float *>(buf) + i * GLDX + k0 + 4 * g;
      const float4 u = *reinterpret_cast<const float4 *>(x), w = *reinterpret_cast<const float4 *>(x + 16);
      f.v[0] = u.x; f.v[1] = u.y; f.v[2] = u.z; f.v[3] = u.w;
      f.v[4] = w.x; f.v[5] = w.y; f.v[6] = w.z; f.v[7] = w.w;
    }
    return f;
  }
  // row i, k-values k0 .. k0+7 (k0 a multiple of 8)
  __device__ static Frag<KIND> frag(const char *buf, int i, int k0) {
    Frag<KIND> f;
    if constexpr (SPLIT) {
      const __bf16 *hi = reinterpret_cast<const __bf16 *>(buf), *lo = hi + 128 * GLDH;
      f.hi = *reinterpret_cast<const bf16x8 *>(hi + i * GLDH + k0);
      f.lo = *reinterpret_cast<const bf16x8 *>(lo + i * GLDH + k0);
    } else {
      float x[8];
      ld8(reinterpret_cast<const float *>(buf) + i * GLDX + k0, x);
#pragma unroll
      for (int j = 0; j < 8; ++j) f.v[j] = x[j];
    }
    return f;
  }
};

// NR x NC fp32 rows (row stride ld) staged, 512 threads.  Transposed, each
// thread takes 4 x 4 blocks, the lanes of a wave consecutive row blocks of
// one column block, so that the transposed rows are written contiguously
template <int MODE, int NR, int NC, bool TR>
__device__ __forceinline__ void stage(char *buf, const float *src, size_t ld, int tid) {
  if constexpr (!TR) {
    constexpr int N4 = NR * NC / 4, PER = N4 / 512;
    static_assert(N4 % 512 == 0, "whole float4 per thread");
    float4 v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + 512 * u, r = e / (NC / 4), c = (e % (NC / 4)) * 4;
      v[u] = *reinterpret_cast<const float4 *>(src + r * ld + c);
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + 512 * u, r = e / (NC / 4), c = (e % (NC / 4)) * 4;
      GStage<MODE>::template put4<false>(buf, r, c, v[u]);
    }
  } else {
    constexpr int RB = NR / 4, NB = RB * (NC / 4), PER = (NB + 511) / 512;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int b = tid + 512 * u;
      if (NB % 512 != 0 && b >= NB) break;
      const int r0 = 4 * (b % RB), c0 = 4 * (b / RB);
      float v[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 x = *reinterpret_cast<const float4 *>(src + (r0 + i) * ld + c0);
        v[i][0] = x.x; v[i][1] = x.y; v[i][2] = x.z; v[i][3] = x.w;
      }
      GStage<MODE>::put4x4t(buf, r0, c0, v);
    }
  }
}
// NR x D input rows of type T (row stride ld elements) staged as fp32 values,
// rows at or past `rows` (>= 1) zero (row_or_zero).
template <int MODE, int NR, bool TR, typename T>
__device__ __forceinline__ void stage_in(char *buf, const T *src, size_t ld, int rows, int tid) {
  constexpr int VE = 16 / (int)sizeof(T);
  if constexpr (!TR) {
    constexpr int NV = NR * D / VE, PER = NV / 512;
    static_assert(NV % 512 == 0, "whole vectors per thread");
    uint4 v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + 512 * u, r = e / (D / VE), c = (e % (D / VE)) * VE;
      v[u] = row_or_zero(src, ((r < rows ? r : rows - 1) * ld + c) * sizeof(T), r < rows);
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + 512 * u, r = e / (D / VE), c = (e % (D / VE)) * VE;
      const T *x = reinterpret_cast<const T *>(&v[u]);
#pragma unroll
      for (int j = 0; j < VE; j += 4)
        GStage<MODE>::template put4<false>(buf, r, c + j,
                                           float4{to_f32(x[j]), to_f32(x[j + 1]), to_f32(x[j + 2]), to_f32(x[j + 3])});
    }
  } else {
    // blocks of 4 rows x one 16-byte vector, the lanes of a wave consecutive
    // row blocks of one column block (as in stage)
    constexpr int RB = NR / 4, NB = RB * (D / VE), PER = (NB + 511) / 512;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int b = tid + 512 * u;
      if (NB % 512 != 0 && b >= NB) break;
      const int r0 = 4 * (b % RB), c0 = VE * (b / RB);
      uint4 w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = row_or_zero(src, ((r0 + i < rows ? r0 + i : rows - 1) * ld + c0) * sizeof(T), r0 + i < rows);
#pragma unroll
      for (int h = 0; h < VE; h += 4) {
        float v[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const T *x = reinterpret_cast<const T *>(&w[i]);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[i][e] = to_f32(x[h + e]);
        }
        GStage<MODE>::put4x4t(buf, r0, c0 + h, v);
      }
    }
  }
}

// the reverse walk: one workgroup of eight waves per (batch, value head),
// wave s holding the 16 columns 16s.. of dh in matrix-core result registers;
// per chunk, from the last to the first, K (row-major, the input rows), W^T
// (staged transposed, split once) and G go to LDS, then
//   Y = K dh,  X = diag(e^{G_last - G}) Y,  dh <- e^{G_last} dh - W^T X + ddh_n
template <int C, typename TI, int MODE> struct BwdWalkLds {
  static constexpr int LDK = D + 16 / (int)sizeof(TI);   // K row stride: 16 bytes of padding put the
                                                         // 16 rows a fragment read touches on distinct banks
  static constexpr int K_OFF = 0;                                    // K rows
  static constexpr int W_OFF = K_OFF + C * LDK * (int)sizeof(TI);    // W^T, staged (split once)
  static constexpr int G_OFF = W_OFF + GStage<MODE>::BYTES;
  static constexpr int BYTES = G_OFF + C * 4;
};

template <int C, typename TI, int MODE, bool RAG>
__device__ __forceinline__ void bwd_walk_body(const BwdArgs &a, size_t bh, char *lds) {
  constexpr int PKD = MODE == MODE_F32 ? P_F32 : P_SPLIT_B;    // K (data) x dh
  constexpr int PS = MODE == MODE_F32 ? P_F32 : P_SPLIT_AB;    // W^T x X
  constexpr int MV = C / 16, MH = D / 16, KBW = D / 32, KBK = C / 32;
  using L = BwdWalkLds<C, TI, MODE>;
  using GS = GStage<MODE>;
  static_assert(PolicyKinds<PS>::a == GS::KIND, "W^T staged as the product's A operand");
  constexpr int LDK = L::LDK;
  TI *sK = reinterpret_cast<TI *>(lds + L::K_OFF);
  char *sW = lds + L::W_OFF;
  float *sG = reinterpret_cast<float *>(lds + L::G_OFF);
  const int b = (int)(bh / a.Hv), hv = (int)(bh % a.Hv), hq = hv / (a.Hv / a.Hqk);
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, g = lane >> 4;
  const int s = __builtin_amdgcn_readfirstlane(tid >> 6), c0 = 16 * s;
  // dh tiles: dh[m] holds rows 16m + 4g + i, column c0 + lr
  f32x4 dh[MH];
#pragma unroll
  for (int m = 0; m < MH; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) dh[m][i] = a.dhT ? a.dhT[(bh * D + 16 * m + 4 * g + i) * D + c0 + lr] : 0.f;
  for (int n = a.N - 1; n >= 0; --n) {
    const size_t cb = bh * a.N + n, t0 = (size_t)b * a.T + (size_t)n * C;
    const int rows = !RAG ? C : (a.T - n * C < C ? a.T - n * C : C);
    // the lane's indices, opaque each chunk: the LDS addresses derived from
    // them are formed where used instead of being hoisted out of the loop
    // (more than the registers hold)
    int tl = tid;
    asm volatile("" : "+v"(tl));
    const int lane = tl & 63, lr = lane & 15, g = lane >> 4;
    __syncthreads();   // every wave past the previous chunk's tiles
    constexpr int VE = 16 / (int)sizeof(TI);
    // (rows past the chunk's tokens read from its last row, then zeroed: a
    // read behind a branch is waited for at once)
    static_assert((C * D / VE) % 512 == 0, "whole vectors per thread");
    {
      uint4 xk[C * D / VE / 512];
#pragma unroll
      for (int u = 0; u < C * D / VE / 512; ++u) {
        const int e = tl + 512 * u, r = e / (D / VE), c = (e % (D / VE)) * VE;
        xk[u] = row_or_zero(a.k, (((t0 + (r < rows ? r : rows - 1)) * a.Hqk + hq) * D + c) * sizeof(TI), r < rows);
      }
#pragma unroll
      for (int u = 0; u < C * D / VE / 512; ++u) {
        const int e = tl + 512 * u, r = e / (D / VE), c = (e % (D / VE)) * VE;
        *reinterpret_cast<uint4 *>(sK + r * LDK + c) = xk[u];
      }
    }
    stage<MODE, C, D, true>(sW, a.W + cb * C * D, D, tl);
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
    // Y = K dh, dh as the B operand split once for all row tiles (two
    // stacked result tiles give lane group g the k-values kk(g, j))
    Frag<PolicyKinds<PKD>::b> db[KBW];
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = dh[2 * kb + j / 4][j % 4];
      db[kb] = make_frag<PolicyKinds<PKD>::b>(x);
    }
    f32x4 y[MV];
#pragma unroll
    for (int mv = 0; mv < MV; ++mv) {
      y[mv] = zero4();
#pragma unroll
      for (int kb = 0; kb < KBW; ++kb) mma(y[mv], kk_frag<TI>(sK + (16 * mv + lr) * LDK + 32 * kb, g), db[kb]);
#pragma unroll
      for (int i = 0; i < 4; ++i) y[mv][i] *= exp2_fast(gl2 - sG[16 * mv + 4 * g + i] * LOG2E);
    }
    // dh <- e^{G_last} dh - W^T X + ddh_n, X split once
    Frag<PolicyKinds<PS>::b> xb[KBK];
#pragma unroll
    for (int kb = 0; kb < KBK; ++kb) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = y[2 * kb + j / 4][j % 4];
      xb[kb] = make_frag<PolicyKinds<PS>::b>(x);
    }
    const float gl = exp2_fast(gl2);
#pragma unroll
    for (int m = 0; m < MH; ++m) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < KBK; ++kb) mma(acc, GS::frag_kk(sW, 16 * m + lr, 32 * kb, g), xb[kb]);
      const float4 dd = *reinterpret_cast<const float4 *>(a.ddh + ((cb * MH + s) * MH + m) * 256 + lane * 4);
      const float ddv[4] = {dd.x, dd.y, dd.z, dd.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) dh[m][i] = gl * dh[m][i] - acc[i] + ddv[i];
    }
  }
  // chunk 0's incoming-state cotangent: that of h0 (one branch per
  // destination: a branch per element made the compiler wait for each store
  // before issuing the next)
  auto put = [&](float *dst) {
#pragma unroll
    for (int m = 0; m < MH; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(size_t)(16 * m + 4 * g + i) * D + c0 + lr] = dh[m][i];
  };
  if (a.dh) put(a.dh + (bh * a.N) * D * D);
  if (a.dh0) put(a.dh0 + bh * D * D);
}

template <int C, typename TI, int MODE, bool RAG>
__global__ __launch_bounds__(512) void bwd_walk_kernel(BwdArgs a) {
  __shared__ __align__(16) char lds[BwdWalkLds<C, TI, MODE>::BYTES];
  bwd_walk_body<C, TI, MODE, RAG>(a, blockIdx.x, lds);
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

template <int C, typename TI, int MODE> struct StatesLds {
  static constexpr int LDKT = C + 8;                                  // K^T row stride (elements)
  static constexpr int KT_OFF = 0;                                    // K^T: row d, the chunk's tokens along k
  static constexpr int W_OFF = KT_OFF + D * LDKT * (int)sizeof(TI);   // W rows, split once
  static constexpr int G_OFF = W_OFF + GStage<MODE>::BYTES;
  static constexpr int BYTES = G_OFF + C * 4;
};

template <int C, typename TI, int MODE, bool RAG>
__device__ __forceinline__ void fwd_states_body(const StatesArgs &a, size_t bh, char *lds) {
  constexpr int PW = MODE == MODE_F32 ? P_F32 : P_SPLIT_AB;   // W (fp32) x h
  constexpr int PK = MODE == MODE_F32 ? P_F32 : P_SPLIT_B;    // K^T (data) x X
  using GS = GStage<MODE>;
  static_assert(PolicyKinds<PW>::a == GS::KIND, "W staged as the product's A operand");
  constexpr int MV = C / 16, MH = D / 16, KBW = D / 32, KBK = C / 32;
  using L = StatesLds<C, TI, MODE>;
  constexpr int LDKT = L::LDKT;
  TI *sKt = reinterpret_cast<TI *>(lds + L::KT_OFF);
  char *sW = lds + L::W_OFF;
  float *sG = reinterpret_cast<float *>(lds + L::G_OFF);
  const int b = (int)(bh / a.Hv), hv = (int)(bh % a.Hv), hq = hv / (a.Hv / a.Hqk);
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, g = lane >> 4;
  const int s = __builtin_amdgcn_readfirstlane(tid >> 6), c0 = 16 * s;
  f32x4 h[MH];   // rows 16m + 4g + i, column c0 + lr
#pragma unroll
  for (int m = 0; m < MH; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) h[m][i] = a.h0 ? a.h0[(bh * D + 16 * m + 4 * g + i) * D + c0 + lr] : 0.f;
  for (int n = 0; n < a.N; ++n) {
    const size_t cb = bh * a.N + n, t0 = (size_t)b * a.T + (size_t)n * C;
    const int rows = !RAG ? C : (a.T - n * C < C ? a.T - n * C : C);
    __syncthreads();
    // K^T: blocks of 4 rows x one 16-byte vector transposed in registers, the
    // lanes of a wave consecutive row blocks, so that each transposed row is
    // written 4 values per lane, contiguous across lanes
    constexpr int VE = 16 / (int)sizeof(TI), RB = C / 4, NB = RB * (D / VE);
    struct Four {
      TI v[4];
    };
    using W4 = typename std::conditional<sizeof(TI) == 2, uint2, uint4>::type;
    for (int bk = tid; bk < NB; bk += 512) {
      const int r0 = 4 * (bk % RB), c = VE * (bk / RB);
      uint4 w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = row_or_zero(a.k, (((t0 + (r0 + i < rows ? r0 + i : rows - 1)) * a.Hqk + hq) * D + c) * sizeof(TI),
                           r0 + i < rows);
#pragma unroll
      for (int j = 0; j < VE; ++j) {
        Four f;
#pragma unroll
        for (int i = 0; i < 4; ++i) f.v[i] = reinterpret_cast<const TI *>(&w[i])[j];
        *reinterpret_cast<W4 *>(sKt + (c + j) * LDKT + r0) = __builtin_bit_cast(W4, f);
      }
    }
    stage<MODE, C, D, false>(sW, a.W + cb * C * D, D, tid);
    if (tid < C) sG[tid] = a.G[cb * C + tid];
#pragma unroll
    for (int m = 0; m < MH; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) a.hs[(cb * D + 16 * m + 4 * g + i) * D + c0 + lr] = h[m][i];
    __syncthreads();
    const float gl2 = sG[C - 1] * LOG2E;
    // X = diag(e^{G_last - G}) (U - W h), h as the B operand split once (U
    // lands in the V' tiles themselves)
    Frag<PolicyKinds<PW>::b> hb[KBW];
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = h[2 * kb + j / 4][j % 4];
      hb[kb] = make_frag<PolicyKinds<PW>::b>(x);
    }
    f32x4 x[MV];
#pragma unroll
    for (int mv = 0; mv < MV; ++mv) {
      // (one row tile's U at a time: hoisted all at once they outgrow the registers)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4; ++i) x[mv][i] = a.U[(cb * C + 16 * mv + 4 * g + i) * D + c0 + lr];
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < KBW; ++kb) mma(acc, GS::frag_kk(sW, 16 * mv + lr, 32 * kb, g), hb[kb]);
#pragma unroll
      for (int i = 0; i < 4; ++i) x[mv][i] = (x[mv][i] - acc[i]) * exp2_fast(gl2 - sG[16 * mv + 4 * g + i] * LOG2E);
    }
    // h <- e^{G_last} h + K^T X, X split once
    Frag<PolicyKinds<PK>::b> xb[KBK];
#pragma unroll
    for (int kb = 0; kb < KBK; ++kb) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = x[2 * kb + j / 4][j % 4];
      xb[kb] = make_frag<PolicyKinds<PK>::b>(v);
    }
    const float gl = exp2_fast(gl2);
#pragma unroll
    for (int m = 0; m < MH; ++m) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < KBK; ++kb) mma(acc, kk_frag<TI>(sKt + (16 * m + lr) * LDKT + 32 * kb, g), xb[kb]);
#pragma unroll
      for (int i = 0; i < 4; ++i) h[m][i] = gl * h[m][i] + acc[i];
    }
  }
}

// The forward-state walk and the reverse walk in one launch: they depend on
// the transform (and the reverse walk on its chunk term) but not on each
// other, and each fills only one workgroup per (batch, value head), so they
// run side by side.  Workgroups [0, B H_v) walk the forward states, the
// next B H_v the cotangents; the two share one LDS buffer.
template <int C, typename TI, int MODE, bool RAG>
__global__ __launch_bounds__(512) void bwd_walks_kernel(StatesArgs sa, BwdArgs ba) {
  constexpr int SB = StatesLds<C, TI, MODE>::BYTES, WB = BwdWalkLds<C, TI, MODE>::BYTES;
  __shared__ __align__(16) char lds[SB > WB ? SB : WB];
  const unsigned nbh = (unsigned)(sa.B * sa.Hv);
  if (blockIdx.x < nbh) fwd_states_body<C, TI, MODE, RAG>(sa, blockIdx.x, lds);
  else bwd_walk_body<C, TI, MODE, RAG>(ba, blockIdx.x - nbh, lds);
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
// per (chunk, value head) at a time (a persistent grid).  Every product is a
// set of 16 x 16 result tiles shared out over the waves, formed from its two
// operands staged whole in LDS (two buffers of up to 128 x 128 fp32, loaded
// with coalesced 16-byte reads, the chunk's inputs converted to fp32 with
// zero rows past the sequence's end -- the identity padding of a partial last
// chunk); either operand may be read transposed from its buffer.  The
// intermediates go to the workgroup's scratch slot between products.
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

template <int C> constexpr size_t grad_slot_floats() { return (size_t)5 * C * D + (size_t)7 * C * C; }

// acc += A B for the 16 x 16 tile (rows i0.. of A, columns j0.. of B) over K
// k-values: A staged with its rows, B with its columns, along the buffer rows.
// Lane (lr, g) takes k = k0 + 8g .. k0 + 8g + 7 of each block of 32.
template <int MODE, int K>
__device__ __forceinline__ void tile_st(f32x4 &acc, const char *A, int i0, const char *B, int j0, int lane) {
  const int lr = lane & 15, g = lane >> 4;
#pragma unroll 2
  for (int k0 = 0; k0 < K; k0 += 32) {
    const int kb = k0 + 8 * g;
    mma(acc, GStage<MODE>::frag(A, i0 + lr, kb), GStage<MODE>::frag(B, j0 + lr, kb));
  }
}

// sums over the 16 lanes of a lane group (the columns of a result tile), and
// over the four lane groups.  Within a group by DPP lane permutations (pairs,
// quads, then the mirrors of half-rows and rows; every lane ends with the
// same sum): as shuffles they went through LDS, a dependent chain of
// permutes per row of every tile.
template <int CTRL>
__device__ __forceinline__ float dpp_from(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum_cols(float x) {
  x += dpp_from<0xB1>(x);    // quad_perm [1, 0, 3, 2]
  x += dpp_from<0x4E>(x);    // quad_perm [2, 3, 0, 1]
  x += dpp_from<0x141>(x);   // row_half_mirror
  x += dpp_from<0x140>(x);   // row_mirror
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
  using GS = GStage<MODE>;
  constexpr int CD = C * D, CC = C * C, DD = D * D, TC = C / 16, TD = D / 16;
  constexpr int NW = 8;                                     // waves
  constexpr int NCD = TC * TD / NW, NCC = TC * TC / NW;     // result tiles per wave: C x D, C x C
  static_assert(NCD * NW == TC * TD && NCC * NW == TC * TC, "whole tiles per wave");
  __shared__ __align__(16) char sA[GS::BYTES];
  __shared__ __align__(16) char sB[GS::BYTES];
  __shared__ float sG[C], sE[C], sS[C], sBt[C], sdG[C], sdB[C];
  const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  float *slot = a.scratch + (size_t)blockIdx.x * grad_slot_floats<C>();
  float *Vp = slot, *dV = Vp + CD, *dW = dV + CD, *dQp = dW + CD, *dKp = dQp + CD;
  float *R = dKp + CD, *Pm = R + CC, *dR = Pm + CC, *dT = dR + CC, *X = dT + CC, *dKk = X + CC, *Kk = dKk + CC;
  const int grp = a.Hv / a.Hqk;
  const int oheads = a.per_value_head ? a.Hv : a.Hqk;
  // each wave's result tiles of a C x D or C x C product: f(row i0, column j0)
  auto for_cd = [&](auto f) {
#pragma unroll 1
    for (int u = 0; u < NCD; ++u) {
      const int t = wv + NW * u;
      f(16 * (t / TD), 16 * (t % TD));
    }
  };
  auto for_cc = [&](auto f) {
#pragma unroll 1
    for (int u = 0; u < NCC; ++u) {
      const int t = wv + NW * u;
      f(16 * (t / TC), 16 * (t % TC));
    }
  };
  // the same, with the memory reads a tile's epilogue needs issued one tile
  // ahead: ld(i0, j0) returns them (registers), f(i0, j0, x) forms the tile.
  // (Read after the tile's products, each read had cost a whole memory
  // latency per tile.)  Past the last tile, ld reads that tile again, unused.
  auto for_tiles_ld = [&](auto n_per_wave, auto tiles_per_row, auto ld, auto f) {
    constexpr int NT = decltype(n_per_wave)::value, TR = decltype(tiles_per_row)::value;
    auto x = ld(16 * (wv / TR), 16 * (wv % TR));
#pragma unroll 1
    for (int u = 0; u < NT; ++u) {
      const int t = wv + NW * u, tn = wv + NW * (u + 1 < NT ? u + 1 : u);
      const auto xn = ld(16 * (tn / TR), 16 * (tn % TR));
      f(16 * (t / TR), 16 * (t % TR), x);
      x = xn;
    }
  };
  auto for_cd_ld = [&](auto ld, auto f) {
    for_tiles_ld(std::integral_constant<int, NCD>{}, std::integral_constant<int, TD>{}, ld, f);
  };
  auto for_cc_ld = [&](auto ld, auto f) {
    for_tiles_ld(std::integral_constant<int, NCC>{}, std::integral_constant<int, TC>{}, ld, f);
  };
  struct E4 {
    float v[4];
  };
  struct E8 {
    float v[4], w[4];
  };

  for (int unit = blockIdx.x; unit < a.units; unit += gridDim.x) {
    // (the thread index made opaque per unit: the per-thread offsets of the
    // staging copies and tile reads are then formed inside the loop, not
    // hoisted out of it into more registers than there are)
    // (from the lane id, counted again each unit, and the wave index: the
    // hardware's thread index would stay live across the whole loop)
    int lid;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lid));
    int tid = 64 * wv + lid;
    int lane = tid & 63, lr = lane & 15, g = lane >> 4;
    // the lane indices made opaque again after each barrier: offsets derived
    // from them are then formed in the phase that uses them, not carried
    // (in registers there are not) from one phase to a later one
    auto lane_fence = [&]() { asm volatile("" : "+v"(tid), "+v"(lane), "+v"(lr), "+v"(g)); };
    // (the divisors too, and in 32 bits: their reciprocals, hoisted out of
    // the loop, had outgrown the registers)
    int Nn = a.N, Hvn = a.Hv, grpn = grp;
    asm volatile("" : "+s"(Nn), "+s"(Hvn), "+s"(grpn));
    const int bhi = unit / Nn, n = unit % Nn, b = bhi / Hvn, hv = bhi % Hvn, hq = hv / grpn;
    const size_t cb = unit, bh = bhi;
    const int oh = a.per_value_head ? hv : hq;
    const size_t t0 = (size_t)b * a.T + (size_t)n * C;
    const int rows = !RAG ? C : (a.T - n * C < C ? a.T - n * C : C);
    const float *Tm = a.Tm + cb * CC, *Wm = a.W + cb * CD, *Um = a.U + cb * CD, *h = a.hs + cb * DD;
    const float *dhn = n + 1 < a.N ? a.dh + (cb + 1) * DD : a.dhT ? a.dhT + bh * DD : g_zero_state;
    const TI *qin = reinterpret_cast<const TI *>(a.q) + (t0 * a.Hqk + hq) * D;
    const TI *kin = reinterpret_cast<const TI *>(a.k) + (t0 * a.Hqk + hq) * D;
    const TI *vin = reinterpret_cast<const TI *>(a.v) + (t0 * a.Hv + hv) * D;
    const float *doin = a.dO + (t0 * a.Hv + hv) * D;
    const size_t ldq = (size_t)a.Hqk * D, ldv = (size_t)a.Hv * D;
    // one input element as fp32 (zero past the sequence's end)
    // (read branch-free from the row clamped into the chunk, then selected:
    // behind a branch, each read was waited for where the branches joined)
    auto in_at = [&](const TI *p, size_t ld, int r, int c) {
      const float x = to_f32(p[(size_t)(r < rows ? r : rows - 1) * ld + c]);
      return r < rows ? x : 0.f;
    };
    auto gam = [&](int r, int c) { return exp2_fast(sG[r] - sG[c]); };   // Gam_rc, c <= r
    // result element (row 4g + i of the tile) helpers
    auto row = [&](int i0, int i) { return i0 + 4 * g + i; };

    __syncthreads();   // the previous unit is done with the LDS
    if (tid < C) {
      const float Gr = a.G[cb * C + tid], Gl = a.G[cb * C + C - 1];
      sG[tid] = Gr * LOG2E;
      sE[tid] = exp2_fast(Gr * LOG2E);
      sS[tid] = exp2_fast((Gl - Gr) * LOG2E);
      const float bt = a.beta[(t0 + (tid < rows ? tid : rows - 1)) * a.Hv + hv];
      sBt[tid] = tid < rows ? bt : 0.f;
      sdG[tid] = 0.f;
      sdB[tid] = 0.f;
    }
    stage_in<MODE, C, false>(sA, qin, ldq, rows, tid);
    stage_in<MODE, C, false>(sB, kin, ldq, rows, tid);
    __syncthreads();
    lane_fence();
    // (1) R = Q K^T, P = R o Gam o [i <= r]; K K^T
    for_cc([&](int i0, int j0) {
      f32x4 acc = zero4();
      tile_st<MODE, D>(acc, sA, i0, sB, j0, lane);
      const int c = j0 + lr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = row(i0, i);
        R[r * C + c] = acc[i];
        Pm[r * C + c] = c <= r ? acc[i] * gam(r, c) : 0.f;
      }
    });
    for_cc([&](int i0, int j0) {
      f32x4 acc = zero4();
      tile_st<MODE, D>(acc, sB, i0, sB, j0, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) Kk[row(i0, i) * C + j0 + lr] = acc[i];
    });
    __syncthreads();
    lane_fence();
    stage<MODE, C, D, false>(sA, Wm, D, tid);
    stage<MODE, D, D, true>(sB, h, D, tid);
    __syncthreads();
    lane_fence();
    // (2) V' = U - W h
    for_cd_ld([&](int i0, int j0) {
      E4 e;
#pragma unroll
      for (int i = 0; i < 4; ++i) e.v[i] = Um[row(i0, i) * D + j0 + lr];
      return e;
    }, [&](int i0, int j0, const E4 &e) {
      f32x4 acc = zero4();
      tile_st<MODE, D>(acc, sA, i0, sB, j0, lane);
      const int c = j0 + lr;
#pragma unroll
      for (int i = 0; i < 4; ++i) Vp[row(i0, i) * D + c] = e.v[i] - acc[i];
    });
    __syncthreads();
    lane_fence();
    stage_in<MODE, C, false>(sA, doin, ldv, rows, tid);
    stage<MODE, D, D, false>(sB, h, D, tid);
    __syncthreads();
    lane_fence();
    // (3) dO h^T: dq's first term E o (dO h^T); dG_r += E_r <q_r, (dO h^T)_r>
    for_cd_ld([&](int i0, int j0) {
      E4 e;
#pragma unroll
      for (int i = 0; i < 4; ++i) e.v[i] = in_at(qin, ldq, row(i0, i), j0 + lr);
      return e;
    }, [&](int i0, int j0, const E4 &e) {
      f32x4 acc = zero4();
      tile_st<MODE, D>(acc, sA, i0, sB, j0, lane);
      const int c = j0 + lr;
      float rs[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = row(i0, i);
        dQp[r * D + c] = sE[r] * acc[i];
        rs[i] = sE[r] * e.v[i] * acc[i];
      }
      add_row_sums(sdG, i0, rs, 1.f, lane);
    });
    __syncthreads();
    lane_fence();
    stage<MODE, C, D, false>(sB, Vp, D, tid);
    __syncthreads();
    lane_fence();
    // (4) dP = (dO V'^T) o [i <= r]: dR = dP o Gam; dG terms of dP o R o Gam
    for_cc_ld([&](int i0, int j0) {
      E4 e;
#pragma unroll
      for (int i = 0; i < 4; ++i) e.v[i] = R[row(i0, i) * C + j0 + lr];
      return e;
    }, [&](int i0, int j0, const E4 &e) {
      f32x4 acc = zero4();
      tile_st<MODE, D>(acc, sA, i0, sB, j0, lane);
      const int c = j0 + lr;
      float tv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = row(i0, i);
        const float gm = c <= r ? gam(r, c) : 0.f;
        dR[r * C + c] = acc[i] * gm;
        tv[i] = acc[i] * e.v[i] * gm;
      }
      add_row_sums(sdG, i0, tv, 1.f, lane);
      add_col_sums(sdG, j0, tv, -1.f, lane);
    });
    __syncthreads();
    lane_fence();
    stage<MODE, C, C, true>(sA, Pm, C, tid);
    stage_in<MODE, C, true>(sB, doin, ldv, rows, tid);
    __syncthreads();
    lane_fence();
    // (5) P^T dO (into dV; (6) adds the second term)
    for_cd([&](int i0, int j0) {
      f32x4 acc = zero4();
      tile_st<MODE, C>(acc, sA, i0, sB, j0, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) dV[row(i0, i) * D + j0 + lr] = acc[i];
    });
    __syncthreads();
    lane_fence();
    stage_in<MODE, C, false>(sA, kin, ldq, rows, tid);
    stage<MODE, D, D, true>(sB, dhn, D, tid);
    __syncthreads();
    lane_fence();
    // (6) dV = P^T dO + diag(s) K dh'
    for_cd_ld([&](int i0, int j0) {
      E4 e;
#pragma unroll
      for (int i = 0; i < 4; ++i) e.v[i] = dV[row(i0, i) * D + j0 + lr];
      return e;
    }, [&](int i0, int j0, const E4 &e) {
      f32x4 acc = zero4();
      tile_st<MODE, D>(acc, sA, i0, sB, j0, lane);
      const int c = j0 + lr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = row(i0, i);
        dV[r * D + c] = e.v[i] + sS[r] * acc[i];
      }
    });
    __syncthreads();
    lane_fence();
    stage<MODE, C, D, false>(sA, Vp, D, tid);
    stage<MODE, D, D, false>(sB, dhn, D, tid);
    __syncthreads();
    lane_fence();
    // (7) V' dh'^T: dk's first term diag(s) V' dh'^T and its dG terms; <h, dh'>
    for_cd_ld([&](int i0, int j0) {
      E4 e;
#pragma unroll
      for (int i = 0; i < 4; ++i) e.v[i] = in_at(kin, ldq, row(i0, i), j0 + lr);
      return e;
    }, [&](int i0, int j0, const E4 &e) {
      f32x4 acc = zero4();
      tile_st<MODE, D>(acc, sA, i0, sB, j0, lane);
      const int c = j0 + lr;
      float dd[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = row(i0, i);
        const float x = sS[r] * acc[i];
        dKp[r * D + c] = x;
        dd[i] = x * e.v[i];
      }
      // dG_r -= dd_r, dG_last += sum_r dd_r
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = sum_cols(dd[i]);
        if (lr == 0) {
          atomicAdd(sdG + row(i0, i), -x);
          atomicAdd(sdG + C - 1, x);
        }
      }
    });
    {
      float hsum = 0.f;
      static_assert((DD / 4) % (64 * NW) == 0, "whole vectors per thread");
#pragma unroll
      for (int u = 0; u < DD / 4 / (64 * NW); ++u) {
        const int e = tid + 64 * NW * u;
        const float4 x = reinterpret_cast<const float4 *>(h)[e], y = reinterpret_cast<const float4 *>(dhn)[e];
        hsum += x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
      }
      hsum = sum_groups(sum_cols(hsum));
      if (lane == 0) atomicAdd(sdG + C - 1, exp2_fast(sG[C - 1]) * hsum);
    }
    __syncthreads();
    lane_fence();
    stage<MODE, C, D, false>(sA, dV, D, tid);
    stage<MODE, D, D, false>(sB, h, D, tid);
    __syncthreads();
    lane_fence();
    // (8) dW = -dV h^T
    for_cd([&](int i0, int j0) {
      f32x4 acc = zero4();
      tile_st<MODE, D>(acc, sA, i0, sB, j0, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) dW[row(i0, i) * D + j0 + lr] = -acc[i];
    });
    __syncthreads();
    lane_fence();
    stage<MODE, C, C, false>(sA, dR, C, tid);
    stage_in<MODE, C, true>(sB, kin, ldq, rows, tid);
    __syncthreads();
    lane_fence();
    // (9) dq = E o (dO h^T) + dR K
    for_cd_ld([&](int i0, int j0) {
      E4 e;
#pragma unroll
      for (int i = 0; i < 4; ++i) e.v[i] = dQp[row(i0, i) * D + j0 + lr];
      return e;
    }, [&](int i0, int j0, const E4 &e) {
      f32x4 acc = zero4();
      tile_st<MODE, C>(acc, sA, i0, sB, j0, lane);
      const int c = j0 + lr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = row(i0, i);
        if (r < rows) a.dq[((t0 + r) * oheads + oh) * D + c] = e.v[i] + acc[i];
      }
    });
    __syncthreads();
    lane_fence();
    stage<MODE, C, C, true>(sA, Tm, C, tid);
    stage<MODE, C, D, true>(sB, dV, D, tid);
    __syncthreads();
    lane_fence();
    // (10) dU~ = T^T dV: dv = diag(beta) dU~, dbeta_r += <dU~_r, v_r>
    for_cd_ld([&](int i0, int j0) {
      E4 e;
#pragma unroll
      for (int i = 0; i < 4; ++i) e.v[i] = in_at(vin, ldv, row(i0, i), j0 + lr);
      return e;
    }, [&](int i0, int j0, const E4 &e) {
      f32x4 acc = zero4();
      tile_st<MODE, C>(acc, sA, i0, sB, j0, lane);
      const int c = j0 + lr;
      float bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = row(i0, i);
        if (r < rows) a.dv[((t0 + r) * a.Hv + hv) * D + c] = sBt[r] * acc[i];
        bv[i] = acc[i] * e.v[i];
      }
      add_row_sums(sdB, i0, bv, 1.f, lane);
    });
    __syncthreads();
    lane_fence();
    stage<MODE, C, D, true>(sB, dW, D, tid);
    __syncthreads();
    lane_fence();
    // (11) dW~ = T^T dW: dk += diag(beta E) dW~; rw_r = <dW~_r, k_r>:
    //      dbeta_r += E_r rw_r, dG_r += beta_r E_r rw_r
    for_cd_ld([&](int i0, int j0) {
      E8 e;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        e.v[i] = dKp[row(i0, i) * D + j0 + lr];
        e.w[i] = in_at(kin, ldq, row(i0, i), j0 + lr);
      }
      return e;
    }, [&](int i0, int j0, const E8 &e) {
      f32x4 acc = zero4();
      tile_st<MODE, C>(acc, sA, i0, sB, j0, lane);
      const int c = j0 + lr;
      float rw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = row(i0, i);
        dKp[r * D + c] = e.v[i] + sBt[r] * sE[r] * acc[i];
        rw[i] = acc[i] * e.w[i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = sum_cols(rw[i]);
        const int r = row(i0, i);
        if (lr == 0) {
          atomicAdd(sdB + r, sE[r] * x);
          atomicAdd(sdG + r, sBt[r] * sE[r] * x);
        }
      }
    });
    __syncthreads();
    lane_fence();
    stage<MODE, C, D, false>(sA, dW, D, tid);
    stage_in<MODE, C, false>(sB, kin, ldq, rows, tid);
    __syncthreads();
    lane_fence();
    // (12) (dW K^T) diag(beta E) (into dT; (13) adds the second term)
    for_cc([&](int i0, int j0) {
      f32x4 acc = zero4();
      tile_st<MODE, D>(acc, sA, i0, sB, j0, lane);
      const int c = j0 + lr;
#pragma unroll
      for (int i = 0; i < 4; ++i) dT[row(i0, i) * C + c] = acc[i] * sE[c] * sBt[c];
    });
    __syncthreads();
    lane_fence();
    stage<MODE, C, D, false>(sA, dV, D, tid);
    stage_in<MODE, C, false>(sB, vin, ldv, rows, tid);
    __syncthreads();
    lane_fence();
    // (13) dT += (dV V^T) diag(beta)
    for_cc_ld([&](int i0, int j0) {
      E4 e;
#pragma unroll
      for (int i = 0; i < 4; ++i) e.v[i] = dT[row(i0, i) * C + j0 + lr];
      return e;
    }, [&](int i0, int j0, const E4 &e) {
      f32x4 acc = zero4();
      tile_st<MODE, D>(acc, sA, i0, sB, j0, lane);
      const int c = j0 + lr;
#pragma unroll
      for (int i = 0; i < 4; ++i) dT[row(i0, i) * C + c] = e.v[i] + acc[i] * sBt[c];
    });
    __syncthreads();
    lane_fence();
    stage<MODE, C, C, false>(sA, dT, C, tid);
    stage<MODE, C, C, false>(sB, Tm, C, tid);
    __syncthreads();
    lane_fence();
    // (14) X = dT T^T
    for_cc([&](int i0, int j0) {
      f32x4 acc = zero4();
      tile_st<MODE, C>(acc, sA, i0, sB, j0, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) X[row(i0, i) * C + j0 + lr] = acc[i];
    });
    __syncthreads();
    lane_fence();
    stage<MODE, C, C, true>(sA, Tm, C, tid);
    stage<MODE, C, C, true>(sB, X, C, tid);
    __syncthreads();
    lane_fence();
    // (15) dS = -strict-lower(T^T X): dbeta, dG terms of diag(beta) dS o K K^T
    //      o Gam, dKk = diag(beta) dS o Gam
    for_cc_ld([&](int i0, int j0) {
      E4 e;
#pragma unroll
      for (int i = 0; i < 4; ++i) e.v[i] = Kk[row(i0, i) * C + j0 + lr];
      return e;
    }, [&](int i0, int j0, const E4 &e) {
      f32x4 acc = zero4();
      tile_st<MODE, C>(acc, sA, i0, sB, j0, lane);
      const int c = j0 + lr;
      float bs[4], tv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = row(i0, i);
        const float ds = c < r ? -acc[i] : 0.f;
        const float gm = c < r ? gam(r, c) : 0.f;
        bs[i] = ds * gm * e.v[i];
        tv[i] = sBt[r] * bs[i];
        dKk[r * C + c] = sBt[r] * ds * gm;
      }
      add_row_sums(sdB, i0, bs, 1.f, lane);
      add_row_sums(sdG, i0, tv, 1.f, lane);
      add_col_sums(sdG, j0, tv, -1.f, lane);
    });
    __syncthreads();
    lane_fence();
    stage<MODE, C, C, true>(sA, dR, C, tid);
    stage_in<MODE, C, true>(sB, qin, ldq, rows, tid);
    __syncthreads();
    lane_fence();
    // (16) dk += dR^T Q
    for_cd_ld([&](int i0, int j0) {
      E4 e;
#pragma unroll
      for (int i = 0; i < 4; ++i) e.v[i] = dKp[row(i0, i) * D + j0 + lr];
      return e;
    }, [&](int i0, int j0, const E4 &e) {
      f32x4 acc = zero4();
      tile_st<MODE, C>(acc, sA, i0, sB, j0, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) dKp[row(i0, i) * D + j0 + lr] = e.v[i] + acc[i];
    });
    __syncthreads();
    lane_fence();
    stage<MODE, C, C, false>(sA, dKk, C, tid);
    stage_in<MODE, C, true>(sB, kin, ldq, rows, tid);
    __syncthreads();
    lane_fence();
    // (17) dk += dKk K
    for_cd_ld([&](int i0, int j0) {
      E4 e;
#pragma unroll
      for (int i = 0; i < 4; ++i) e.v[i] = dKp[row(i0, i) * D + j0 + lr];
      return e;
    }, [&](int i0, int j0, const E4 &e) {
      f32x4 acc = zero4();
      tile_st<MODE, C>(acc, sA, i0, sB, j0, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) dKp[row(i0, i) * D + j0 + lr] = e.v[i] + acc[i];
    });
    __syncthreads();
    lane_fence();
    stage<MODE, C, C, true>(sA, dKk, C, tid);
    __syncthreads();
    lane_fence();
    // (18) dk = diag(s) V' dh'^T + diag(beta E) dW~ + dR^T Q + dKk K + dKk^T K;
    //      dg = reverse cumulative sum of dG; dbeta
    for_cd_ld([&](int i0, int j0) {
      E4 e;
#pragma unroll
      for (int i = 0; i < 4; ++i) e.v[i] = dKp[row(i0, i) * D + j0 + lr];
      return e;
    }, [&](int i0, int j0, const E4 &e) {
      f32x4 acc = zero4();
      tile_st<MODE, C>(acc, sA, i0, sB, j0, lane);
      const int c = j0 + lr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = row(i0, i);
        if (r < rows) a.dk[((t0 + r) * oheads + oh) * D + c] = e.v[i] + acc[i];
      }
    });
    // dg = the reverse cumulative sum of dG: a suffix scan over each wave's
    // 64 entries, the first wave adding the second's total (C = 128)
    if (tid < C) {
      const int ln = tid & 63;
      float x = sdG[tid];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_down(x, off, 64);
        x += ln + off < 64 ? y : 0.f;
      }
      if (C > 64 && tid < 64) {
        float t = sdG[64 + ln];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) t += __shfl_xor(t, off, 64);
        x += t;
      }
      if (tid < rows) {
        a.dg[(t0 + tid) * a.Hv + hv] = x;
        a.dbeta[(t0 + tid) * a.Hv + hv] = sdB[tid];
      }
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
