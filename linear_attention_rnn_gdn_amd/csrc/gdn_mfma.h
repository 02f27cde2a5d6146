// gdn_mfma.h -- gfx950 matrix-core building blocks for the GDN kernels.
//
// Every product in the kernels is built from one 16x16 output tile per wave
// and a contraction (k) loop in blocks of 32.  Operands are staged in LDS; for
// a k-block each lane fetches 8 consecutive k-values of one row of A and of
// one column of B:
//     lane l:  A row  = l % 16,  k = 8*(l/16) + j   (j = 0..7)
//              B col  = l % 16,  k = 8*(l/16) + j
//     result:  lane l holds D[4*(l/16) + i][l % 16], i = 0..3
// This is the operand layout of v_mfma_f32_16x16x32_bf16.  The fp32 matrix
// core instruction v_mfma_f32_16x16x4_f32 takes one k-value per lane group;
// feeding it j = 0..7 in turn covers the same 32 k-values (the k order of a
// sum is free as long as A and B agree), so both precisions share one
// fetch layout and one result layout.
//
// Precision policies for one product (chosen per product, see the kernels):
//   P_BF16      both operands rounded to bf16 (exact when they are bf16 data)
//   P_SPLIT_A   A = a_hi + a_lo (two bf16), B bf16: 2 bf16 MFMAs
//   P_SPLIT_B   A bf16, B split: 2 bf16 MFMAs
//   P_SPLIT_AB  both split, a_lo*b_lo dropped: 3 bf16 MFMAs (~fp32 accuracy)
//   P_F32       fp32 matrix-core products (exact fp32 multiply)
#pragma once
#include <hip/hip_runtime.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

enum : int { P_BF16 = 0, P_SPLIT_A = 1, P_SPLIT_B = 2, P_SPLIT_AB = 3, P_F32 = 4 };

// A zero the compiler cannot see through, held in a VGPR.  Added to the
// address of a wave-uniform load it keeps the load on the vector memory path:
// a scalar (SMEM) load shares the lgkm counter with LDS and can return out of
// order, so while one is in flight every LDS wait becomes lgkmcnt(0) and
// stalls for the full memory latency.
__device__ __forceinline__ int vgpr_zero() {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}

// Workgroup barrier for LDS traffic only.  __syncthreads() is a workgroup
// memory fence as well and drains every outstanding global load and store
// (s_waitcnt vmcnt(0)) at each barrier, which would serialise the prefetch of
// the next chunk with the compute of this one.  Here only the LDS counter is
// drained; global data never passes between waves of a workgroup.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Global stores with the nontemporal hint, for tensors that one launch writes
// once and a later launch reads: the walk's copies of h and V' for the output
// stage, and o.  With plain stores the walk's dirty lines sit in L2 next to
// the operands it keeps re-reading (and each store's completion, which every
// later wait on the memory counter includes, takes longer); streamed, the
// walk runs about a quarter faster.  Prep's outputs are the exception: the
// walk that follows reads them at once, and with plain stores they are still
// in the memory-side cache then (measured over whole steps: the walk runs in
// two thirds of the time).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
template <typename T>
__device__ __forceinline__ void st16(void *p, const T &v) {
  static_assert(sizeof(T) == 16, "16-byte store");
  *reinterpret_cast<u32x4 *>(p) = __builtin_bit_cast(u32x4, v);
}
template <typename T>
__device__ __forceinline__ void st16_stream(void *p, const T &v) {
  static_assert(sizeof(T) == 16, "16-byte store");
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4 *>(p));
}
template <typename T>
__device__ __forceinline__ void st8_stream(void *p, const T &v) {
  static_assert(sizeof(T) == 8, "8-byte store");
  __builtin_nontemporal_store(__builtin_bit_cast(u32x2, v), reinterpret_cast<u32x2 *>(p));
}

// Round 8 fp32 values to bf16 (round to nearest even), two per packed
// convert.  to_bf16x8_split also returns the rounding remainders x - hi,
// rounded the same way (exact differences in fp32); the widened high halves
// come from the packed words by a shift (element 2p) and a mask (element
// 2p + 1), so a value costs about two instructions less than converting it
// alone and widening it back.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ unsigned pk_bf16(float x0, float x1) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{x0, x1}, bf16x2));
}
__device__ __forceinline__ bf16x8 to_bf16x8(const float (&x)[8]) {
  const uint4 u{pk_bf16(x[0], x[1]), pk_bf16(x[2], x[3]), pk_bf16(x[4], x[5]), pk_bf16(x[6], x[7])};
  return __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ void to_bf16x8_split(const float (&x)[8], bf16x8 &hi, bf16x8 &lo) {
  unsigned h[4], l[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    h[p] = pk_bf16(x[2 * p], x[2 * p + 1]);
    const float h0 = __builtin_bit_cast(float, h[p] << 16);
    const float h1 = __builtin_bit_cast(float, h[p] & 0xffff0000u);
    l[p] = pk_bf16(x[2 * p] - h0, x[2 * p + 1] - h1);
  }
  hi = __builtin_bit_cast(bf16x8, uint4{h[0], h[1], h[2], h[3]});
  lo = __builtin_bit_cast(bf16x8, uint4{l[0], l[1], l[2], l[3]});
}

template <int P>
__device__ __forceinline__ void mma_k32(f32x4 &c, const float (&a)[8], const float (&b)[8]) {
  if constexpr (P == P_F32) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
  } else {
    bf16x8 ah, bh, al, bl;
    if constexpr (P == P_SPLIT_A || P == P_SPLIT_AB) to_bf16x8_split(a, ah, al);
    else ah = to_bf16x8(a);
    if constexpr (P == P_SPLIT_B || P == P_SPLIT_AB) to_bf16x8_split(b, bh, bl);
    else bh = to_bf16x8(b);
    // small terms first
    if constexpr (P == P_SPLIT_A || P == P_SPLIT_AB) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, c, 0, 0, 0);
    if constexpr (P == P_SPLIT_B || P == P_SPLIT_AB) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, c, 0, 0, 0);
  }
}

// Operand fragments: an operand is converted (or split) once and can then
// feed several MFMAs.  Kinds: F_BF16 (rounded to bf16), F_SPLIT (hi + lo
// bf16), F_F32 (kept fp32 for the fp32 matrix-core instruction).
enum : int { F_BF16 = 0, F_SPLIT = 1, F_F32 = 2 };
template <int K> struct Frag;
template <> struct Frag<F_BF16> { bf16x8 hi; };
template <> struct Frag<F_SPLIT> { bf16x8 hi, lo; };
template <> struct Frag<F_F32> { float v[8]; };

// operand kinds of each product policy: A side, B side
template <int P> struct PolicyKinds;
template <> struct PolicyKinds<P_BF16> { static constexpr int a = F_BF16, b = F_BF16; };
template <> struct PolicyKinds<P_SPLIT_A> { static constexpr int a = F_SPLIT, b = F_BF16; };
template <> struct PolicyKinds<P_SPLIT_B> { static constexpr int a = F_BF16, b = F_SPLIT; };
template <> struct PolicyKinds<P_SPLIT_AB> { static constexpr int a = F_SPLIT, b = F_SPLIT; };
template <> struct PolicyKinds<P_F32> { static constexpr int a = F_F32, b = F_F32; };

template <int K>
__device__ __forceinline__ Frag<K> make_frag(const float (&x)[8]) {
  Frag<K> f;
  if constexpr (K == F_F32) {
#pragma unroll
    for (int j = 0; j < 8; ++j) f.v[j] = x[j];
  } else if constexpr (K == F_SPLIT) {
    to_bf16x8_split(x, f.hi, f.lo);
  } else {
    f.hi = to_bf16x8(x);
  }
  return f;
}

// c += A B for one k-block, with the instruction count the operand kinds need
// (lo x lo products are dropped; small terms are accumulated first).
template <int KA, int KB>
__device__ __forceinline__ void mma(f32x4 &c, const Frag<KA> &a, const Frag<KB> &b) {
  if constexpr (KA == F_F32 || KB == F_F32) {
    static_assert(KA == F_F32 && KB == F_F32, "fp32 operands pair with fp32 operands");
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
  } else {
    if constexpr (KA == F_SPLIT) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, c, 0, 0, 0);
    if constexpr (KB == F_SPLIT) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, c, 0, 0, 0);
  }
}

// 8 consecutive LDS elements -> float[8]  (p 16-byte aligned)
__device__ __forceinline__ void ld8(const float *p, float (&x)[8]) {
  const float4 u = *reinterpret_cast<const float4 *>(p);
  const float4 w = *reinterpret_cast<const float4 *>(p + 4);
  x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
  x[4] = w.x; x[5] = w.y; x[6] = w.z; x[7] = w.w;
}
__device__ __forceinline__ void ld8(const __bf16 *p, float (&x)[8]) {
  const bf16x8 u = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = (float)u[j];
}
// 8 LDS elements with a stride
template <typename T>
__device__ __forceinline__ void ld8s(const T *p, int stride, float (&x)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = (float)p[j * stride];
}

// LDS -> operand fragment.  Exact bf16 data become a bf16 fragment with one
// 16-byte read and no conversion.
template <int K>
__device__ __forceinline__ Frag<K> lds_frag(const float *p) {
  float x[8];
  ld8(p, x);
  return make_frag<K>(x);
}
template <int K>
__device__ __forceinline__ Frag<K> lds_frag(const __bf16 *p) {
  if constexpr (K == F_BF16) {
    Frag<K> f;
    f.hi = *reinterpret_cast<const bf16x8 *>(p);
    return f;
  } else {
    float x[8];
    ld8(p, x);
    return make_frag<K>(x);
  }
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

}  // namespace gdn
