// Device-side building blocks of the gfx950 linear-attention kernels: bf16
// conversion, the 16x16x32 bf16 MFMA, XOR-swizzled LDS tile addressing and the
// RoPE rotation with a double-precision angle reduction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

constexpr int kD = 128;     // head dimension (D_k = D_v)
constexpr int kHalf = 64;   // RoPE frequencies per head (rotate-half pairs)

typedef short bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(uint32_t h16) { return __uint_as_float(h16 << 16); }
__device__ __forceinline__ float bf2f_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf2f_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even float -> bf16 (gfx950 converts in hardware).
__device__ __forceinline__ uint32_t f2bf(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}
// Two floats -> packed bf16 pair (one v_cvt_pk_bf16_f32).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// acc + a.lo * b.lo + a.hi * b.hi for packed bf16 pairs, fp32 accumulate.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc,
                                         false);
}

// D = A(16x32) * B(32x16) + C with bf16 inputs and fp32 accumulation.
// Lane l supplies A[l % 16][8 (l / 16) + e] and B[8 (l / 16) + e][l % 16] for
// e = 0..7, and receives D[4 (l / 16) + r][l % 16] for r = 0..3.
__device__ __forceinline__ f32x4 mma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ bf16x8 as_bf16x8(uint2 lo, uint2 hi) {
  return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Pack two accumulator tiles (4 rows each) into one 8-element bf16 operand.
__device__ __forceinline__ bf16x8 pack8(const f32x4& a, const f32x4& b) {
  return __builtin_bit_cast(bf16x8, make_uint4(pack2(a[0], a[1]), pack2(a[2], a[3]),
                                               pack2(b[0], b[1]), pack2(b[2], b[3])));
}

// ---------------------------------------------------------------------------
// Global load of 8 bytes that are read once (non-temporal hint).
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 ld_stream(const void* p) {
  const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(x.x, x.y);
}

template <typename T>
__device__ __forceinline__ T lds_ld(const uint8_t* base, int off) {
  return *reinterpret_cast<const T*>(base + off);
}
template <typename T>
__device__ __forceinline__ void lds_st(uint8_t* base, int off, T v) {
  *reinterpret_cast<T*>(base + off) = v;
}

// ---------------------------------------------------------------------------
// RoPE rotation e^{i p theta} for an integer position p.  The angle is carried in
// revolutions: rev = p * (theta / 2 pi) is formed in double precision and reduced
// to [-1/2, 1/2] (error ~1e-11 revolutions for p up to millions); the hardware
// sine/cosine (argument in revolutions) then act on the small reduced value.
__device__ __forceinline__ float2 rope_rotation(int64_t p, double rev_per_pos) {
  double rev = (double)p * rev_per_pos;
  rev -= rint(rev);
  const float r = (float)rev;
  return make_float2(__builtin_amdgcn_cosf(r), __builtin_amdgcn_sinf(r));
}

__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
  return make_float2(a.x * b.x - a.y * b.y, a.y * b.x + a.x * b.y);
}

// sigmoid(x) = 1 / (1 + e^{-x}) with the hardware exp and reciprocal (~1 ulp each).
__device__ __forceinline__ float sigmoidf_(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

// 1 / sqrt(x) (hardware reciprocal square root, ~1 ulp).
__device__ __forceinline__ float rsqrt_(float x) { return __builtin_amdgcn_rsqf(x); }

}  // namespace la
