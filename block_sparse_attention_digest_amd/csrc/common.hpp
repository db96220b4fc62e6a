// Device helpers shared by the gfx950 kernels of libscoutattn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

constexpr int kWave = 64;  // CDNA wavefront width

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));  // four bf16 MFMA operand

// ---- bfloat16 <-> float ------------------------------------------------------------------
// A 32-bit word holds two bf16 values: element 0 in the low half, element 1 in the high half.
// Loads of data read once per pass (K/V pages, digests), marked non-temporal so that they
// are kept out of the caches' working set in favour of data that is read again.
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load_stream8(const void* p) {
  typedef unsigned int v2u __attribute__((ext_vector_type(2)));
  const v2u v = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(p));
  return make_uint2(v.x, v.y);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Eight bf16 values (one 16-byte vector) widened to float.
__device__ __forceinline__ void bf16x8_to_f32(const uint4& v, float* f) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// double -> bf16 bits with ONE rounding, to nearest even, directly from the 53-bit
// significand (going through float would round twice).  bf16 keeps 8 significant bits
// and float's exponent range; below 2^-126 the spacing stays 2^-133.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
  int exp = (int)((u >> 52) & 0x7ff);
  uint64_t frac = u & ((1ull << 52) - 1);
  if (exp == 0x7ff) return frac ? 0x7fc0u : (sign | 0x7f80u);   // NaN, +-inf
  if (exp == 0) return sign;                                     // +-0 and f64 subnormals
  int e = exp - 1023;                                           // unbiased exponent
  uint64_t mant = frac | (1ull << 52);                          // 53-bit significand
  if (e >= -126) {
    uint32_t keep = (uint32_t)(mant >> 45);                      // 8 significant bits
    uint64_t rem = mant & ((1ull << 45) - 1);
    const uint64_t half = 1ull << 44;
    if (rem > half || (rem == half && (keep & 1u))) keep += 1;
    if (keep == 256u) { keep = 128u; e += 1; }
    if (e > 127) return sign | 0x7f80u;                          // overflow to infinity
    return sign | ((uint32_t)(e + 127) << 7) | (keep & 127u);
  }
  // subnormal range: value = n * 2^-133 with n = mant * 2^(e + 81)
  int shift = -(e + 81);                                         // >= 46
  if (shift > 60) return sign;                                   // < half of 2^-133
  uint64_t n = mant >> shift;
  uint64_t rem = mant & ((1ull << shift) - 1);
  uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (n & 1ull))) n += 1;
  return sign | (uint32_t)n;                                     // n == 128 is 2^-126
}

// ---- order-preserving keys -------------------------------------------------------------
// Monotone map float -> uint32 (a < b  <=>  key(a) < key(b)); -0 and +0 map alike.
__device__ __forceinline__ uint32_t order_key(float f) {
  f = f + 0.0f;  // -0 + 0 = +0 under round-to-nearest
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---- cross-lane exchange without LDS ------------------------------------------------------
// DPP row permutations (within 16-lane rows) and the gfx950 permlane swaps (across rows).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within each 8
constexpr int kDppMirror = 0x140;     // lane i <- lane 15-i within each 16
constexpr int kDppRor8 = 0x128;       // lane i <- lane i^8 within each 16

__device__ __forceinline__ float xor8(float v) { return dpp<kDppRor8>(v); }

// {v of this lane, v of lane^16} summed / maxed, via v_permlane16_swap
__device__ __forceinline__ float sum_xor16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float max_xor16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
// {v of this lane, v of lane^32}, via v_permlane32_swap
__device__ __forceinline__ float sum_xor32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

// Sum within aligned groups of W lanes (W a power of two <= 64); every lane gets its
// group's sum.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  if (W >= 2) v += dpp<kDppXor1>(v);
  if (W >= 4) v += dpp<kDppXor2>(v);
  if (W >= 8) v += dpp<kDppHalfMirror>(v);
  if (W >= 16) v += dpp<kDppMirror>(v);
  if (W >= 32) v = sum_xor16(v);
  if (W >= 64) v = sum_xor32(v);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup barrier that orders LDS accesses only: a wave waits for its own LDS writes, not
// for its global loads in flight (which a __syncthreads would drain).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace sa
