// Block digests [ScoutAttention, arXiv:2603.27138, HTML Sec. 2.2]: the mean of K over a
// block (MoBA-style) or the channel-wise min and max of K over a block (Quest-style).
//
// One wavefront per (sequence, KV head, block).  The block's page [bs][d] is read with
// 16-byte loads: LPR lanes cover one token row and the wave covers TPI rows per load, so
// every load instruction reads TPI*d*elem contiguous bytes.  The mean accumulates in
// float64, where sums of bf16 keys are exact, and is rounded once to the stored dtype;
// min/max are exact in any precision.  HBM-bound: the page is read once and d (or 2d)
// values are written.
#include "common.hpp"
#include "kernels.hpp"

namespace sa {
namespace {

template <typename T>
struct Vec;
template <>
struct Vec<uint16_t> {  // eight bf16
  static constexpr int N = 8;
  __device__ static void load(const uint16_t* p, float* f) {
    bf16x8_to_f32(*reinterpret_cast<const uint4*>(p), f);
  }
};
template <>
struct Vec<float> {  // four float
  static constexpr int N = 4;
  __device__ static void load(const float* p, float* f) {
    float4 v = *reinterpret_cast<const float4*>(p);
    f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
  }
};

__device__ __forceinline__ void store_vals(uint16_t* dst, const float* f, int n) {
  // values are exact bf16 (min/max of bf16 keys): take the high half of the float
  uint32_t w[4];
  for (int i = 0; i < n / 2; ++i)
    w[i] = (__float_as_uint(f[2 * i]) >> 16) | (__float_as_uint(f[2 * i + 1]) & 0xffff0000u);
  *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ void store_vals(float* dst, const float* f, int) {
  *reinterpret_cast<float4*>(dst) = make_float4(f[0], f[1], f[2], f[3]);
}
__device__ __forceinline__ void store_mean(uint16_t* dst, const double* v, int n) {
  uint32_t w[4];
  for (int i = 0; i < n / 2; ++i)
    w[i] = f64_to_bf16_rne(v[2 * i]) | (f64_to_bf16_rne(v[2 * i + 1]) << 16);
  *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ void store_mean(float* dst, const double* v, int) {
  *reinterpret_cast<float4*>(dst) =
      make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
}

template <typename T, int D, int BS, bool MINMAX>
__global__ __launch_bounds__(256) void digest_kernel(const T* __restrict__ k_pool,
                                                     const int32_t* __restrict__ table,
                                                     const int32_t* __restrict__ seq_lens,
                                                     T* __restrict__ dig, int Hkv,
                                                     int max_blocks, long total) {
  constexpr int VEC = Vec<T>::N;
  constexpr int LPR = D / VEC;        // lanes per token row
  constexpr int TPI = kWave / LPR;    // token rows per load instruction
  constexpr int ITERS = BS / TPI;
  const int lane = threadIdx.x % kWave;
  const long gw = (long)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (gw >= total) return;
  const int pair = (int)(gw / max_blocks);
  const int b = (int)(gw % max_blocks);
  const int len = seq_lens[pair / Hkv];
  if (b * BS >= len) return;
  const int page = table[gw];
  if (page < 0) return;
  const int nvalid = min(BS, len - b * BS);
  const int cg = lane % LPR, ts = lane / LPR;
  const T* src = k_pool + (size_t)page * BS * D + cg * VEC;

  if constexpr (MINMAX) {
    float mn[VEC], mx[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) { mn[i] = INFINITY; mx[i] = -INFINITY; }
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int t = it * TPI + ts;
      if (t < nvalid) {
        float f[VEC];
        Vec<T>::load(src + (size_t)t * D, f);
#pragma unroll
        for (int i = 0; i < VEC; ++i) { mn[i] = fminf(mn[i], f[i]); mx[i] = fmaxf(mx[i], f[i]); }
      }
    }
#pragma unroll
    for (int o = LPR; o < kWave; o <<= 1) {
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        mn[i] = fminf(mn[i], __shfl_xor(mn[i], o, kWave));
        mx[i] = fmaxf(mx[i], __shfl_xor(mx[i], o, kWave));
      }
    }
    if (ts == 0) {
      T* dst = dig + (size_t)gw * 2 * D + cg * VEC;
      store_vals(dst, mn, VEC);
      store_vals(dst + D, mx, VEC);
    }
  } else {
    double acc[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] = 0.0;
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int t = it * TPI + ts;
      if (t < nvalid) {
        float f[VEC];
        Vec<T>::load(src + (size_t)t * D, f);
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc[i] += (double)f[i];
      }
    }
#pragma unroll
    for (int o = LPR; o < kWave; o <<= 1) {
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] += __shfl_xor(acc[i], o, kWave);
    }
    if (ts == 0) {
      double v[VEC];
#pragma unroll
      for (int i = 0; i < VEC; ++i) v[i] = acc[i] / (double)nvalid;
      store_mean(dig + (size_t)gw * D + cg * VEC, v, VEC);
    }
  }
}

template <typename T, int D, int BS>
hipError_t launch_typed(const Shape& s, bool minmax, const void* k_pool, const int32_t* table,
                        const int32_t* lens, void* dig, hipStream_t stream) {
  const long total = (long)s.B * s.Hkv * s.max_blocks;
  const int waves_per_wg = 4;
  const dim3 grid((unsigned)((total + waves_per_wg - 1) / waves_per_wg));
  const dim3 block(waves_per_wg * kWave);
  if (minmax)
    hipLaunchKernelGGL((digest_kernel<T, D, BS, true>), grid, block, 0, stream,
                       (const T*)k_pool, table, lens, (T*)dig, s.Hkv, s.max_blocks, total);
  else
    hipLaunchKernelGGL((digest_kernel<T, D, BS, false>), grid, block, 0, stream,
                       (const T*)k_pool, table, lens, (T*)dig, s.Hkv, s.max_blocks, total);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dtype(const Shape& s, bool minmax, const void* k, const int32_t* t,
                        const int32_t* l, void* dig, hipStream_t st) {
  if (s.d == 128)
    return s.bs == 32 ? launch_typed<T, 128, 32>(s, minmax, k, t, l, dig, st)
                      : launch_typed<T, 128, 16>(s, minmax, k, t, l, dig, st);
  return s.bs == 32 ? launch_typed<T, 64, 32>(s, minmax, k, t, l, dig, st)
                    : launch_typed<T, 64, 16>(s, minmax, k, t, l, dig, st);
}

}  // namespace

hipError_t launch_build_digests(const Shape& s, bool minmax, const void* k_pool,
                                const int32_t* block_table, const int32_t* seq_lens,
                                void* digests, hipStream_t stream) {
  if (s.bf16)
    return launch_dtype<uint16_t>(s, minmax, k_pool, block_table, seq_lens, digests, stream);
  return launch_dtype<float>(s, minmax, k_pool, block_table, seq_lens, digests, stream);
}

}  // namespace sa
