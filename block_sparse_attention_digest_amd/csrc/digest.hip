// Block digests [ScoutAttention, arXiv:2603.27138, HTML Sec. 2.2]: the mean of K over a
// block (MoBA-style) or the channel-wise min and max of K over a block (Quest-style).
//
// One wavefront per (sequence, KV head, block).  K pages are chunk-major ([d/x][bs][x], x
// elements per 16-byte chunk), so one page is d/x chunk rows of bs tokens each.  Each load
// instruction reads 8 chunks x 8 tokens: lane l takes chunk 8 cg + l / 8 and token
// 8 tg + l % 8, so every group of 8 lanes reads one whole 128-byte line.  A lane keeps its
// chunk's running sums (or min/max) over its tokens; the 8 lanes of a chunk then combine
// theirs with cross-lane exchanges.  The mean accumulates in float64, where sums of bf16
// keys are exact, and is rounded once to the stored dtype; min/max are exact in any
// precision.  HBM-bound: the page is read once and d (or 2d) values are written.
#include "common.hpp"
#include "kernels.hpp"

namespace sa {
namespace {

template <typename T>
struct Vec;
template <>
struct Vec<uint16_t> {  // eight bf16 per 16-byte chunk
  static constexpr int N = 8;
  __device__ static void widen(const uint4& v, float* f) { bf16x8_to_f32(v, f); }
};
template <>
struct Vec<float> {  // four float per 16-byte chunk
  static constexpr int N = 4;
  __device__ static void widen(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
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
  constexpr int VEC = Vec<T>::N;  // elements per 16-byte chunk
  constexpr int NC = D / VEC;     // chunks per token
  constexpr int CG = NC / 8;      // chunk groups: 8 chunks per load instruction
  constexpr int TG = BS / 8;      // token groups: 8 tokens (one 128-byte line) per chunk
  static_assert(NC % 8 == 0 && BS % 8 == 0, "page shape");
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
  const T* src = k_pool + (size_t)page * BS * D;
  const int cl = lane / 8, tl = lane % 8;  // chunk within the group, token within the group

  // the whole page in flight at once (CG * TG <= 16 loads of 16 bytes per lane)
  uint4 raw[CG][TG];
#pragma unroll
  for (int cg = 0; cg < CG; ++cg)
#pragma unroll
    for (int tg = 0; tg < TG; ++tg)
      raw[cg][tg] = *reinterpret_cast<const uint4*>(
          src + ((size_t)(8 * cg + cl) * BS + 8 * tg + tl) * VEC);

  if constexpr (MINMAX) {
    float mn[CG][VEC], mx[CG][VEC];
#pragma unroll
    for (int cg = 0; cg < CG; ++cg) {
#pragma unroll
      for (int i = 0; i < VEC; ++i) { mn[cg][i] = INFINITY; mx[cg][i] = -INFINITY; }
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) {
        if (8 * tg + tl < nvalid) {
          float f[VEC];
          Vec<T>::widen(raw[cg][tg], f);
#pragma unroll
          for (int i = 0; i < VEC; ++i) {
            mn[cg][i] = fminf(mn[cg][i], f[i]);
            mx[cg][i] = fmaxf(mx[cg][i], f[i]);
          }
        }
      }
#pragma unroll
      for (int o = 1; o < 8; o <<= 1)
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          mn[cg][i] = fminf(mn[cg][i], __shfl_xor(mn[cg][i], o, kWave));
          mx[cg][i] = fmaxf(mx[cg][i], __shfl_xor(mx[cg][i], o, kWave));
        }
      if (tl == 0) {
        T* dst = dig + (size_t)gw * 2 * D + (8 * cg + cl) * VEC;
        store_vals(dst, mn[cg], VEC);
        store_vals(dst + D, mx[cg], VEC);
      }
    }
  } else {
#pragma unroll
    for (int cg = 0; cg < CG; ++cg) {
      double acc[VEC];
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] = 0.0;
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) {
        if (8 * tg + tl < nvalid) {
          float f[VEC];
          Vec<T>::widen(raw[cg][tg], f);
#pragma unroll
          for (int i = 0; i < VEC; ++i) acc[i] += (double)f[i];
        }
      }
#pragma unroll
      for (int o = 1; o < 8; o <<= 1)
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc[i] += __shfl_xor(acc[i], o, kWave);
      if (tl == 0) {
        double v[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) v[i] = acc[i] / (double)nvalid;
        store_mean(dig + (size_t)gw * D + (8 * cg + cl) * VEC, v, VEC);
      }
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
