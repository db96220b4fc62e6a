// Layout conversions into the orders the decode kernels stream (pure data movement, no
// arithmetic).  Both run once per buffer -- K when a page is written, W_Q when the weights
// are loaded -- and are not part of the per-token decode path.
//
//   K pages: token rows [P][bs][d] -> chunk-major [P][d/x][bs][x], x = 16 bytes of elements.
//     A 16-token slice of one chunk is 256 contiguous bytes, so the attention kernel's
//     matrix-core operand loads (16 tokens x 16 bytes per 16 lanes) read whole cache lines.
//   V pages: token rows [P][bs][d] -> [P][bs/16][d][16]: each 16-token half of a page is
//     channel-major with its 16 tokens contiguous, so a 16-channel x 16-token matrix-core
//     operand tile of V^T is 512 contiguous bytes.
//   W_Q: [n][k] -> [n/16][k/32][64][8], one v_mfma_f32_16x16x32_bf16 B operand (16 output
//     features x 32 inputs, lane l holding feature l % 16 and inputs 8 (l / 16) .. + 7) per
//     contiguous kilobyte, so one GEMM load instruction reads 1 KiB of consecutive bytes.
#include "common.hpp"
#include "kernels.hpp"

namespace sa {
namespace {

// One thread per 16-byte chunk of the destination (consecutive threads write consecutive
// chunks; their sources are one token row apart).
__global__ __launch_bounds__(256) void pack_k_kernel(const uint4* __restrict__ src,
                                                     uint4* __restrict__ dst, long total,
                                                     int bs, int nc) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const long per_page = (long)bs * nc;
  const long page = i / per_page;
  const int r = (int)(i % per_page);
  const int c = r / bs, t = r % bs;
  dst[i] = src[page * per_page + (long)t * nc + c];
}

// One thread per 16 bytes (8 bf16) of the packed weight.
__global__ __launch_bounds__(256) void pack_w_kernel(const uint4* __restrict__ src,
                                                     uint4* __restrict__ dst, long total,
                                                     int k) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int ksteps = k / 32;
  const int lane = (int)(i % 64);
  const long tile = i / 64;
  const long a = tile / ksteps;
  const int b = (int)(tile % ksteps);
  const long row = 16 * a + lane % 16;
  const long col = 32L * b + 8 * (lane / 16);
  dst[i] = src[(row * k + col) / 8];
}

// One workgroup per 16-token half-page (16 x d elements): 16-byte reads of the token rows
// into LDS, then 16-byte writes of the channel-major result, each gathering one channel's
// consecutive tokens from LDS.
template <typename T>
__global__ __launch_bounds__(256) void pack_v_kernel(const T* __restrict__ src,
                                                     T* __restrict__ dst, int d) {
  constexpr int E = 16 / sizeof(T);  // elements per 16-byte chunk
  extern __shared__ uint4 tile[];   // [16][d] elements
  const T* s = src + (size_t)blockIdx.x * 16 * d;
  T* o = dst + (size_t)blockIdx.x * 16 * d;
  const int chunks = 16 * d / E;
  for (int c = threadIdx.x; c < chunks; c += blockDim.x)
    tile[c] = *reinterpret_cast<const uint4*>(s + (size_t)c * E);
  __syncthreads();
  const T* t = reinterpret_cast<const T*>(tile);
  for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
    const int ch = c / (16 / E), t0 = (c % (16 / E)) * E;  // channel, first token
    T v[E];
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = t[(t0 + e) * d + ch];
    uint4 w;
    __builtin_memcpy(&w, v, sizeof(w));
    *reinterpret_cast<uint4*>(o + (size_t)c * E) = w;
  }
}

}  // namespace

hipError_t launch_pack_v(const Shape& s, const void* v_rows, void* v_pool, hipStream_t stream) {
  const dim3 grid((unsigned)((long)s.P * (s.bs / 16))), block(256);
  const size_t lds = (size_t)16 * s.d * (s.bf16 ? 2 : 4);
  if (s.bf16)
    hipLaunchKernelGGL(pack_v_kernel<uint16_t>, grid, block, lds, stream,
                       (const uint16_t*)v_rows, (uint16_t*)v_pool, s.d);
  else
    hipLaunchKernelGGL(pack_v_kernel<float>, grid, block, lds, stream, (const float*)v_rows,
                       (float*)v_pool, s.d);
  return hipGetLastError();
}

hipError_t launch_pack_k(const Shape& s, const void* k_rows, void* k_pool, hipStream_t stream) {
  const int nc = s.d * (s.bf16 ? 2 : 4) / 16;
  const long total = (long)s.P * s.bs * nc;
  hipLaunchKernelGGL(pack_k_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     stream, (const uint4*)k_rows, (uint4*)k_pool, total, s.bs, nc);
  return hipGetLastError();
}

hipError_t launch_pack_w(int n, int k, const void* w, void* w_packed, hipStream_t stream) {
  const long total = (long)n * k / 8;
  hipLaunchKernelGGL(pack_w_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     stream, (const uint4*)w, (uint4*)w_packed, total, k);
  return hipGetLastError();
}

}  // namespace sa
