// Layer-ahead query prediction Q_pred^{i+1} = W_Q^{i+1} X^i [ScoutAttention,
// arXiv:2603.27138, HTML Sec. 3.3; Algorithm 1], and the true query Q^i = W_Q^i X^i, as a
// skinny GEMM q[m][n] = x[m][k] . w[n][k]^T with bf16 operands and float32 accumulation.
//
// m is the batch (8..40 rows), so the product is bound by streaming W from HBM, not by
// the matrix cores: each workgroup owns a 64-column tile of n (16 columns per wave) and a
// slice of k, and computes every row of x against it with v_mfma_f32_16x16x32_bf16.  W is
// read once, 16 contiguous bytes per lane per k-step, eight k-steps in flight per wave.
// Several k-slices per tile give enough workgroups to cover the chip; their float32
// partials are summed in a fixed order by a second kernel, so results are deterministic.
// Two weight matrices that share x (Q^i and Q_pred^{i+1}) run as one launch.
#include "common.hpp"
#include "kernels.hpp"

namespace sa {
namespace {

constexpr int kTileN = 64;  // columns per workgroup (4 waves x 16)
constexpr int kUnroll = 8;  // k-steps of 32 loaded ahead

template <int MT>
__global__ __launch_bounds__(256) void gemm_kernel(const uint16_t* __restrict__ x,
                                                   const uint16_t* __restrict__ w0,
                                                   const uint16_t* __restrict__ w1, int m,
                                                   int n, int k, int kslice, int n_total,
                                                   float* __restrict__ out0,
                                                   float* __restrict__ out1, int ksplit,
                                                   float* __restrict__ partials) {
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int col_g = blockIdx.x * kTileN + wave * 16 + (lane % 16);  // in [0, n_total)
  const int prob = col_g >= n ? 1 : 0;
  const int col = col_g - prob * n;
  const uint16_t* w = prob ? w1 : w0;
  const int ks = blockIdx.y;
  const int k0 = ks * kslice;
  const int k1 = min(k, k0 + kslice);
  const int row0 = blockIdx.z * 16 * MT;
  const int kq = 8 * (lane / 16);  // this lane's 8 k-values within a 32-wide step

  const uint16_t* wrow = w + (size_t)col * k + kq;
  const uint16_t* xrow[MT];
  bool xvalid[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int r = row0 + 16 * t + (lane % 16);
    xvalid[t] = r < m;
    xrow[t] = x + (size_t)(xvalid[t] ? r : 0) * k + kq;
  }

  floatx4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};

  int kk = k0;
  for (; kk + 32 * kUnroll <= k1; kk += 32 * kUnroll) {
    uint4 bw[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      bw[u] = *reinterpret_cast<const uint4*>(wrow + kk + 32 * u);
    uint4 ax[kUnroll][MT];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int t = 0; t < MT; ++t)
        ax[u][t] = xvalid[t] ? *reinterpret_cast<const uint4*>(xrow[t] + kk + 32 * u)
                             : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const bf16x8 b = __builtin_bit_cast(bf16x8, bw[u]);
#pragma unroll
      for (int t = 0; t < MT; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ax[u][t]),
                                                         b, acc[t], 0, 0, 0);
    }
  }
  for (; kk < k1; kk += 32) {
    const bf16x8 b = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(wrow + kk));
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const uint4 a = xvalid[t] ? *reinterpret_cast<const uint4*>(xrow[t] + kk)
                                : make_uint4(0, 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), b,
                                                       acc[t], 0, 0, 0);
    }
  }

  // acc[t][r] holds row row0 + 16t + 4*(lane/16) + r, column col_g
#pragma unroll
  for (int t = 0; t < MT; ++t) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row0 + 16 * t + 4 * (lane / 16) + r;
      if (row < m) {
        if (ksplit == 1) {
          float* out = prob ? out1 : out0;
          out[(size_t)row * n + col] = acc[t][r];
        } else {
          partials[((size_t)ks * m + row) * n_total + col_g] = acc[t][r];
        }
      }
    }
  }
}

// Sum of the k-slice partials in slice order; four consecutive columns per thread.
__global__ __launch_bounds__(256) void gemm_reduce_kernel(const float* __restrict__ partials,
                                                          int m, int n, int n_total, int ksplit,
                                                          float* __restrict__ out0,
                                                          float* __restrict__ out1) {
  const long i4 = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long total4 = (long)m * n_total / 4;
  if (i4 >= total4) return;
  const long e = i4 * 4;
  const int row = (int)(e / n_total);
  const int col_g = (int)(e % n_total);
  float4 s = *reinterpret_cast<const float4*>(partials + e);
  for (int ks = 1; ks < ksplit; ++ks) {
    const float4 v =
        *reinterpret_cast<const float4*>(partials + (size_t)ks * m * n_total + e);
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  const int prob = col_g >= n ? 1 : 0;
  float* out = prob ? out1 : out0;
  *reinterpret_cast<float4*>(out + (size_t)row * n + (col_g - prob * n)) = s;
}

}  // namespace

GemmPlan gemm_plan(int m, int n_total, int k) {
  const int tiles = n_total / kTileN;
  const int row_groups = (m + 63) / 64;
  const int ksteps64 = k / 64;
  int ksplit = (768 + tiles * row_groups - 1) / (tiles * row_groups);
  ksplit = ksplit < 1 ? 1 : ksplit;
  const int max_split = ksteps64 / 4 > 0 ? ksteps64 / 4 : 1;  // slices of >= 256 columns
  ksplit = ksplit > max_split ? max_split : ksplit;
  const int kslice = 64 * ((ksteps64 + ksplit - 1) / ksplit);
  ksplit = (k + kslice - 1) / kslice;
  GemmPlan p;
  p.ksplit = ksplit;
  p.kslice = kslice;
  p.ws_bytes = ksplit > 1 ? (size_t)ksplit * m * n_total * sizeof(float) : 0;
  return p;
}

hipError_t launch_gemm(int m, int n, int k, const void* x, int nprob, const void* w0,
                       float* q0, const void* w1, float* q1, float* ws, const GemmPlan& plan,
                       hipStream_t stream) {
  const int n_total = n * nprob;
  const int mt = m >= 64 ? 4 : (m + 15) / 16;
  const dim3 grid(n_total / kTileN, plan.ksplit, (m + 63) / 64);
  const dim3 block(256);
  const uint16_t* X = (const uint16_t*)x;
  const uint16_t* W0 = (const uint16_t*)w0;
  const uint16_t* W1 = (const uint16_t*)(nprob > 1 ? w1 : w0);
  float* Q1 = nprob > 1 ? q1 : q0;
  switch (mt) {
    case 1: hipLaunchKernelGGL(gemm_kernel<1>, grid, block, 0, stream, X, W0, W1, m, n, k,
                               plan.kslice, n_total, q0, Q1, plan.ksplit, ws); break;
    case 2: hipLaunchKernelGGL(gemm_kernel<2>, grid, block, 0, stream, X, W0, W1, m, n, k,
                               plan.kslice, n_total, q0, Q1, plan.ksplit, ws); break;
    case 3: hipLaunchKernelGGL(gemm_kernel<3>, grid, block, 0, stream, X, W0, W1, m, n, k,
                               plan.kslice, n_total, q0, Q1, plan.ksplit, ws); break;
    default: hipLaunchKernelGGL(gemm_kernel<4>, grid, block, 0, stream, X, W0, W1, m, n, k,
                                plan.kslice, n_total, q0, Q1, plan.ksplit, ws); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.ksplit == 1) return e;
  const long total4 = (long)m * n_total / 4;
  hipLaunchKernelGGL(gemm_reduce_kernel, dim3((unsigned)((total4 + 255) / 256)), dim3(256), 0,
                     stream, ws, m, n, n_total, plan.ksplit, q0, Q1);
  return hipGetLastError();
}

}  // namespace sa
