// Layer-ahead query prediction Q_pred^{i+1} = W_Q^{i+1} X^i [ScoutAttention,
// arXiv:2603.27138, HTML Sec. 3.3; Algorithm 1], and the true query Q^i = W_Q^i X^i, as a
// skinny GEMM q[m][n] = x[m][k] . w[n][k]^T with bf16 operands and float32 accumulation.
//
// m is the batch (8..40 rows), so the product is bound by streaming W from HBM, not by the
// matrix cores.  A workgroup of 8 waves owns 128 columns of n (16 per wave) and one slice
// of k.  The slice of x it needs (at most 64 rows) is staged once in LDS and shared by the
// 8 waves, so HBM and L2 carry W once and x only once per workgroup.  W arrives packed
// (launch_pack_w): the v_mfma_f32_16x16x32_bf16 B operand of one 16-column tile and one
// 32-wide k-step is a contiguous kilobyte, so each wave streams its W with 16-byte loads
// that cover whole cache lines, straight into B operands, keeping the next 8 k-steps in
// flight (double-buffered registers) while the current 8 are multiplied.  Several k-slices per column tile give enough workgroups to cover the chip;
// their float32 partials are summed in slice order by a second kernel, so results are
// deterministic.  Two weight matrices that share x (Q^i and Q_pred^{i+1}) run as one launch.
#include "common.hpp"
#include "kernels.hpp"

namespace sa {
namespace {

constexpr int kWaves = 8;
constexpr int kTileN = 16 * kWaves;  // columns per workgroup
constexpr int kGroup = 8;            // k-steps (of 32) per register buffer
constexpr int kLdsBytes = 64 * 1024;
constexpr int kPad = 8;              // bf16 elements of padding per LDS row

template <int MT>
__global__ __launch_bounds__(512) void gemm_kernel(const uint16_t* __restrict__ x,
                                                   const uint16_t* __restrict__ w0,
                                                   const uint16_t* __restrict__ w1, int m,
                                                   int n, int k, int kslice, int n_total,
                                                   float* __restrict__ out0,
                                                   float* __restrict__ out1, int ksplit,
                                                   float* __restrict__ partials) {
  extern __shared__ uint16_t xs[];  // [16*MT][kslice + kPad]
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // scalar branches
  const int col_g = blockIdx.x * kTileN + wave * 16 + (lane % 16);  // in [0, n_total)
  const int prob = col_g >= n ? 1 : 0;  // the same for the 16 columns of a wave (16 | n)
  const int col = min(col_g - prob * n, n - 1);  // clamped for waves past n_total
  const uint16_t* w = prob ? w1 : w0;
  const int ks = blockIdx.y;
  const int k0 = ks * kslice;
  const int k1 = min(k, k0 + kslice);
  const int klen = k1 - k0;
  const int row0 = blockIdx.z * 16 * MT;
  const int ldx = kslice + kPad;

  // stage x[row0 .. row0+16MT)[k0 .. k1) in LDS (rows past m are zero)
  {
    const int chunks_per_row = klen / 8;
    const int total = 16 * MT * chunks_per_row;
    for (int c = threadIdx.x; c < total; c += blockDim.x) {
      const int r = c / chunks_per_row, q8 = c % chunks_per_row;
      const int gr = row0 + r;
      const uint4 v = gr < m ? *reinterpret_cast<const uint4*>(x + (size_t)gr * k + k0 + 8 * q8)
                             : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(xs + r * ldx + 8 * q8) = v;
    }
  }

  const int kq = 8 * (lane / 16);  // this lane's 8 k-values within a 32-wide step
  // packed tile (col / 16, k-step): 512 elements, this lane's 8 at lane * 8
  const uint16_t* wtile = w + ((size_t)(col / 16) * (k / 32) + k0 / 32) * 512 + lane * 8;
  const int nsteps = klen / 32;

  floatx4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Loads are issued unconditionally (k-steps past the slice are clamped to its last
  // step and their B operand zeroed), so every path has the same loads in flight and the
  // compiler waits only for the group being multiplied.
  uint4 wa[kGroup], wb[kGroup];
  auto load_group = [&](uint4* dst, int s0) {
#pragma unroll
    for (int u = 0; u < kGroup; ++u)
      dst[u] = *reinterpret_cast<const uint4*>(wtile + 512 * min(s0 + u, nsteps - 1));
  };
  auto mma_group = [&](const uint4* src, int s0) {
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      const int st = min(s0 + u, nsteps - 1);
      const uint4 bw = s0 + u < nsteps ? src[u] : make_uint4(0, 0, 0, 0);
      const bf16x8 b = __builtin_bit_cast(bf16x8, bw);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const uint4 a = *reinterpret_cast<const uint4*>(
            xs + (16 * t + (lane % 16)) * ldx + 32 * st + kq);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), b,
                                                         acc[t], 0, 0, 0);
      }
    }
  };

  // a wave whose 16 columns lie past n_total (last tile) only helps stage x
  const bool live = blockIdx.x * kTileN + wave * 16 < n_total;
  if (live) load_group(wa, 0);
  __syncthreads();  // x slice staged
  if (!live) return;
  // Both halves always run (a group past the slice multiplies zeros): with no early exit
  // the compiler cannot sink a group's loads down to the block that uses them, and the
  // scheduling barriers keep it from moving them within the iteration.
  for (int s0 = 0; s0 < nsteps; s0 += 2 * kGroup) {
    load_group(wb, s0 + kGroup);
    __builtin_amdgcn_sched_barrier(0);
    mma_group(wa, s0);
    load_group(wa, s0 + 2 * kGroup);
    __builtin_amdgcn_sched_barrier(0);
    mma_group(wb, s0 + kGroup);
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

int row_tiles(int m) { return m >= 64 ? 4 : (m + 15) / 16; }

}  // namespace

GemmPlan gemm_plan(int m, int n_total, int k) {
  const int mt = row_tiles(m);
  const int groups = (n_total + kTileN - 1) / kTileN;
  const int row_groups = (m + 63) / 64;
  // k-slice: a multiple of 64 whose x tile fits the LDS budget
  const int max_slice = ((kLdsBytes / (16 * mt * 2) - kPad) / 64) * 64;
  int ksplit = (640 + groups * row_groups - 1) / (groups * row_groups);  // ~640+ workgroups
  ksplit = ksplit < 1 ? 1 : ksplit;
  const int ksteps64 = k / 64;
  if (ksplit > ksteps64) ksplit = ksteps64;
  int kslice = 64 * ((ksteps64 + ksplit - 1) / ksplit);
  if (kslice > max_slice) kslice = max_slice;
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
  const int mt = row_tiles(m);
  const dim3 grid((n_total + kTileN - 1) / kTileN, plan.ksplit, (m + 63) / 64);
  const dim3 block(kWaves * kWave);
  const size_t lds = (size_t)16 * mt * (plan.kslice + kPad) * sizeof(uint16_t);
  const uint16_t* X = (const uint16_t*)x;
  const uint16_t* W0 = (const uint16_t*)w0;
  const uint16_t* W1 = (const uint16_t*)(nprob > 1 ? w1 : w0);
  float* Q1 = nprob > 1 ? q1 : q0;
  switch (mt) {
    case 1: hipLaunchKernelGGL(gemm_kernel<1>, grid, block, lds, stream, X, W0, W1, m, n, k,
                               plan.kslice, n_total, q0, Q1, plan.ksplit, ws); break;
    case 2: hipLaunchKernelGGL(gemm_kernel<2>, grid, block, lds, stream, X, W0, W1, m, n, k,
                               plan.kslice, n_total, q0, Q1, plan.ksplit, ws); break;
    case 3: hipLaunchKernelGGL(gemm_kernel<3>, grid, block, lds, stream, X, W0, W1, m, n, k,
                               plan.kslice, n_total, q0, Q1, plan.ksplit, ws); break;
    default: hipLaunchKernelGGL(gemm_kernel<4>, grid, block, lds, stream, X, W0, W1, m, n, k,
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
