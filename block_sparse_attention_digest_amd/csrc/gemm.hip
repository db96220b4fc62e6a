// Layer-ahead query prediction Q_pred^{i+1} = W_Q^{i+1} X^i [ScoutAttention,
// arXiv:2603.27138, HTML Sec. 3.3; Algorithm 1], and the true query Q^i = W_Q^i X^i, as a
// skinny GEMM q[m][n] = x[m][k] . w[n][k]^T with bf16 operands and float32 accumulation.
//
// m is the batch (8..40 rows), so the product is bound by streaming W from HBM, not by the
// matrix cores.  The work is cut into units of one 16-column tile x one k-slice; each unit
// belongs to one workgroup, where kpw waves split its k-slice (their sums are combined in
// LDS at the end, in a fixed order).  A wave streams its W (packed by launch_pack_w: the
// v_mfma_f32_16x16x32_bf16 B operand of one tile and one 32-wide k-step is a contiguous
// kilobyte) with 16-byte loads that cover whole cache lines, straight into B operands,
// with up to 24 k-steps in flight.  A workgroup's waves own consecutive tiles of the same
// k-slice, so the slice of x they share (at most 64 rows) is staged once in LDS, by
// global-to-LDS loads issued just ahead of the W stream (so the staging overlaps it) --
// up to 160 KiB, so one k-slice can be long and the float32 partials of the slices stay a
// small fraction of the W bytes.  The partials are summed in slice order -- by a second
// kernel in the stand-alone call, by the kernels that read the query in the decode step --
// so results are deterministic.  The plan sizes the grid to about
// one workgroup per CU, so the whole product is one round of long-lived waves.  Two weight
// matrices that share x (Q^i and Q_pred^{i+1}) can run as one launch.
#include <hip/hip_ext.h>

#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace sa {
namespace {

constexpr int kGroup = 8;            // k-steps (of 32) per register buffer
// waves per workgroup: small workgroups (about 122 VGPRs per wave, at most two waves on a
// SIMD) leave room on every CU for an attention or selection workgroup running beside them
constexpr int kMaxWpg = 5;
constexpr int kTargetUnits = 1024;   // >= 4 long-lived waves per CU
constexpr int kCUs = 256;

template <int MT>
__global__ __launch_bounds__(kMaxWpg * kWave) void gemm_kernel(const uint16_t* __restrict__ x,
                                                    const uint16_t* __restrict__ w0,
                                                    const uint16_t* __restrict__ w1, int m,
                                                    int n, int k, int kslice, int n_total,
                                                    int tiles, int tpw, float* __restrict__ out0,
                                                    float* __restrict__ out1, int ksplit,
                                                    float* __restrict__ partials) {
  extern __shared__ uint16_t xs[];  // [kslice/32][MT][64 lanes][8]; later the kpw combine
  const int lane = threadIdx.x % kWave;
  const int kpw = blockDim.x / kWave / tpw;  // waves per tile
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // scalar branches
  const int tw = wave % tpw, kpart = wave / tpw;
  const int unit0 = blockIdx.x * tpw;  // units are (k-slice, tile), slice-major
  const int ks = unit0 / tiles;        // one slice per workgroup (tiles % tpw == 0)
  const int tile = unit0 % tiles + tw;
  const int col_g = tile * 16 + (lane % 16);  // in [0, n_total)
  const int prob = tile * 16 >= n ? 1 : 0;    // the same for the 16 columns (16 | n)
  const int col = col_g - prob * n;
  const uint16_t* w = prob ? w1 : w0;
  const int k0 = ks * kslice;                 // slices are full: k0 + kslice <= k
  const int row0 = blockIdx.y * 16 * MT;

  const int nsteps = kslice / 32 / kpw;  // this wave's k-steps: part kpart of the slice
  const int step0 = kpart * nsteps;      // first k-step of the part within the slice
  // packed tile (col / 16, k-step): 512 elements, this lane's 8 at lane * 8
  const uint16_t* wtile =
      w + ((size_t)(col / 16) * (k / 32) + k0 / 32 + step0) * 512 + lane * 8;

  floatx4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};

  // 1. The x slice goes straight from global memory into LDS, in matrix-core operand order:
  //    the A operand of row tile t and k-step s (rows 16t + l % 16, k-values 32s + 8(l / 16)
  //    .. + 7 for lane l) is the kilobyte at xs + (s MT + t) 512, lane l's 16 bytes at
  //    l * 8, so each load instruction fills one kilobyte and every later operand read is
  //    lane-contiguous.  Rows past m read row m - 1: a row of A feeds only its own output
  //    row, and those rows are not stored.  The waves of the workgroup share the chunks.
  {
    const int nst = kslice / 32;
    const int waves = blockDim.x / kWave;
    const int row = min(row0 + (lane % 16), m - 1) - row0;  // row within tile 0
    const uint16_t* xl = x + (size_t)k0 + 8 * (lane / 16);
    for (int j = wave; j < MT * nst; j += waves) {
      const int st = j / MT, t = j % MT;
      const int r = min(row0 + 16 * t + row, m - 1);
      __builtin_amdgcn_global_load_lds(xl + (size_t)r * k + 32 * st, xs + (size_t)j * 512, 16,
                                       0, 0);
    }
  }
  // 2. W streams through three register groups (24 k-steps in flight: the whole part, for
  //    parts of up to 24 k-steps), issued right behind the x slice so the slice's staging
  //    overlaps the stream; each group is refilled right after it is multiplied.  All three
  //    thirds always run (a group past the part multiplies zeros and its refill re-reads the
  //    last step, a cached line): with no early exit the compiler cannot sink a group's loads
  //    down to the block that uses them, and the scheduling barriers keep it from moving
  //    them within the iteration.  Loads are unconditional (k-steps past the part clamp to
  //    its last step and their B operand is zeroed), so every path has the same loads in
  //    flight and the compiler waits only for the group being multiplied.
  uint4 wa[kGroup], wb[kGroup], wc[kGroup];
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
            xs + ((size_t)(step0 + st) * MT + t) * 512 + lane * 8);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), b,
                                                         acc[t], 0, 0, 0);
      }
    }
  };
  __builtin_amdgcn_sched_barrier(0);  // the x slice's loads go first
  load_group(wa, 0);
  load_group(wb, kGroup);
  load_group(wc, 2 * kGroup);
  __syncthreads();  // x slice staged (waits for the W loads in flight too)
  __builtin_amdgcn_sched_barrier(0);
  // (a do-while: nsteps >= 1, and a loop guard would let the compiler sink the loads above
  // past it, below the barrier)
  int s0 = 0;
  do {
    mma_group(wa, s0);
    load_group(wa, s0 + 3 * kGroup);
    __builtin_amdgcn_sched_barrier(0);
    mma_group(wb, s0 + kGroup);
    load_group(wb, s0 + 4 * kGroup);
    __builtin_amdgcn_sched_barrier(0);
    mma_group(wc, s0 + 2 * kGroup);
    load_group(wc, s0 + 5 * kGroup);
    __builtin_amdgcn_sched_barrier(0);
    s0 += 3 * kGroup;
  } while (s0 < nsteps);

  // combine the kpw parts of each tile in LDS (part order is fixed: deterministic)
  if (kpw > 1) {
    floatx4* red = reinterpret_cast<floatx4*>(xs);  // [tpw][kpw-1][MT][64]
    __syncthreads();  // every wave is done with the x slice
    if (kpart > 0) {
#pragma unroll
      for (int t = 0; t < MT; ++t)
        red[((tw * (kpw - 1) + kpart - 1) * MT + t) * kWave + lane] = acc[t];
    }
    __syncthreads();
    if (kpart > 0) return;
    for (int p = 1; p < kpw; ++p) {
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const floatx4 v = red[((tw * (kpw - 1) + p - 1) * MT + t) * kWave + lane];
        acc[t] += v;
      }
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

// Sum of the k-slice partials in slice order; four consecutive columns per thread.  All
// slices are loaded before the sum (up to kMaxSlices in flight), so the kernel waits for
// memory once.
constexpr int kMaxSlices = 8;
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
  const size_t slice = (size_t)m * n_total;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k0 = 0; k0 < ksplit; k0 += kMaxSlices) {
    float4 v[kMaxSlices];
#pragma unroll
    for (int j = 0; j < kMaxSlices; ++j)
      v[j] = *reinterpret_cast<const float4*>(partials + min(k0 + j, ksplit - 1) * slice + e);
#pragma unroll
    for (int j = 0; j < kMaxSlices; ++j) {
      if (k0 + j < ksplit) {
        s.x += v[j].x; s.y += v[j].y; s.z += v[j].z; s.w += v[j].w;
      }
    }
  }
  const int prob = col_g >= n ? 1 : 0;
  float* out = prob ? out1 : out0;
  *reinterpret_cast<float4*>(out + (size_t)row * n + (col_g - prob * n)) = s;
}

int row_tiles(int m) { return m >= 64 ? 4 : (m + 15) / 16; }

}  // namespace

GemmPlan gemm_plan(int m, int n_total, int k) {
  const int mt = row_tiles(m);
  const int tiles = n_total / 16;
  const int ksteps64 = k / 64;
  const size_t lds_max = 160 * 1024;
  // fewest k-slices (a divisor of k/64, so slices are equal) that give enough units and
  // whose x slice fits the LDS of one workgroup
  int ksplit = 0;
  for (int d = 1; d <= ksteps64; ++d) {
    if (ksteps64 % d) continue;
    const size_t lds = (size_t)16 * mt * (k / d) * sizeof(uint16_t);
    if (lds > lds_max) continue;
    ksplit = d;
    if ((long)tiles * d >= kTargetUnits) break;
  }
  const int units = tiles * ksplit;
  // tiles per workgroup: a divisor of the tile count (so a workgroup stays in one slice),
  // as large as keeps about one workgroup per CU
  int tpw = 1;
  for (int v = 1; v <= kMaxWpg; ++v)
    if (tiles % v == 0 && units / v >= kCUs) tpw = v;
  // waves per tile: split the slice further while each part keeps two register groups
  const int steps = k / ksplit / 32;
  int kpw = 1;
  for (int v = 2; v * tpw <= kMaxWpg; ++v)
    if (steps % v == 0 && steps / v >= 2 * kGroup) kpw = v;
  GemmPlan p;
  p.ksplit = ksplit;
  p.kslice = k / ksplit;
  p.tpw = tpw;
  p.kpw = kpw;
  p.ws_bytes = ksplit > 1 ? (size_t)ksplit * m * n_total * sizeof(float) : 0;
  return p;
}

hipError_t launch_gemm(int m, int n, int k, const void* x, int nprob, const void* w0,
                       float* q0, const void* w1, float* q1, float* ws, const GemmPlan& plan,
                       hipStream_t stream, bool sum_slices, hipEvent_t ev_start,
                       hipEvent_t ev_stop) {
  const int n_total = n * nprob;
  const int mt = row_tiles(m);
  const int tiles = n_total / 16;
  const dim3 grid(tiles * plan.ksplit / plan.tpw, (m + 63) / 64);
  const dim3 block(plan.tpw * plan.kpw * kWave);
  const size_t lds = std::max((size_t)16 * mt * plan.kslice * sizeof(uint16_t),
                              (size_t)plan.tpw * (plan.kpw - 1) * mt * kWave * 16);
  const uint16_t* X = (const uint16_t*)x;
  const uint16_t* W0 = (const uint16_t*)w0;
  const uint16_t* W1 = (const uint16_t*)(nprob > 1 ? w1 : w0);
  float* Q1 = nprob > 1 ? q1 : q0;
  // hipExtLaunchKernelGGL records the (optional) events at the kernel's own start and end
#define SA_GEMM_CASE(MT)                                                                    \
  case MT:                                                                                  \
    hipExtLaunchKernelGGL(gemm_kernel<MT>, grid, block, lds, stream, ev_start, ev_stop, 0,  \
                          X, W0, W1, m, n, k, plan.kslice, n_total, tiles, plan.tpw, q0,    \
                          Q1, plan.ksplit, ws);                                             \
    break;
  switch (mt) {
    SA_GEMM_CASE(1) SA_GEMM_CASE(2) SA_GEMM_CASE(3) default: SA_GEMM_CASE(4)
  }
#undef SA_GEMM_CASE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.ksplit == 1 || !sum_slices) return e;
  const long total4 = (long)m * n_total / 4;
  hipLaunchKernelGGL(gemm_reduce_kernel, dim3((unsigned)((total4 + 255) / 256)), dim3(256), 0,
                     stream, ws, m, n, n_total, plan.ksplit, q0, Q1);
  return hipGetLastError();
}

// One float4 of one row per thread: the k-slice partials summed in slice order.  `out` may be
// page-locked host memory the device addresses (the query handed to the CPU side).
__global__ __launch_bounds__(256) void gather_query_kernel(QParts q, int rows, int n,
                                                           const int32_t* __restrict__ n_cpu,
                                                           int group_cols, int Hkv,
                                                           float* __restrict__ out) {
  const long i4 = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int n4 = n / 4;
  if (i4 >= (long)rows * n4) return;
  const int row = (int)(i4 / n4);
  const int col = (int)(i4 % n4) * 4;
  // with n_cpu, only the query heads of (row, KV head) pairs that offloaded something
  if (n_cpu && n_cpu[(size_t)row * Hkv + col / group_cols] <= 0) return;
  const float* src = q.base + (size_t)row * q.row_stride + col;
  float4 s = *reinterpret_cast<const float4*>(src);
  for (int p = 1; p < q.parts; ++p) {
    const float4 v = *reinterpret_cast<const float4*>(src + (size_t)p * q.part_stride);
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  *reinterpret_cast<float4*>(out + (size_t)row * n + col) = s;
}

hipError_t launch_gather_query(const QParts& q, int rows, int n, float* out, hipStream_t stream,
                               const int32_t* n_cpu, int group_cols, int Hkv) {
  const long total4 = (long)rows * (n / 4);
  if (total4 == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_query_kernel, dim3((unsigned)((total4 + 255) / 256)), dim3(256), 0,
                     stream, q, rows, n, n_cpu, group_cols, Hkv, out);
  return hipGetLastError();
}

QParts gemm_result(const GemmPlan& plan, int m, int n, int nprob, int prob, const float* q,
                   const float* ws) {
  if (plan.ksplit == 1) return plain_query(q, n);  // written straight to q
  const size_t n_total = (size_t)n * nprob;
  return QParts{ws + (size_t)prob * n, plan.ksplit, (size_t)m * n_total, n_total};
}

}  // namespace sa
