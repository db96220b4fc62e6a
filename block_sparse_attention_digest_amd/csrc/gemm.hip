// Layer-ahead query prediction Q_pred^{i+1} = W_Q^{i+1} X^i [ScoutAttention,
// arXiv:2603.27138, HTML Sec. 3.3; Algorithm 1], and the true query Q^i = W_Q^i X^i, as a
// skinny GEMM q[m][n] = x[m][k] . w[n][k]^T with bf16 operands and float32 accumulation.
//
// m is the batch (8..40 rows), so the product is bound by streaming W from memory, not by
// the matrix cores.  A workgroup owns TPW 16-column tiles and one k-slice; its kpw waves
// split the k-slice into kpw parts, and each wave multiplies its part for all TPW tiles, so
// an x operand (the v_mfma_f32_16x16x32_bf16 A operand: 16 rows x 32 k-values, 16 bytes a
// lane) is loaded once per wave and used for every tile.  Both operands go straight from
// memory into registers -- x rows as A operands, W (packed by launch_pack_w: the B operand
// of one tile and one 32-wide k-step is a contiguous kilobyte) as B operands -- five k-steps
// (four with 64 rows) ahead of the matrix cores, so no wave waits for another before its
// first product.  The tile count is a template parameter, so the product loop has no
// branches.  At the end each wave writes its part of the workgroup's output block
// row-major into LDS; the parts are summed in part order, and the workgroup stores its
// block (its slice's float32 partial) as whole rows of float4.  The partials are summed in
// slice order -- by a second kernel in the stand-alone call, by the kernels that read the
// query in the decode step -- so results are deterministic.  The plan sizes the grid to
// about one workgroup per CU, of four waves (one per SIMD) unless the caller asks for up to
// five, so the whole product is one round of short-lived waves.  Two weight matrices that
// share x (Q^i and Q_pred^{i+1}) can run as one launch.
#include <hip/hip_ext.h>

#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace sa {
namespace {

// waves per workgroup: up to five (the plan takes four unless told otherwise: one per SIMD
// of a CU); small workgroups also leave room on every CU for an attention or selection
// workgroup running beside them.  The kernel is built for two waves per SIMD (at most 256
// registers a wave): with more, the compiler keeps values in the accumulation registers and
// copies them inside the product loop.
constexpr int kMaxWpg = 5;
constexpr int kMaxTpw = 5;           // 16-column tiles per workgroup (and per wave)
constexpr int kCUs = 256;

// floats per row of a wave's part in LDS: the block's 16 TPW columns and 4 more, so the four
// row quads a store instruction writes fall in different banks
constexpr int red_stride(int tpw) { return 16 * tpw + 4; }

template <int MT, int TPW>
__global__ __launch_bounds__(kMaxWpg * kWave, 2) void gemm_kernel(const uint16_t* __restrict__ x,
                                                    const uint16_t* __restrict__ w0,
                                                    const uint16_t* __restrict__ w1, int m,
                                                    int n, int k, int kslice, int tiles,
                                                    float* __restrict__ out0,
                                                    float* __restrict__ out1, int ksplit,
                                                    float* __restrict__ partials) {
  extern __shared__ float4 red4[];  // [kpw][16 MT][RS] floats: every part's sums, row-major
  constexpr int RS = red_stride(TPW);
  const int lane = threadIdx.x % kWave;
  const int kpw = blockDim.x / kWave;  // waves per workgroup: the parts of the k-slice
  const int kpart = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int groups = tiles / TPW;
  const int ks = blockIdx.x / groups;        // the k-slice
  const int tile0 = (blockIdx.x % groups) * TPW;
  const int n_total = tiles * 16;
  const int row0 = blockIdx.y * 16 * MT;
  const int mr = min(16 * MT, m - row0);     // rows of this row group
  const int nsteps = kslice / 32 / kpw;      // this wave's k-steps
  const int kk0 = ks * kslice + kpart * nsteps * 32;  // its first k

  // A operand of row tile t, k-step s: lane l holds row 16t + l % 16 (rows past m read row
  // m - 1: a row of A feeds only its own output row, and those rows are not stored),
  // k-values 8 (l / 16) .. + 7
  const uint16_t* xa[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t)
    xa[t] = x + (size_t)min(row0 + 16 * t + lane % 16, m - 1) * k + kk0 + 8 * (lane / 16);
  // B operand of tile tt, k-step s: the packed kilobyte (tile, k-step), lane l's 8 values
  const uint16_t* wb[TPW];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int tile = tile0 + tt;
    const int prob = tile * 16 >= n ? 1 : 0;  // (16 | n: the same for the tile's columns)
    const uint16_t* w = prob ? w1 : w0;
    wb[tt] = w + ((size_t)(tile - prob * n / 16) * (k / 32) + kk0 / 32) * 512 + lane * 8;
  }

  floatx4 acc[TPW][MT];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[tt][t] = floatx4{0.f, 0.f, 0.f, 0.f};

  // kAhead register sets rotate, each holding one k-step's operands; a set is refilled
  // right after it is multiplied, while the k-steps of the other sets are in flight.  Loads
  // are unconditional (k-steps past the part clamp to its last step; the B operands of such
  // steps are zeroed), so the loop has the same loads in flight on every path and the
  // compiler waits only for the set being multiplied; the scheduling barriers keep it from
  // sinking loads.  The last round issues no loads.
  constexpr int kAhead = MT >= 4 ? 4 : 5;
  struct Set {
    uint4 a[MT];
    uint4 b[TPW];
  };
  Set rs[kAhead];
  auto load = [&](Set& r, int st) {
    const int sc = min(st, nsteps - 1);
#pragma unroll
    for (int t = 0; t < MT; ++t) r.a[t] = *reinterpret_cast<const uint4*>(xa[t] + 32 * sc);
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) r.b[tt] = *reinterpret_cast<const uint4*>(wb[tt] + 512 * sc);
  };
  auto mma = [&](const Set& r, int st) {
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      const uint4 bw = st < nsteps ? r.b[tt] : make_uint4(0, 0, 0, 0);
      const bf16x8 b = __builtin_bit_cast(bf16x8, bw);
#pragma unroll
      for (int t = 0; t < MT; ++t)
        acc[tt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, r.a[t]),
                                                             b, acc[tt][t], 0, 0, 0);
    }
  };
#pragma unroll
  for (int u = 0; u < kAhead; ++u) load(rs[u], u);
  __builtin_amdgcn_sched_barrier(0);
  int s0 = 0;
  for (; s0 + kAhead < nsteps; s0 += kAhead) {
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      mma(rs[u], s0 + u);
      load(rs[u], s0 + u + kAhead);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int u = 0; u < kAhead; ++u)
    if (s0 + u < nsteps) mma(rs[u], s0 + u);  // (uniform)

  // acc[tt][t][r] holds row 16t + 4 (lane / 16) + r of the block, column 16 tt + lane % 16:
  // the wave writes its part row-major, every row (rows past mr hold sums of the repeated
  // last row and are never read; writing them keeps the stores unpredicated)
  float* red = reinterpret_cast<float*>(red4);
  float* mine = red + (size_t)kpart * 16 * MT * RS;
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        mine[(16 * t + 4 * (lane / 16) + r) * RS + 16 * tt + lane % 16] = acc[tt][t][r];
  __syncthreads();
  // the block, mr rows x 4 TPW float4: each sums the kpw parts in part order (deterministic)
  // and stores whole rows
  const int units = mr * 4 * TPW;
  for (int u = threadIdx.x; u < units; u += blockDim.x) {
    const int row = u / (4 * TPW), c4 = u % (4 * TPW);
    float4 s = red4[(row * RS) / 4 + c4];
    for (int p = 1; p < kpw; ++p) {
      const float4 v = red4[((p * 16 * MT + row) * RS) / 4 + c4];
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    const int col_g = tile0 * 16 + 4 * c4;  // in [0, n_total); a float4 stays in one tile
    if (ksplit == 1) {
      const int prob = col_g >= n ? 1 : 0;
      float* out = prob ? out1 : out0;
      *reinterpret_cast<float4*>(out + (size_t)(row0 + row) * n + col_g - prob * n) = s;
    } else {
      *reinterpret_cast<float4*>(partials + ((size_t)ks * m + row0 + row) * n_total + col_g) = s;
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

GemmPlan gemm_plan(int m, int n_total, int k, int max_waves) {
  const int tiles = n_total / 16;
  const int ksteps64 = k / 64;
  const int row_groups = (m + 63) / 64;
  // tiles per workgroup: 5 when they divide the tile count, else 4 (the entry points take
  // n % 64 == 0, so the tile count is a multiple of 4; any other count gets tpw = 0, which
  // launch_gemm refuses)
  const int tpw = tiles % kMaxTpw == 0 ? kMaxTpw : tiles % 4 == 0 ? 4 : 0;
  const int groups = tpw ? tiles / tpw : 1;
  // fewest k-slices (a divisor of k/64, so slices are equal) that give about one workgroup
  // per CU, and at most kMaxSplit of them (the consumers sum the slices' partials)
  constexpr int kMaxSplit = 16;
  int ksplit = 1;
  for (int d = 1; d <= ksteps64 && d <= kMaxSplit; ++d) {
    if (ksteps64 % d) continue;
    ksplit = d;
    if ((long)groups * row_groups * d >= kCUs) break;
  }
  // waves per workgroup: the most, up to max_waves, that split the slice's k-steps evenly
  const int steps = k / ksplit / 32;
  int kpw = 1;
  for (int v = 2; v <= std::min(max_waves, kMaxWpg); ++v)
    if (steps % v == 0) kpw = v;
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
  if (plan.tpw != 4 && plan.tpw != kMaxTpw) return hipErrorInvalidValue;
  const int mt = row_tiles(m);
  const int tiles = n_total / 16;
  const dim3 grid(tiles / plan.tpw * plan.ksplit, (m + 16 * mt - 1) / (16 * mt));
  const dim3 block(plan.kpw * kWave);
  // every wave's part of the block, all 16 mt rows
  const size_t lds = (size_t)plan.kpw * 16 * mt * red_stride(plan.tpw) * sizeof(float);
  const uint16_t* X = (const uint16_t*)x;
  const uint16_t* W0 = (const uint16_t*)w0;
  const uint16_t* W1 = (const uint16_t*)(nprob > 1 ? w1 : w0);
  float* Q1 = nprob > 1 ? q1 : q0;
  // hipExtLaunchKernelGGL records the (optional) events at the kernel's own start and end
#define SA_GEMM_LAUNCH(MT, TPW)                                                             \
  hipExtLaunchKernelGGL((gemm_kernel<MT, TPW>), grid, block, lds, stream, ev_start, ev_stop, \
                        0, X, W0, W1, m, n, k, plan.kslice, tiles, q0, Q1, plan.ksplit, ws)
#define SA_GEMM_TPW(MT)    \
  if (plan.tpw == 4) {     \
    SA_GEMM_LAUNCH(MT, 4); \
  } else {                 \
    SA_GEMM_LAUNCH(MT, 5); \
  }
  switch (mt) {
    case 1: SA_GEMM_TPW(1) break;
    case 2: SA_GEMM_TPW(2) break;
    case 3: SA_GEMM_TPW(3) break;
    default: SA_GEMM_TPW(4) break;
  }
#undef SA_GEMM_TPW
#undef SA_GEMM_LAUNCH
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
