// GPU-side partial attention over the resident selected blocks, A_gpu = GPUATTN(Q, B_gpu),
// and its FlashAttention-style merge with the host partials, A = MERGE(A_gpu, A_cpu)
// [ScoutAttention, arXiv:2603.27138, HTML Sec. 3.2; Algorithm 1].
//
// Work split: balanced persistent waves.  The selected resident blocks of all (sequence,
// KV head) pairs are laid end to end (an exclusive prefix sum of n_gpu over the pairs, T
// blocks in all) and wave w of the W waves in the grid streams blocks
// [floor(w T / W), floor((w+1) T / W)), crossing pair boundaries as it goes.  Every wave
// gets the same number of blocks whatever the per-pair counts are, so the chip streams
// until the end with no partial last round.  For each pair its range touches a wave keeps
// one online softmax and writes one un-normalised partial (o, m, l) per query head; the
// partial of wave w for pair p lives in slot w + p, which is unique because the waves'
// ranges are ordered.  The reduce kernel combines a pair's partials (waves covering the
// pair's block range) and, when given, the host partial.
//
// bf16 path, per 16-token step of a wave (one MFMA tile: a block of 16, or half of 32):
//   * the page and valid-token count of up to 64 upcoming blocks (of one or more pairs) sit
//     in lane registers, looked up in one round per window from the page list when the
//     selection wrote one (else list entry, then block table);
//   * K (16 x d) is loaded straight into MFMA A-operand registers: lane l holds token
//     l % 16 and 8 consecutive channels (16 bytes).  K pages are chunk-major (the bs
//     tokens' values of 8 channels are 16 * bs contiguous bytes), so the 16 lanes that load
//     one chunk for 16 tokens read 256 contiguous bytes -- whole cache lines;
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16.  Q's columns are the G heads split into a
//     bf16 high part (columns 0..7) and a bf16 low part q - hi (columns 8..15); adding the
//     two results recovers q . k to about 2^-17 relative, so the float32 query keeps its
//     precision while K stays bf16;
//   * the softmax runs on the MFMA output layout (lane l: column l % 16, four tokens) with
//     DPP / permlane exchanges;
//   * O^T += V^T P on v_mfma_f32_16x16x16_bf16: V^T is the A operand (lane l: channel
//     l % 16 of a 16-channel group, four tokens -- 8 contiguous bytes of a V page stored as
//     [bs/16][d][16]), and P is the B operand straight from the softmax registers (its
//     layout is the S^T layout), split like Q into bf16(p) (columns 0..7) and p - bf16(p)
//     (columns 8..15);
//   * the two steps after the one being computed are in flight; all of a step's loads are
//     issued unconditionally (clamped to valid rows) so that the waits before a step cover
//     that step only, and the pipeline runs on across pair boundaries.
// float32 path (small fp32 workloads): the same balanced ranges, one block at a time, K
// (chunk-major, four channels per chunk) and V staged through LDS and plain per-lane dot
// products.
//
// Internal log2 domain: logits are scaled by scale * log2(e) and exponentiated with exp2;
// m is reported in natural-log units.
#include <hip/hip_ext.h>

#include "common.hpp"
#include "kernels.hpp"

namespace sa {
namespace {

constexpr int kAttnWaves = 4;            // waves per workgroup (bf16 path)
constexpr int kQStage = 4;               // pairs whose summed queries a workgroup stages
constexpr int kPartGroup = 4;            // query parts loaded together
constexpr int kStep = 16;                // tokens per wave step (one MFMA tile)
constexpr int kWavesPerCU = 8;           // resident waves per CU the grid is sized for
constexpr int kMaxWaves = 256 * kWavesPerCU;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Workspace: prefix [npairs + 1] ints, then per slot (W + npairs slots) and head: o [D]
// floats, then (m_log2, l) pairs.
struct PartialView {
  int* pfx;
  float* o;
  float* ml;
};
__host__ __device__ inline size_t prefix_bytes(int npairs) {
  return ((size_t)(npairs + 1) * sizeof(int) + 255) & ~(size_t)255;
}
__host__ __device__ inline PartialView partial_view(float* base, int npairs, int W, int G, int D) {
  PartialView v;
  v.pfx = reinterpret_cast<int*>(base);
  v.o = reinterpret_cast<float*>(reinterpret_cast<char*>(base) + prefix_bytes(npairs));
  v.ml = v.o + (size_t)(W + npairs) * G * D;
  return v;
}

// first global block of wave w, and the wave holding global block g
__device__ __forceinline__ int wave_start(int w, int T, int W) {
  return (int)((long long)w * T / W);
}
__device__ __forceinline__ int wave_of(int g, int T, int W) {
  return (int)(((long long)(g + 1) * W + T - 1) / T) - 1;
}

// Exclusive prefix sum of n_gpu over the pairs into LDS pfx[0..npairs] (pfx[npairs] = T);
// counts are taken clamped into [0, cap] (cap = the list stride), so no count read from
// memory can move an index past the lists.  Every thread of the workgroup takes part; ends
// with a barrier.
__device__ __forceinline__ int clamp_count(int n, int cap) { return min(max(n, 0), cap); }
__device__ void pair_prefix(const int32_t* __restrict__ n_gpu, int npairs, int cap, int* pfx,
                            int* wave_tot) {
  const int nt = blockDim.x, tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave, nw = nt / kWave;
  const int per = (npairs + nt - 1) / nt;
  const int p0 = min(npairs, tid * per), p1 = min(npairs, p0 + per);
  int local = 0;
  for (int p = p0; p < p1; ++p) local += clamp_count(n_gpu[p], cap);
  int incl = local;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += t;
  }
  if (lane == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wave_tot[w];
  int run = base + incl - local;
  for (int p = p0; p < p1; ++p) {
    pfx[p] = run;
    run += clamp_count(n_gpu[p], cap);
  }
  if (tid == nt - 1) {
    int tot = 0;
    for (int w = 0; w < nw; ++w) tot += wave_tot[w];
    pfx[npairs] = tot;
  }
  __syncthreads();
}

// The same prefix computed by each wave on its own, for npairs <= kWave * kPrefixRun: lane i
// sums the counts of pairs [i r, i r + r) (r = ceil(npairs / kWave)) and one wave scan joins
// the runs.  The waves of a workgroup all write the same values, and each reads the array
// only after writing all of it itself, so no barrier is needed.  Returns T = pfx[npairs].
constexpr int kPrefixRun = 8;
__device__ int wave_prefix(const int32_t* __restrict__ n_gpu, int npairs, int cap, int* pfx) {
  const int lane = threadIdx.x % kWave;
  const int per = (npairs + kWave - 1) / kWave;
  const int p0 = lane * per;
  int v[kPrefixRun];
  int local = 0;
#pragma unroll
  for (int u = 0; u < kPrefixRun; ++u) {  // loads unconditional, indexes clamped
    const int c = n_gpu[min(p0 + u, npairs - 1)];
    v[u] = u < per && p0 + u < npairs ? clamp_count(c, cap) : 0;
    local += v[u];
  }
  int incl = local;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += t;
  }
  int run = incl - local;
#pragma unroll
  for (int u = 0; u < kPrefixRun; ++u) {
    if (u < per && p0 + u < npairs) pfx[p0 + u] = run;
    run += v[u];
  }
  const int T = __builtin_amdgcn_readlane(incl, kWave - 1);
  if (lane == 0) pfx[npairs] = T;
  return T;
}

// last pair p with pfx[p] <= g (the pair holding global block g when g < T)
__device__ __forceinline__ int pair_of(const int* pfx, int npairs, int g) {
  int lo = 0, hi = npairs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pfx[mid] <= g) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The query rows of pairs [q_lo, q_lo + q_n) summed from their parts, in part order, for
// staging in LDS.  Every thread of the workgroup takes kSlots float4 of them.  stage_load
// only issues the loads of the first kPartGroup parts (all in flight together), so the
// caller can issue other loads before stage_store sums them (loading any further parts) and
// writes the sums out.
template <int G, int D>
struct QStage {
  static constexpr int kPerPair = G * D / 4;  // float4 per pair
  static constexpr int kSlots = (kQStage * kPerPair + 255) / 256;
  const float* src[kSlots];
  float4 t[kPartGroup][kSlots];
};
template <int G, int D>
__device__ __forceinline__ void stage_load_group(const QParts& q, int p0, QStage<G, D>& st) {
#pragma unroll
  for (int u = 0; u < kPartGroup; ++u)
#pragma unroll
    for (int j = 0; j < QStage<G, D>::kSlots; ++j)
      st.t[u][j] = *reinterpret_cast<const float4*>(
          st.src[j] + (size_t)min(p0 + u, q.parts - 1) * q.part_stride);
}
template <int G, int D>
__device__ __forceinline__ void stage_load(const QParts& q, int Hkv, int q_lo, int q_n,
                                           QStage<G, D>& st) {
  constexpr int kPerPair = QStage<G, D>::kPerPair;
  const int total = max(q_n, 1) * kPerPair;  // q_n = 0: a re-read of pair q_lo, unused
#pragma unroll
  for (int j = 0; j < QStage<G, D>::kSlots; ++j) {
    const int i = min((int)threadIdx.x + j * (int)blockDim.x, total - 1);  // past the end: a re-read
    const int pair = q_lo + i / kPerPair, e = i % kPerPair;
    st.src[j] = q.base + (size_t)(pair / Hkv) * q.row_stride + (size_t)(pair % Hkv) * G * D + 4 * e;
  }
  stage_load_group(q, 0, st);
}
// adds parts p0 + u (u = u0 .. kPartGroup - 1) that exist; branch-free selects on the
// uniform part count keep the waits on these loads exact
template <int G, int D>
__device__ __forceinline__ void stage_sum_group(const QParts& q, int p0, int u0,
                                                const QStage<G, D>& st,
                                                float4 (&acc)[QStage<G, D>::kSlots]) {
#pragma unroll
  for (int u = 0; u < kPartGroup; ++u) {
    if (u < u0) continue;
    const bool use = p0 + u < q.parts;
#pragma unroll
    for (int j = 0; j < QStage<G, D>::kSlots; ++j) {
      const float4 t = st.t[u][j];
      acc[j].x = use ? acc[j].x + t.x : acc[j].x;
      acc[j].y = use ? acc[j].y + t.y : acc[j].y;
      acc[j].z = use ? acc[j].z + t.z : acc[j].z;
      acc[j].w = use ? acc[j].w + t.w : acc[j].w;
    }
  }
}
template <int G, int D>
__device__ __forceinline__ void stage_store(const QParts& q, int q_n, QStage<G, D>& st,
                                            float* q_lds) {
  constexpr int kSlots = QStage<G, D>::kSlots;
  float4 acc[kSlots];
#pragma unroll
  for (int j = 0; j < kSlots; ++j) acc[j] = st.t[0][j];
  stage_sum_group(q, 0, 1, st, acc);
  for (int p0 = kPartGroup; p0 < q.parts; p0 += kPartGroup) {  // more parts: one group at a time
    stage_load_group(q, p0, st);
    stage_sum_group(q, p0, 0, st, acc);
  }
  const int total = q_n * QStage<G, D>::kPerPair;
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    const int i = (int)threadIdx.x + j * (int)blockDim.x;
    if (i < total) *reinterpret_cast<float4*>(q_lds + 4 * i) = acc[j];
  }
}

template <int D, int BS, int G>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(
    const QParts q, const uint16_t* __restrict__ k_pool,
    const uint16_t* __restrict__ v_pool, const int32_t* __restrict__ table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ gpu_blocks,
    const int32_t* __restrict__ gpu_pages, const int32_t* __restrict__ n_gpu, int list_stride,
    int Hkv, int max_blocks, int P, int npairs, int W, float scale_log2,
    float* __restrict__ ws) {
  constexpr int KS = D / 32;          // MFMA k-steps over the head dimension (S = K Q^T)
  constexpr int CG = D / 16;          // 16-channel groups of the output (O^T += V^T P)
  constexpr int HPB = BS / kStep;     // 16-token steps per block (1, 2 or 4)

  extern __shared__ int pfx[];        // [npairs + 1]
  __shared__ float q_lds[kQStage * G * D];
  __shared__ int wave_tot[kAttnWaves];

  const int lane = threadIdx.x % kWave;
  // wave-uniform values are made explicitly scalar so that every loop below branches on
  // scalars: a loop exit the compiler takes for lane-divergent ends in exec-masked flow
  // blocks, where it drains all loads in flight (vmcnt(0)) at the loop header
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  int T;
  if (npairs <= kWave * kPrefixRun) {  // (uniform)
    T = wave_prefix(n_gpu, npairs, list_stride, pfx);
  } else {
    pair_prefix(n_gpu, npairs, list_stride, pfx, wave_tot);
    T = pfx[npairs];
  }
  T = __builtin_amdgcn_readfirstlane(T);
  const PartialView part = partial_view(ws, npairs, W, G, D);
  if (blockIdx.x == 0 && wave == 0)
    for (int i = lane; i <= npairs; i += kWave) part.pfx[i] = pfx[i];
  const int gw = blockIdx.x * kAttnWaves + wave;
  if (T == 0) return;
  // the queries of the first kQStage pairs the workgroup's block range touches
  int q_lo = 0, q_n = 0;
  {
    const int lo = wave_start(blockIdx.x * kAttnWaves, T, W);
    const int hi = wave_start((blockIdx.x + 1) * kAttnWaves, T, W);
    if (lo < hi) {
      q_lo = __builtin_amdgcn_readfirstlane(pair_of(pfx, npairs, lo));
      q_n = min(kQStage, __builtin_amdgcn_readfirstlane(pair_of(pfx, npairs, hi - 1)) - q_lo + 1);
    }
  }
  const int b0 = wave_start(gw, T, W), b1 = wave_start(gw + 1, T, W);

  // The wave's range is walked in windows of up to 64 blocks; a window may span several
  // pairs.  Lane j looks up window block j in one pass (its pair by a short scan of the
  // prefix, then list entry, valid tokens and page -- from the page list when one is
  // given, else from the block table), so a pair change costs no new lookup.
  int l_blk = 0, l_len = 0, l_page = 0;
  auto lookup = [&](int wb, int nw, int pstart) {
    const int g = wb + min(lane, nw - 1);
    int pj = pstart;
    while (pfx[pj + 1] <= g) ++pj;
    const size_t idx = (size_t)pj * list_stride + (g - pfx[pj]);
    // entries are taken clamped into range: a bad list gives wrong numbers, never an access
    // outside the pools
    l_blk = min(max(gpu_blocks[idx], 0), max_blocks - 1);
    l_len = seq_lens[pj / Hkv];
    l_page = gpu_pages ? gpu_pages[idx] : table[(size_t)pj * max_blocks + l_blk];
    l_page = min(max(l_page, 0), P - 1);
  };
  // The first window's lookup and the query staging loads are issued together (a wave with
  // no blocks looks up the last block, unused).
  const int gfirst = min(b0, T - 1);
  int p = __builtin_amdgcn_readfirstlane(pair_of(pfx, npairs, gfirst));
  lookup(gfirst, b0 < b1 ? min(kWave, b1 - b0) : 1, p);
  QStage<G, D> qst;
  stage_load<G, D>(q, Hkv, q_lo, q_n, qst);
  __builtin_amdgcn_sched_barrier(0);  // issued here, ahead of the first window's K/V loads

  const int c16 = lane % 16;   // MFMA column (head / hi-lo) and token row in the tile
  const int kq = lane / 16;    // MFMA k-group
  const int hcol = c16 & 7;    // head of this MFMA column

  // Q^T as the MFMA B operand (hi columns 0..7, lo 8..15), set when a pair's blocks begin
  // from its float rows: staged pairs from LDS; any other pair (a workgroup range crossing
  // more than kQStage pairs) summed from its parts in global memory.
  bf16x8 qb[KS];
  auto set_q = [&](int pair) {
    const int row = hcol < G ? hcol : 0;
    float4 qr[KS][2];
    if (pair - q_lo < q_n && pair >= q_lo) {
      const float* qrow = q_lds + ((pair - q_lo) * G + row) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        qr[ks][0] = *reinterpret_cast<const float4*>(qrow + 32 * ks + 8 * kq);
        qr[ks][1] = *reinterpret_cast<const float4*>(qrow + 32 * ks + 8 * kq + 4);
      }
    } else {
      const float* qrow = q.base + (size_t)(pair / Hkv) * q.row_stride +
                          ((size_t)(pair % Hkv) * G + row) * D;
      for (int part = 0; part < q.parts; ++part) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const float4 v = *reinterpret_cast<const float4*>(
                qrow + (size_t)part * q.part_stride + 32 * ks + 8 * kq + 4 * hh);
            if (part == 0) {
              qr[ks][hh] = v;
            } else {
              qr[ks][hh].x += v.x; qr[ks][hh].y += v.y;
              qr[ks][hh].z += v.z; qr[ks][hh].w += v.w;
            }
          }
      }
    }
    const bool live = hcol < G;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float v[8];
      *reinterpret_cast<float4*>(v) = qr[ks][0];
      *reinterpret_cast<float4*>(v + 4) = qr[ks][1];
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t half[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float x = live ? v[2 * i + j] : 0.f;
          const uint32_t hi = f32_to_bf16_rne(x);
          half[j] = c16 < 8 ? hi : f32_to_bf16_rne(x - __uint_as_float(hi << 16));
        }
        w[i] = half[0] | (half[1] << 16);
      }
      qb[ks] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
    }
  };

  // Online softmax state of MFMA column c16 (head hcol): m and this lane's share of l
  // (its four tokens of every step), and O^T as CG MFMA accumulator tiles, o[cg][r] =
  // O^T[channel 16 cg + 4 kq + r][column c16].  Columns 0..7 accumulate V^T P_hi and
  // columns 8..15 V^T P_lo for the same heads; o = their sum.
  float m_run = -INFINITY;   // log2 units, uniform over the column's lanes
  float l_lane = 0.f;
  floatx4 o[CG];
  auto reset = [&]() {
    m_run = -INFINITY;
    l_lane = 0.f;
#pragma unroll
    for (int cg = 0; cg < CG; ++cg) o[cg] = floatx4{0.f, 0.f, 0.f, 0.f};
  };
  auto finalize = [&](int pair) {  // write this wave's partial for `pair` to slot gw + pair
    const float l_w = sum_xor32(sum_xor16(l_lane));  // the column's four kq lanes
    const size_t slot = (size_t)(gw + pair) * G;
    float* dst = part.o + (slot + (c16 < G ? c16 : 0)) * D + 4 * kq;
#pragma unroll
    for (int cg = 0; cg < CG; ++cg) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = o[cg][r] + xor8(o[cg][r]);  // hi + lo columns
      if (c16 < G)
        *reinterpret_cast<float4*>(dst + 16 * cg) = make_float4(v[0], v[1], v[2], v[3]);
    }
    if (lane < G) {  // lane g: c16 = g, kq = 0
      part.ml[(slot + lane) * 2 + 0] = m_run;
      part.ml[(slot + lane) * 2 + 1] = l_w;
    }
  };

  // One 16-token step in registers, both as MFMA A operands: the K tile (lane l: token
  // l % 16, channels 32 ks + 8 kq .. + 7) and the V^T tiles (lane l: channel 16 cg + l % 16,
  // tokens 4 kq .. + 3 of the step).
  struct StepRegs {
    uint4 k[KS];
    uint2 v[CG];
    int nval;
  };
  int w_page = 0, w_nval = 0;  // lane j: page and valid tokens of block (window start + j)
  // Every load is issued unconditionally, so the number of loads in flight is the same on
  // every path and the compiler waits only for the step being computed, never for the one
  // in flight.  The K/V of a step are read once (non-temporal loads); a padding step past a
  // window's end reads the first step of pool page 0 instead, the same lines for every wave,
  // so that after the first they come from the cache rather than from HBM.
  auto load_step = [&](int j, int hh, StepRegs& R, bool pad) {
    const int page = pad ? 0 : __builtin_amdgcn_readlane(w_page, j);
    hh = pad ? 0 : hh;
    R.nval = __builtin_amdgcn_readlane(w_nval, j) - kStep * hh;  // valid tokens of the step
    // chunk 4 ks + kq (channels 32 ks + 8 kq .. + 7) of token kStep hh + c16
    const uint16_t* src = k_pool + (size_t)page * BS * D + ((size_t)kq * BS + kStep * hh + c16) * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      R.k[ks] = load_stream16(src + (size_t)ks * 4 * BS * 8);
    // V half-page hh is [D][16]: channel 16 cg + c16, tokens 4 kq .. + 3 (8 bytes); the 64
    // lanes of one tile read 512 contiguous bytes
    const uint16_t* vsrc = v_pool + ((size_t)page * HPB + hh) * D * kStep + c16 * kStep + 4 * kq;
#pragma unroll
    for (int cg = 0; cg < CG; ++cg)
      R.v[cg] = load_stream8(vsrc + (size_t)cg * 16 * kStep);
  };

  auto compute_step = [&](const StepRegs& R) {
    // S^T tile: acc[r] = logit of token 4kq + r for MFMA column c16
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, R.k[ks]), qb[ks],
                                                    acc, 0, 0, 0);
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float tot = acc[r] + xor8(acc[r]);  // hi + lo columns
      sc[r] = 4 * kq + r < R.nval ? tot * scale_log2 : -INFINITY;
    }
    // online softmax for head hcol (the column's 16 tokens are on its four kq lanes)
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = max_xor32(max_xor16(mx));
    const float m_new = fmaxf(m_run, mx);
    const bool none = m_new == -INFINITY;
    const float alpha = none ? 1.f : fast_exp2(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = none ? 0.f : fast_exp2(sc[r] - m_new);
      sc[r] = p;
      psum += p;
    }
    l_lane = l_lane * alpha + psum;
    m_run = m_new;
    // P as the B operand of O^T += V^T P, straight from this layout (lane l: column c16,
    // tokens 4 kq .. + 3): bf16(p) in columns 0..7, the rounding remainder p - bf16(p) in
    // columns 8..15, so the two column halves together carry p to about 2^-17
    uint32_t pw[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      uint32_t half[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float x = sc[2 * i + j];
        const uint32_t hi = f32_to_bf16_rne(x);
        half[j] = c16 < 8 ? hi : f32_to_bf16_rne(x - __uint_as_float(hi << 16));
      }
      pw[i] = half[0] | (half[1] << 16);
    }
    const shortx4 pb = __builtin_bit_cast(shortx4, make_uint2(pw[0], pw[1]));
    // tokens past the valid ones may hold anything (a partly filled page): their V is zeroed
    // (their p is already 0), so no stale NaN reaches the sum
    uint2 keep = make_uint2(~0u, ~0u);
    if (R.nval < kStep) {
      const int n = R.nval - 4 * kq;  // valid tokens among this lane's four
      keep.x = n >= 2 ? ~0u : (n == 1 ? 0xffffu : 0u);
      keep.y = n >= 4 ? ~0u : (n == 3 ? 0xffffu : 0u);
    }
#pragma unroll
    for (int cg = 0; cg < CG; ++cg) {
      o[cg] *= alpha;
      const uint2 v = make_uint2(R.v[cg].x & keep.x, R.v[cg].y & keep.y);
      o[cg] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(shortx4, v), pb,
                                                        o[cg], 0, 0, 0);
    }
  };

  // The steps of a window run as one software pipeline across pair boundaries: before the
  // first step of a pair's block is computed, the previous pair's partial is written and
  // the new pair's query set, while that step's loads and the next ones are in flight.
  // (The pair after p that holds blocks: the one holding block pfx[p + 1].)
  auto next_pair = [&](int pp) {
    const int end = __builtin_amdgcn_readfirstlane(pfx[pp + 1]);
    while (pp < npairs - 1 && __builtin_amdgcn_readfirstlane(pfx[pp + 1]) <= end) ++pp;
    return pp;
  };
  // A window's pages and valid-token counts go to lane registers and the loads of its first
  // two steps are issued.  The steps past the window's end are padding loads (see
  // load_step), so every path has the same loads in flight.
  StepRegs ra, rb, rc;
  int nw = 1, nst = 1;
  auto ld = [&](int st, StepRegs& R) {
    const int sc = min(st, nst - 1);
    load_step(sc / HPB, sc % HPB, R, st >= nst);
  };
  auto open_window = [&](int wb) {
    nw = max(1, min(kWave, b1 - wb));
    w_page = l_page;
    w_nval = min(BS, l_len - l_blk * BS);
    nst = nw * HPB;
    ld(0, ra);
    ld(1, rb);
  };
  // The first window opens before the staged queries are written out, so its loads are in
  // flight while the workgroup meets at the staging barrier (which orders LDS only).  A wave
  // with no blocks has loaded its clamped lookup's page and stops there.
  open_window(b0);
  if (q_n > 0) {  // (uniform over the workgroup)
    stage_store<G, D>(q, q_n, qst, q_lds);
    lds_barrier();
  }
  if (b0 >= b1) return;

  bool open = false;  // a partial of pair p is being accumulated
  for (int wb = b0; wb < b1; wb += kWave) {
    if (wb != b0) {
      lookup(wb, min(kWave, b1 - wb), p);
      open_window(wb);
    }
    int bnd = __builtin_amdgcn_readfirstlane(pfx[p + 1]) - wb;  // first block of the next pair
    // before step s (block s / HPB): switch pairs at a pair's first block
    auto enter = [&](int s) {
      if (s % HPB == 0 && s / HPB == bnd) {
        finalize(p);
        open = false;
        p = next_pair(p);
        bnd = __builtin_amdgcn_readfirstlane(pfx[p + 1]) - wb;
      }
      if (!open) {
        set_q(p);
        reset();
        open = true;
      }
    };
    // HPB steps per block; a step past the block's valid tokens is fully masked.  Three
    // steps per iteration, the two after the one being computed in flight (so a wave keeps
    // the memory busy on its own once its SIMD neighbour has finished); the scheduling
    // barriers keep the compiler from sinking the loads to their use.
    for (int st = 0; st < nst; st += 3) {
      ld(st + 2, rc);
      __builtin_amdgcn_sched_barrier(0);
      enter(st);
      compute_step(ra);
      ld(st + 3, ra);
      __builtin_amdgcn_sched_barrier(0);
      if (st + 1 < nst) {
        enter(st + 1);
        compute_step(rb);
      }
      ld(st + 4, rb);
      __builtin_amdgcn_sched_barrier(0);
      if (st + 2 < nst) {
        enter(st + 2);
        compute_step(rc);
      }
    }
    if (nw == bnd) {  // pair p ends with the window
      finalize(p);
      open = false;
      p = next_pair(p);
    }
  }
  if (open) finalize(p);  // the range ended inside pair p
}

// float32 KV: one wave per workgroup, the same balanced ranges, one block at a time.
template <int D, int BS>
__global__ __launch_bounds__(64) void attn_f32_kernel(
    const QParts q, const float* __restrict__ k_pool,
    const float* __restrict__ v_pool, const int32_t* __restrict__ table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ gpu_blocks,
    const int32_t* __restrict__ n_gpu, int list_stride, int Hkv, int G, int max_blocks,
    int P, int npairs, int W, float scale_log2, float* __restrict__ ws) {
  constexpr int CPL = D / kWave;  // channels per lane (1 or 2)
  extern __shared__ int pfx[];    // [npairs + 1]
  __shared__ float qs[8][D];
  __shared__ float ks[BS][D + 1];
  __shared__ float vs[BS][D];
  __shared__ float sc[8][BS];
  __shared__ int wave_tot[1];
  const int lane = threadIdx.x;
  pair_prefix(n_gpu, npairs, list_stride, pfx, wave_tot);
  const PartialView part = partial_view(ws, npairs, W, G, D);
  if (blockIdx.x == 0)
    for (int i = lane; i <= npairs; i += kWave) part.pfx[i] = pfx[i];
  const int T = pfx[npairs];
  const int gw = blockIdx.x;
  if (T == 0) return;
  const int b0 = wave_start(gw, T, W), b1 = wave_start(gw + 1, T, W);
  if (b0 >= b1) return;
  float m_run[8], l_run[8], o[8][CPL];
  auto reset = [&]() {
    for (int g = 0; g < 8; ++g) {
      m_run[g] = -INFINITY;
      l_run[g] = 0.f;
      for (int c = 0; c < CPL; ++c) o[g][c] = 0.f;
    }
  };
  auto finalize = [&](int pair) {
    const size_t slot = (size_t)(gw + pair) * G;
    for (int g = 0; g < G; ++g) {
      for (int c = 0; c < CPL; ++c) part.o[(slot + g) * D + lane + kWave * c] = o[g][c];
      if (lane == 0) {
        part.ml[(slot + g) * 2 + 0] = m_run[g];
        part.ml[(slot + g) * 2 + 1] = l_run[g];
      }
    }
  };
  reset();
  int cur_pair = -1;
  int p = pair_of(pfx, npairs, b0);
  for (int g_blk = b0; g_blk < b1; ++g_blk) {
    while (pfx[p + 1] <= g_blk) ++p;
    if (p != cur_pair) {
      if (cur_pair >= 0) { finalize(cur_pair); reset(); }
      cur_pair = p;
      const int s = p / Hkv, h = p % Hkv;
      __syncthreads();
      const float* qrow = q.base + (size_t)s * q.row_stride + (size_t)h * G * D;
      for (int i = lane; i < G * D; i += kWave) {
        float v = qrow[i];
        for (int part = 1; part < q.parts; ++part) v += qrow[(size_t)part * q.part_stride + i];
        qs[i / D][i % D] = v;
      }
    }
    const int blk = min(max(gpu_blocks[(size_t)p * list_stride + (g_blk - pfx[p])], 0),
                        max_blocks - 1);
    const int page = min(max(table[(size_t)p * max_blocks + blk], 0), P - 1);
    const int nval = min(BS, seq_lens[p / Hkv] - blk * BS);
    __syncthreads();
    for (int i = lane; i < BS * D; i += kWave) {
      // K is chunk-major: element i is channel 4 (i / 4BS) + i % 4 of token (i / 4) % BS;
      // V is [BS/16][D][16]: element i is channel (i / 16) % D of token 16 (i / 16D) + i % 16
      ks[(i / 4) % BS][4 * (i / (4 * BS)) + i % 4] =
          __builtin_nontemporal_load(k_pool + (size_t)page * BS * D + i);
      vs[16 * (i / (16 * D)) + i % 16][(i / 16) % D] =
          __builtin_nontemporal_load(v_pool + (size_t)page * BS * D + i);
    }
    __syncthreads();
    for (int i = lane; i < G * BS; i += kWave) {
      const int g = i / BS, t = i % BS;
      float acc = 0.f;
      for (int c = 0; c < D; ++c) acc = fmaf(qs[g][c], ks[t][c], acc);
      sc[g][t] = t < nval ? acc * scale_log2 : -INFINITY;
    }
    __syncthreads();
    for (int g = 0; g < G; ++g) {
      float mx = -INFINITY;
      for (int t = 0; t < BS; ++t) mx = fmaxf(mx, sc[g][t]);
      const float m_new = fmaxf(m_run[g], mx);           // finite: nval >= 1
      const float alpha = fast_exp2(m_run[g] - m_new);   // 0 on the first block
      float ps = 0.f;
      float acc[CPL];
      for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
      // only the valid tokens: the rest of a partly filled page may hold anything, and a
      // zero weight times a stale NaN or infinity would still poison the sum
      for (int t = 0; t < nval; ++t) {
        const float pr = fast_exp2(sc[g][t] - m_new);
        ps += pr;
        for (int c = 0; c < CPL; ++c) acc[c] = fmaf(pr, vs[t][lane + kWave * c], acc[c]);
      }
      l_run[g] = l_run[g] * alpha + ps;
      for (int c = 0; c < CPL; ++c) o[g][c] = o[g][c] * alpha + acc[c];
      m_run[g] = m_new;
    }
  }
  if (cur_pair >= 0) finalize(cur_pair);
}

// One wave per (sequence, query head) row: combine the partials of the waves that covered
// the pair's blocks and, when given, the host partial; write the normalised output.  The
// loads come in two rounds: first the pair's count and prefix and the host partial, then
// every covering wave's (m, l) (one per lane) together with the o vectors of the first
// kPre of them (a pair usually spans fewer waves); only pairs covered by more waves than
// that read further o vectors one by one.
template <int D>
__global__ __launch_bounds__(256) void reduce_kernel(
    const float* __restrict__ ws, int npairs, int W, int G, int Hkv, int rows, int cap,
    const int32_t* __restrict__ n_gpu, const float* __restrict__ host_o,
    const float* __restrict__ host_m, const float* __restrict__ host_l,
    const int32_t* __restrict__ n_cpu, float* __restrict__ o, float* __restrict__ m,
    float* __restrict__ l) {
  constexpr int CPL = D / kWave;
  constexpr int kPre = 16;
  const int lane = threadIdx.x % kWave;
  const int row = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (row >= rows) return;
  const int Hq = Hkv * G;
  const int s = row / Hq, qh = row % Hq;
  const int pair = s * Hkv + qh / G, g = qh % G;
  const PartialView part = partial_view(const_cast<float*>(ws), npairs, W, G, D);

  // first loads: the pair's block count and prefix, its offloaded count and the host
  // partial's (m, l); the host o vector (possibly over the host link) is read in the second
  // round, and only for a pair with something offloaded
  const int ng = clamp_count(n_gpu[pair], cap);
  const int P = part.pfx[pair];
  const int T = part.pfx[npairs];
  const bool host_ptr = host_o != nullptr;
  float mh = -INFINITY, lh = 0.f;
  float ho[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) ho[i] = 0.f;
  int nc = 1;
  if (host_ptr) {
    mh = host_m[row] * kLog2e;
    lh = host_l[row];
    if (n_cpu) nc = n_cpu[pair];
  }
  // an empty host partial, or one for a pair with nothing offloaded, contributes nothing
  if (!host_ptr || nc <= 0 || !(lh > 0.f)) mh = -INFINITY;
  if (mh != -INFINITY) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) ho[i] = host_o[(size_t)row * D + lane + kWave * i];
  }

  int w_lo = 0, nslot = 0;
  if (ng > 0) {
    w_lo = wave_of(P, T, W);
    nslot = wave_of(P + ng - 1, T, W) - w_lo + 1;
  }
  // a covering wave with an empty range (possible when W > T) wrote no partial
  // (with no more waves than blocks every wave has a block)
  auto slot_live = [&](int j) {
    const int w = w_lo + j;
    return j < nslot && (W <= T || wave_start(w, T, W) < wave_start(w + 1, T, W));
  };
  auto o_of = [&](int j, int i) {  // o of covering wave j (index clamped into the slots)
    const size_t sl = (size_t)(w_lo + j + pair) * G + g;
    return part.o[sl * D + lane + kWave * i];
  };

  // second loads: (m, l) of the covering waves, one per lane, and the first kPre o vectors
  float M = mh, L = 0.f;
  float acc[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) acc[i] = 0.f;
  float ob[kPre][CPL];
#pragma unroll
  for (int j = 0; j < kPre; ++j)
#pragma unroll
    for (int i = 0; i < CPL; ++i) ob[j][i] = o_of(max(0, min(j, nslot - 1)), i);
  for (int j0 = 0; j0 < nslot; j0 += kWave) {
    const bool live = slot_live(j0 + lane);
    float mw = -INFINITY, lw = 0.f;
    if (live) {
      const size_t sl = (size_t)(w_lo + j0 + lane + pair) * G + g;
      mw = part.ml[sl * 2];
      lw = part.ml[sl * 2 + 1];
    }
    float mx = max_xor32(max_xor16(mw));
    mx = fmaxf(mx, dpp<kDppMirror>(mx));
    mx = fmaxf(mx, dpp<kDppHalfMirror>(mx));
    mx = fmaxf(mx, dpp<kDppXor2>(mx));
    mx = fmaxf(mx, dpp<kDppXor1>(mx));
    // rescale what is accumulated so far to the new running maximum
    const float Mn = fmaxf(M, mx);
    if (Mn != -INFINITY) {
      const float r = M == -INFINITY ? 0.f : fast_exp2(M - Mn);
      L *= r;
#pragma unroll
      for (int i = 0; i < CPL; ++i) acc[i] *= r;
      const float wt = mw == -INFINITY ? 0.f : fast_exp2(mw - Mn);
      L += group_sum<kWave>(wt * lw);
      const int cnt = min(kWave, nslot - j0);
      for (int j = 0; j < cnt; ++j) {
        const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt), j));
        if (wj == 0.f) continue;  // (a stale slot may hold anything: skip, do not scale)
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          const float v = j0 + j < kPre ? ob[min(j0 + j, kPre - 1)][i] : o_of(j0 + j, i);
          acc[i] = fmaf(wj, v, acc[i]);
        }
      }
    }
    M = Mn;
  }
  if (mh != -INFINITY) {  // the host partial, at the final maximum
    const float wt = lh * fast_exp2(mh - M);
    L += wt;
#pragma unroll
    for (int i = 0; i < CPL; ++i) acc[i] = fmaf(wt, ho[i], acc[i]);
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) o[(size_t)row * D + lane + kWave * i] = acc[i] * inv;
  if (lane == 0) {
    if (m) m[row] = M == -INFINITY ? -INFINITY : M * kLn2;
    if (l) l[row] = L;
  }
}

// Elementwise merge of two normalised partials, one wave per row.
__global__ __launch_bounds__(256) void merge_kernel(int rows, int d, const float* o_a,
                                                    const float* m_a, const float* l_a,
                                                    const float* o_b, const float* m_b,
                                                    const float* l_b, float* o, float* m,
                                                    float* l) {
  const int lane = threadIdx.x % kWave;
  const int row = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (row >= rows) return;
  const float ma = m_a[row], mb = m_b[row];
  const float la = l_a[row], lb = l_b[row];
  const float M = fmaxf(ma, mb);
  float wa = 0.f, wb = 0.f;
  if (M != -INFINITY) {
    if (ma != -INFINITY) wa = la * expf(ma - M);
    if (mb != -INFINITY) wb = lb * expf(mb - M);
  }
  const float L = wa + wb;
  const float inv = L > 0.f ? 1.f / L : 0.f;
  for (int c = lane; c < d; c += kWave) {
    const size_t i = (size_t)row * d + c;
    o[i] = (wa * o_a[i] + wb * o_b[i]) * inv;
  }
  // all lanes have read m_a / l_a before lane 0 overwrites them (outputs may alias a)
  __builtin_amdgcn_wave_barrier();
  if (lane == 0) {
    m[row] = L > 0.f ? M : -INFINITY;
    l[row] = L;
  }
}

template <int D, int BS>
hipError_t attn_bf16_g(const Shape& s, const AttnPlan& p, const QParts& q, const void* k,
                       const void* v, const int32_t* t, const int32_t* lens,
                       const int32_t* gb, const int32_t* gp, const int32_t* ng, int stride,
                       float sl2,
                       float* ws, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  const int npairs = s.B * s.Hkv;
  const dim3 grid(p.waves / kAttnWaves), block(kAttnWaves * kWave);
  const size_t lds = (size_t)(npairs + 1) * sizeof(int);
  // hipExtLaunchKernelGGL records the (optional) events at the kernel's own start and end
#define SA_ATTN_CASE(GG)                                                                     \
  case GG:                                                                                   \
    hipExtLaunchKernelGGL((attn_bf16_kernel<D, BS, GG>), grid, block, lds, st, e0, e1, 0, q, \
                          (const uint16_t*)k, (const uint16_t*)v, t, lens, gb, gp, ng, stride,\
                          s.Hkv, s.max_blocks, s.P, npairs, p.waves, sl2, ws);               \
    break;
  switch (s.G) {
    SA_ATTN_CASE(1) SA_ATTN_CASE(2) SA_ATTN_CASE(3) SA_ATTN_CASE(4)
    SA_ATTN_CASE(5) SA_ATTN_CASE(6) SA_ATTN_CASE(7) SA_ATTN_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef SA_ATTN_CASE
  return hipGetLastError();
}

template <int D, int BS>
hipError_t attn_f32(const Shape& s, const AttnPlan& p, const QParts& q, const void* k,
                    const void* v, const int32_t* t, const int32_t* lens, const int32_t* gb,
                    const int32_t*, const int32_t* ng, int stride, float sl2, float* ws,
                    hipStream_t st,
                    hipEvent_t e0, hipEvent_t e1) {
  const int npairs = s.B * s.Hkv;
  const size_t lds = (size_t)(npairs + 1) * sizeof(int);
  hipExtLaunchKernelGGL((attn_f32_kernel<D, BS>), dim3(p.waves), dim3(kWave), lds, st, e0, e1,
                        0, q, (const float*)k, (const float*)v, t, lens, gb, ng, stride, s.Hkv,
                        s.G, s.max_blocks, s.P, npairs, p.waves, sl2, ws);
  return hipGetLastError();
}

}  // namespace

AttnPlan attn_plan(const Shape& s, int list_stride) {
  AttnPlan p;
  const int npairs = s.B * s.Hkv;
  const long most = (long)npairs * list_stride;  // upper bound of the resident selected blocks
  // about four of those blocks a wave, at most kMaxWaves waves: with fewer blocks a wave the
  // prologue's dependent loads dominate (a layer of 64 pairs and 3072 resident blocks: 16.4 µs
  // at 1024 waves, 18.5 at 2048, 18.3 at 512)
  const long want = (most + 3) / 4;
  int w = (int)(want < kMaxWaves ? want : kMaxWaves);
  if (s.bf16) w = (w + kAttnWaves - 1) / kAttnWaves * kAttnWaves;
  p.waves = w < 1 ? 1 : w;
  p.list_stride = list_stride;
  p.ws_bytes = prefix_bytes(npairs) +
               (size_t)(p.waves + npairs) * s.G * (s.d + 2) * sizeof(float);
  return p;
}

hipError_t launch_attention(const Shape& s, const AttnPlan& plan, const QParts& q,
                            const void* k_pool, const void* v_pool,
                            const int32_t* block_table, const int32_t* seq_lens,
                            const int32_t* gpu_blocks, const int32_t* gpu_pages,
                            const int32_t* n_gpu, int list_stride, float scale,
                            float* partials, hipStream_t stream, hipEvent_t ev_start,
                            hipEvent_t ev_stop) {
  const float sl2 = scale * kLog2e;
#define SA_ARGS plan, q, k_pool, v_pool, block_table, seq_lens, gpu_blocks, gpu_pages, n_gpu, \
                list_stride, sl2, partials, stream, ev_start, ev_stop
#define SA_BY_BS(FN, D)                                   \
  (s.bs == 64   ? FN<D, 64>(s, SA_ARGS)                    \
   : s.bs == 32 ? FN<D, 32>(s, SA_ARGS)                    \
                : FN<D, 16>(s, SA_ARGS))
  if (s.bf16) return s.d == 128 ? SA_BY_BS(attn_bf16_g, 128) : SA_BY_BS(attn_bf16_g, 64);
  return s.d == 128 ? SA_BY_BS(attn_f32, 128) : SA_BY_BS(attn_f32, 64);
#undef SA_BY_BS
#undef SA_ARGS
}

hipError_t launch_reduce(const Shape& s, const AttnPlan& plan, const int32_t* n_gpu,
                         const float* partials, const float* host_o, const float* host_m,
                         const float* host_l, const int32_t* n_cpu, float* o, float* m,
                         float* l, hipStream_t stream) {
  const int rows = s.B * s.Hq;
  const int npairs = s.B * s.Hkv;
  const dim3 grid((rows + 3) / 4), block(256);
  if (s.d == 128)
    hipLaunchKernelGGL(reduce_kernel<128>, grid, block, 0, stream, partials, npairs,
                       plan.waves, s.G, s.Hkv, rows, plan.list_stride, n_gpu, host_o, host_m,
                       host_l, n_cpu, o, m, l);
  else
    hipLaunchKernelGGL(reduce_kernel<64>, grid, block, 0, stream, partials, npairs, plan.waves,
                       s.G, s.Hkv, rows, plan.list_stride, n_gpu, host_o, host_m, host_l, n_cpu,
                       o, m, l);
  return hipGetLastError();
}

hipError_t launch_merge(int rows, int d, const float* o_a, const float* m_a, const float* l_a,
                        const float* o_b, const float* m_b, const float* l_b, float* o,
                        float* m, float* l, hipStream_t stream) {
  hipLaunchKernelGGL(merge_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream, rows, d, o_a,
                     m_a, l_a, o_b, m_b, l_b, o, m, l);
  return hipGetLastError();
}

}  // namespace sa
