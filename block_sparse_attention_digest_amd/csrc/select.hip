// Block selection of ScoutAttention [arXiv:2603.27138, HTML Sec. 2.2 and 3.2; Algorithm 1]:
//   B_pred = TopK(Q K_digest^T) per (sequence, KV head), then B_cpu = B_pred \ B_gpu.
//
// score_kernel: every block's score against the digests.  The G query heads of a KV head
//   are folded into per-channel coefficients first -- the group sum sum_g q_g for mean
//   digests, and for min/max digests
//     sum_g max(q_gc min_c, q_gc max_c) = (sum_g max(q_gc, 0)) max_c + (sum_g min(q_gc, 0)) min_c
//   (exact, since max_c >= min_c) -- so each digest element costs one or two FMAs.  A digest
//   row is read by 16-byte loads across LPR lanes and reduced across them with shuffles;
//   every load of a wave (8-16 KiB) is issued before the first is used.  HBM-bound: every
//   digest byte is read once.
// topk_split_kernel: one workgroup per (sequence, KV head).  A histogram of the score values
//   over 256 equal-width buckets locates the bucket holding the k-th largest score; the few
//   scores in that bucket are ranked exactly by (score, lower index first).  Crowded
//   buckets (e.g. all scores equal) fall back to an exact MSB-first radix select on
//   order-preserving 32-bit keys.  The selected blocks are compacted in ascending order and
//   split by the block table into the resident and offloaded lists.
#include "common.hpp"
#include "kernels.hpp"

namespace sa {
namespace {

constexpr int kScoreWaves = 4;

// digest rows per load instruction, loads in flight per lane, blocks per workgroup
template <typename T, int D, bool MINMAX>
struct ScoreShape;
template <typename T>
struct Digest;
template <>
struct Digest<uint16_t> {  // eight bf16 per 16-byte vector
  static constexpr int N = 8;
  __device__ static uint4 load(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
  __device__ static void widen(const uint4& v, float* f) { bf16x8_to_f32(v, f); }
};
template <>
struct Digest<float> {  // four float per 16-byte vector
  static constexpr int N = 4;
  __device__ static uint4 load(const float* p) { return *reinterpret_cast<const uint4*>(p); }
  __device__ static void widen(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
};

template <typename T, int D, bool MINMAX>
struct ScoreShape {
  static constexpr int VEC = Digest<T>::N;
  static constexpr int LPR = D / VEC;       // lanes per digest row
  static constexpr int BPI = kWave / LPR;   // blocks per load instruction
  static constexpr int U = MINMAX ? 8 : 16; // block loads in flight per lane
  static constexpr int BPW = kScoreWaves * U * BPI;  // blocks per workgroup
};

template <typename T, int D, bool MINMAX>
__global__ __launch_bounds__(256) void score_kernel(const float* __restrict__ q,
                                                    const T* __restrict__ dig,
                                                    const int32_t* __restrict__ seq_lens,
                                                    float* __restrict__ scores, int Hkv, int G,
                                                    int bs, int max_blocks) {
  using S = ScoreShape<T, D, MINMAX>;
  constexpr int VEC = S::VEC, LPR = S::LPR, BPI = S::BPI, U = S::U;
  constexpr int ROW = MINMAX ? 2 * D : D;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int pair = blockIdx.y;
  const int s = pair / Hkv, h = pair % Hkv;
  const int nb = (seq_lens[s] + bs - 1) / bs;
  const int wg_b0 = blockIdx.x * S::BPW;
  if (wg_b0 >= nb) return;
  const int cg = lane % LPR, bi = lane / LPR;

  // block indices of this lane's loads; all of them are issued before any is used
  int bidx[U];
  uint4 raw[U][MINMAX ? 2 : 1];
  const T* base = dig + (size_t)pair * max_blocks * ROW + cg * VEC;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int b = wg_b0 + (u * kScoreWaves + wave) * BPI + bi;
    bidx[u] = b;
    if (b < nb) {
      raw[u][0] = Digest<T>::load(base + (size_t)b * ROW);
      if (MINMAX) raw[u][MINMAX ? 1 : 0] = Digest<T>::load(base + (size_t)b * ROW + D);
    }
  }

  // per-channel coefficients of this lane's VEC channels
  float ca[VEC], cb[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) { ca[i] = 0.f; cb[i] = 0.f; }
  const float* qg = q + ((size_t)s * Hkv * G + (size_t)h * G) * D + cg * VEC;
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      const float v = qg[(size_t)g * D + i];
      if (MINMAX) { ca[i] += fmaxf(v, 0.f); cb[i] += fminf(v, 0.f); }
      else ca[i] += v;
    }
  }

  float* out = scores + (size_t)pair * max_blocks;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float acc = 0.f;
    if (bidx[u] < nb) {
      float lo_or_mean[VEC];
      Digest<T>::widen(raw[u][0], lo_or_mean);
      if (MINMAX) {  // digest row 0 = min, row 1 = max
        float hi[VEC];
        Digest<T>::widen(raw[u][MINMAX ? 1 : 0], hi);
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc = fmaf(ca[i], hi[i], acc);
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc = fmaf(cb[i], lo_or_mean[i], acc);
      } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc = fmaf(ca[i], lo_or_mean[i], acc);
      }
    }
    acc = group_sum<LPR>(acc);
    if (cg == 0 && bidx[u] < nb) out[bidx[u]] = acc;
  }
}

// Inclusive prefix sum over the 256 threads of a workgroup.
__device__ __forceinline__ uint32_t block_scan_incl(uint32_t v, uint32_t* tmp) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  if (lane == kWave - 1) tmp[wave] = v;
  __syncthreads();
  uint32_t add = 0;
  for (int w = 0; w < wave; ++w) add += tmp[w];
  __syncthreads();
  return v + add;
}

constexpr int kMaxCand = 256;  // boundary-bucket candidates ranked directly
constexpr uint8_t kSelected = 1, kResident = 2;  // per-block flag bits

__global__ __launch_bounds__(256) void topk_split_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens, int bs,
    int max_blocks, int Hkv, int top_k, const int32_t* __restrict__ table,
    int32_t* __restrict__ gpu_blocks, int32_t* __restrict__ n_gpu,
    int32_t* __restrict__ cpu_blocks, int32_t* __restrict__ n_cpu) {
  extern __shared__ uint32_t smem[];
  uint32_t* keys = smem;                                          // [max_blocks]
  uint8_t* flag = reinterpret_cast<uint8_t*>(smem + max_blocks);  // [max_blocks]
  __shared__ uint32_t hist[256];
  __shared__ uint32_t tmp[4];
  __shared__ float red_lo[4], red_hi[4];
  __shared__ uint32_t cand_key[kMaxCand];
  __shared__ int cand_idx[kMaxCand];
  __shared__ uint32_t sel_digit, sel_remaining, sel_count, ncand, tot_res, tot_off;

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int pair = blockIdx.x;
  const int s = pair / Hkv;
  const int nb = (seq_lens[s] + bs - 1) / bs;
  const uint32_t ks = (uint32_t)min(top_k, nb);
  const float* sc = scores + (size_t)pair * max_blocks;

  // keys and residency bits in LDS (scores and block table read together, coalesced), and
  // the range of the scores
  const int32_t* trow = table + (size_t)pair * max_blocks;
  float lo = INFINITY, hi = -INFINITY;
#pragma unroll 8
  for (int i = tid; i < nb; i += 256) {
    const float v = sc[i];
    const int32_t page = trow[i];
    keys[i] = order_key(v);
    flag[i] = page >= 0 ? kResident : 0;
    lo = fminf(lo, v);
    hi = fmaxf(hi, v);
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, o, kWave));
    hi = fmaxf(hi, __shfl_xor(hi, o, kWave));
  }
  if (lane == 0) { red_lo[wave] = lo; red_hi[wave] = hi; }
  hist[tid] = 0;
  if (tid == 0) ncand = 0;
  __syncthreads();
  lo = fminf(fminf(red_lo[0], red_lo[1]), fminf(red_lo[2], red_lo[3]));
  hi = fmaxf(fmaxf(red_hi[0], red_hi[1]), fmaxf(red_hi[2], red_hi[3]));
  const float span = hi - lo;
  const bool bucketed = span > 0.f && span < INFINITY;
  const float to_bucket = bucketed ? 256.f / span : 0.f;

  // Fast path: a histogram of the score VALUE over 256 equal-width buckets.  The map
  // v -> (v - lo) * 256 / span is monotone, so every block of a higher bucket outscores
  // every block of a lower one; the k-th largest lies in the bucket B found by a suffix
  // count, and only B's few members need an exact (score, index) ranking.
  uint32_t B = 0, r = 0, cnt = 0xffffffffu;
  if (bucketed) {
    for (int i = tid; i < nb; i += 256) {
      const int b = min(255, (int)((sc[i] - lo) * to_bucket));
      atomicAdd(&hist[b], 1u);
    }
    __syncthreads();
    const uint32_t c = hist[255 - tid];
    const uint32_t cge = block_scan_incl(c, tmp);
    const uint32_t cgt = cge - c;
    if (cgt < ks && cge >= ks) {
      sel_digit = 255u - (uint32_t)tid;
      sel_remaining = ks - cgt;
      sel_count = c;
    }
    __syncthreads();
    B = sel_digit;
    r = sel_remaining;
    cnt = sel_count;
  }
  if (cnt <= (uint32_t)kMaxCand) {
    for (int i = tid; i < nb; i += 256) {
      const uint32_t b = (uint32_t)min(255, (int)((sc[i] - lo) * to_bucket));
      if (b > B) flag[i] |= kSelected;
      if (b == B) {
        const uint32_t pos = atomicAdd(&ncand, 1u);
        cand_key[pos] = keys[i];
        cand_idx[pos] = i;
      }
    }
    __syncthreads();
    for (uint32_t c = tid; c < cnt; c += 256) {
      const uint32_t key = cand_key[c];
      const int idx = cand_idx[c];
      uint32_t rank = 0;
      for (uint32_t j = 0; j < cnt; ++j) {
        const uint32_t kj = cand_key[j];
        rank += kj > key || (kj == key && cand_idx[j] < idx);
      }
      if (rank < r) flag[idx] |= kSelected;
    }
    __syncthreads();
  } else {
    // General path (all scores equal, or a crowded bucket): exact radix select of the
    // ks-th largest key, 8 bits per pass from the top.
    uint32_t prefix = 0, mask = 0, remaining = ks;
    for (int shift = 24; shift >= 0; shift -= 8) {
      hist[tid] = 0;
      __syncthreads();
      for (int i = tid; i < nb; i += 256) {
        const uint32_t kv = keys[i];
        if ((kv & mask) == prefix) atomicAdd(&hist[(kv >> shift) & 255u], 1u);
      }
      __syncthreads();
      const uint32_t c = hist[255 - tid];
      const uint32_t cge = block_scan_incl(c, tmp);
      const uint32_t cgt = cge - c;
      if (cgt < remaining && cge >= remaining) {
        sel_digit = 255u - (uint32_t)tid;
        sel_remaining = remaining - cgt;
      }
      __syncthreads();
      prefix |= sel_digit << shift;
      mask |= 255u << shift;
      remaining = sel_remaining;
      __syncthreads();
    }
    const uint32_t thr = prefix;         // the ks-th largest key
    const uint32_t take_eq = remaining;  // keys equal to thr that are selected
    const int per = (nb + 255) / 256;
    const int i0 = min(nb, tid * per), i1 = min(nb, i0 + per);
    uint32_t ties = 0;
    for (int i = i0; i < i1; ++i) ties += keys[i] == thr;
    const uint32_t tie_base = block_scan_incl(ties, tmp) - ties;
    uint32_t seen = 0;
    for (int i = i0; i < i1; ++i) {
      const uint32_t kv = keys[i];
      bool sel = kv > thr;
      if (kv == thr) { sel = tie_base + seen < take_eq; ++seen; }
      if (sel) flag[i] |= kSelected;
    }
    __syncthreads();
  }

  // ascending compaction of the selected blocks, split by residency
  const int per = (nb + 255) / 256;
  const int i0 = min(nb, tid * per), i1 = min(nb, i0 + per);
  uint32_t cnt_res = 0, cnt_off = 0;
  for (int i = i0; i < i1; ++i) {
    const uint8_t f = flag[i];
    cnt_res += f == (kSelected | kResident);
    cnt_off += f == kSelected;
  }
  const uint32_t packed = cnt_res | (cnt_off << 16);
  const uint32_t incl = block_scan_incl(packed, tmp);
  uint32_t pos_res = (incl - packed) & 0xffffu, pos_off = (incl - packed) >> 16;
  if (tid == 255) { tot_res = incl & 0xffffu; tot_off = incl >> 16; }
  int32_t* grow = gpu_blocks + (size_t)pair * top_k;
  int32_t* crow = cpu_blocks + (size_t)pair * top_k;
  for (int i = i0; i < i1; ++i) {
    const uint8_t f = flag[i];
    if (f == (kSelected | kResident)) grow[pos_res++] = i;
    else if (f == kSelected) crow[pos_off++] = i;
  }
  __syncthreads();
  const int nr = (int)tot_res, no = (int)tot_off;
  for (int j = nr + tid; j < top_k; j += 256) grow[j] = -1;
  for (int j = no + tid; j < top_k; j += 256) crow[j] = -1;
  if (tid == 0) { n_gpu[pair] = nr; n_cpu[pair] = no; }
}

template <typename T, int D>
hipError_t score_typed(const Shape& s, bool minmax, const float* q, const void* dig,
                       const int32_t* lens, float* scores, hipStream_t st) {
  const int bpw_mean = ScoreShape<T, D, false>::BPW, bpw_mm = ScoreShape<T, D, true>::BPW;
  const int bpw = minmax ? bpw_mm : bpw_mean;
  const dim3 grid((s.max_blocks + bpw - 1) / bpw, s.B * s.Hkv);
  if (minmax)
    hipLaunchKernelGGL((score_kernel<T, D, true>), grid, dim3(256), 0, st, q, (const T*)dig,
                       lens, scores, s.Hkv, s.G, s.bs, s.max_blocks);
  else
    hipLaunchKernelGGL((score_kernel<T, D, false>), grid, dim3(256), 0, st, q, (const T*)dig,
                       lens, scores, s.Hkv, s.G, s.bs, s.max_blocks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score(const Shape& s, bool minmax, const float* q, const void* digests,
                        const int32_t* seq_lens, float* scores, hipStream_t stream) {
  if (s.bf16)
    return s.d == 128 ? score_typed<uint16_t, 128>(s, minmax, q, digests, seq_lens, scores, stream)
                      : score_typed<uint16_t, 64>(s, minmax, q, digests, seq_lens, scores, stream);
  return s.d == 128 ? score_typed<float, 128>(s, minmax, q, digests, seq_lens, scores, stream)
                    : score_typed<float, 64>(s, minmax, q, digests, seq_lens, scores, stream);
}

hipError_t launch_topk_split(const Shape& s, const float* scores, const int32_t* seq_lens,
                             int top_k, const int32_t* block_table, int32_t* gpu_blocks,
                             int32_t* n_gpu, int32_t* cpu_blocks, int32_t* n_cpu,
                             hipStream_t stream) {
  const size_t lds = (size_t)s.max_blocks * 5;  // keys (4 B) + flags (1 B)
  hipLaunchKernelGGL(topk_split_kernel, dim3(s.B * s.Hkv), dim3(256), lds, stream, scores,
                     seq_lens, s.bs, s.max_blocks, s.Hkv, top_k, block_table, gpu_blocks,
                     n_gpu, cpu_blocks, n_cpu);
  return hipGetLastError();
}

}  // namespace sa
