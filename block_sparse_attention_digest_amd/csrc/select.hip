// Block selection of ScoutAttention [arXiv:2603.27138, HTML Sec. 2.2 and 3.2; Algorithm 1]:
//   B_pred = TopK(Q K_digest^T) per (sequence, KV head), then B_cpu = B_pred \ B_gpu.
//
// score_kernel: every block's score against the digests.  The G query heads of a KV head
//   are folded into per-channel coefficients first -- the group sum sum_g q_g for mean
//   digests, and for min/max digests
//     sum_g max(q_gc min_c, q_gc max_c) = (sum_g max(q_gc, 0)) max_c + (sum_g min(q_gc, 0)) min_c
//   (exact, since max_c >= min_c) -- so each digest element costs one or two FMAs.  A digest
//   row is read by 16-byte loads across LPR lanes and reduced across them with shuffles;
//   four loads per lane are in flight.  HBM-bound: every digest byte is read once.
// topk_split_kernel: one workgroup per (sequence, KV head).  The scores become
//   order-preserving 32-bit keys in LDS; an MSB-first radix select (4 passes of 8 bits)
//   finds the exact k-th largest key; selected blocks (ties at the threshold taken in index
//   order) are compacted in ascending order and split by the block table into the resident
//   and offloaded lists.
#include "common.hpp"
#include "kernels.hpp"

namespace sa {
namespace {

constexpr int kScoreUnroll = 4;
constexpr int kBlocksPerWG = 256;

template <typename T>
struct Digest;
template <>
struct Digest<uint16_t> {
  static constexpr int N = 8;
  __device__ static void load(const uint16_t* p, float* f) {
    bf16x8_to_f32(*reinterpret_cast<const uint4*>(p), f);
  }
};
template <>
struct Digest<float> {
  static constexpr int N = 4;
  __device__ static void load(const float* p, float* f) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
  }
};

template <typename T, int D, bool MINMAX>
__global__ __launch_bounds__(256) void score_kernel(const float* __restrict__ q,
                                                    const T* __restrict__ dig,
                                                    const int32_t* __restrict__ seq_lens,
                                                    float* __restrict__ scores, int Hkv, int G,
                                                    int bs, int max_blocks) {
  constexpr int VEC = Digest<T>::N;
  constexpr int LPR = D / VEC;       // lanes per digest row
  constexpr int BPI = kWave / LPR;   // blocks per load instruction
  constexpr int ROW = MINMAX ? 2 * D : D;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int pair = blockIdx.y;
  const int s = pair / Hkv, h = pair % Hkv;
  const int nb = (seq_lens[s] + bs - 1) / bs;
  const int wg_b0 = blockIdx.x * kBlocksPerWG;
  if (wg_b0 >= nb) return;
  const int cg = lane % LPR, bi = lane / LPR;

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

  const T* base = dig + (size_t)pair * max_blocks * ROW + cg * VEC;
  float* out = scores + (size_t)pair * max_blocks;
  constexpr int kWaves = 4;
  constexpr int kPerIter = kWaves * kScoreUnroll * BPI;
  for (int it0 = wg_b0; it0 < min(nb, wg_b0 + kBlocksPerWG); it0 += kPerIter) {
    float vals[kScoreUnroll][MINMAX ? 2 : 1][VEC];
    int bidx[kScoreUnroll];
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      const int b = it0 + (u * kWaves + wave) * BPI + bi;
      bidx[u] = b;
      if (b < nb) {
        Digest<T>::load(base + (size_t)b * ROW, vals[u][0]);
        if (MINMAX) Digest<T>::load(base + (size_t)b * ROW + D, vals[u][MINMAX ? 1 : 0]);
      }
    }
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      float acc = 0.f;
      if (bidx[u] < nb) {
        if (MINMAX) {
#pragma unroll
          for (int i = 0; i < VEC; ++i) acc = fmaf(ca[i], vals[u][MINMAX ? 1 : 0][i], acc);
#pragma unroll
          for (int i = 0; i < VEC; ++i) acc = fmaf(cb[i], vals[u][0][i], acc);
        } else {
#pragma unroll
          for (int i = 0; i < VEC; ++i) acc = fmaf(ca[i], vals[u][0][i], acc);
        }
      }
      acc = group_sum<LPR>(acc);
      if (cg == 0 && bidx[u] < nb) out[bidx[u]] = acc;
    }
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

__global__ __launch_bounds__(256) void topk_split_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens, int bs,
    int max_blocks, int Hkv, int top_k, const int32_t* __restrict__ table,
    int32_t* __restrict__ gpu_blocks, int32_t* __restrict__ n_gpu,
    int32_t* __restrict__ cpu_blocks, int32_t* __restrict__ n_cpu) {
  extern __shared__ uint32_t smem[];
  uint32_t* keys = smem;                                    // [max_blocks]
  uint8_t* flag = reinterpret_cast<uint8_t*>(smem + max_blocks);  // [max_blocks]
  __shared__ uint32_t hist[256];
  __shared__ uint32_t tmp[4];
  __shared__ uint32_t sel_digit, sel_remaining, tot_res, tot_off;

  const int tid = threadIdx.x;
  const int pair = blockIdx.x;
  const int s = pair / Hkv;
  const int nb = (seq_lens[s] + bs - 1) / bs;
  const int ks = min(top_k, nb);
  const float* sc = scores + (size_t)pair * max_blocks;
  for (int i = tid; i < nb; i += 256) keys[i] = order_key(sc[i]);

  // radix select of the ks-th largest key
  uint32_t prefix = 0, mask = 0, remaining = (uint32_t)ks;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < nb; i += 256) {
      const uint32_t kv = keys[i];
      if ((kv & mask) == prefix) atomicAdd(&hist[(kv >> shift) & 255u], 1u);
    }
    __syncthreads();
    const uint32_t c = hist[255 - tid];           // thread 0 holds the highest digit
    const uint32_t cge = block_scan_incl(c, tmp);  // keys with digit >= 255 - tid
    const uint32_t cgt = cge - c;                  // keys with digit >  255 - tid
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
  const uint32_t thr = prefix;   // the ks-th largest key
  const uint32_t take_eq = remaining;  // how many keys equal to thr are selected

  // contiguous index range of this thread
  const int per = (nb + 255) / 256;
  const int i0 = min(nb, tid * per), i1 = min(nb, i0 + per);
  uint32_t ties = 0;
  for (int i = i0; i < i1; ++i) ties += keys[i] == thr;
  const uint32_t tie_base = block_scan_incl(ties, tmp) - ties;
  uint32_t seen = 0, cnt_res = 0, cnt_off = 0;
  const int32_t* trow = table + (size_t)pair * max_blocks;
  for (int i = i0; i < i1; ++i) {
    const uint32_t kv = keys[i];
    bool sel = kv > thr;
    if (kv == thr) { sel = tie_base + seen < take_eq; ++seen; }
    uint8_t f = 0;
    if (sel) {
      if (trow[i] >= 0) { f = 1; ++cnt_res; } else { f = 2; ++cnt_off; }
    }
    flag[i] = f;
  }
  const uint32_t packed = cnt_res | (cnt_off << 16);
  const uint32_t incl = block_scan_incl(packed, tmp);
  uint32_t pos_res = (incl - packed) & 0xffffu, pos_off = (incl - packed) >> 16;
  if (tid == 255) { tot_res = incl & 0xffffu; tot_off = incl >> 16; }
  int32_t* grow = gpu_blocks + (size_t)pair * top_k;
  int32_t* crow = cpu_blocks + (size_t)pair * top_k;
  for (int i = i0; i < i1; ++i) {
    const uint8_t f = flag[i];
    if (f == 1) grow[pos_res++] = i;
    else if (f == 2) crow[pos_off++] = i;
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
  const dim3 grid((s.max_blocks + kBlocksPerWG - 1) / kBlocksPerWG, s.B * s.Hkv);
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
