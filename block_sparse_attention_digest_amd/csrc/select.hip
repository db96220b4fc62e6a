// Block selection of ScoutAttention [arXiv:2603.27138, HTML Sec. 2.2 and 3.2; Algorithm 1]:
//   B_pred = TopK(Q K_digest^T) per (sequence, KV head), then B_cpu = B_pred \ B_gpu.
//
// One workgroup of 8 waves per (sequence, KV head) does the whole selection:
//   1. scoring: the G query heads of the KV head are folded into per-channel coefficients
//      -- the group sum sum_g q_g for mean digests, and for min/max digests
//        sum_g max(q_gc min_c, q_gc max_c) = (sum_g max(q_gc, 0)) max_c + (sum_g min(q_gc, 0)) min_c
//      (exact, since max_c >= min_c) -- so a digest element costs one or two FMAs.  The
//      query rows (all their parts), the first digest batch and the pair's block-table
//      entries are requested together in one round: the workgroup sums the query parts into
//      LDS and each lane reads its coefficients from there behind an LDS-only barrier, while
//      the digests are already in flight.  Each wave streams a contiguous share of the
//      pair's digest rows with 16-byte loads, the next batch of 8 loads in flight while the
//      current one is reduced (DPP row sums; loads are unconditional so the waits cover one
//      batch); the scores stay in LDS.  Every pair's workgroup is resident at once, so HBM
//      bandwidth is shared evenly and the whole digest set streams in one pass.
//   2. top-k: a histogram of the score values over 256 equal-width buckets locates the
//      bucket holding the k-th largest score; the few scores in that bucket are ranked
//      exactly by (score, lower index first).  Crowded buckets (e.g. all scores equal) fall
//      back to an exact MSB-first radix select on order-preserving 32-bit keys.
//   3. split: the selected blocks are compacted in ascending order and split by the block
//      table (read during step 1) into the resident and offloaded lists; the offloaded list
//      can also be written straight into a host mirror (the hand-off of Algorithm 1), and
//      the pages of the resident list next to it (so attention skips the table lookup).
#include "common.hpp"
#include "kernels.hpp"

namespace sa {
namespace {

constexpr int kSelWaves = 8;
constexpr int kSelThreads = kSelWaves * kWave;
constexpr int kBatch = 8;        // 16-byte loads per lane per batch
constexpr int kMaxCand = 256;    // boundary-bucket candidates ranked directly
constexpr int kSelPartGroup = 4; // query parts loaded together
constexpr int kTblRun = 8;       // block-table entries a thread holds in registers
constexpr int kMaxGroup = 8;     // query heads per KV head
constexpr uint8_t kSelected = 1, kResident = 2;  // per-block flag bits

template <typename T>
struct Digest;
template <>
struct Digest<uint16_t> {  // eight bf16 per 16-byte vector
  static constexpr int N = 8;
  __device__ static void widen(const uint4& v, float* f) { bf16x8_to_f32(v, f); }
};
template <>
struct Digest<float> {  // four float per 16-byte vector
  static constexpr int N = 4;
  __device__ static void widen(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
};

// Inclusive prefix sum over all threads of the workgroup.
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

// The bucket (0..255) of score v when [lo, hi] is split into 256 equal-width buckets.  The
// map is monotone in v, so a higher bucket means a strictly larger score.
__device__ __forceinline__ int bucket_of(float v, float lo, float to_bucket) {
  return min(255, (int)((v - lo) * to_bucket));
}

__device__ __forceinline__ float wave_min(float v) {
  v = fminf(v, dpp<kDppMirror>(v));
  v = fminf(v, dpp<kDppHalfMirror>(v));
  v = fminf(v, dpp<kDppXor2>(v));
  v = fminf(v, dpp<kDppXor1>(v));
  auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fminf(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
  auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fminf(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<kDppMirror>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppXor1>(v));
  return max_xor32(max_xor16(v));
}

template <typename T, int D, bool MINMAX>
__global__ __launch_bounds__(kSelThreads, 2) void select_kernel(
    const QParts q, const T* __restrict__ dig, const int32_t* __restrict__ seq_lens,
    int Hkv, int G, int bs, int max_blocks, int top_k, const int32_t* __restrict__ table,
    int32_t* __restrict__ gpu_blocks, int32_t* __restrict__ n_gpu,
    int32_t* __restrict__ cpu_blocks, int32_t* __restrict__ n_cpu,
    float* __restrict__ scores_out, int32_t* __restrict__ cpu_blocks_host,
    int32_t* __restrict__ n_cpu_host, int32_t* __restrict__ gpu_pages) {
  constexpr int VEC = Digest<T>::N;
  constexpr int LPR = D / VEC;             // lanes per digest row
  constexpr int BPI = kWave / LPR;         // blocks per load instruction
  constexpr int LPB = MINMAX ? 2 : 1;      // loads per block row
  constexpr int BPB = kBatch / LPB * BPI;  // blocks per batch (per wave)
  constexpr int ROW = LPB * D;

  extern __shared__ float sc[];                                 // [max_blocks] scores
  uint8_t* flag = reinterpret_cast<uint8_t*>(sc + max_blocks);  // [max_blocks]
  // [max_blocks] block-table entries, kept only when the pages are written out
  int32_t* pg = reinterpret_cast<int32_t*>(sc + max_blocks + (max_blocks + 3) / 4);
  __shared__ uint32_t hist[256];
  __shared__ uint32_t tmp[kSelWaves];
  __shared__ float red_lo[kSelWaves], red_hi[kSelWaves];
  __shared__ uint32_t cand_key[kMaxCand];
  __shared__ int cand_idx[kMaxCand];
  __shared__ uint32_t sel_digit, sel_remaining, sel_count, ncand, tot_res, tot_off;
  __shared__ float4 q_sum[kMaxGroup * D / 4];  // the pair's G query rows, parts summed

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // scalar loop bounds
  const int pair = blockIdx.x;
  const int s = pair / Hkv, h = pair % Hkv;

  // The pair's query rows come first, in one round: thread t loads float4 t of the G rows
  // (G D / 4 <= kSelThreads), its first kSelPartGroup parts at once (indexes clamped, so every
  // thread issues the same loads).
  constexpr int kQ4 = D / 4;
  const bool q_own = tid < G * kQ4;
  const float* qsrc = q.base + (size_t)s * q.row_stride + (size_t)h * G * D +
                      4 * (size_t)(q_own ? tid : 0);
  float4 qp[kSelPartGroup];
#pragma unroll
  for (int u = 0; u < kSelPartGroup; ++u)
    qp[u] = *reinterpret_cast<const float4*>(qsrc + (size_t)min(u, q.parts - 1) * q.part_stride);
  __builtin_amdgcn_sched_barrier(0);  // issued ahead of the digest and table loads
  // blocks of the sequence, clamped to the table's span (a bad length cannot move a read
  // past the pair's rows)
  const int nb = min(max((seq_lens[s] + bs - 1) / bs, 0), max_blocks);
  const uint32_t ks = (uint32_t)min(top_k, nb);
  const int cg = lane % LPR, bi = lane / LPR;

  // this wave's contiguous share of the pair's blocks
  const int per_wave = (nb + kSelWaves - 1) / kSelWaves;
  const int wb0 = min(nb, wave * per_wave), wb1 = min(nb, wb0 + per_wave);
  const T* base = dig + (size_t)pair * max_blocks * ROW + cg * VEC;
  uint4 bufa[kBatch], bufb[kBatch];
  // Loads are issued unconditionally (rows past the range clamped to its last row, their
  // scores discarded), so the waits before a batch cover that batch only.
  auto load_batch = [&](int b_first, uint4* buf) {
#pragma unroll
    for (int u = 0; u < kBatch / LPB; ++u) {
      const int b = max(min(b_first + u * BPI + bi, wb1 - 1), 0);
#pragma unroll
      for (int r = 0; r < LPB; ++r)
        buf[u * LPB + r] = *reinterpret_cast<const uint4*>(base + (size_t)b * ROW + r * D);
    }
  };
  load_batch(wb0, bufa);  // (a wave with no rows re-reads a valid one, unused)

  // residency of every block: the block table is read while the digests stream, into
  // registers (kTblRun entries per thread) that are only consumed after the scoring
  const int32_t* trow = table + (size_t)pair * max_blocks;
  const bool tbl_regs = nb > 0 && nb <= kTblRun * kSelThreads;  // (uniform)
  int32_t tbl[kTblRun];  // (loads unconditional, indexes clamped to a valid entry)
#pragma unroll
  for (int u = 0; u < kTblRun; ++u) tbl[u] = trow[max(min(tid + u * kSelThreads, nb - 1), 0)];
  if (tid < 256) hist[tid] = 0;
  if (tid == 0) ncand = 0;

  // each query element is the sum of its parts, taken in part order
  {
    float4 v = qp[0];
    auto add = [&](const float4& w, bool use) {
      v.x = use ? v.x + w.x : v.x; v.y = use ? v.y + w.y : v.y;
      v.z = use ? v.z + w.z : v.z; v.w = use ? v.w + w.w : v.w;
    };
#pragma unroll
    for (int u = 1; u < kSelPartGroup; ++u) add(qp[u], u < q.parts);
    for (int p0 = kSelPartGroup; p0 < q.parts; p0 += kSelPartGroup) {  // more parts (rare)
#pragma unroll
      for (int u = 0; u < kSelPartGroup; ++u)
        qp[u] = *reinterpret_cast<const float4*>(qsrc + (size_t)min(p0 + u, q.parts - 1) *
                                                            q.part_stride);
#pragma unroll
      for (int u = 0; u < kSelPartGroup; ++u) add(qp[u], p0 + u < q.parts);
    }
    if (q_own) q_sum[tid] = v;
  }
  lds_barrier();  // the summed rows are visible; the digest loads stay in flight

  // per-channel coefficients of this lane's VEC channels, summed over the heads in order
  float ca[VEC], cb[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) { ca[i] = 0.f; cb[i] = 0.f; }
  for (int g = 0; g < G; ++g) {
    float v[VEC];
#pragma unroll
    for (int i = 0; i < VEC; i += 4)
      *reinterpret_cast<float4*>(v + i) = q_sum[g * kQ4 + (cg * VEC + i) / 4];
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      if (MINMAX) { ca[i] += fmaxf(v[i], 0.f); cb[i] += fminf(v[i], 0.f); }
      else ca[i] += v[i];
    }
  }

  float lo = INFINITY, hi = -INFINITY;
  auto score_batch = [&](int b_first, const uint4* buf) {
#pragma unroll
    for (int u = 0; u < kBatch / LPB; ++u) {
      const int b = b_first + u * BPI + bi;
      float acc = 0.f;
      {
        float x[VEC];
        Digest<T>::widen(buf[u * LPB], x);
        if (MINMAX) {  // digest row 0 = min, row 1 = max
          float y[VEC];
          Digest<T>::widen(buf[u * LPB + (MINMAX ? 1 : 0)], y);
#pragma unroll
          for (int i = 0; i < VEC; ++i) acc = fmaf(ca[i], y[i], acc);
#pragma unroll
          for (int i = 0; i < VEC; ++i) acc = fmaf(cb[i], x[i], acc);
        } else {
#pragma unroll
          for (int i = 0; i < VEC; ++i) acc = fmaf(ca[i], x[i], acc);
        }
      }
      acc = group_sum<LPR>(acc);
      if (b < wb1) {
        lo = fminf(lo, acc);
        hi = fmaxf(hi, acc);
        if (cg == 0) {
          sc[b] = acc;
          if (scores_out) scores_out[(size_t)pair * max_blocks + b] = acc;
        }
      }
    }
  };
  // the scheduling barriers keep the compiler from sinking a batch's loads to their use
  for (int b = wb0; b < wb1; b += 2 * BPB) {
    load_batch(min(b + BPB, wb1 - 1), bufb);
    __builtin_amdgcn_sched_barrier(0);
    score_batch(b, bufa);
    load_batch(min(b + 2 * BPB, wb1 - 1), bufa);
    __builtin_amdgcn_sched_barrier(0);
    if (b + BPB < wb1) score_batch(b + BPB, bufb);
  }
  // the residency flags (and pages), from the table entries read at the start
  if (tbl_regs) {
#pragma unroll
    for (int u = 0; u < kTblRun; ++u) {
      const int i = tid + u * kSelThreads;
      if (i < nb) {
        flag[i] = tbl[u] >= 0 ? kResident : 0;
        if (gpu_pages) pg[i] = tbl[u];
      }
    }
  } else {
    for (int i = tid; i < nb; i += kSelThreads) {
      const int32_t e = trow[i];
      flag[i] = e >= 0 ? kResident : 0;
      if (gpu_pages) pg[i] = e;
    }
  }
  lo = wave_min(lo);
  hi = wave_max(hi);
  if (lane == 0) { red_lo[wave] = lo; red_hi[wave] = hi; }
  __syncthreads();  // scores, flags, histogram reset and the per-wave ranges are visible
  lo = red_lo[0];
  hi = red_hi[0];
  for (int w = 1; w < kSelWaves; ++w) { lo = fminf(lo, red_lo[w]); hi = fmaxf(hi, red_hi[w]); }
  const float span = hi - lo;
  const bool bucketed = span > 0.f && span < INFINITY;
  const float to_bucket = bucketed ? 256.f / span : 0.f;

  // top-k, fast path: histogram of score values, exact ranking inside the boundary bucket
  uint32_t B = 0, r = 0, cnt = 0xffffffffu;
  if (bucketed) {
    for (int i = tid; i < nb; i += kSelThreads) atomicAdd(&hist[bucket_of(sc[i], lo, to_bucket)], 1u);
    __syncthreads();
    const uint32_t c = tid < 256 ? hist[255 - tid] : 0u;  // thread 0: the highest bucket
    const uint32_t cge = block_scan_incl(c, tmp);
    const uint32_t cgt = cge - c;
    if (tid < 256 && cgt < ks && cge >= ks) {
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
    for (int i = tid; i < nb; i += kSelThreads) {
      const uint32_t b = (uint32_t)bucket_of(sc[i], lo, to_bucket);
      if (b > B) flag[i] |= kSelected;
      if (b == B) {
        const uint32_t pos = atomicAdd(&ncand, 1u);
        cand_key[pos] = order_key(sc[i]);
        cand_idx[pos] = i;
      }
    }
    __syncthreads();
    for (uint32_t c = tid; c < cnt; c += kSelThreads) {
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
    // General path: exact radix select of the ks-th largest key, 8 bits per pass.
    uint32_t prefix = 0, mask = 0, remaining = ks;
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int i = tid; i < nb; i += kSelThreads) {
        const uint32_t kv = order_key(sc[i]);
        if ((kv & mask) == prefix) atomicAdd(&hist[(kv >> shift) & 255u], 1u);
      }
      __syncthreads();
      const uint32_t c = tid < 256 ? hist[255 - tid] : 0u;
      const uint32_t cge = block_scan_incl(c, tmp);
      const uint32_t cgt = cge - c;
      if (tid < 256 && cgt < remaining && cge >= remaining) {
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
    const int per = (nb + kSelThreads - 1) / kSelThreads;
    const int i0 = min(nb, tid * per), i1 = min(nb, i0 + per);
    uint32_t ties = 0;
    for (int i = i0; i < i1; ++i) ties += order_key(sc[i]) == thr;
    const uint32_t tie_base = block_scan_incl(ties, tmp) - ties;
    uint32_t seen = 0;
    for (int i = i0; i < i1; ++i) {
      const uint32_t kv = order_key(sc[i]);
      bool sel = kv > thr;
      if (kv == thr) { sel = tie_base + seen < take_eq; ++seen; }
      if (sel) flag[i] |= kSelected;
    }
    __syncthreads();
  }

  // ascending compaction of the selected blocks, split by residency.  The offloaded list
  // is assembled in LDS (over the scores, no longer needed) and then written out with
  // coalesced stores, to device memory and, when given, straight into the host mirror
  // (coherent page-locked host memory, which the device writes through without caching,
  // so the values are in host memory once the kernel has completed): the hand-off needs
  // no copy.
  const int per = (nb + kSelThreads - 1) / kSelThreads;
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
  if (tid == kSelThreads - 1) { tot_res = incl & 0xffffu; tot_off = incl >> 16; }
  int32_t* grow = gpu_blocks + (size_t)pair * top_k;
  int32_t* prow = gpu_pages ? gpu_pages + (size_t)pair * top_k : nullptr;
  int32_t* off_lds = reinterpret_cast<int32_t*>(sc);  // [top_k] <= [max_blocks]
  for (int i = i0; i < i1; ++i) {
    const uint8_t f = flag[i];
    if (f == (kSelected | kResident)) {
      grow[pos_res] = i;
      if (prow) prow[pos_res] = pg[i];
      ++pos_res;
    } else if (f == kSelected) {
      off_lds[pos_off++] = i;
    }
  }
  __syncthreads();
  const int nr = (int)tot_res, no = (int)tot_off;
  for (int j = nr + tid; j < top_k; j += kSelThreads) {
    grow[j] = -1;
    if (prow) prow[j] = -1;
  }
  int32_t* crow = cpu_blocks + (size_t)pair * top_k;
  int32_t* hrow = cpu_blocks_host ? cpu_blocks_host + (size_t)pair * top_k : nullptr;
  for (int j = tid; j < top_k; j += kSelThreads) {
    const int32_t v = j < no ? off_lds[j] : -1;
    crow[j] = v;
    if (hrow) hrow[j] = v;
  }
  if (tid == 0) {
    n_gpu[pair] = nr;
    n_cpu[pair] = no;
    if (n_cpu_host) n_cpu_host[pair] = no;
  }
}

template <typename T, int D>
hipError_t select_typed(const Shape& s, bool minmax, const QParts& q, const void* dig,
                        const int32_t* lens, int top_k, const int32_t* table, int32_t* gb,
                        int32_t* ng, int32_t* cb, int32_t* nc, float* scores, int32_t* cbh,
                        int32_t* nch, int32_t* gp, hipStream_t st) {
  // scores, flags (padded to a float boundary) and, when pages are written, table entries
  const size_t lds = (size_t)(s.max_blocks + (s.max_blocks + 3) / 4) * sizeof(float) +
                     (gp ? (size_t)s.max_blocks * sizeof(int32_t) : 0);
  const dim3 grid(s.B * s.Hkv), block(kSelThreads);
  if (minmax)
    hipLaunchKernelGGL((select_kernel<T, D, true>), grid, block, lds, st, q, (const T*)dig,
                       lens, s.Hkv, s.G, s.bs, s.max_blocks, top_k, table, gb, ng, cb, nc,
                       scores, cbh, nch, gp);
  else
    hipLaunchKernelGGL((select_kernel<T, D, false>), grid, block, lds, st, q, (const T*)dig,
                       lens, s.Hkv, s.G, s.bs, s.max_blocks, top_k, table, gb, ng, cb, nc,
                       scores, cbh, nch, gp);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select(const Shape& s, bool minmax, const QParts& q, const void* digests,
                         const int32_t* seq_lens, int top_k, const int32_t* block_table,
                         int32_t* gpu_blocks, int32_t* n_gpu, int32_t* cpu_blocks,
                         int32_t* n_cpu, float* scores_or_null, int32_t* cpu_blocks_host,
                         int32_t* n_cpu_host, int32_t* gpu_pages, hipStream_t stream) {
#define SA_SEL_ARGS s, minmax, q, digests, seq_lens, top_k, block_table, gpu_blocks, n_gpu, \
                    cpu_blocks, n_cpu, scores_or_null, cpu_blocks_host, n_cpu_host, gpu_pages, \
                    stream
  if (s.bf16)
    return s.d == 128 ? select_typed<uint16_t, 128>(SA_SEL_ARGS)
                      : select_typed<uint16_t, 64>(SA_SEL_ARGS);
  return s.d == 128 ? select_typed<float, 128>(SA_SEL_ARGS) : select_typed<float, 64>(SA_SEL_ARGS);
#undef SA_SEL_ARGS
}

}  // namespace sa
