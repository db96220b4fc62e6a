// Block selection of ScoutAttention [arXiv:2603.27138, HTML Sec. 2.2 and 3.2; Algorithm 1]:
//   B_pred = TopK(Q K_digest^T) per (sequence, KV head), then B_cpu = B_pred \ B_gpu.
//
// Work split: whole (sequence, KV head) pairs go one to an 8-wave workgroup, in as many
// full rounds of one per CU as the pairs fill; the pairs left over are cut into pieces,
// about one per CU in all, one workgroup each.  So every CU streams about the same digest
// bytes (at the 40-layer decode shape: 320 pairs on 256 CUs, each CU one whole pair plus a
// quarter of one of the 64 others), where one workgroup per pair would put two pairs on a
// quarter of the CUs and end with them.  The pieces come first in the grid and are short,
// so their hand-over (step 3) is over while the whole pairs still stream.
//   1. scoring: the G query heads of the KV head are folded into per-channel coefficients
//      -- the group sum sum_g q_g for mean digests, and for min/max digests
//        sum_g max(q_gc min_c, q_gc max_c) = (sum_g max(q_gc, 0)) max_c + (sum_g min(q_gc, 0)) min_c
//      (exact, since max_c >= min_c) -- so a digest element costs one or two FMAs.  The
//      query rows (all their parts), the first digest batch and the item's block-table
//      entries are requested together in one round: the workgroup sums the query parts into
//      LDS and each lane reads its coefficients from there behind an LDS-only barrier, while
//      the digests are already in flight.  The waves stream the item's rows in batches of
//      8 coalesced 16-byte loads per lane, the next batch in flight while the current one is
//      reduced (DPP row sums; loads are unconditional so the waits cover one batch); after
//      its first two batches a wave takes each next batch from a counter in LDS, so the
//      waves of a workgroup run out of rows together rather than each at the end of a
//      fixed share (under load, one wave's latency differs from another's by microseconds).
//      The scores stay in LDS.
//   2. top-k: a histogram of the score values over 256 equal-width buckets locates the
//      bucket holding the k-th largest score; the few scores in that bucket are ranked
//      exactly by (score, lower position first).  A crowded bucket (e.g. all scores equal)
//      falls back to an exact MSB-first radix select on order-preserving 32-bit keys.
//   3. hand-over (pieces only): each piece selects its own top min(k, rows) -- every block
//      of the pair's selection that lies in the piece is among them -- and writes them, in
//      ascending block order with their scores and block-table entries, to the workspace
//      with device-scope stores (written through to the memory all XCDs share); it waits
//      until they have completed and only then counts itself in on the pair's arrival
//      counter (a device-scope atomic add).  The piece that counts last has therefore every
//      other piece's candidates in memory: it reads them back with device-scope loads (in
//      piece order, so still ascending by block), resets the counter to zero for the next
//      launch, and selects the pair's top-k among them (step 2 again).  No workgroup ever
//      waits for another.
//   4. split: the selected blocks are compacted in ascending order and split by the block
//      table into the resident and offloaded lists; the offloaded list can also be written
//      straight into a host mirror (the hand-off of Algorithm 1), and the pages of the
//      resident list next to it (so attention skips the table lookup).
#include <hip/hip_ext.h>

#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace sa {
namespace {

constexpr int kSelWaves = 8;
constexpr int kSelThreads = kSelWaves * kWave;
static_assert(kSelThreads >= 256, "a thread per histogram bucket");
constexpr int kBatch = 8;        // 16-byte loads per lane per batch
constexpr int kMaxCand = 256;    // boundary-bucket candidates ranked directly
constexpr int kSelPartGroup = 4; // query parts loaded together
constexpr int kTblRun = 8;       // block-table entries a thread holds in registers
constexpr int kMaxRows = kTblRun * kSelThreads;  // rows of one item: its entries fit them
constexpr int kMinChunkRows = 64;
constexpr int kCUs = 256;        // compute units of the chip (one round of whole pairs)
constexpr size_t kWholeBytes = 192 << 10;  // digest bytes of a pair one CU takes whole
constexpr int kMaxGroup = 8;     // query heads per KV head
// two workgroups per CU at once (a whole pair's beside a piece's): 4 waves per SIMD
constexpr int kSelWavesPerSimd = 4;
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

// Device-scope accesses of the chunks' hand-over: stores written through to (and loads
// served from) the memory every XCD shares, so no L2 cache holds a stale copy.
__device__ __forceinline__ void store_device(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_device(uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

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

// The hand-over buffers in the workspace: per pair and block, a piece's candidates at
// the piece's own rows (score, block-table entry, block index), the candidate count of every
// (pair, piece), then the arrival counters [pairs] (zero between launches).
struct Handover {
  uint32_t* score;  // [pairs][max_blocks]
  uint32_t* page;   // [pairs][max_blocks]
  uint32_t* blk;    // [pairs][max_blocks]
  uint32_t* n;      // [pairs][nchunk]
  uint32_t* count;  // [pairs]
};

template <typename T, int D, bool MINMAX>
__global__ __launch_bounds__(kSelThreads, kSelWavesPerSimd) void select_kernel(
    const QParts q, const T* __restrict__ dig, const int32_t* __restrict__ seq_lens,
    int Hkv, int G, int bs, int max_blocks, int top_k, int whole, int split, int chunk,
    int nchunk, const int32_t* __restrict__ table, int32_t* __restrict__ gpu_blocks,
    int32_t* __restrict__ n_gpu, int32_t* __restrict__ cpu_blocks,
    int32_t* __restrict__ n_cpu, float* __restrict__ scores_out,
    int32_t* __restrict__ cpu_blocks_host, int32_t* __restrict__ n_cpu_host,
    int32_t* __restrict__ gpu_pages, Handover xs) {
  constexpr int VEC = Digest<T>::N;
  constexpr int LPR = D / VEC;             // lanes per digest row
  constexpr int BPI = kWave / LPR;         // blocks per load instruction
  constexpr int LPB = MINMAX ? 2 : 1;      // loads per block row
  constexpr int BPB = kBatch / LPB * BPI;  // blocks per batch (per wave)
  constexpr int ROW = LPB * D;

  // per position j < max_blocks: score, block-table entry, block index (the last piece's
  // candidates; elsewhere the position is the block) and flags
  extern __shared__ float sc[];
  int32_t* pg = reinterpret_cast<int32_t*>(sc + max_blocks);
  uint16_t* bk = reinterpret_cast<uint16_t*>(pg + max_blocks);
  uint8_t* flag = reinterpret_cast<uint8_t*>(bk + max_blocks);
  __shared__ uint32_t hist[256];
  __shared__ uint32_t tmp[kSelWaves];
  __shared__ float red_lo[kSelWaves], red_hi[kSelWaves];
  __shared__ uint32_t cand_key[kMaxCand];
  __shared__ int cand_idx[kMaxCand];
  __shared__ uint32_t sel_digit, sel_remaining, sel_count, ncand, tot_a, tot_b, arrived;
  __shared__ uint32_t next_row;                 // the next unscored batch of the item
  __shared__ float4 q_sum[kMaxGroup * D / 4];   // the pair's G query rows, parts summed

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // scalar loop bounds
  // work item: the first split * nchunk workgroups take the pieces of pairs [whole, whole +
  // split), the rest one whole pair each (pairs [0, whole))
  const bool whole_item = (int)blockIdx.x >= split * nchunk;
  const int pair = whole_item ? (int)blockIdx.x - split * nchunk : whole + (int)blockIdx.x / nchunk;
  const int ck = whole_item ? 0 : (int)blockIdx.x % nchunk;
  const int s = pair / Hkv, h = pair % Hkv;

  // blocks of the sequence, clamped to the table's span (a bad length cannot move a read
  // past the pair's rows), and the pieces that hold them (at least one, which also handles
  // a pair without blocks)
  const int nb = min(max((seq_lens[s] + bs - 1) / bs, 0), max_blocks);
  const int live = whole_item ? 1 : max(1, (nb + chunk - 1) / chunk);
  if (ck >= live) return;  // (uniform) a piece past the sequence's blocks
  const bool alone = live == 1;
  const int r0 = ck * chunk, r1 = alone ? nb : min(nb, r0 + chunk);  // this item's rows
  const uint32_t ks = (uint32_t)min(top_k, nb);

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
  const int cg = lane % LPR, bi = lane / LPR;

  const T* base = dig + (size_t)pair * max_blocks * ROW + cg * VEC;
  uint4 bufa[kBatch], bufb[kBatch];
  // Batch [b, b + BPB) of the item's rows.  Loads are issued unconditionally (rows past the
  // item clamped to its last row, their scores discarded), so the waits before a batch cover
  // that batch only.
  auto load_batch = [&](int b_first, uint4* buf) {
#pragma unroll
    for (int u = 0; u < kBatch / LPB; ++u) {
      const int b = max(min(b_first + u * BPI + bi, r1 - 1), 0);
#pragma unroll
      for (int r = 0; r < LPB; ++r)
        buf[u * LPB + r] = load_stream16(base + (size_t)b * ROW + r * D);
    }
  };
  // the first two batches of a wave are fixed; later ones come from next_row
  int cur = r0 + wave * BPB, nxt = r0 + (kSelWaves + wave) * BPB;
  load_batch(cur, bufa);  // (a wave with no rows re-reads a valid one, unused)

  // the item's block-table entries are read while the digests stream, into registers
  // (row r0 + tid + u * kSelThreads in entry u) that are only consumed after the scoring
  const int32_t* trow = table + (size_t)pair * max_blocks;
  int32_t tbl[kTblRun];  // (loads unconditional, indexes clamped to a valid entry)
#pragma unroll
  for (int u = 0; u < kTblRun; ++u) tbl[u] = trow[max(min(r0 + tid + u * kSelThreads, r1 - 1), 0)];
  if (tid == 0) next_row = (uint32_t)(r0 + 2 * kSelWaves * BPB);

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
  lds_barrier();  // the summed rows and next_row are visible; the digest loads stay in flight

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
      if (b < r1) {
        lo = fminf(lo, acc);
        hi = fmaxf(hi, acc);
        if (cg == 0) {
          sc[b] = acc;
          if (scores_out) scores_out[(size_t)pair * max_blocks + b] = acc;
        }
      }
    }
  };
  // a batch from the counter: lane 0 asks, and the answer is read (made scalar) only when
  // it is needed, two batches later
  auto take = [&]() {
    uint32_t v = 0;
    if (lane == 0) v = atomicAdd(&next_row, (uint32_t)BPB);
    return v;
  };
  auto scalar = [](uint32_t v) { return (int)__builtin_amdgcn_readfirstlane(v); };
  // the scheduling barriers keep the compiler from sinking a batch's loads to their use
  while (cur < r1) {
    load_batch(nxt, bufb);
    const uint32_t t1 = take();
    __builtin_amdgcn_sched_barrier(0);
    score_batch(cur, bufa);
    if (nxt >= r1) break;
    const int after = scalar(t1);
    load_batch(after, bufa);
    const uint32_t t2 = take();
    __builtin_amdgcn_sched_barrier(0);
    score_batch(nxt, bufb);
    cur = after;
    nxt = scalar(t2);
  }

  // flags (and pages) of the item's rows, from the table entries read at the start
#pragma unroll
  for (int u = 0; u < kTblRun; ++u) {
    const int i = r0 + tid + u * kSelThreads;
    if (i < r1) {
      flag[i] = tbl[u] >= 0 ? kResident : 0;
      pg[i] = tbl[u];
    }
  }
  lo = wave_min(lo);
  hi = wave_max(hi);
  if (lane == 0) { red_lo[wave] = lo; red_hi[wave] = hi; }
  __syncthreads();  // scores, flags and the per-wave ranges are visible
  lo = red_lo[0];
  hi = red_hi[0];
  for (int w = 1; w < kSelWaves; ++w) { lo = fminf(lo, red_lo[w]); hi = fmaxf(hi, red_hi[w]); }

  // Marks, in flag, the kk largest of sc[b0 .. b0 + n) (equal scores: the lower position
  // first), whose minimum and maximum are lo and hi.  Every thread calls it.
  auto topk = [&](int b0, int n, uint32_t kk, float lo, float hi) {
    if (kk >= (uint32_t)n) {  // all of them (also none)
      for (int i = tid; i < n; i += kSelThreads) flag[b0 + i] |= kSelected;
      __syncthreads();
      return;
    }
    if (tid < 256) hist[tid] = 0;
    if (tid == 0) ncand = 0;
    __syncthreads();
    const float span = hi - lo;
    const bool bucketed = span > 0.f && span < INFINITY;
    const float to_bucket = bucketed ? 256.f / span : 0.f;
    // fast path: histogram of score values, exact ranking inside the boundary bucket
    uint32_t B = 0, r = 0, cnt = 0xffffffffu;
    if (bucketed) {
      for (int i = tid; i < n; i += kSelThreads)
        atomicAdd(&hist[bucket_of(sc[b0 + i], lo, to_bucket)], 1u);
      __syncthreads();
      const uint32_t c = tid < 256 ? hist[255 - tid] : 0u;  // thread 0: the highest bucket
      const uint32_t cge = block_scan_incl(c, tmp);
      const uint32_t cgt = cge - c;
      if (tid < 256 && cgt < kk && cge >= kk) {
        sel_digit = 255u - (uint32_t)tid;
        sel_remaining = kk - cgt;
        sel_count = c;
      }
      __syncthreads();
      B = sel_digit;
      r = sel_remaining;
      cnt = sel_count;
    }
    if (cnt <= (uint32_t)kMaxCand) {
      for (int i = tid; i < n; i += kSelThreads) {
        const uint32_t b = (uint32_t)bucket_of(sc[b0 + i], lo, to_bucket);
        if (b > B) flag[b0 + i] |= kSelected;
        if (b == B) {
          const uint32_t pos = atomicAdd(&ncand, 1u);
          cand_key[pos] = order_key(sc[b0 + i]);
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
        if (rank < r) flag[b0 + idx] |= kSelected;
      }
      __syncthreads();
    } else {
      // General path: exact radix select of the kk-th largest key, 8 bits per pass.
      uint32_t prefix = 0, mask = 0, remaining = kk;
      for (int shift = 24; shift >= 0; shift -= 8) {
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += kSelThreads) {
          const uint32_t kv = order_key(sc[b0 + i]);
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
      const uint32_t thr = prefix;         // the kk-th largest key
      const uint32_t take_eq = remaining;  // keys equal to thr that are selected
      const int per = (n + kSelThreads - 1) / kSelThreads;
      const int i0 = min(n, tid * per), i1 = min(n, i0 + per);
      uint32_t ties = 0;
      for (int i = i0; i < i1; ++i) ties += order_key(sc[b0 + i]) == thr;
      const uint32_t tie_base = block_scan_incl(ties, tmp) - ties;
      uint32_t seen = 0;
      for (int i = i0; i < i1; ++i) {
        const uint32_t kv = order_key(sc[b0 + i]);
        bool sel = kv > thr;
        if (kv == thr) { sel = tie_base + seen < take_eq; ++seen; }
        if (sel) flag[b0 + i] |= kSelected;
      }
      __syncthreads();
    }
  };

  int n = nb;        // positions the final selection runs over
  bool cand = false; // positions hold the pieces' candidates (block index in bk)
  if (!alone) {
    // 3. hand-over: this piece's top min(k, rows), ascending, to the workspace
    topk(r0, r1 - r0, min(ks, (uint32_t)(r1 - r0)), lo, hi);
    const int per = (r1 - r0 + kSelThreads - 1) / kSelThreads;
    const int i0 = min(r1, r0 + tid * per), i1 = min(r1, i0 + per);
    uint32_t mine = 0;
    for (int i = i0; i < i1; ++i) mine += flag[i] & kSelected;
    uint32_t pos = block_scan_incl(mine, tmp) - mine;
    const size_t row0 = (size_t)pair * max_blocks;
    for (int i = i0; i < i1; ++i) {
      if (flag[i] & kSelected) {
        const size_t at = row0 + r0 + pos++;
        store_device(xs.score + at, __float_as_uint(sc[i]));
        store_device(xs.page + at, (uint32_t)pg[i]);
        store_device(xs.blk + at, (uint32_t)i);
      }
    }
    if (tid == kSelThreads - 1)
      store_device(xs.n + (size_t)pair * nchunk + ck, pos);  // (the last thread's end = count)
    __builtin_amdgcn_s_waitcnt(0);  // every store of this thread has completed
    __syncthreads();                // ... and of every thread of the workgroup
    if (tid == 0)
      arrived = __hip_atomic_fetch_add(xs.count + pair, 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (arrived != (uint32_t)(live - 1)) return;  // (uniform) another piece comes later
    // the last piece: every other piece's candidates are in memory; gather them in piece
    // order (ascending by block) into positions 0 .. n
    if (tid == 0) store_device(xs.count + pair, 0u);
    n = 0;
    lo = INFINITY;
    hi = -INFINITY;
    for (int c = 0; c < live; ++c) {
      // (a count read back is clamped to the piece and to the positions left)
      const int nc = min(min((int)load_device(xs.n + (size_t)pair * nchunk + c), chunk),
                         max_blocks - n);
      const size_t src = row0 + (size_t)c * chunk;
      for (int j = tid; j < nc; j += kSelThreads) {
        const float v = __uint_as_float(load_device(xs.score + src + j));
        const int32_t e = (int32_t)load_device(xs.page + src + j);
        const uint32_t b = load_device(xs.blk + src + j);
        sc[n + j] = v;
        pg[n + j] = e;
        bk[n + j] = (uint16_t)min(b, (uint32_t)(max_blocks - 1));
        flag[n + j] = e >= 0 ? kResident : 0;
        lo = fminf(lo, v);
        hi = fmaxf(hi, v);
      }
      n += nc;
    }
    cand = true;
    lo = wave_min(lo);
    hi = wave_max(hi);
    if (lane == 0) { red_lo[wave] = lo; red_hi[wave] = hi; }
    __syncthreads();
    lo = red_lo[0];
    hi = red_hi[0];
    for (int w = 1; w < kSelWaves; ++w) { lo = fminf(lo, red_lo[w]); hi = fmaxf(hi, red_hi[w]); }
  }
  topk(0, n, ks, lo, hi);

  // 4. ascending compaction of the selected positions, split by residency.  The offloaded
  // list is assembled in LDS (over the scores, no longer needed) and then written out with
  // coalesced stores, to device memory and, when given, straight into the host mirror
  // (coherent page-locked host memory, which the device writes through without caching,
  // so the values are in host memory once the kernel has completed): the hand-off needs
  // no copy.
  const int per = (n + kSelThreads - 1) / kSelThreads;
  const int i0 = min(n, tid * per), i1 = min(n, i0 + per);
  uint32_t cnt_res = 0, cnt_off = 0;
  for (int i = i0; i < i1; ++i) {
    const uint8_t f = flag[i];
    cnt_res += f == (kSelected | kResident);
    cnt_off += f == kSelected;
  }
  const uint32_t packed = cnt_res | (cnt_off << 16);
  const uint32_t incl = block_scan_incl(packed, tmp);
  uint32_t pos_res = (incl - packed) & 0xffffu, pos_off = (incl - packed) >> 16;
  if (tid == kSelThreads - 1) { tot_a = incl & 0xffffu; tot_b = incl >> 16; }
  int32_t* grow = gpu_blocks + (size_t)pair * top_k;
  int32_t* prow = gpu_pages ? gpu_pages + (size_t)pair * top_k : nullptr;
  int32_t* off_lds = reinterpret_cast<int32_t*>(sc);  // [top_k] <= [max_blocks]
  __syncthreads();  // (every score read before off_lds overwrites them)
  for (int i = i0; i < i1; ++i) {
    const uint8_t f = flag[i];
    const int32_t blk = cand ? (int32_t)bk[i] : i;
    if (f == (kSelected | kResident)) {
      grow[pos_res] = blk;
      if (prow) prow[pos_res] = pg[i];
      ++pos_res;
    } else if (f == kSelected) {
      off_lds[pos_off++] = blk;
    }
  }
  __syncthreads();
  const int nr = (int)tot_a, no = (int)tot_b;
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
hipError_t select_typed(const Shape& s, const SelectPlan& p, bool minmax, const QParts& q,
                        const void* dig, const int32_t* lens, int top_k, const int32_t* table,
                        int32_t* gb, int32_t* ng, int32_t* cb, int32_t* nc, float* scores,
                        int32_t* cbh, int32_t* nch, int32_t* gp, void* ws, hipStream_t st,
                        hipEvent_t e0, hipEvent_t e1) {
  // per position: score, table entry, block index (16 bits), flags
  const size_t lds = (size_t)s.max_blocks * (sizeof(float) + sizeof(int32_t) + 2 + 1);
  const size_t pairs = (size_t)s.B * s.Hkv, rows = pairs * s.max_blocks;
  Handover xs{};
  if (p.split > 0 && p.nchunk > 1) {
    xs.score = static_cast<uint32_t*>(ws);
    xs.page = xs.score + rows;
    xs.blk = xs.page + rows;
    xs.n = xs.blk + rows;
    xs.count = xs.n + pairs * p.nchunk;
  }
  const dim3 grid(p.whole + p.split * p.nchunk), block(kSelThreads);
  // hipExtLaunchKernelGGL records the (optional) events at the kernel's own start and end
  if (minmax)
    hipExtLaunchKernelGGL((select_kernel<T, D, true>), grid, block, lds, st, e0, e1, 0, q,
                          (const T*)dig, lens, s.Hkv, s.G, s.bs, s.max_blocks, top_k, p.whole,
                          p.split, p.chunk, p.nchunk, table, gb, ng, cb, nc, scores, cbh, nch,
                          gp, xs);
  else
    hipExtLaunchKernelGGL((select_kernel<T, D, false>), grid, block, lds, st, e0, e1, 0, q,
                          (const T*)dig, lens, s.Hkv, s.G, s.bs, s.max_blocks, top_k, p.whole,
                          p.split, p.chunk, p.nchunk, table, gb, ng, cb, nc, scores, cbh, nch,
                          gp, xs);
  return hipGetLastError();
}

}  // namespace

SelectPlan select_plan(const Shape& s, bool minmax) {
  SelectPlan p;
  const int pairs = s.B * s.Hkv;
  // whole pairs: as many full rounds of one per CU as there are (a pair's rows must fit
  // the table registers of one workgroup).  With no more pairs than CUs and small pairs, all
  // of them whole: one CU streams such a pair (at most kWholeBytes of digests) in about the
  // time a piece's hand-over takes.
  const size_t pair_bytes = (size_t)s.max_blocks * s.d * (s.bf16 ? 2 : 4) * (minmax ? 2 : 1);
  if (s.max_blocks <= kMaxRows && pairs <= kCUs && pair_bytes <= kWholeBytes)
    p.whole = pairs;
  else
    p.whole = s.max_blocks <= kMaxRows ? pairs / kCUs * kCUs : 0;
  p.split = pairs - p.whole;
  // the other pairs in pieces, about one piece per CU in all
  const int pieces = p.split > 0 ? std::max(1, (kCUs + p.split - 1) / p.split) : 1;
  int rows = (s.max_blocks + pieces - 1) / pieces;
  rows = std::min(std::max(rows, kMinChunkRows), kMaxRows);
  p.chunk = rows;
  p.nchunk = p.split > 0 ? (s.max_blocks + rows - 1) / rows : 1;
  // hand-over candidates (score, table entry, block) [pairs][max_blocks], their counts
  // [pairs][nchunk], then the counters [pairs]
  p.ws_bytes = p.split > 0 && p.nchunk > 1
                   ? (size_t)pairs * (3 * (size_t)s.max_blocks + p.nchunk + 1) * sizeof(uint32_t)
                   : 0;
  return p;
}

hipError_t launch_select(const Shape& s, const SelectPlan& plan, bool minmax, const QParts& q,
                         const void* digests, const int32_t* seq_lens, int top_k,
                         const int32_t* block_table, int32_t* gpu_blocks, int32_t* n_gpu,
                         int32_t* cpu_blocks, int32_t* n_cpu, float* scores_or_null,
                         int32_t* cpu_blocks_host, int32_t* n_cpu_host, int32_t* gpu_pages,
                         void* ws, hipStream_t stream, hipEvent_t ev_start,
                         hipEvent_t ev_stop) {
#define SA_SEL_ARGS s, plan, minmax, q, digests, seq_lens, top_k, block_table, gpu_blocks, \
                    n_gpu, cpu_blocks, n_cpu, scores_or_null, cpu_blocks_host, n_cpu_host, \
                    gpu_pages, ws, stream, ev_start, ev_stop
  if (s.bf16)
    return s.d == 128 ? select_typed<uint16_t, 128>(SA_SEL_ARGS)
                      : select_typed<uint16_t, 64>(SA_SEL_ARGS);
  return s.d == 128 ? select_typed<float, 128>(SA_SEL_ARGS) : select_typed<float, 64>(SA_SEL_ARGS);
#undef SA_SEL_ARGS
}

}  // namespace sa
