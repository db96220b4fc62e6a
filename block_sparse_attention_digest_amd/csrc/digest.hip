// Block digests [ScoutAttention, arXiv:2603.27138, HTML Sec. 2.2]: the mean of K over a
// block (MoBA-style) or the channel-wise min and max of K over a block (Quest-style).
//
// Persistent waves walk the (sequence, KV head, block) slots.  K pages are chunk-major
// ([d/x][bs][x], x elements per 16-byte chunk), so one page is d/x chunk rows of bs tokens
// each.  Each load instruction reads 8 chunks x 8 tokens: lane l takes chunk 8 cg + l / 8
// and token 8 tg + l % 8, so every group of 8 lanes reads one whole 128-byte line.  A lane
// keeps its chunk's running sums (or min/max) over its tokens; the 8 lanes of a chunk then
// combine theirs with a reduce-scatter, after which each lane owns (and writes) one
// channel.  The mean accumulates in float64, where sums of bf16 keys are exact, and is
// rounded once to the stored dtype; min/max are exact in any precision.  HBM-bound: the
// page is read once and d (or 2d) values are written.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace sa {
namespace {

constexpr int kDigestWaves = 4;  // waves per workgroup of the build

template <typename T>
struct Vec;
template <>
struct Vec<uint16_t> {  // eight bf16 per 16-byte chunk
  static constexpr int N = 8;
  __device__ static void widen(const uint4& v, float* f) { bf16x8_to_f32(v, f); }
};
template <>
struct Vec<float> {  // four float per 16-byte chunk
  static constexpr int N = 4;
  __device__ static void widen(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
};

// One exchange step: a lane keeps H of its 2H values (the upper half when `upper`) and adds
// the partner's copy of them (lane ^ mask).
template <int H, typename V, typename Op>
__device__ __forceinline__ void halve(V* v, bool upper, int mask, Op op) {
#pragma unroll
  for (int i = 0; i < H; ++i) {
    const V send = upper ? v[i] : v[H + i];
    const V keep = upper ? v[H + i] : v[i];
    v[i] = op(keep, __shfl_xor(send, mask, kWave));
  }
}

// Reduce-scatter over the 8 lanes of a chunk (tl = lane % 8) of N = 8 or 4 values per lane:
// each exchange halves what a lane keeps (the upper lane of a pair keeps the upper half);
// once one value is left the last exchange adds it whole.  Lane tl ends with element
// (tl * N) / 8 of the chunk, reduced over the 8 lanes.
template <int N, typename V, typename Op>
__device__ __forceinline__ V reduce_scatter8(V (&v)[N], int tl, Op op) {
  static_assert(N == 8 || N == 4, "chunk width");
  if constexpr (N == 8) {
    halve<4>(v, tl & 4, 4, op);
    halve<2>(v, tl & 2, 2, op);
    halve<1>(v, tl & 1, 1, op);
  } else {
    halve<2>(v, tl & 4, 4, op);
    halve<1>(v, tl & 2, 2, op);
    v[0] = op(v[0], __shfl_xor(v[0], 1, kWave));
  }
  return v[0];
}

__device__ __forceinline__ void store_one(uint16_t* dst, float f) {
  *dst = (uint16_t)(__float_as_uint(f) >> 16);  // exact bf16 (a min or max of bf16 keys)
}
__device__ __forceinline__ void store_one(float* dst, float f) { *dst = f; }
__device__ __forceinline__ void store_mean1(uint16_t* dst, double v) {
  *dst = (uint16_t)f64_to_bf16_rne(v);
}
__device__ __forceinline__ void store_mean1(float* dst, double v) { *dst = (float)v; }

// Page geometry of one instantiation.  A lane holds CGS x TG loads of 16 bytes at a time:
// the whole page when that is at most 8 loads, else the page in SL channel slabs of CGS
// chunk groups each (channels are digested independently, so a slab is a unit of its own;
// two slabs in flight per wave keep the registers within reach of two waves per SIMD).
template <typename T, int D, int BS>
struct PageGeom {
  static constexpr int VEC = Vec<T>::N;  // elements per 16-byte chunk
  static constexpr int NC = D / VEC;     // chunks per token
  static constexpr int CG = NC / 8;      // chunk groups: 8 chunks per load instruction
  static constexpr int TG = BS / 8;      // token groups: 8 tokens (one 128-byte line) per chunk
  static constexpr int SL = CG * TG > 8 ? CG * TG / 8 : 1;    // channel slabs per page
  static constexpr int CGS = CG / SL;                          // chunk groups per slab
  static_assert(NC % 8 == 0 && BS % 8 == 0 && CG % SL == 0, "page shape");
};

// The digest of slab `slab` of one block, from its loads already in registers (raw),
// written to slot gidx.
template <typename T, int D, int BS, bool MINMAX>
__device__ __forceinline__ void digest_block(
    const uint4 (&raw)[PageGeom<T, D, BS>::CGS][BS / 8], int nvalid, T* __restrict__ dig,
    long gidx, int cl, int tl, int slab) {
  using PG = PageGeom<T, D, BS>;
  constexpr int VEC = PG::VEC, CGS = PG::CGS, TG = PG::TG;
  const int e = tl * VEC / 8;                          // this lane's element of its chunk
  const bool writer = (tl * VEC) % 8 == 0;             // one lane per element
#pragma unroll
  for (int cs = 0; cs < CGS; ++cs) {
    const int cg = CGS * slab + cs;
    const int ch = (8 * cg + cl) * VEC + e;            // this lane's channel
    if constexpr (MINMAX) {
      float mn[VEC], mx[VEC];
#pragma unroll
      for (int i = 0; i < VEC; ++i) { mn[i] = INFINITY; mx[i] = -INFINITY; }
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) {  // tokens past the valid ones are left out
        const bool ok = 8 * tg + tl < nvalid;
        float f[VEC];
        Vec<T>::widen(raw[cs][tg], f);
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          mn[i] = fminf(mn[i], ok ? f[i] : INFINITY);
          mx[i] = fmaxf(mx[i], ok ? f[i] : -INFINITY);
        }
      }
      const float lo = reduce_scatter8<VEC>(mn, tl, [](float a, float b) { return fminf(a, b); });
      const float hi = reduce_scatter8<VEC>(mx, tl, [](float a, float b) { return fmaxf(a, b); });
      if (writer) {
        T* dst = dig + (size_t)gidx * 2 * D + ch;
        store_one(dst, lo);
        store_one(dst + D, hi);
      }
    } else {
      double acc[VEC];
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] = 0.0;
      if (nvalid >= BS) {  // a full block (all but a sequence's last)
#pragma unroll
        for (int tg = 0; tg < TG; ++tg) {
          float f[VEC];
          Vec<T>::widen(raw[cs][tg], f);
#pragma unroll
          for (int i = 0; i < VEC; ++i) acc[i] += (double)f[i];
        }
      } else {
#pragma unroll
        for (int tg = 0; tg < TG; ++tg) {  // tokens past the valid ones add 0
          const bool ok = 8 * tg + tl < nvalid;
          float f[VEC];
          Vec<T>::widen(raw[cs][tg], f);
#pragma unroll
          for (int i = 0; i < VEC; ++i) acc[i] += (double)(ok ? f[i] : 0.f);
        }
      }
      const double sum = reduce_scatter8<VEC>(acc, tl, [](double a, double b) { return a + b; });
      if (writer) store_mean1(dig + (size_t)gidx * D + ch, sum / (double)nvalid);
    }
  }
}

// Block count of each (sequence, KV head) pair, nb = ceil(len / BS) clamped into
// [0, max_blocks] (a negative or oversize length folded in before the division), and their
// exclusive prefix over the pairs into LDS pfx[0..npairs] (pfx[npairs] = the blocks of all
// sequences).  Every thread of the workgroup takes part; ends with a barrier.
template <int BS>
__device__ void block_count_prefix(const int32_t* __restrict__ seq_lens, int Hkv, int npairs,
                                   int max_blocks, int* pfx, int* wave_tot) {
  const int nt = blockDim.x, tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave, nw = nt / kWave;
  const int per = (npairs + nt - 1) / nt;
  const int p0 = min(npairs, tid * per), p1 = min(npairs, p0 + per);
  auto nb_of = [&](int p) {
    const int len = min(max(seq_lens[p / Hkv], 0), max_blocks * BS);
    return (len + BS - 1) / BS;
  };
  int local = 0;
  for (int p = p0; p < p1; ++p) local += nb_of(p);
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
    run += nb_of(p);
  }
  if (tid == nt - 1) {
    int tot = 0;
    for (int w = 0; w < nw; ++w) tot += wave_tot[w];
    pfx[npairs] = tot;
  }
  __syncthreads();
}

// Persistent waves over the blocks inside the sequences: the blocks of all (sequence, KV
// head) pairs laid end to end (Nb of them, by the prefix of the pairs' block counts), wave w
// of W takes [w Nb / W, (w + 1) Nb / W), so every wave has the same number of blocks whatever
// the sequence lengths (slots past a sequence's end are never visited).  It walks its range
// in windows of 64: lane j finds window block j's pair by a short forward scan of the prefix
// and reads its table entry and sequence length (one coalesced round); the resident blocks of
// the window are then digested in order, the next unit's page loads in flight while the
// current one is reduced.  Blocks without a page in the pool are skipped (their digests are
// not written).
template <typename T, int D, int BS, bool MINMAX>
__global__ __launch_bounds__(256) void digest_kernel(const T* __restrict__ k_pool,
                                                     const int32_t* __restrict__ table,
                                                     const int32_t* __restrict__ seq_lens,
                                                     T* __restrict__ dig, int Hkv, int npairs,
                                                     int max_blocks, int P, int W) {
  using PG = PageGeom<T, D, BS>;
  constexpr int VEC = PG::VEC, CGS = PG::CGS, TG = PG::TG, SL = PG::SL;
  extern __shared__ int pfx[];  // [npairs + 1]
  __shared__ int wave_tot[kDigestWaves];
  block_count_prefix<BS>(seq_lens, Hkv, npairs, max_blocks, pfx, wave_tot);
  const int Nb = pfx[npairs];
  const int lane = threadIdx.x % kWave;
  const int gw = blockIdx.x * kDigestWaves + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int i0 = (int)((long)gw * Nb / W), i1 = (int)((long)(gw + 1) * Nb / W);
  if (i0 >= i1) return;
  const int cl = lane / 8, tl = lane % 8;  // chunk within the group, token within the group

  // one slab of a page at once (CGS * TG <= 8 loads of 16 bytes per lane), read once
  // (non-temporal loads); the padding load after a window's last slab reads slab 0 of pool
  // page 0, the same lines for every wave, so that after the first they come from the cache
  auto load_slab = [&](int page, int slab, uint4 (&raw)[CGS][TG], bool pad) {
    page = pad ? 0 : page;
    slab = pad ? 0 : slab;
    const T* src = k_pool + (size_t)page * BS * D;
#pragma unroll
    for (int cs = 0; cs < CGS; ++cs)
#pragma unroll
      for (int tg = 0; tg < TG; ++tg)
        raw[cs][tg] =
            load_stream16(src + ((size_t)(8 * (CGS * slab + cs) + cl) * BS + 8 * tg + tl) * VEC);
  };

  // the pair of the wave's first block (pairs without blocks are passed over)
  int p = 0;
  {
    int lo = 0, hi = npairs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pfx[mid] <= i0) lo = mid; else hi = mid - 1;
    }
    p = __builtin_amdgcn_readfirstlane(lo);
  }
  for (int w0 = i0; w0 < i1; w0 += kWave) {
    const int g = min(w0 + lane, i1 - 1);
    int pj = p;
    while (pfx[pj + 1] <= g) ++pj;  // ends: pfx[npairs] = Nb > g
    const int b = g - pfx[pj];      // < the pair's block count <= max_blocks
    const int slot = pj * max_blocks + b;
    const int page_l = table[slot];
    const int len = seq_lens[pj / Hkv];
    const bool live = w0 + lane < i1 && page_l >= 0 && page_l < P;
    const int nval_l = min(BS, len - b * BS);  // >= 1: b < ceil(len / BS)
    p = __builtin_amdgcn_readlane(pj, kWave - 1);
    uint64_t mask = __ballot(live);
    if (mask == 0) continue;
    // the slabs of the window's resident blocks in order; the next slab is loaded before
    // the current one is reduced (past the last, a padding load)
    int j = __builtin_ctzll(mask);
    mask &= mask - 1;
    int sl = 0;
    uint4 cur[CGS][TG], nxt[CGS][TG];
    load_slab(__builtin_amdgcn_readlane(page_l, j), 0, cur, false);
    while (true) {
      int jn = j, sn = sl + 1;
      const bool last = sn == SL && !mask;
      if (sn == SL) {
        sn = last ? sl : 0;
        jn = last ? j : __builtin_ctzll(mask);
      }
      load_slab(__builtin_amdgcn_readlane(page_l, jn), sn, nxt, last);
      __builtin_amdgcn_sched_barrier(0);
      digest_block<T, D, BS, MINMAX>(cur, __builtin_amdgcn_readlane(nval_l, j), dig,
                                     __builtin_amdgcn_readlane(slot, j), cl, tl, sl);
      if (last) break;
      if (sn == 0) mask &= mask - 1;  // block jn begins
      j = jn;
      sl = sn;
#pragma unroll
      for (int cs = 0; cs < CGS; ++cs)
#pragma unroll
        for (int tg = 0; tg < TG; ++tg) cur[cs][tg] = nxt[cs][tg];
    }
  }
}

// Digest maintenance during decode: one wave per (sequence, KV head) recomputes the digest of
// the block that holds the sequence's last token, from its page, with the same arithmetic
// as the full build (so the entry is bit-identical to what digest_kernel writes).  A pair
// whose last block is not resident (or names a page outside the pool) is left unchanged.
template <typename T, int D, int BS, bool MINMAX>
__global__ __launch_bounds__(256) void refresh_kernel(const T* __restrict__ k_pool,
                                                      const int32_t* __restrict__ table,
                                                      const int32_t* __restrict__ seq_lens,
                                                      T* __restrict__ dig, int Hkv, int npairs,
                                                      int max_blocks, int P) {
  using PG = PageGeom<T, D, BS>;
  constexpr int VEC = PG::VEC, CGS = PG::CGS, TG = PG::TG;
  const int lane = threadIdx.x % kWave;
  const int pair = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (pair >= npairs) return;
  const int len = seq_lens[pair / Hkv];
  if (len < 1) return;
  const int b = min((len - 1) / BS, max_blocks - 1);
  const int page = table[(size_t)pair * max_blocks + b];
  if (page < 0 || page >= P) return;
  const int cl = lane / 8, tl = lane % 8;
  const T* src = k_pool + (size_t)page * BS * D;
#pragma unroll
  for (int sl = 0; sl < PG::SL; ++sl) {
    uint4 raw[CGS][TG];
#pragma unroll
    for (int cs = 0; cs < CGS; ++cs)
#pragma unroll
      for (int tg = 0; tg < TG; ++tg)
        raw[cs][tg] =
            load_stream16(src + ((size_t)(8 * (CGS * sl + cs) + cl) * BS + 8 * tg + tl) * VEC);
    digest_block<T, D, BS, MINMAX>(raw, min(BS, len - b * BS), dig,
                                   (long)pair * max_blocks + b, cl, tl, sl);
  }
}

// Waves the device holds at once for this kernel with `lds` bytes of dynamic LDS per
// workgroup (all CUs at full occupancy).
template <typename K>
int resident_waves(K kernel, int block, size_t lds) {
  int per_cu = 0, cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, lds) != hipSuccess ||
      per_cu < 1 || cus < 1)
    return 2048;  // any grid covers the blocks; this one keeps the chip busy
  return per_cu * cus * (block / kWave);
}

template <typename T, int D, int BS, bool MINMAX>
hipError_t launch_kind(const Shape& s, const void* k_pool, const int32_t* table,
                       const int32_t* lens, void* dig, hipStream_t stream) {
  const int npairs = s.B * s.Hkv;
  const int block = kDigestWaves * kWave;
  const size_t lds = (size_t)(npairs + 1) * sizeof(int);
  auto kernel = digest_kernel<T, D, BS, MINMAX>;
  // every wave resident at once (the block count is on the device: waves past it exit)
  const int waves = resident_waves(kernel, block, lds);
  const dim3 grid((unsigned)((waves + kDigestWaves - 1) / kDigestWaves));
  hipLaunchKernelGGL(kernel, grid, dim3(block), lds, stream, (const T*)k_pool, table, lens,
                     (T*)dig, s.Hkv, npairs, s.max_blocks, s.P, (int)grid.x * kDigestWaves);
  return hipGetLastError();
}

template <typename T, int D, int BS>
hipError_t launch_typed(const Shape& s, bool minmax, const void* k_pool, const int32_t* table,
                        const int32_t* lens, void* dig, hipStream_t stream) {
  return minmax ? launch_kind<T, D, BS, true>(s, k_pool, table, lens, dig, stream)
                : launch_kind<T, D, BS, false>(s, k_pool, table, lens, dig, stream);
}

template <typename T>
hipError_t launch_dtype(const Shape& s, bool minmax, const void* k, const int32_t* t,
                        const int32_t* l, void* dig, hipStream_t st) {
#define SA_BY_BS(FN, D)                                                  \
  (s.bs == 64   ? FN<T, D, 64>(s, minmax, k, t, l, dig, st)               \
   : s.bs == 32 ? FN<T, D, 32>(s, minmax, k, t, l, dig, st)               \
                : FN<T, D, 16>(s, minmax, k, t, l, dig, st))
  return s.d == 128 ? SA_BY_BS(launch_typed, 128) : SA_BY_BS(launch_typed, 64);
}

template <typename T, int D, int BS>
hipError_t refresh_typed(const Shape& s, bool minmax, const void* k, const int32_t* t,
                         const int32_t* l, void* dig, hipStream_t st) {
  const int npairs = s.B * s.Hkv;
  const dim3 grid((npairs + 3) / 4), block(256);
  if (minmax)
    hipLaunchKernelGGL((refresh_kernel<T, D, BS, true>), grid, block, 0, st, (const T*)k, t, l,
                       (T*)dig, s.Hkv, npairs, s.max_blocks, s.P);
  else
    hipLaunchKernelGGL((refresh_kernel<T, D, BS, false>), grid, block, 0, st, (const T*)k, t, l,
                       (T*)dig, s.Hkv, npairs, s.max_blocks, s.P);
  return hipGetLastError();
}

template <typename T>
hipError_t refresh_dtype(const Shape& s, bool minmax, const void* k, const int32_t* t,
                         const int32_t* l, void* dig, hipStream_t st) {
  return s.d == 128 ? SA_BY_BS(refresh_typed, 128) : SA_BY_BS(refresh_typed, 64);
#undef SA_BY_BS
}

}  // namespace

hipError_t launch_refresh_digests(const Shape& s, bool minmax, const void* k_pool,
                                  const int32_t* block_table, const int32_t* seq_lens,
                                  void* digests, hipStream_t stream) {
  if (s.bf16)
    return refresh_dtype<uint16_t>(s, minmax, k_pool, block_table, seq_lens, digests, stream);
  return refresh_dtype<float>(s, minmax, k_pool, block_table, seq_lens, digests, stream);
}

hipError_t launch_build_digests(const Shape& s, bool minmax, const void* k_pool,
                                const int32_t* block_table, const int32_t* seq_lens,
                                void* digests, hipStream_t stream) {
  if (s.bf16)
    return launch_dtype<uint16_t>(s, minmax, k_pool, block_table, seq_lens, digests, stream);
  return launch_dtype<float>(s, minmax, k_pool, block_table, seq_lens, digests, stream);
}

}  // namespace sa
