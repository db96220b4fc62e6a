// Periodic KV recall [arXiv:2603.27138, HTML Sec. 3.4]: offloaded blocks that the current
// selection needs come back from host memory into GPU pages, so the share of the budget the
// CPU attends stays small.  Two launches:
//   recall_plan_kernel -- one wave per (sequence, KV head): which blocks move where, if the
//     layer is due (optionally: its offloaded selected blocks above a threshold).  The
//     candidates are the pair's offloaded selected blocks (cpu list order) that lie inside the
//     sequence, are not resident and have a host page; the evicted blocks are the resident
//     blocks outside the current selection, in ascending order; candidate t takes the page of
//     evicted block t.  The block table is updated in place and the copies are listed.
//   recall_copy_kernel -- one workgroup per listed copy: the block's keys and values are read
//     from page-locked host memory (16-byte reads of the token rows, staged in LDS) and
//     written into the page in the pool layouts: K chunk-major [d/x][bs][x], V [bs/16][d][16].
#include "common.hpp"
#include "kernels.hpp"

namespace sa {
namespace {

constexpr int kCopyThreads = 256;

__global__ __launch_bounds__(kWave) void recall_plan_kernel(
    const int* __restrict__ seq_lens, int Hkv, int bs, int max_blocks, int num_pages,
    int* __restrict__ block_table, const int* __restrict__ gpu_blocks,
    const int* __restrict__ n_gpu, const int* __restrict__ cpu_blocks,
    const int* __restrict__ n_cpu, int list_stride, const int* __restrict__ host_table,
    int host_pages, int max_recall, long threshold, int2* __restrict__ copies,
    int* __restrict__ n_recalled) {
  extern __shared__ int lds[];
  const int words = (max_blocks + 31) / 32;
  unsigned* sel = reinterpret_cast<unsigned*>(lds);  // selection bitmap over the blocks
  int* cand = lds + words;                             // [max_recall] blocks to bring back
  int* vict = cand + max_recall;                       // [max_recall] blocks to evict
  const int pair = blockIdx.x;
  const int lane = threadIdx.x;
  const int len = seq_lens[pair / Hkv];
  const int nb = len > 0 ? min((len + bs - 1) / bs, max_blocks) : 0;
  int* tab = block_table + (size_t)pair * max_blocks;
  const int* htab = host_table + (size_t)pair * max_blocks;
  const int* gl = gpu_blocks + (size_t)pair * list_stride;
  const int* cl = cpu_blocks + (size_t)pair * list_stride;
  const int ng = min(max(n_gpu[pair], 0), list_stride);
  const int nc = min(max(n_cpu[pair], 0), list_stride);

  // the trigger (threshold >= 0): the layer's offloaded selected blocks, over all pairs, must
  // exceed it, or nothing moves; every workgroup counts them itself
  if (threshold >= 0) {
    long total = 0;
    const int pairs = gridDim.x;
    for (int p = lane; p < pairs; p += kWave) total += min(max(n_cpu[p], 0), list_stride);
    for (int off = kWave / 2; off > 0; off >>= 1) total += __shfl_xor(total, off);
    if (total <= threshold) {
      if (lane == 0) n_recalled[pair] = 0;
      return;
    }
  }
  for (int w = lane; w < words; w += kWave) sel[w] = 0u;
  __syncthreads();
  for (int j = lane; j < ng + nc; j += kWave) {
    const int b = j < ng ? gl[j] : cl[j - ng];
    if (b >= 0 && b < max_blocks) atomicOr(&sel[b >> 5], 1u << (b & 31));
  }
  __syncthreads();

  const unsigned long long below = (1ull << lane) - 1ull;
  // candidates, in list order
  int ncand = 0;
  for (int j0 = 0; j0 < nc && ncand < max_recall; j0 += kWave) {
    const int j = j0 + lane;
    const int b = j < nc ? cl[j] : -1;
    const bool ok = b >= 0 && b < nb && tab[b] < 0 && htab[b] >= 0 && htab[b] < host_pages;
    const unsigned long long m = __ballot(ok);
    const int r = ncand + __popcll(m & below);
    if (ok && r < max_recall) cand[r] = b;
    ncand += __popcll(m);
  }
  ncand = min(ncand, max_recall);
  // evicted blocks: resident, with a valid page, not selected, ascending
  int nvict = 0;
  for (int b0 = 0; b0 < nb && nvict < ncand; b0 += kWave) {
    const int b = b0 + lane;
    bool ok = false;
    if (b < nb) {
      const int page = tab[b];
      ok = page >= 0 && page < num_pages && !((sel[b >> 5] >> (b & 31)) & 1u);
    }
    const unsigned long long m = __ballot(ok);
    const int r = nvict + __popcll(m & below);
    if (ok && r < ncand) vict[r] = b;
    nvict += __popcll(m);
  }
  const int n = min(ncand, nvict);
  __syncthreads();
  // the evicted and recalled blocks are disjoint (outside and inside the selection), so
  // each lane's table entries are its own
  for (int t = lane; t < n; t += kWave) {
    const int v = vict[t], b = cand[t];
    const int page = tab[v];
    tab[v] = -1;
    tab[b] = page;
    copies[(size_t)pair * max_recall + t] = make_int2(page, htab[b]);
  }
  if (lane == 0) n_recalled[pair] = n;
}

template <typename T>
__global__ __launch_bounds__(kCopyThreads) void recall_copy_kernel(
    const int* __restrict__ n_recalled, const int2* __restrict__ copies, int max_recall,
    const T* __restrict__ k_host, const T* __restrict__ v_host, T* __restrict__ k_pool,
    T* __restrict__ v_pool, int bs, int d) {
  constexpr int E = 16 / sizeof(T);  // elements per 16-byte chunk
  extern __shared__ uint4 stage[];   // [2][bs * d / E]: the host rows of K, then of V
  const int pair = blockIdx.y, t = blockIdx.x;
  if (t >= n_recalled[pair]) return;  // the whole workgroup leaves together
  const int2 cp = copies[(size_t)pair * max_recall + t];  // (pool page, host page)
  const int nc = d / E;         // chunks per token row
  const int chunks = bs * nc;   // chunks per page
  const size_t page_elems = (size_t)bs * d;
  const uint4* ks = reinterpret_cast<const uint4*>(k_host + (size_t)cp.y * page_elems);
  const uint4* vs = reinterpret_cast<const uint4*>(v_host + (size_t)cp.y * page_elems);
  for (int c = threadIdx.x; c < chunks; c += kCopyThreads) {
    stage[c] = ks[c];
    stage[chunks + c] = vs[c];
  }
  __syncthreads();
  // K: destination chunk i holds chunk c = i / bs of token i % bs
  uint4* kd = reinterpret_cast<uint4*>(k_pool + (size_t)cp.x * page_elems);
  for (int i = threadIdx.x; i < chunks; i += kCopyThreads)
    kd[i] = stage[(i % bs) * nc + i / bs];
  // V: destination chunk i is in 16-token half h; it holds E consecutive tokens of one channel
  T* vd = v_pool + (size_t)cp.x * page_elems;
  const T* vt = reinterpret_cast<const T*>(stage + chunks);
  const int per_half = 16 * d / E;
  for (int i = threadIdx.x; i < chunks; i += kCopyThreads) {
    const int h = i / per_half, r = i % per_half;
    const int ch = r / (16 / E), t0 = h * 16 + (r % (16 / E)) * E;
    T v[E];
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = vt[(size_t)(t0 + e) * d + ch];
    uint4 w;
    __builtin_memcpy(&w, v, sizeof(w));
    *reinterpret_cast<uint4*>(vd + (size_t)i * E) = w;
  }
}

}  // namespace

size_t recall_plan_lds_bytes(const Shape& s, int max_recall) {
  return sizeof(int) * ((size_t)(s.max_blocks + 31) / 32 + 2 * (size_t)max_recall);
}

hipError_t launch_recall(const Shape& s, int list_stride, int max_recall, const int* seq_lens,
                         int* block_table, const int* gpu_blocks, const int* n_gpu,
                         const int* cpu_blocks, const int* n_cpu, const void* k_host,
                         const void* v_host, const int* host_table, int host_pages,
                         void* k_pool, void* v_pool, int* n_recalled, void* copies,
                         long threshold, hipStream_t stream) {
  const int pairs = s.B * s.Hkv;
  int2* cp = static_cast<int2*>(copies);
  hipLaunchKernelGGL(recall_plan_kernel, dim3(pairs), dim3(kWave),
                     recall_plan_lds_bytes(s, max_recall), stream, seq_lens, s.Hkv, s.bs,
                     s.max_blocks, s.P, block_table, gpu_blocks, n_gpu, cpu_blocks, n_cpu,
                     list_stride, host_table, host_pages, max_recall, threshold, cp,
                     n_recalled);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(max_recall, pairs), block(kCopyThreads);
  const size_t lds = 2 * (size_t)s.bs * s.d * (s.bf16 ? 2 : 4);
  if (s.bf16)
    hipLaunchKernelGGL(recall_copy_kernel<uint16_t>, grid, block, lds, stream, n_recalled, cp,
                       max_recall, static_cast<const uint16_t*>(k_host),
                       static_cast<const uint16_t*>(v_host), static_cast<uint16_t*>(k_pool),
                       static_cast<uint16_t*>(v_pool), s.bs, s.d);
  else
    hipLaunchKernelGGL(recall_copy_kernel<float>, grid, block, lds, stream, n_recalled, cp,
                       max_recall, static_cast<const float*>(k_host),
                       static_cast<const float*>(v_host), static_cast<float*>(k_pool),
                       static_cast<float*>(v_pool), s.bs, s.d);
  return hipGetLastError();
}

}  // namespace sa
