// Dense paged decode attention (FullKV, the pages' uncompressed baseline [arXiv:2603.27138,
// HTML Sec. 4]): every block of every sequence is attended.  The block-sparse attention kernel
// already streams whatever list it is given, split evenly over the waves of the grid, which is
// the schedule a dense kernel wants too; so the dense call builds the list of every resident
// block of each (sequence, KV head) and runs that kernel and its reduce.  Blocks without a
// page are left out, so the call is FullKV exactly when every block is resident.
#include "common.hpp"
#include "kernels.hpp"

namespace sa {
namespace {

// One wave per (sequence, KV head): the resident blocks below nb_s, ascending, compacted with
// a ballot per 64 blocks.
__global__ __launch_bounds__(kWave) void dense_lists_kernel(const int* __restrict__ seq_lens,
                                                            const int* __restrict__ block_table,
                                                            int Hkv, int bs, int max_blocks,
                                                            int num_pages, int* __restrict__ lists,
                                                            int* __restrict__ counts) {
  const int pair = blockIdx.x;
  const int lane = threadIdx.x;
  const int len = seq_lens[pair / Hkv];
  const int nb = len > 0 ? min((len + bs - 1) / bs, max_blocks) : 0;
  const int* tab = block_table + (size_t)pair * max_blocks;
  int* out = lists + (size_t)pair * max_blocks;
  const unsigned long long below = (1ull << lane) - 1ull;
  int n = 0;
  for (int b0 = 0; b0 < nb; b0 += kWave) {
    const int b = b0 + lane;
    bool ok = false;
    if (b < nb) {
      const int page = tab[b];
      ok = page >= 0 && page < num_pages;
    }
    const unsigned long long m = __ballot(ok);
    if (ok) out[n + __popcll(m & below)] = b;
    n += __popcll(m);
  }
  if (lane == 0) counts[pair] = n;
}

}  // namespace

hipError_t launch_dense_lists(const Shape& s, const int* seq_lens, const int* block_table,
                              int* lists, int* counts, hipStream_t stream) {
  hipLaunchKernelGGL(dense_lists_kernel, dim3(s.B * s.Hkv), dim3(kWave), 0, stream, seq_lens,
                     block_table, s.Hkv, s.bs, s.max_blocks, s.P, lists, counts);
  return hipGetLastError();
}

}  // namespace sa
