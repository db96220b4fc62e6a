// Host-side (CPU) part of the library: the partial attention over offloaded blocks.
#pragma once

#include <cstddef>
#include <cstdint>

namespace sa {

// Arguments of the host partial attention, all host memory (shapes as in the C ABI).
struct HostAttnArgs {
  int B, Hq, Hkv, G, d, bs, max_blocks, host_pages, list_stride;
  bool bf16;
  float scale;
  const float* q;            // [B][Hq][d]
  const void* k_host;        // [host_pages][bs][d], KV dtype
  const void* v_host;        // [host_pages][bs][d], KV dtype
  const int32_t* host_table; // [B][Hkv][max_blocks]: host page of each block, or -1
  const int32_t* seq_lens;   // [B]
  const int32_t* cpu_blocks; // [B][Hkv][list_stride]
  const int32_t* n_cpu;      // [B][Hkv]
  float* o;                  // [B][Hq][d]
  float* m;                  // [B][Hq]
  float* l;                  // [B][Hq]
};

// worker threads for a request (<= 0: the machine's hardware threads)
int host_threads(int requested);
// computes every (sequence, query head) partial; blocks until done
void host_partial_attention(const HostAttnArgs& args, int threads);

}  // namespace sa
