// Host-side (CPU) part of the library: the partial attention over offloaded blocks.
#pragma once

#include <atomic>
#include <condition_variable>
#include <cstddef>
#include <cstdint>
#include <mutex>
#include <thread>
#include <vector>

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
// computes every (sequence, query head) partial; blocks until done; throws if no thread could
// run
void host_partial_attention(const HostAttnArgs& args, int threads);

// A fixed set of worker threads for repeated host partials (one per decode layer): threads-1
// workers wait between jobs, and the thread that calls run() works beside them.  run() is not
// reentrant: one job at a time.
class HostPool {
 public:
  explicit HostPool(int threads);
  ~HostPool();
  HostPool(const HostPool&) = delete;
  HostPool& operator=(const HostPool&) = delete;
  // computes every (sequence, query head) partial of `args`; blocks until done; false if no
  // thread could run (out of memory)
  bool run(const HostAttnArgs& args);
  int threads() const { return (int)workers_.size() + 1; }

 private:
  void loop();
  std::mutex mu_;
  std::condition_variable start_, done_;
  std::atomic<const HostAttnArgs*> job_{nullptr};
  std::atomic<uint64_t> gen_{0};
  std::atomic<int> busy_{0};
  std::atomic<bool> stop_{false};
  std::atomic<int> next_{0};
  std::vector<float> own_buf_;  // the block buffers of the thread that calls run()
  std::vector<std::thread> workers_;
};

}  // namespace sa
