// Host-side (CPU) part of the library: the partial attention over offloaded blocks.
#pragma once

#include <atomic>
#include <condition_variable>
#include <cstddef>
#include <cstdint>
#include <functional>
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

// The flag hand-off of the offload step: a host thread that serves each layer whose ready
// flag the GPU has advanced -- it runs the layer's task, then sets the layer's done flag to
// the ready value it served -- while a bounded wait on the GPU holds the layer's merge until
// done equals ready.  The flags are caller-owned words both sides see (page-locked, coherent
// memory): ready[0, L) (advanced only by the GPU), done[L, 2L) (written only here), and word
// 2L, where the GPU's wait records a timeout.  Every ready value seen gets its done flag
// written: after the task, or after a failed task (the layer's partial then empty), and at
// shutdown for a layer raised but not yet served (partial empty).  The thread needs no job
// posted by the host, so a step may be replayed from a graph.  Pending layers are served in
// cyclic layer order from the last one served.
class FlagDispatcher {
 public:
  using Task = std::function<bool(int)>;   // runs the layer's CPU side; false: it failed
  using Empty = std::function<void(int)>;  // writes the layer's empty partial
  FlagDispatcher(uint32_t* flags, int layers, Task task, Empty empty);  // zeroes the flags
  ~FlagDispatcher();
  FlagDispatcher(const FlagDispatcher&) = delete;
  FlagDispatcher& operator=(const FlagDispatcher&) = delete;
  // waits until every layer's done flag equals its ready flag
  void drain() const;
  int64_t failures() const { return failures_.load(); }
  bool gpu_timed_out() const;
  uint32_t* flags() const { return flags_; }
  int layers() const { return layers_; }

 private:
  void loop();
  uint32_t* flags_;
  int layers_;
  Task task_;
  Empty empty_;
  std::atomic<bool> stop_{false};
  std::atomic<int64_t> failures_{0};
  std::thread thread_;
};

}  // namespace sa
