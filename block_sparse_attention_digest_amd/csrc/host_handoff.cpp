// The host half of the offload step's flag hand-off (the GPU half is the signal and bounded
// wait kernels): one dispatcher thread per plan serves every layer whose ready flag the GPU
// has advanced, and always ends by writing the layer's done flag.  Host-only code (no HIP
// calls): the flags are plain words in memory the device also maps.
#include <chrono>
#include <utility>

#include "host.hpp"

namespace sa {
namespace {

inline uint32_t load_acquire(const uint32_t* p) { return __atomic_load_n(p, __ATOMIC_ACQUIRE); }
inline void store_release(uint32_t* p, uint32_t v) { __atomic_store_n(p, v, __ATOMIC_RELEASE); }

}  // namespace

FlagDispatcher::FlagDispatcher(uint32_t* flags, int layers, Task task, Empty empty)
    : flags_(flags), layers_(layers), task_(std::move(task)), empty_(std::move(empty)) {
  for (int i = 0; i < 2 * layers + 1; ++i) store_release(flags_ + i, 0);
  thread_ = std::thread([this] { loop(); });
}

FlagDispatcher::~FlagDispatcher() {
  stop_.store(true);
  thread_.join();
}

bool FlagDispatcher::gpu_timed_out() const { return load_acquire(flags_ + 2 * layers_) != 0; }

void FlagDispatcher::drain() const {
  for (int j = 0; j < layers_; ++j)
    while (load_acquire(flags_ + layers_ + j) != load_acquire(flags_ + j) && !stop_.load())
      std::this_thread::sleep_for(std::chrono::microseconds(20));
}

void FlagDispatcher::loop() {
  using clk = std::chrono::steady_clock;
  // A layer's flag usually comes within a layer of GPU work after the last one: the thread
  // yields for the first 200 us of an idle spell, then sleeps 20 us at a time, and after
  // 10 ms of idleness 200 us at a time (between steps it need not hold a core).
  auto idle_since = clk::now();
  int next = 0;
  while (!stop_.load()) {
    int j = -1;
    uint32_t v = 0;
    for (int t = 0; t < layers_; ++t) {
      const int c = (next + t) % layers_;
      v = load_acquire(flags_ + c);
      if (v != load_acquire(flags_ + layers_ + c)) {
        j = c;
        break;
      }
    }
    if (j < 0) {
      const auto idle = clk::now() - idle_since;
      if (idle < std::chrono::microseconds(200))
        std::this_thread::yield();
      else
        std::this_thread::sleep_for(std::chrono::microseconds(
            idle < std::chrono::milliseconds(10) ? 20 : 200));
      continue;
    }
    if (!task_(j)) ++failures_;  // a failed task has written the empty partial
    store_release(flags_ + layers_ + j, v);
    next = (j + 1) % layers_;
    idle_since = clk::now();
  }
  // stopping: close every layer raised but not served
  for (int j = 0; j < layers_; ++j) {
    const uint32_t v = load_acquire(flags_ + j);
    if (v != load_acquire(flags_ + layers_ + j)) {
      empty_(j);
      store_release(flags_ + layers_ + j, v);
    }
  }
}

}  // namespace sa
