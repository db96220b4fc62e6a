// Stream-ordered flags in memory the host shares (page-locked, coherent), for the offload
// step's hand-over of each layer's CPU side [ScoutAttention, arXiv:2603.27138, HTML Sec. 3.3:
// the CPU computes its partial of layer i while the GPU works one layer ahead, and the GPU
// merges the two at layer i].
//
// signal_kernel advances a counter flag (ready = ready + 1) once everything before it on its
// stream has finished (its writes are then visible to the host); only the device writes it,
// in stream order, so the counter needs no atomic update.  wait_kernel holds its stream until
// a second flag (done, written by the host) equals the counter: one lane polls with a
// system-scope load, pausing between reads, and gives up after a bounded number of rounds --
// it then records the timeout in a word the host reads and returns -- so the wait ends
// whatever the host does.  Neither kernel takes a value from the host, so both can be
// captured in a graph and replayed.
#include "common.hpp"
#include "kernels.hpp"

namespace sa {
namespace {

__global__ __launch_bounds__(64) void signal_kernel(uint32_t* ready) {
  if (threadIdx.x == 0) {
    const uint32_t v = __hip_atomic_load(ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_store(ready, v + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

__global__ __launch_bounds__(64) void wait_kernel(const uint32_t* done, const uint32_t* ready,
                                                  uint32_t rounds, uint32_t* timeouts) {
  if (threadIdx.x != 0) return;
  const uint32_t want = __hip_atomic_load(ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  for (uint32_t r = 0; r < rounds; ++r) {
    if (__hip_atomic_load(done, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_SYSTEM) == want) return;
    __builtin_amdgcn_s_sleep(127);  // 127 x 64 shader clocks between reads
  }
  if (__hip_atomic_load(done, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_SYSTEM) != want)
    __hip_atomic_store(timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

}  // namespace

uint32_t wait_rounds(int ms) {
  // a round is a read over the host link (about a microsecond) and an 8128-clock pause (3.4 us
  // at 2.4 GHz, longer at lower clocks): counted as 4 us, so the bound is about `ms`
  const long r = (long)ms * 250;
  return (uint32_t)(r < 1 ? 1 : (r > 0x7fffffffL ? 0x7fffffffL : r));
}

hipError_t launch_signal(uint32_t* ready, hipStream_t stream) {
  hipLaunchKernelGGL(signal_kernel, dim3(1), dim3(kWave), 0, stream, ready);
  return hipGetLastError();
}

hipError_t launch_wait(const uint32_t* done, const uint32_t* ready, uint32_t rounds,
                       uint32_t* timeouts, hipStream_t stream) {
  hipLaunchKernelGGL(wait_kernel, dim3(1), dim3(kWave), 0, stream, done, ready, rounds,
                     timeouts);
  return hipGetLastError();
}

}  // namespace sa
