// Host-side partial attention over the offloaded selected blocks -- the CPU half of
// ScoutAttention's collaborative attention, A_cpu = CPUATTN(Q, B_cpu) [arXiv:2603.27138,
// HTML Sec. 3.2 and 3.3; Algorithm 1]: the blocks of the top-k selection that are not
// resident on the GPU are attended on the CPU, next to the host memory that holds them, and
// the GPU merges that partial with its own.
//
// One task per (sequence, KV head): the G query heads that share the KV head walk the pair's
// offloaded blocks together, so each key and value row is read from memory once per pair.
// Each head keeps an online softmax in float32 (running maximum m, sum l, and the unscaled
// output row); the result is the normalised partial (o, m, l) with m in natural-log units,
// the form the GPU merge takes.  Tasks go to worker threads through an atomic counter, so
// pairs with many offloaded blocks do not hold the others up; a pair is always computed by
// one thread in one order, so the result does not depend on the thread count.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

#include "host.hpp"

namespace sa {
namespace {

constexpr int kMaxGroup = 8;  // query heads per KV head

inline float to_f32(float v) { return v; }
inline float to_f32(uint16_t v) {  // bfloat16 bit pattern
  const uint32_t u = (uint32_t)v << 16;
  float f;
  std::memcpy(&f, &u, sizeof f);
  return f;
}

// dot product with eight independent partial sums (so the compiler can keep them in SIMD
// lanes); d is a multiple of 8
inline float dot(const float* a, const float* b, int d) {
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < d; c += 8)
    for (int i = 0; i < 8; ++i) s[i] += a[c + i] * b[c + i];
  return ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
}

template <typename T>
void attend_pair(const HostAttnArgs& a, int pair, float* kf, float* vf, float* acc) {
  const int G = a.G, D = a.d, BS = a.bs;
  const int s = pair / a.Hkv, h = pair % a.Hkv;
  const int len = a.seq_lens[s];
  const int n = std::min(std::max(a.n_cpu[pair], 0), a.list_stride);
  const T* K = static_cast<const T*>(a.k_host);
  const T* V = static_cast<const T*>(a.v_host);
  const float* q = a.q + ((size_t)s * a.Hq + (size_t)h * G) * D;
  float m[kMaxGroup], l[kMaxGroup];
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
  }
  std::fill(acc, acc + (size_t)G * D, 0.f);
  for (int j = 0; j < n; ++j) {
    // list entries, host pages and lengths outside their ranges are skipped
    const int b = a.cpu_blocks[(size_t)pair * a.list_stride + j];
    if (b < 0 || b >= a.max_blocks) continue;
    const int page = a.host_table[(size_t)pair * a.max_blocks + b];
    if (page < 0 || page >= a.host_pages) continue;
    const int nval = std::min(BS, len - b * BS);
    for (int t = 0; t < nval; ++t) {
      const T* kr = K + ((size_t)page * BS + t) * D;
      const T* vr = V + ((size_t)page * BS + t) * D;
      for (int c = 0; c < D; ++c) {
        kf[c] = to_f32(kr[c]);
        vf[c] = to_f32(vr[c]);
      }
      for (int g = 0; g < G; ++g) {
        const float z = dot(q + (size_t)g * D, kf, D) * a.scale;
        float* o = acc + (size_t)g * D;
        if (z > m[g]) {  // a new maximum: rescale what is accumulated so far
          const float alpha = std::exp(m[g] - z);  // 0 for the first token (m = -inf)
          l[g] = l[g] * alpha + 1.f;
          for (int c = 0; c < D; ++c) o[c] = o[c] * alpha + vf[c];
          m[g] = z;
        } else {
          const float p = std::exp(z - m[g]);
          l[g] += p;
          for (int c = 0; c < D; ++c) o[c] += p * vf[c];
        }
      }
    }
  }
  for (int g = 0; g < G; ++g) {
    const size_t row = (size_t)s * a.Hq + (size_t)h * G + g;
    float* o_out = a.o + row * D;
    if (l[g] > 0.f) {
      const float inv = 1.f / l[g];
      for (int c = 0; c < D; ++c) o_out[c] = acc[(size_t)g * D + c] * inv;
      a.m[row] = m[g];
      a.l[row] = l[g];
    } else {  // nothing offloaded for this pair: the empty partial
      std::fill(o_out, o_out + D, 0.f);
      a.m[row] = -INFINITY;
      a.l[row] = 0.f;
    }
  }
}

template <typename T>
void run(const HostAttnArgs& a, int threads) {
  const int npairs = a.B * a.Hkv;
  std::atomic<int> next{0};
  auto worker = [&]() {
    std::vector<float> buf((size_t)(2 + a.G) * a.d);
    for (int p = next.fetch_add(1); p < npairs; p = next.fetch_add(1))
      attend_pair<T>(a, p, buf.data(), buf.data() + a.d, buf.data() + 2 * a.d);
  };
  threads = std::max(1, std::min(threads, npairs));
  std::vector<std::thread> pool;
  pool.reserve(threads - 1);
  for (int t = 1; t < threads; ++t) pool.emplace_back(worker);
  worker();  // the calling thread works too
  for (auto& th : pool) th.join();
}

}  // namespace

int host_threads(int requested) {
  if (requested > 0) return requested;
  const unsigned hw = std::thread::hardware_concurrency();
  return hw > 0 ? (int)hw : 1;
}

void host_partial_attention(const HostAttnArgs& a, int threads) {
  if (a.bf16)
    run<uint16_t>(a, threads);
  else
    run<float>(a, threads);
}

}  // namespace sa
