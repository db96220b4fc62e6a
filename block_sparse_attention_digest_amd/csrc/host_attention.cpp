// Host-side partial attention over the offloaded selected blocks -- the CPU half of
// ScoutAttention's collaborative attention, A_cpu = CPUATTN(Q, B_cpu) [arXiv:2603.27138,
// HTML Sec. 3.2 and 3.3; Algorithm 1]: the blocks of the top-k selection that are not
// resident on the GPU are attended on the CPU, next to the host memory that holds them, and
// the GPU merges that partial with its own.
//
// One task per (sequence, KV head): the G query heads that share the KV head walk the pair's
// offloaded blocks together, so each key and value row is read from memory once per pair.
// Each head keeps an online softmax in float32 (running maximum m, sum l, and the unscaled
// output row), updated once per block; the result is the normalised partial (o, m, l) with m
// in natural-log units,
// the form the GPU merge takes.  Tasks go to worker threads through an atomic counter, so
// pairs with many offloaded blocks do not hold the others up; a pair is always computed by
// one thread in one order, so the result does not depend on the thread count.
#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <condition_variable>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <stdexcept>
#include <thread>
#include <type_traits>
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

// W floats as one vector value (W = 8: two SSE registers or one AVX register; W = 16: one
// AVX-512 register where the build has it)
template <int W>
struct VecT {
  typedef float type __attribute__((vector_size(W * sizeof(float))));
};
template <int W>
using vecf = typename VecT<W>::type;

template <int W>
inline __attribute__((always_inline)) vecf<W> loadv(const float* p) {
  vecf<W> v;
  std::memcpy(&v, p, sizeof v);
  return v;
}
template <int W>
inline __attribute__((always_inline)) void storev(float* p, vecf<W> v) {
  std::memcpy(p, &v, sizeof v);
}
template <int W>
inline __attribute__((always_inline)) float hsum(vecf<W> s) {
  float t = 0.f;
  for (int i = 0; i < W; ++i) t += s[i];
  return t;
}

// One block of one pair for the G query heads: the block's rows converted to float (bf16
// keys and values), the block's G x nval logits (each key row read once for all heads), one
// online-softmax update per head (one rescale of the running output per block, not per
// token), then P V with a 2W-column strip of the G output rows held in registers across the
// block's tokens.  The head dimension is a multiple of 2W.  z holds G rows of zs logits.
template <typename T, int G, int W>
inline __attribute__((always_inline)) void block_body(const float* q, const void* k_rows,
                                                      const void* v_rows, float* kf, float* vf,
                                                      int nval, int D, float scale, float* m,
                                                      float* l, float* acc, float* z, int zs) {
  const float* K;
  const float* V;
  if constexpr (std::is_same<T, float>::value) {
    K = static_cast<const float*>(k_rows);
    V = static_cast<const float*>(v_rows);
  } else {
    const T* kr = static_cast<const T*>(k_rows);
    const T* vr = static_cast<const T*>(v_rows);
    const size_t n = (size_t)nval * D;
    for (size_t i = 0; i < n; ++i) {
      kf[i] = to_f32(kr[i]);
      vf[i] = to_f32(vr[i]);
    }
    K = kf;
    V = vf;
  }
  for (int t = 0; t < nval; ++t) {
    const float* kt = K + (size_t)t * D;
    vecf<W> s[G];
    for (int g = 0; g < G; ++g) s[g] = vecf<W>{};
    for (int c = 0; c < D; c += W) {
      const vecf<W> k = loadv<W>(kt + c);
      for (int g = 0; g < G; ++g) s[g] += loadv<W>(q + (size_t)g * D + c) * k;
    }
    for (int g = 0; g < G; ++g) z[g * zs + t] = hsum<W>(s[g]) * scale;
  }
  float alpha[G];
  for (int g = 0; g < G; ++g) {
    float* zg = z + g * zs;
    float mb = zg[0];
    for (int t = 1; t < nval; ++t) mb = std::max(mb, zg[t]);
    const float m_new = std::max(m[g], mb);
    alpha[g] = std::exp(m[g] - m_new);  // 0 for the first block (m = -inf)
    float psum = 0.f;
    for (int t = 0; t < nval; ++t) {
      zg[t] = std::exp(zg[t] - m_new);
      psum += zg[t];
    }
    l[g] = l[g] * alpha[g] + psum;
    m[g] = m_new;
  }
  for (int c0 = 0; c0 < D; c0 += 2 * W) {
    vecf<W> o[G][2];
    for (int g = 0; g < G; ++g) {
      float* ag = acc + (size_t)g * D + c0;
      o[g][0] = loadv<W>(ag) * alpha[g];
      o[g][1] = loadv<W>(ag + W) * alpha[g];
    }
    for (int t = 0; t < nval; ++t) {
      const float* vt = V + (size_t)t * D + c0;
      const vecf<W> v0 = loadv<W>(vt), v1 = loadv<W>(vt + W);
      for (int g = 0; g < G; ++g) {
        const float p = z[g * zs + t];
        o[g][0] += p * v0;
        o[g][1] += p * v1;
      }
    }
    for (int g = 0; g < G; ++g) {
      float* ag = acc + (size_t)g * D + c0;
      storev<W>(ag, o[g][0]);
      storev<W>(ag + W, o[g][1]);
    }
  }
}

#define SA_BLOCK_ARGS                                                                       \
  const float *q, const void *k_rows, const void *v_rows, float *kf, float *vf, int nval,  \
      int D, float scale, float *m, float *l, float *acc, float *z, int zs
#define SA_BLOCK_PASS q, k_rows, v_rows, kf, vf, nval, D, scale, m, l, acc, z, zs

template <typename T, int G>
__attribute__((target("avx512f,avx512bw,avx512vl,avx512dq,fma"))) void block_avx512(
    SA_BLOCK_ARGS) {
  block_body<T, G, 16>(SA_BLOCK_PASS);
}

template <typename T, int G>
__attribute__((target("avx2,fma"))) void block_avx2(SA_BLOCK_ARGS) {
  block_body<T, G, 8>(SA_BLOCK_PASS);
}

template <typename T, int G>
void block_base(SA_BLOCK_ARGS) {
  block_body<T, G, 8>(SA_BLOCK_PASS);
}

using BlockFn = void (*)(SA_BLOCK_ARGS);
#undef SA_BLOCK_ARGS
#undef SA_BLOCK_PASS

enum class Isa { base, avx2, avx512 };

// The widest build the CPU runs, or a narrower one named by SCOUTATTN_HOST_ISA ("base",
// "avx2"; read once), so that every build can be checked on one machine.
Isa host_isa() {
  static const Isa isa = [] {
    Isa best = Isa::base;
    if (__builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
        __builtin_cpu_supports("avx512vl") && __builtin_cpu_supports("avx512dq") &&
        __builtin_cpu_supports("fma"))
      best = Isa::avx512;
    else if (__builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma"))
      best = Isa::avx2;
    const char* want = std::getenv("SCOUTATTN_HOST_ISA");
    if (want && std::strcmp(want, "base") == 0) return Isa::base;
    if (want && std::strcmp(want, "avx2") == 0 && best != Isa::base) return Isa::avx2;
    return best;
  }();
  return isa;
}

// the block routine for a KV type and group size, in the widest build the CPU runs
template <typename T>
BlockFn pick_block(int G) {
  const Isa isa = host_isa();
  switch (G) {
#define SA_HOST_G(n)                                    \
  case n:                                               \
    return isa == Isa::avx512 ? block_avx512<T, n>      \
           : isa == Isa::avx2 ? block_avx2<T, n>        \
                              : block_base<T, n>;
    SA_HOST_G(1) SA_HOST_G(2) SA_HOST_G(3) SA_HOST_G(4)
    SA_HOST_G(5) SA_HOST_G(6) SA_HOST_G(7) SA_HOST_G(8)
#undef SA_HOST_G
  }
  return nullptr;
}

template <typename T>
void attend_pair(const HostAttnArgs& a, BlockFn block, int pair, float* kf, float* vf,
                 float* acc, float* z) {
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
    if (nval <= 0) continue;
    block(q, K + (size_t)page * BS * D, V + (size_t)page * BS * D, kf, vf, nval, D, a.scale, m,
          l, acc, z, BS);
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

// Takes pairs from `next` until none is left, with this thread's own block buffers in `buf`:
// one block of K and V as float, the G output rows, the G x bs logits.
template <typename T>
void work(const HostAttnArgs& a, std::atomic<int>& next, std::vector<float>& buf) {
  const BlockFn block = pick_block<T>(a.G);
  const int npairs = a.B * a.Hkv;
  const size_t blk = (size_t)a.bs * a.d;
  buf.resize(2 * blk + (size_t)a.G * a.d + (size_t)a.G * a.bs);
  float* kf = buf.data();
  float* vf = kf + blk;
  float* acc = vf + blk;
  float* z = acc + (size_t)a.G * a.d;
  for (int p = next.fetch_add(1); p < npairs; p = next.fetch_add(1))
    attend_pair<T>(a, block, p, kf, vf, acc, z);
}

// false if this thread could not take part (its buffers could not be allocated); the pairs
// it would have taken are then left to the other threads
bool work_any(const HostAttnArgs& a, std::atomic<int>& next, std::vector<float>& buf) noexcept {
  try {
    if (a.bf16)
      work<uint16_t>(a, next, buf);
    else
      work<float>(a, next, buf);
    return true;
  } catch (...) {
    return false;
  }
}

// Spins until pred() holds or `us` microseconds have passed; returns pred().  Waking a thread
// that sleeps on a condition variable costs tens of microseconds, which a layer's host task
// (well under a millisecond when little is offloaded) would pay twice.  The spin yields rather
// than pausing: with as many workers as CPUs, a spinning worker must give way to the runtime's
// own threads (the one that starts the next host task among them).
template <class Pred>
bool spin_until(Pred pred, int us) {
  const auto end = std::chrono::steady_clock::now() + std::chrono::microseconds(us);
  for (unsigned i = 0;; ++i) {
    if (pred()) return true;
    std::this_thread::yield();
    if ((i & 63) == 63 && std::chrono::steady_clock::now() > end) return pred();
  }
}

constexpr int kSpinUs = 300;  // about two GPU layers of the 40-layer decode step

}  // namespace

int host_threads(int requested) {
  if (requested > 0) return requested;
  const unsigned hw = std::thread::hardware_concurrency();
  return hw > 0 ? (int)hw : 1;
}

void host_partial_attention(const HostAttnArgs& a, int threads) {
  std::atomic<int> next{0};
  std::atomic<bool> ok{true};
  threads = std::max(1, std::min(threads, a.B * a.Hkv));
  std::vector<std::thread> pool;
  pool.reserve(threads - 1);
  for (int t = 1; t < threads; ++t)
    pool.emplace_back([&] {
      std::vector<float> buf;
      if (!work_any(a, next, buf)) ok = false;
    });
  std::vector<float> buf;
  if (!work_any(a, next, buf)) ok = false;  // the calling thread works too
  for (auto& th : pool) th.join();
  // a thread that failed took no pair, so a pair is left only if every thread failed
  if (next.load() < a.B * a.Hkv) throw std::runtime_error("no worker thread could run");
}

// ---- persistent workers ----------------------------------------------------------------------
// run() publishes one job and bumps the generation (under the mutex, so a sleeping worker cannot
// miss it); every worker takes part in each generation exactly once (run() returns only when
// all of them have reported back), so a job's arguments stay valid while any worker reads them.
// Between jobs a worker spins for a short while before it sleeps, and so does run() while it
// waits for the last worker.

HostPool::HostPool(int threads) {
  threads = std::max(1, threads);
  workers_.reserve(threads - 1);
  for (int t = 1; t < threads; ++t) workers_.emplace_back([this] { loop(); });
}

HostPool::~HostPool() {
  {
    std::lock_guard<std::mutex> lk(mu_);
    stop_.store(true);
  }
  start_.notify_all();
  for (auto& th : workers_) th.join();
}

void HostPool::loop() {
  uint64_t seen = 0;
  std::vector<float> buf;  // this worker's block buffers, kept across jobs
  auto ready = [&] { return stop_.load(std::memory_order_acquire) ||
                            gen_.load(std::memory_order_acquire) != seen; };
  for (;;) {
    if (!spin_until(ready, kSpinUs)) {
      std::unique_lock<std::mutex> lk(mu_);
      start_.wait(lk, ready);
    }
    if (stop_.load(std::memory_order_acquire)) return;
    seen = gen_.load(std::memory_order_acquire);
    work_any(*job_.load(std::memory_order_acquire), next_, buf);  // a failure leaves its
                                                                  // pairs to the others
    if (busy_.fetch_sub(1, std::memory_order_acq_rel) == 1) {
      std::lock_guard<std::mutex> lk(mu_);
      done_.notify_one();
    }
  }
}

bool HostPool::run(const HostAttnArgs& a) {
  job_.store(&a, std::memory_order_relaxed);
  next_.store(0, std::memory_order_relaxed);
  busy_.store((int)workers_.size(), std::memory_order_relaxed);
  {
    std::lock_guard<std::mutex> lk(mu_);
    gen_.fetch_add(1, std::memory_order_release);
  }
  start_.notify_all();
  work_any(a, next_, own_buf_);  // the calling thread works too
  auto finished = [&] { return busy_.load(std::memory_order_acquire) == 0; };
  if (!spin_until(finished, kSpinUs)) {
    std::unique_lock<std::mutex> lk(mu_);
    done_.wait(lk, finished);
  }
  job_.store(nullptr, std::memory_order_relaxed);
  // a thread that failed took no pair, and a pair taken is always finished: the job is
  // whole unless every thread failed
  return next_.load() >= a.B * a.Hkv;
}

}  // namespace sa
