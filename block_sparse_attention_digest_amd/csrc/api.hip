// C ABI of libscoutattn: argument checks, workspace layout and kernel dispatch for the
// GPU-side decode path of ScoutAttention [arXiv:2603.27138, HTML Sec. 3.2-3.3;
// Algorithm 1].  Every argument is checked here, on the host, before anything is launched.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/scoutattn.h"
#include <exception>

#include "host.hpp"
#include "kernels.hpp"

namespace {

thread_local std::string g_err;

// Kernel profiling events of the calling thread, per stage (sa_profile_kernels).
struct ProfileEvents {
  std::vector<hipEvent_t> start, stop;
  size_t next = 0;
};
thread_local ProfileEvents g_prof[SA_PROFILE_STAGES];

// Events that order the streams of sa_decode_step, created on first use and reused by
// every later call on the same thread (re-recording an event does not affect waits
// enqueued before it, so one event per fork/join point of a call is enough).  Creating
// and destroying events on every call would block the host.  They live as long as the
// thread: destroying them from a thread-exit destructor could run after the HIP runtime
// itself has shut down.
struct EventPool {
  std::vector<hipEvent_t> ev;
  size_t next = 0;
};
thread_local EventPool g_events;

void next_profile_events(hipEvent_t* e0, hipEvent_t* e1,
                         sa_profile_stage stage = SA_PROFILE_ATTENTION) {
  ProfileEvents& P = g_prof[stage];
  *e0 = *e1 = nullptr;
  if (P.next < P.start.size()) {
    *e0 = P.start[P.next];
    *e1 = P.stop[P.next];
    ++P.next;
  }
}

sa_status fail(sa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

sa_status ok() {
  g_err.clear();
  return SA_OK;
}

sa_status hip_fail(hipError_t e, const char* what) {
  return fail(SA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kMaxBlocks = 8192;  // LDS budget of the top-k workgroup
constexpr int kMaxPairs = 8192;   // LDS budget of the attention workgroups' pair prefix

sa_status check_dims(const sa_dims* d, sa::Shape* s) {
  if (!d) return fail(SA_ERR_INVALID_ARG, "dims is NULL");
  if (d->batch < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1 || d->head_dim < 1 ||
      d->block_size < 1 || d->max_blocks < 1 || d->num_pages < 1)
    return fail(SA_ERR_INVALID_ARG,
                "dims: batch, heads, head_dim, block_size, max_blocks, num_pages must be >= 1");
  if (d->num_q_heads % d->num_kv_heads != 0)
    return fail(SA_ERR_INVALID_ARG, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
                d->num_q_heads, d->num_kv_heads);
  const int G = d->num_q_heads / d->num_kv_heads;
  if (G > 8) return fail(SA_ERR_UNSUPPORTED, "query heads per KV head %d > 8", G);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(SA_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", d->head_dim);
  if (d->block_size != 16 && d->block_size != 32 && d->block_size != 64)
    return fail(SA_ERR_UNSUPPORTED, "block_size %d not in {16, 32, 64}", d->block_size);
  if (d->max_blocks > kMaxBlocks)
    return fail(SA_ERR_UNSUPPORTED, "max_blocks %d > %d", d->max_blocks, kMaxBlocks);
  if ((long)d->batch * d->num_kv_heads > kMaxPairs)
    return fail(SA_ERR_UNSUPPORTED, "batch * num_kv_heads %ld > %d",
                (long)d->batch * d->num_kv_heads, kMaxPairs);
  if (d->kv_dtype != SA_F32 && d->kv_dtype != SA_BF16)
    return fail(SA_ERR_UNSUPPORTED, "kv_dtype %d is neither SA_F32 nor SA_BF16", (int)d->kv_dtype);
  s->B = d->batch;
  s->Hq = d->num_q_heads;
  s->Hkv = d->num_kv_heads;
  s->G = G;
  s->d = d->head_dim;
  s->bs = d->block_size;
  s->max_blocks = d->max_blocks;
  s->P = d->num_pages;
  s->bf16 = d->kv_dtype == SA_BF16;
  return SA_OK;
}

sa_status check_kind(sa_digest_kind k) {
  if (k != SA_DIGEST_MEAN && k != SA_DIGEST_MINMAX)
    return fail(SA_ERR_INVALID_ARG, "unknown digest kind %d", (int)k);
  return SA_OK;
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of selection + attention: first the selection's hand-over buffers (their
// counters stay zero between calls), then the attention partials.  The selection region is
// sized for the larger of the two digest kinds, so one workspace serves both.
struct Layout {
  size_t sel, parts, total;
  sa::AttnPlan plan;
};
size_t select_ws_bytes(const sa::Shape& s) {
  return align_up(std::max(sa::select_plan(s, false).ws_bytes, sa::select_plan(s, true).ws_bytes));
}
Layout layout(const sa::Shape& s, int top_k) {
  Layout L;
  L.plan = sa::attn_plan(s, top_k);
  L.sel = 0;
  L.parts = select_ws_bytes(s);
  L.total = L.parts + align_up(L.plan.ws_bytes);
  return L;
}

sa_status check_gemm_shape(int32_t m, int32_t n, int32_t k) {
  if (m < 1 || n < 1 || k < 1) return fail(SA_ERR_INVALID_ARG, "GEMM sizes must be >= 1");
  if (m > 256) return fail(SA_ERR_UNSUPPORTED, "GEMM m = %d > 256", m);
  if (n % 64 != 0 || k % 64 != 0)
    return fail(SA_ERR_UNSUPPORTED, "GEMM n (%d) and k (%d) must be multiples of 64", n, k);
  return SA_OK;
}

#define SA_CHECK(expr)                \
  do {                                \
    sa_status st_ = (expr);           \
    if (st_ != SA_OK) return st_;     \
  } while (0)
#define SA_NOT_NULL(p) \
  do { if (!(p)) return fail(SA_ERR_INVALID_ARG, "%s is NULL", #p); } while (0)
// buffers the kernels read or write with 16-byte vector accesses
#define SA_ALIGNED16(p)                                                              \
  do {                                                                               \
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0)                                    \
      return fail(SA_ERR_INVALID_ARG, "%s is not 16-byte aligned", #p);               \
  } while (0)
#define SA_HIP(expr, what)                       \
  do {                                           \
    hipError_t e_ = (expr);                      \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

sa_status check_scale(float scale) {
  if (!(std::isfinite(scale) && scale > 0.f))
    return fail(SA_ERR_INVALID_ARG, "scale must be finite and > 0");
  return SA_OK;
}

// selection of one layer: scores, top-k and split in one launch (scores written out only
// when asked for); sel_ws is the selection region of a Layout
sa_status run_select(const sa::Shape& s, bool minmax, const sa::QParts& q, const void* digests,
                     const int32_t* seq_lens, int top_k, const int32_t* block_table,
                     int32_t* gpu_blocks, int32_t* n_gpu, int32_t* cpu_blocks, int32_t* n_cpu,
                     float* scores, int32_t* cpu_blocks_host, int32_t* n_cpu_host,
                     int32_t* gpu_pages, void* sel_ws, hipStream_t stream) {
  hipEvent_t e0, e1;
  next_profile_events(&e0, &e1, SA_PROFILE_SELECT);
  SA_HIP(sa::launch_select(s, sa::select_plan(s, minmax), minmax, q, digests, seq_lens, top_k,
                           block_table, gpu_blocks, n_gpu, cpu_blocks, n_cpu, scores,
                           cpu_blocks_host, n_cpu_host, gpu_pages, sel_ws, stream, e0, e1),
         "select kernel");
  return SA_OK;
}

}  // namespace

// The attention partials of sa_decode_attend_merge_noalloc live here, not in a caller
// workspace: kScratchBytes per GPU, which every GPU the library runs on holds (zero-filled
// when the code object loads) until the process ends.  In host code `scratch` is only a
// stand-in for the symbol, never a device address: the address each GPU's copy has is
// looked up once per device (scratch_address) and only that is passed to kernels.
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current GPU's scratch (looked up on this device's first call).
sa_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(SA_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SA_OK;
}
}  // namespace

extern "C" {

int sa_abi_version(void) { return SA_ABI_VERSION; }

const char* sa_last_error(void) { return g_err.c_str(); }

sa_status sa_profile_kernels(sa_profile_stage stage, const hipEvent_t* start,
                             const hipEvent_t* stop, int32_t n) {
  if ((int)stage < 0 || (int)stage >= SA_PROFILE_STAGES)
    return fail(SA_ERR_INVALID_ARG, "unknown profile stage %d", (int)stage);
  if (n < 0) return fail(SA_ERR_INVALID_ARG, "n %d < 0", n);
  if (n > 0 && (!start || !stop)) return fail(SA_ERR_INVALID_ARG, "event arrays are NULL");
  ProfileEvents& P = g_prof[stage];
  P.start.assign(start, start + n);
  P.stop.assign(stop, stop + n);
  P.next = 0;
  for (int32_t i = 0; i < n; ++i)
    if (!P.start[i] || !P.stop[i]) {
      P.start.clear();
      P.stop.clear();
      return fail(SA_ERR_INVALID_ARG, "event %d is NULL", i);
    }
  return ok();
}

sa_status sa_profile_attention(const hipEvent_t* start, const hipEvent_t* stop, int32_t n) {
  return sa_profile_kernels(SA_PROFILE_ATTENTION, start, stop, n);
}

const char* sa_status_string(sa_status status) {
  switch (status) {
    case SA_OK: return "SA_OK";
    case SA_ERR_INVALID_ARG: return "SA_ERR_INVALID_ARG";
    case SA_ERR_UNSUPPORTED: return "SA_ERR_UNSUPPORTED";
    case SA_ERR_WORKSPACE: return "SA_ERR_WORKSPACE";
    case SA_ERR_HIP: return "SA_ERR_HIP";
  }
  return "unknown status";
}

sa_status sa_pack_k_pages(const sa_dims* dims, const void* k_rows, void* k_pool,
                          hipStream_t stream) {
  sa::Shape s;
  SA_CHECK(check_dims(dims, &s));
  SA_NOT_NULL(k_rows);
  SA_NOT_NULL(k_pool);
  SA_ALIGNED16(k_rows);
  SA_ALIGNED16(k_pool);
  const size_t bytes = (size_t)s.P * s.bs * s.d * (s.bf16 ? 2 : 4);
  const char* a = (const char*)k_rows;
  const char* b = (const char*)k_pool;
  if (a < b + bytes && b < a + bytes) return fail(SA_ERR_INVALID_ARG, "k_rows and k_pool overlap");
  SA_HIP(sa::launch_pack_k(s, k_rows, k_pool, stream), "K pack kernel");
  return ok();
}

sa_status sa_pack_v_pages(const sa_dims* dims, const void* v_rows, void* v_pool,
                          hipStream_t stream) {
  sa::Shape s;
  SA_CHECK(check_dims(dims, &s));
  SA_NOT_NULL(v_rows);
  SA_NOT_NULL(v_pool);
  SA_ALIGNED16(v_rows);
  SA_ALIGNED16(v_pool);
  const size_t bytes = (size_t)s.P * s.bs * s.d * (s.bf16 ? 2 : 4);
  const char* a = (const char*)v_rows;
  const char* b = (const char*)v_pool;
  if (a < b + bytes && b < a + bytes) return fail(SA_ERR_INVALID_ARG, "v_rows and v_pool overlap");
  SA_HIP(sa::launch_pack_v(s, v_rows, v_pool, stream), "V pack kernel");
  return ok();
}

sa_status sa_pack_weight(int32_t n, int32_t k, const void* w, void* w_packed,
                         hipStream_t stream) {
  if (n < 32 || k < 32) return fail(SA_ERR_INVALID_ARG, "weight sizes n %d, k %d must be >= 32", n, k);
  if (n % 16 != 0 || k % 32 != 0)
    return fail(SA_ERR_UNSUPPORTED, "weight n (%d) must be a multiple of 16 and k (%d) of 32", n, k);
  SA_NOT_NULL(w);
  SA_NOT_NULL(w_packed);
  SA_ALIGNED16(w);
  SA_ALIGNED16(w_packed);
  const size_t bytes = (size_t)n * k * 2;
  const char* a = (const char*)w;
  const char* b = (const char*)w_packed;
  if (a < b + bytes && b < a + bytes) return fail(SA_ERR_INVALID_ARG, "w and w_packed overlap");
  SA_HIP(sa::launch_pack_w(n, k, w, w_packed, stream), "weight pack kernel");
  return ok();
}

sa_status sa_build_digests(const sa_dims* dims, sa_digest_kind kind, const void* k_pool,
                           const int32_t* block_table, const int32_t* seq_lens,
                           void* digests, hipStream_t stream) {
  sa::Shape s;
  SA_CHECK(check_dims(dims, &s));
  SA_CHECK(check_kind(kind));
  SA_NOT_NULL(k_pool);
  SA_NOT_NULL(block_table);
  SA_NOT_NULL(seq_lens);
  SA_NOT_NULL(digests);
  SA_ALIGNED16(k_pool);
  SA_ALIGNED16(digests);
  SA_HIP(sa::launch_build_digests(s, kind == SA_DIGEST_MINMAX, k_pool, block_table, seq_lens,
                                  digests, stream),
         "digest kernel");
  return ok();
}

sa_status sa_refresh_last_digests(const sa_dims* dims, sa_digest_kind kind,
                                  const void* k_pool, const int32_t* block_table,
                                  const int32_t* seq_lens, void* digests, hipStream_t stream) {
  sa::Shape s;
  SA_CHECK(check_dims(dims, &s));
  SA_CHECK(check_kind(kind));
  SA_NOT_NULL(k_pool);
  SA_NOT_NULL(block_table);
  SA_NOT_NULL(seq_lens);
  SA_NOT_NULL(digests);
  SA_ALIGNED16(k_pool);
  SA_ALIGNED16(digests);
  SA_HIP(sa::launch_refresh_digests(s, kind == SA_DIGEST_MINMAX, k_pool, block_table,
                                    seq_lens, digests, stream),
         "digest refresh kernel");
  return ok();
}

size_t sa_predict_query_workspace_bytes(int32_t m, int32_t n, int32_t k) {
  if (check_gemm_shape(m, n, k) != SA_OK) return 0;
  return sa::gemm_plan(m, n, k).ws_bytes;
}

sa_status sa_predict_query(int32_t m, int32_t n, int32_t k, const void* x,
                           const void* w_packed, float* q, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  SA_CHECK(check_gemm_shape(m, n, k));
  SA_NOT_NULL(x);
  SA_NOT_NULL(w_packed);
  const void* w = w_packed;
  SA_NOT_NULL(q);
  SA_ALIGNED16(x);
  SA_ALIGNED16(w_packed);
  SA_ALIGNED16(q);
  SA_ALIGNED16(ws);
  const sa::GemmPlan plan = sa::gemm_plan(m, n, k);
  if (plan.ws_bytes > 0 && (!ws || ws_bytes < plan.ws_bytes))
    return fail(SA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, plan.ws_bytes);
  hipEvent_t e0, e1;
  next_profile_events(&e0, &e1, SA_PROFILE_GEMM);
  SA_HIP(sa::launch_gemm(m, n, k, x, 1, w, q, nullptr, nullptr, (float*)ws, plan, stream, true,
                         e0, e1),
         "GEMM kernel");
  return ok();
}

size_t sa_workspace_bytes(const sa_dims* dims, int32_t top_k) {
  sa::Shape s;
  if (check_dims(dims, &s) != SA_OK) return 0;
  if (top_k < 1 || top_k > s.max_blocks) {
    fail(SA_ERR_INVALID_ARG, "top_k %d outside [1, max_blocks]", top_k);
    return 0;
  }
  return layout(s, top_k).total;
}

sa_status sa_select_blocks(const sa_dims* dims, sa_digest_kind kind, const float* q,
                           const void* digests, const int32_t* seq_lens, int32_t top_k,
                           const int32_t* block_table, int32_t* gpu_blocks, int32_t* n_gpu,
                           int32_t* cpu_blocks, int32_t* n_cpu, float* scores, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  sa::Shape s;
  SA_CHECK(check_dims(dims, &s));
  SA_CHECK(check_kind(kind));
  SA_NOT_NULL(q);
  SA_NOT_NULL(digests);
  SA_NOT_NULL(seq_lens);
  SA_NOT_NULL(block_table);
  SA_NOT_NULL(gpu_blocks);
  SA_NOT_NULL(n_gpu);
  SA_NOT_NULL(cpu_blocks);
  SA_NOT_NULL(n_cpu);
  SA_ALIGNED16(q);
  SA_ALIGNED16(digests);
  SA_ALIGNED16(ws);
  if (top_k < 1 || top_k > s.max_blocks)
    return fail(SA_ERR_INVALID_ARG, "top_k %d outside [1, max_blocks = %d]", top_k, s.max_blocks);
  const Layout L = layout(s, top_k);
  if (!ws || ws_bytes < L.total)
    return fail(SA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, L.total);
  SA_CHECK(run_select(s, kind == SA_DIGEST_MINMAX, sa::plain_query(q, s.Hq * s.d), digests,
                      seq_lens, top_k, block_table,
                      gpu_blocks, n_gpu, cpu_blocks, n_cpu, scores, nullptr, nullptr, nullptr,
                      (char*)ws + L.sel, stream));
  return ok();
}

// The attention stage with its merge: every argument is checked on the host, then the
// partials go to `ws` (a caller workspace laid out as Layout says), or, with noalloc, to the
// current GPU's scratch, which must hold them.
static sa_status decode_common(const sa_dims* dims, const float* q, const void* k_pool,
                               const void* v_pool, const int32_t* block_table,
                               const int32_t* seq_lens, const int32_t* gpu_blocks,
                               const int32_t* n_gpu, int32_t list_stride, float scale,
                               const float* host_o, const float* host_m, const float* host_l,
                               const int32_t* n_cpu, float* o, float* m, float* l, void* ws,
                               size_t ws_bytes, hipStream_t stream, bool noalloc = false) {
  sa::Shape s;
  SA_CHECK(check_dims(dims, &s));
  SA_NOT_NULL(q);
  SA_NOT_NULL(k_pool);
  SA_NOT_NULL(v_pool);
  SA_NOT_NULL(block_table);
  SA_NOT_NULL(seq_lens);
  SA_NOT_NULL(gpu_blocks);
  SA_NOT_NULL(n_gpu);
  SA_NOT_NULL(o);
  SA_CHECK(check_scale(scale));
  SA_ALIGNED16(q);
  SA_ALIGNED16(k_pool);
  SA_ALIGNED16(v_pool);
  SA_ALIGNED16(ws);
  if (list_stride < 1 || list_stride > s.max_blocks)
    return fail(SA_ERR_INVALID_ARG, "list_stride %d outside [1, max_blocks = %d]", list_stride,
                s.max_blocks);
  const Layout L = layout(s, list_stride);
  float* parts = nullptr;
  if (noalloc) {
    if (L.plan.ws_bytes > kScratchBytes)
      return fail(SA_ERR_WORKSPACE,
                  "the attention partials of this shape need %zu bytes, more than the %zu "
                  "bytes of scratch the library holds per GPU (use sa_decode_attend_merge)",
                  L.plan.ws_bytes, kScratchBytes);
    void* ptr = nullptr;
    SA_CHECK(scratch_address(&ptr));
    parts = static_cast<float*>(ptr);
  } else {
    if (!ws || ws_bytes < L.total)
      return fail(SA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, L.total);
    parts = (float*)((char*)ws + L.parts);
  }
  hipEvent_t e0, e1;
  next_profile_events(&e0, &e1);
  SA_HIP(sa::launch_attention(s, L.plan, sa::plain_query(q, s.Hq * s.d), k_pool, v_pool,
                              block_table, seq_lens, gpu_blocks, nullptr, n_gpu, list_stride,
                              scale, parts, stream, e0, e1),
         "attention kernel");
  SA_HIP(sa::launch_reduce(s, L.plan, n_gpu, parts, host_o, host_m, host_l, n_cpu, o, m, l,
                           stream),
         "reduce kernel");
  return ok();
}

sa_status sa_sparse_decode(const sa_dims* dims, const float* q, const void* k_pool,
                           const void* v_pool, const int32_t* block_table,
                           const int32_t* seq_lens, const int32_t* gpu_blocks,
                           const int32_t* n_gpu, int32_t list_stride, float scale, float* o,
                           float* m, float* l, void* ws, size_t ws_bytes, hipStream_t stream) {
  return decode_common(dims, q, k_pool, v_pool, block_table, seq_lens, gpu_blocks, n_gpu,
                       list_stride, scale, nullptr, nullptr, nullptr, nullptr, o, m, l, ws,
                       ws_bytes, stream);
}

sa_status sa_decode_attend_merge(const sa_dims* dims, const float* q, const void* k_pool,
                                 const void* v_pool, const int32_t* block_table,
                                 const int32_t* seq_lens, const int32_t* gpu_blocks,
                                 const int32_t* n_gpu, int32_t list_stride, float scale,
                                 const float* host_o, const float* host_m,
                                 const float* host_l, const int32_t* n_cpu, float* o,
                                 float* m, float* l, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
  SA_NOT_NULL(host_o);
  SA_NOT_NULL(host_m);
  SA_NOT_NULL(host_l);
  return decode_common(dims, q, k_pool, v_pool, block_table, seq_lens, gpu_blocks, n_gpu,
                       list_stride, scale, host_o, host_m, host_l, n_cpu, o, m, l, ws,
                       ws_bytes, stream);
}

sa_status sa_decode_attend_merge_noalloc(const sa_dims* dims, const float* q,
                                         const void* k_pool, const void* v_pool,
                                         const int32_t* block_table, const int32_t* seq_lens,
                                         const int32_t* gpu_blocks, const int32_t* n_gpu,
                                         int32_t list_stride, float scale, const float* host_o,
                                         const float* host_m, const float* host_l,
                                         const int32_t* n_cpu, float* o, float* m, float* l,
                                         hipStream_t stream) {
  SA_NOT_NULL(host_o);
  SA_NOT_NULL(host_m);
  SA_NOT_NULL(host_l);
  return decode_common(dims, q, k_pool, v_pool, block_table, seq_lens, gpu_blocks, n_gpu,
                       list_stride, scale, host_o, host_m, host_l, n_cpu, o, m, l, nullptr, 0,
                       stream, true);
}

sa_status sa_merge(int32_t rows, int32_t d, const float* o_a, const float* m_a,
                   const float* l_a, const float* o_b, const float* m_b, const float* l_b,
                   float* o, float* m, float* l, hipStream_t stream) {
  if (rows < 1) return fail(SA_ERR_INVALID_ARG, "rows %d < 1", rows);
  if (d < 1 || d > 1024) return fail(SA_ERR_INVALID_ARG, "d %d outside [1, 1024]", d);
  SA_NOT_NULL(o_a);
  SA_NOT_NULL(m_a);
  SA_NOT_NULL(l_a);
  SA_NOT_NULL(o_b);
  SA_NOT_NULL(m_b);
  SA_NOT_NULL(l_b);
  SA_NOT_NULL(o);
  SA_NOT_NULL(m);
  SA_NOT_NULL(l);
  SA_HIP(sa::launch_merge(rows, d, o_a, m_a, l_a, o_b, m_b, l_b, o, m, l, stream),
         "merge kernel");
  return ok();
}

// ---- dense (FullKV) attention -----------------------------------------------------------------

// workspace: the lists [pairs][max_blocks], the counts [pairs], then the attention partials
static size_t dense_lists_bytes(const sa::Shape& s) {
  return align_up((size_t)s.B * s.Hkv * (s.max_blocks + 1) * sizeof(int32_t));
}

size_t sa_dense_workspace_bytes(const sa_dims* dims) {
  sa::Shape s;
  if (check_dims(dims, &s) != SA_OK) return 0;
  return dense_lists_bytes(s) + layout(s, s.max_blocks).total;
}

sa_status sa_dense_decode(const sa_dims* dims, const float* q, const void* k_pool,
                          const void* v_pool, const int32_t* block_table,
                          const int32_t* seq_lens, float scale, float* o, float* m, float* l,
                          void* ws, size_t ws_bytes, hipStream_t stream) {
  sa::Shape s;
  SA_CHECK(check_dims(dims, &s));
  SA_CHECK(check_scale(scale));
  SA_NOT_NULL(q);
  SA_NOT_NULL(k_pool);
  SA_NOT_NULL(v_pool);
  SA_NOT_NULL(block_table);
  SA_NOT_NULL(seq_lens);
  SA_NOT_NULL(o);
  SA_ALIGNED16(q);
  SA_ALIGNED16(k_pool);
  SA_ALIGNED16(v_pool);
  SA_ALIGNED16(ws);
  const size_t need = sa_dense_workspace_bytes(dims);
  if (!ws || ws_bytes < need)
    return fail(SA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, need);
  int32_t* lists = (int32_t*)ws;
  int32_t* counts = lists + (size_t)s.B * s.Hkv * s.max_blocks;
  float* parts = (float*)((char*)ws + dense_lists_bytes(s));
  const Layout L = layout(s, s.max_blocks);
  SA_HIP(sa::launch_dense_lists(s, seq_lens, block_table, lists, counts, stream),
         "dense list kernel");
  hipEvent_t e0, e1;
  next_profile_events(&e0, &e1);
  SA_HIP(sa::launch_attention(s, L.plan, sa::plain_query(q, s.Hq * s.d), k_pool, v_pool,
                              block_table, seq_lens, lists, nullptr, counts, s.max_blocks, scale,
                              parts, stream, e0, e1),
         "attention kernel");
  SA_HIP(sa::launch_reduce(s, L.plan, counts, parts, nullptr, nullptr, nullptr, nullptr, o, m, l,
                           stream),
         "reduce kernel");
  return ok();
}

// ---- periodic recall -------------------------------------------------------------------------

static constexpr int kMaxRecall = 4096;  // blocks moved per pair by one recall, at most

size_t sa_recall_workspace_bytes(const sa_dims* dims, int32_t max_recall) {
  sa::Shape s;
  if (check_dims(dims, &s) != SA_OK) return 0;
  if (max_recall < 1 || max_recall > kMaxRecall) {
    fail(SA_ERR_INVALID_ARG, "max_recall %d outside [1, %d]", max_recall, kMaxRecall);
    return 0;
  }
  return align_up((size_t)s.B * s.Hkv * max_recall * 2 * sizeof(int32_t));
}

sa_status sa_recall_blocks(const sa_dims* dims, int32_t list_stride, int32_t max_recall,
                           const int32_t* seq_lens, int32_t* block_table,
                           const int32_t* gpu_blocks, const int32_t* n_gpu,
                           const int32_t* cpu_blocks, const int32_t* n_cpu, const void* k_host,
                           const void* v_host, const int32_t* host_table, int32_t host_pages,
                           void* k_pool, void* v_pool, int32_t* n_recalled, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  sa::Shape s;
  SA_CHECK(check_dims(dims, &s));
  if (list_stride < 1 || list_stride > s.max_blocks)
    return fail(SA_ERR_INVALID_ARG, "list_stride %d outside [1, max_blocks = %d]", list_stride,
                s.max_blocks);
  if (max_recall < 1 || max_recall > kMaxRecall)
    return fail(SA_ERR_INVALID_ARG, "max_recall %d outside [1, %d]", max_recall, kMaxRecall);
  if (sa::recall_plan_lds_bytes(s, max_recall) > 64 * 1024)
    return fail(SA_ERR_UNSUPPORTED, "max_blocks %d with max_recall %d exceeds the plan's LDS",
                s.max_blocks, max_recall);
  if (host_pages < 1) return fail(SA_ERR_INVALID_ARG, "host_pages %d < 1", host_pages);
  SA_NOT_NULL(seq_lens);
  SA_NOT_NULL(block_table);
  SA_NOT_NULL(gpu_blocks);
  SA_NOT_NULL(n_gpu);
  SA_NOT_NULL(cpu_blocks);
  SA_NOT_NULL(n_cpu);
  SA_NOT_NULL(k_host);
  SA_NOT_NULL(v_host);
  SA_NOT_NULL(host_table);
  SA_NOT_NULL(k_pool);
  SA_NOT_NULL(v_pool);
  SA_NOT_NULL(n_recalled);
  SA_ALIGNED16(k_host);
  SA_ALIGNED16(v_host);
  SA_ALIGNED16(k_pool);
  SA_ALIGNED16(v_pool);
  SA_ALIGNED16(ws);
  const size_t need = sa_recall_workspace_bytes(dims, max_recall);
  if (!ws || ws_bytes < need)
    return fail(SA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, need);
  SA_HIP(sa::launch_recall(s, list_stride, max_recall, seq_lens, block_table, gpu_blocks, n_gpu,
                           cpu_blocks, n_cpu, k_host, v_host, host_table, host_pages, k_pool,
                           v_pool, n_recalled, ws, -1, stream),
         "recall kernels");
  return ok();
}

// ---- the host side: partial attention over the offloaded blocks ------------------------------

static sa::HostAttnArgs host_args(const sa::Shape& s, int host_pages, int list_stride,
                                  float scale, const float* q, const void* k_host,
                                  const void* v_host, const int32_t* host_table,
                                  const int32_t* seq_lens, const int32_t* cpu_blocks,
                                  const int32_t* n_cpu, float* o, float* m, float* l) {
  sa::HostAttnArgs a;
  a.B = s.B;
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.G = s.G;
  a.d = s.d;
  a.bs = s.bs;
  a.max_blocks = s.max_blocks;
  a.host_pages = host_pages;
  a.list_stride = list_stride;
  a.bf16 = s.bf16;
  a.scale = scale;
  a.q = q;
  a.k_host = k_host;
  a.v_host = v_host;
  a.host_table = host_table;
  a.seq_lens = seq_lens;
  a.cpu_blocks = cpu_blocks;
  a.n_cpu = n_cpu;
  a.o = o;
  a.m = m;
  a.l = l;
  return a;
}

sa_status sa_host_partial_attention(const sa_dims* dims, int32_t host_pages,
                                    const float* q_host, const void* k_host,
                                    const void* v_host, const int32_t* host_table,
                                    const int32_t* seq_lens_host,
                                    const int32_t* cpu_blocks_host, const int32_t* n_cpu_host,
                                    int32_t list_stride, float scale, float* o_host,
                                    float* m_host, float* l_host, int32_t num_threads) {
  sa::Shape s;
  SA_CHECK(check_dims(dims, &s));
  SA_CHECK(check_scale(scale));
  if (host_pages < 1) return fail(SA_ERR_INVALID_ARG, "host_pages %d < 1", host_pages);
  if (list_stride < 1 || list_stride > s.max_blocks)
    return fail(SA_ERR_INVALID_ARG, "list_stride %d outside [1, max_blocks = %d]", list_stride,
                s.max_blocks);
  if (num_threads < 0) return fail(SA_ERR_INVALID_ARG, "num_threads %d < 0", num_threads);
  SA_NOT_NULL(q_host);
  SA_NOT_NULL(k_host);
  SA_NOT_NULL(v_host);
  SA_NOT_NULL(host_table);
  SA_NOT_NULL(seq_lens_host);
  SA_NOT_NULL(cpu_blocks_host);
  SA_NOT_NULL(n_cpu_host);
  SA_NOT_NULL(o_host);
  SA_NOT_NULL(m_host);
  SA_NOT_NULL(l_host);
  const sa::HostAttnArgs a =
      host_args(s, host_pages, list_stride, scale, q_host, k_host, v_host, host_table,
                seq_lens_host, cpu_blocks_host, n_cpu_host, o_host, m_host, l_host);
  try {
    sa::host_partial_attention(a, sa::host_threads(num_threads));
  } catch (const std::exception& e) {  // (thread creation; no exception crosses the ABI)
    return fail(SA_ERR_INVALID_ARG, "host worker failed: %s", e.what());
  }
  return ok();
}

// ---- the host plan: the CPU side of the step, as HIP host tasks ------------------------------


struct sa_host_plan {
  struct Task {
    sa_host_plan* plan;
    int layer;
  };
  sa::Shape s;
  int top_k = 0;
  float scale = 0.f;
  const int32_t* seq_lens = nullptr;
  std::vector<sa_host_layer> layers;
  std::vector<Task> tasks;  // the host functions' arguments (stable addresses)
  std::unique_ptr<sa::HostPool> pool;
  std::atomic<int64_t> runs{0}, busy_ns{0};
  std::atomic<bool> failed{false};
  // periodic recall inside the step (sa_host_plan_set_recall); off while `recall` is empty
  std::vector<sa_recall_layer> recall;
  int max_recall = 0;
  long recall_threshold = 0;  // the layer recalls when its offloaded selected blocks exceed it
  void* recall_ws = nullptr;
  // overlap mode: a step leaves its recalls running; layer i's event, recorded after its
  // recall, is waited for by the next step's selection of layer i
  bool recall_overlap = false;
  std::vector<hipEvent_t> recall_done;
  std::vector<char> recall_pending;
  // flag hand-off (sa_host_plan_set_handoff): the dispatcher thread, and the GPU wait bound
  std::unique_ptr<sa::FlagDispatcher> flags;
  uint32_t wait_rounds = 0;
  ~sa_host_plan() {
    flags.reset();  // joins the dispatcher before the tasks and the pool it uses go
    for (hipEvent_t e : recall_done) hipEventDestroy(e);
  }
};

// The empty partial of a layer: o = 0, m = -inf, l = 0 for every row.
static void empty_partial(const sa_host_plan& P, int layer) {
  const sa_host_layer& H = P.layers[layer];
  const size_t rows = (size_t)P.s.B * P.s.Hq;
  std::fill(H.o_host, H.o_host + rows * P.s.d, 0.f);
  std::fill(H.m_host, H.m_host + rows, -INFINITY);
  std::fill(H.l_host, H.l_host + rows, 0.f);
}

// A layer's host task: A_cpu on the plan's workers; false if no worker could run (the
// partial is then the empty one).
static bool host_task(const sa_host_plan::Task& t) {
  sa_host_plan& P = *t.plan;
  const sa_host_layer& H = P.layers[t.layer];
  const auto t0 = std::chrono::steady_clock::now();
  const sa::HostAttnArgs a =
      host_args(P.s, H.host_pages, P.top_k, P.scale, H.q_host, H.k_host, H.v_host,
                H.host_table, P.seq_lens, H.cpu_blocks_host, H.n_cpu_host, H.o_host, H.m_host,
                H.l_host);
  const bool done = P.pool->run(a);
  if (!done) {
    P.failed = true;
    empty_partial(P, t.layer);
  }
  const auto dt = std::chrono::steady_clock::now() - t0;
  P.busy_ns += std::chrono::duration_cast<std::chrono::nanoseconds>(dt).count();
  ++P.runs;
  return done;
}

// The host task as a HIP host function: it runs on the runtime's callback thread and holds
// its stream until it returns; it makes no HIP call.  A failure shows in sa_host_plan_stats.
static void run_host_task(void* arg) { host_task(*static_cast<const sa_host_plan::Task*>(arg)); }

sa_status sa_host_plan_create(const sa_dims* dims, int32_t top_k, float scale,
                              const int32_t* seq_lens_host, int32_t num_layers,
                              const sa_host_layer* layers, int32_t num_threads,
                              sa_host_plan** plan) {
  SA_NOT_NULL(plan);
  *plan = nullptr;
  sa::Shape s;
  SA_CHECK(check_dims(dims, &s));
  SA_CHECK(check_scale(scale));
  if (top_k < 1 || top_k > s.max_blocks)
    return fail(SA_ERR_INVALID_ARG, "top_k %d outside [1, max_blocks = %d]", top_k, s.max_blocks);
  SA_NOT_NULL(seq_lens_host);
  SA_NOT_NULL(layers);
  if (num_layers < 1) return fail(SA_ERR_INVALID_ARG, "num_layers %d < 1", num_layers);
  if (num_threads < 0) return fail(SA_ERR_INVALID_ARG, "num_threads %d < 0", num_threads);
  for (int i = 0; i < num_layers; ++i) {
    const sa_host_layer& H = layers[i];
    if (!H.k_host || !H.v_host || !H.host_table || !H.q_host || !H.cpu_blocks_host ||
        !H.n_cpu_host || !H.o_host || !H.m_host || !H.l_host)
      return fail(SA_ERR_INVALID_ARG, "host layer %d: a pointer is NULL", i);
    if (H.host_pages < 1)
      return fail(SA_ERR_INVALID_ARG, "host layer %d: host_pages %d < 1", i, H.host_pages);
  }
  try {
    auto P = std::make_unique<sa_host_plan>();
    P->s = s;
    P->top_k = top_k;
    P->scale = scale;
    P->seq_lens = seq_lens_host;
    P->layers.assign(layers, layers + num_layers);
    P->tasks.resize(num_layers);
    for (int i = 0; i < num_layers; ++i) P->tasks[i] = {P.get(), i};
    P->pool = std::make_unique<sa::HostPool>(sa::host_threads(num_threads));
    *plan = P.release();
  } catch (const std::exception& e) {  // allocation or thread creation
    return fail(SA_ERR_INVALID_ARG, "host plan: %s", e.what());
  }
  return ok();
}

sa_status sa_host_plan_run(sa_host_plan* plan, int32_t layer) {
  SA_NOT_NULL(plan);
  if (layer < 0 || layer >= (int)plan->layers.size())
    return fail(SA_ERR_INVALID_ARG, "layer %d outside [0, %d)", layer, (int)plan->layers.size());
  if (!host_task(plan->tasks[layer]))
    return fail(SA_ERR_HIP, "the host task could not run (out of memory)");
  return ok();
}

sa_status sa_host_plan_set_recall(sa_host_plan* plan, int32_t max_recall, float beta,
                                  const sa_recall_layer* layers, void* ws, size_t ws_bytes,
                                  int32_t overlap) {
  SA_NOT_NULL(plan);
  for (hipEvent_t e : plan->recall_done)  // a step may still be recalling: let it finish
    if (hipEventSynchronize(e) != hipSuccess) return fail(SA_ERR_HIP, "hipEventSynchronize");
  std::fill(plan->recall_pending.begin(), plan->recall_pending.end(), 0);
  if (!layers) {
    plan->recall.clear();
    plan->recall_overlap = false;
    return ok();
  }
  if (max_recall < 1 || max_recall > kMaxRecall)
    return fail(SA_ERR_INVALID_ARG, "max_recall %d outside [1, %d]", max_recall, kMaxRecall);
  if (!(beta >= 0.f)) return fail(SA_ERR_INVALID_ARG, "beta must be >= 0");
  if (sa::recall_plan_lds_bytes(plan->s, max_recall) > 64 * 1024)
    return fail(SA_ERR_UNSUPPORTED, "max_blocks %d with max_recall %d exceeds the plan's LDS",
                plan->s.max_blocks, max_recall);
  const size_t need = align_up((size_t)plan->s.B * plan->s.Hkv * max_recall * 2 * sizeof(int32_t));
  if (!ws || ws_bytes < need)
    return fail(SA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, need);
  const int L = (int)plan->layers.size();
  for (int i = 0; i < L; ++i)
    if (layers[i].host_table_dev && !layers[i].n_recalled)
      return fail(SA_ERR_INVALID_ARG, "recall layer %d: n_recalled is NULL", i);
  try {
    plan->recall.assign(layers, layers + L);
  } catch (const std::exception& e) {
    return fail(SA_ERR_INVALID_ARG, "recall layers: %s", e.what());
  }
  plan->max_recall = max_recall;
  // ratio > beta  <=>  total > beta * pairs * top_k  <=>  total > floor(beta * pairs * top_k)
  plan->recall_threshold =
      (long)std::floor((double)beta * (double)plan->s.B * plan->s.Hkv * plan->top_k);
  plan->recall_ws = ws;
  plan->recall_overlap = overlap != 0;
  if (plan->recall_overlap && plan->recall_done.empty()) {
    for (int i = 0; i < L; ++i) {
      hipEvent_t e;
      SA_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming), "hipEventCreate");
      plan->recall_done.push_back(e);
    }
    plan->recall_pending.assign(L, 0);
  }
  return ok();
}

sa_status sa_host_plan_set_handoff(sa_host_plan* plan, sa_handoff mode, uint32_t* flags,
                                   int32_t gpu_wait_ms) {
  SA_NOT_NULL(plan);
  if (mode != SA_HANDOFF_HOST_FUNC && mode != SA_HANDOFF_FLAGS)
    return fail(SA_ERR_INVALID_ARG, "handoff mode %d is neither SA_HANDOFF_HOST_FUNC nor "
                "SA_HANDOFF_FLAGS", (int)mode);
  if (mode == SA_HANDOFF_FLAGS) {
    SA_NOT_NULL(flags);
    if ((uintptr_t)flags % alignof(uint32_t) != 0)
      return fail(SA_ERR_INVALID_ARG, "flags is not 4-byte aligned");
    if (gpu_wait_ms < 1) return fail(SA_ERR_INVALID_ARG, "gpu_wait_ms %d < 1", gpu_wait_ms);
  }
  plan->flags.reset();  // (serves or closes the layers still raised)
  if (mode == SA_HANDOFF_HOST_FUNC) return ok();
  try {
    sa_host_plan* P = plan;
    plan->flags = std::make_unique<sa::FlagDispatcher>(
        flags, (int)plan->layers.size(), [P](int layer) { return host_task(P->tasks[layer]); },
        [P](int layer) { empty_partial(*P, layer); });
  } catch (const std::exception& e) {  // thread creation
    return fail(SA_ERR_INVALID_ARG, "handoff dispatcher: %s", e.what());
  }
  plan->wait_rounds = sa::wait_rounds(gpu_wait_ms);
  return ok();
}

sa_status sa_stream_signal(uint32_t* counter, hipStream_t stream) {
  SA_NOT_NULL(counter);
  if ((uintptr_t)counter % alignof(uint32_t) != 0)
    return fail(SA_ERR_INVALID_ARG, "counter is not 4-byte aligned");
  SA_HIP(sa::launch_signal(counter, stream), "signal kernel");
  return ok();
}

sa_status sa_stream_wait(const uint32_t* flag, const uint32_t* counter, int32_t wait_ms,
                         uint32_t* timeouts, hipStream_t stream) {
  SA_NOT_NULL(flag);
  SA_NOT_NULL(counter);
  SA_NOT_NULL(timeouts);
  if ((uintptr_t)flag % alignof(uint32_t) != 0 || (uintptr_t)counter % alignof(uint32_t) != 0 ||
      (uintptr_t)timeouts % alignof(uint32_t) != 0)
    return fail(SA_ERR_INVALID_ARG, "flag, counter or timeouts is not 4-byte aligned");
  if (wait_ms < 1) return fail(SA_ERR_INVALID_ARG, "wait_ms %d < 1", wait_ms);
  SA_HIP(sa::launch_wait(flag, counter, sa::wait_rounds(wait_ms), timeouts, stream),
         "wait kernel");
  return ok();
}

sa_status sa_host_plan_destroy(sa_host_plan* plan) {
  delete plan;  // joins the dispatcher and the workers
  return ok();
}

sa_status sa_host_plan_stats(const sa_host_plan* plan, int64_t* tasks, double* busy_seconds) {
  SA_NOT_NULL(plan);
  const sa::FlagDispatcher* D = plan->flags.get();
  if (D) D->drain();
  if (tasks) *tasks = plan->runs.load();
  if (busy_seconds) *busy_seconds = 1e-9 * (double)plan->busy_ns.load();
  if (plan->failed.load())
    return fail(SA_ERR_HIP, "a host task could not run (out of memory); its partial is empty");
  if (D && D->gpu_timed_out())
    return fail(SA_ERR_HIP, "a GPU wait for a done flag timed out; that layer's merge read "
                "its host partial before it was complete");
  return ok();
}

// ---- the layer-ahead step -------------------------------------------------------------------

namespace {
struct StepLayout {
  size_t q_true, q_pred[2], gemm[2], pages[2], sel, total;
  sa::GemmPlan plan_dual, plan_single;
  Layout sel_layout;
};
StepLayout step_layout(const sa::Shape& s, int hidden, int top_k) {
  StepLayout L;
  const int n = s.Hq * s.d;
  L.plan_dual = sa::gemm_plan(s.B, 2 * n, hidden);
  L.plan_single = sa::gemm_plan(s.B, n, hidden);
  const size_t qbytes = align_up((size_t)s.B * n * sizeof(float));
  L.q_true = 0;
  L.q_pred[0] = qbytes;      // Q_pred of even target layers
  L.q_pred[1] = 2 * qbytes;  // Q_pred of odd target layers
  // GEMM slice partials: one buffer for the main stream, one for the side stream
  const size_t gbytes = align_up(std::max(L.plan_dual.ws_bytes, L.plan_single.ws_bytes));
  L.gemm[0] = 3 * qbytes;
  L.gemm[1] = L.gemm[0] + gbytes;
  // pages of the resident lists, written by the selection for the attention kernel; two
  // buffers (by layer parity), as the next layer's selection runs during this attention
  const size_t pbytes = align_up((size_t)s.B * s.Hkv * top_k * sizeof(int32_t));
  L.pages[0] = L.gemm[1] + gbytes;
  L.pages[1] = L.pages[0] + pbytes;
  L.sel = L.pages[1] + pbytes;
  L.sel_layout = layout(s, top_k);
  L.total = L.sel + L.sel_layout.total;
  return L;
}
}  // namespace

size_t sa_step_workspace_bytes(const sa_dims* dims, int32_t hidden, int32_t top_k) {
  sa::Shape s;
  if (check_dims(dims, &s) != SA_OK) return 0;
  if (check_gemm_shape(s.B, s.Hq * s.d, hidden) != SA_OK) return 0;
  if (top_k < 1 || top_k > s.max_blocks) {
    fail(SA_ERR_INVALID_ARG, "top_k %d outside [1, max_blocks]", top_k);
    return 0;
  }
  return step_layout(s, hidden, top_k).total;
}

// The step, with its CPU side given (plan NULL: each layer's host_o/m/l) or computed by the
// plan's host tasks on host_stream.
static sa_status step_impl(const sa_dims* dims, sa_digest_kind kind, int32_t hidden,
                           int32_t top_k, float scale, const int32_t* seq_lens,
                           int32_t num_layers, const sa_layer* layers, void* ws,
                           size_t ws_bytes, hipStream_t stream, hipStream_t side_stream,
                           sa_host_plan* plan, hipStream_t host_stream,
                           hipStream_t recall_stream) {
  sa::Shape s;
  SA_CHECK(check_dims(dims, &s));
  SA_CHECK(check_kind(kind));
  SA_CHECK(check_gemm_shape(s.B, s.Hq * s.d, hidden));
  SA_CHECK(check_scale(scale));
  SA_NOT_NULL(seq_lens);
  SA_NOT_NULL(layers);
  if (num_layers < 1) return fail(SA_ERR_INVALID_ARG, "num_layers %d < 1", num_layers);
  if (top_k < 1 || top_k > s.max_blocks)
    return fail(SA_ERR_INVALID_ARG, "top_k %d outside [1, max_blocks = %d]", top_k, s.max_blocks);
  for (int i = 0; i < num_layers; ++i) {
    const sa_layer& L = layers[i];
    if (!L.x || !L.w_q || !L.digests || !L.block_table || !L.k_pool || !L.v_pool ||
        !L.gpu_blocks || !L.n_gpu || !L.cpu_blocks || !L.n_cpu || !L.out_o)
      return fail(SA_ERR_INVALID_ARG, "layer %d: a required pointer is NULL", i);
    for (const void* v : {L.x, L.w_q, L.digests, L.k_pool, L.v_pool})
      if (reinterpret_cast<uintptr_t>(v) % 16 != 0)
        return fail(SA_ERR_INVALID_ARG,
                    "layer %d: x, w_q, digests, k_pool and v_pool must be 16-byte aligned", i);
    if (plan) continue;  // the plan's host buffers take the place of the rest
    if (!L.host_o || !L.host_m || !L.host_l)
      return fail(SA_ERR_INVALID_ARG, "layer %d: a host partial pointer is NULL", i);
    if ((L.cpu_blocks_host == nullptr) != (L.n_cpu_host == nullptr))
      return fail(SA_ERR_INVALID_ARG,
                  "layer %d: cpu_blocks_host and n_cpu_host must both be set or both NULL", i);
  }
  if (side_stream == stream) side_stream = nullptr;
  if (plan) {
    const sa::Shape& p = plan->s;
    if (p.B != s.B || p.Hq != s.Hq || p.Hkv != s.Hkv || p.d != s.d || p.bs != s.bs ||
        p.max_blocks != s.max_blocks || p.bf16 != s.bf16)
      return fail(SA_ERR_INVALID_ARG, "the host plan was made for other dims");
    if (plan->top_k != top_k || plan->scale != scale ||
        (int)plan->layers.size() != num_layers)
      return fail(SA_ERR_INVALID_ARG,
                  "the host plan was made for another top_k, scale or number of layers");
    if (!plan->flags && (!host_stream || host_stream == stream || host_stream == side_stream))
      return fail(SA_ERR_INVALID_ARG, "host_stream must be a stream of its own");
    if (!plan->recall.empty() &&
        (!recall_stream || recall_stream == stream || recall_stream == side_stream ||
         recall_stream == host_stream))
      return fail(SA_ERR_INVALID_ARG,
                  "the plan recalls: recall_stream must be a stream of its own");
  }
  const bool recalls = plan && !plan->recall.empty();
  const bool overlap = recalls && plan->recall_overlap;
  sa::FlagDispatcher* flags = plan ? plan->flags.get() : nullptr;
  if (overlap) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    SA_HIP(hipStreamIsCapturing(stream, &cs), "hipStreamIsCapturing");
    if (cs != hipStreamCaptureStatusNone)
      return fail(SA_ERR_INVALID_ARG,
                  "recalls that overlap the next step cannot be captured (set overlap 0)");
  }
  StepLayout SL = step_layout(s, hidden, top_k);
  if (!ws || ws_bytes < SL.total)
    return fail(SA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, SL.total);
  SA_ALIGNED16(ws);
  // The GEMMs share the CUs with the selection and the attention.  Where the selection ranks
  // 4096 blocks or more per (sequence, KV head) it sets the step's pace, and five-wave GEMM
  // workgroups leave it more room than four.  Measured on the 40-layer step: blocks of 16
  // (4096 a pair) 5.24 against 5.55 ms; blocks of 32 (2048 a pair) 4.29 against 4.42 ms
  // with mean digests and 4.50 against 4.63-4.68 ms with min/max digests (which stream as
  // many bytes as blocks of 16) in favour of four; blocks of 64, four.  The wave count does
  // not change the workspace.
  if (s.max_blocks >= 4096) {
    SL.plan_dual = sa::gemm_plan(s.B, 2 * s.Hq * s.d, hidden, 5);
    SL.plan_single = sa::gemm_plan(s.B, s.Hq * s.d, hidden, 5);
  }

  char* base = (char*)ws;
  float* q_true = (float*)(base + SL.q_true);
  float* q_pred[2] = {(float*)(base + SL.q_pred[0]), (float*)(base + SL.q_pred[1])};
  float* gemm_ws[2] = {(float*)(base + SL.gemm[0]), (float*)(base + SL.gemm[1])};
  int32_t* pages[2] = {(int32_t*)(base + SL.pages[0]), (int32_t*)(base + SL.pages[1])};
  char* sel_base = base + SL.sel;
  float* parts = (float*)(sel_base + SL.sel_layout.parts);
  // the selections of the step run one after another (each stream is in order, and the
  // side stream's selection of layer i+1 starts after layer i's), so they share one region
  void* sel_ws = sel_base + SL.sel_layout.sel;
  const bool minmax = kind == SA_DIGEST_MINMAX;
  const int n = s.Hq * s.d;
  hipStream_t sel_stream = side_stream ? side_stream : stream;

  g_events.next = 0;
  auto new_event = [&](hipEvent_t* ev) -> sa_status {
    if (g_events.next == g_events.ev.size()) {
      hipEvent_t e;
      SA_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming), "hipEventCreate");
      g_events.ev.push_back(e);
    }
    *ev = g_events.ev[g_events.next++];
    return SA_OK;
  };
  // `to` waits for the work enqueued so far on `from`
  auto order = [&](hipStream_t from, hipStream_t to) -> sa_status {
    if (from == to) return SA_OK;
    hipEvent_t ev;
    SA_CHECK(new_event(&ev));
    SA_HIP(hipEventRecord(ev, from), "hipEventRecord");
    SA_HIP(hipStreamWaitEvent(to, ev, 0), "hipStreamWaitEvent");
    return SA_OK;
  };
  // the CPU side of layer j, once its lists are selected on `from`: the query it attends
  // with goes to the plan's host buffer, then a host task on host_stream computes A_cpu^j
  std::vector<hipEvent_t> host_done(plan ? num_layers : 0, nullptr);
  // (only the query heads of pairs that offloaded something: the host reads no other)
  auto spawn_host = [&](int j, const sa::QParts& q, hipStream_t from) -> sa_status {
    const sa_host_layer& H = plan->layers[j];
    SA_HIP(sa::launch_gather_query(q, s.B, n, H.q_host, from, layers[j].n_cpu, s.G * s.d,
                                   s.Hkv),
           "query gather kernel");
    if (flags) {  // advance ready[j] once the lists and the query are written
      SA_HIP(sa::launch_signal(flags->flags() + j, from), "signal kernel");
      return SA_OK;
    }
    SA_CHECK(order(from, host_stream));
    SA_HIP(hipLaunchHostFunc(host_stream, run_host_task, &plan->tasks[j]), "hipLaunchHostFunc");
    SA_CHECK(new_event(&host_done[j]));
    SA_HIP(hipEventRecord(host_done[j], host_stream), "hipEventRecord");
    return SA_OK;
  };
  // where the selection of layer j hands its offloaded lists over
  auto mirror_blocks = [&](int j) {
    return plan ? plan->layers[j].cpu_blocks_host : layers[j].cpu_blocks_host;
  };
  auto mirror_n = [&](int j) { return plan ? plan->layers[j].n_cpu_host : layers[j].n_cpu_host; };
  // overlap mode: the selection of layer j (which rewrites the lists layer j's pending recall
  // reads, and reads the table it writes) waits for that recall first
  auto after_recall = [&](int j, hipStream_t on) -> sa_status {
    if (!overlap || !plan->recall_pending[j]) return SA_OK;
    SA_HIP(hipStreamWaitEvent(on, plan->recall_done[j], 0), "hipStreamWaitEvent");
    plan->recall_pending[j] = 0;
    return SA_OK;
  };
  sa_status st = SA_OK;
  hipEvent_t sel_done = nullptr;  // side stream: the selection of this layer is done
  hipEvent_t sel_next = nullptr;  // ... and of the coming layer
  for (int i = 0; i < num_layers && st == SA_OK; ++i) {
    const sa_layer& L = layers[i];
    const bool has_next = i + 1 < num_layers;
    // Q_pred alternates between two buffers, so a prediction never overwrites the query a
    // selection may still be reading.
    float* qp = q_pred[(i + 1) & 1];
    hipError_t e;
    // 0. with a side stream, the layer-ahead work for layer i+1 (below) may start as soon
    //    as X^i exists, i.e. once the previous layer is done on `stream`
    if (side_stream && has_next && i > 0) {
      st = order(stream, side_stream);
      if (st != SA_OK) break;
    }
    // 1. Q^i = W_Q^i X^i on `stream`.  Without a side stream, Q_pred^{i+1} = W_Q^{i+1} X^i
    //    comes from the same launch (both weights share X^i).  The GEMMs leave their k-slice
    //    partials; the selection and attention kernels sum them as they read the query.
    sa::QParts q_cur, q_next{};
    hipEvent_t g0, g1;
    next_profile_events(&g0, &g1, SA_PROFILE_GEMM);
    if (side_stream || !has_next) {
      e = sa::launch_gemm(s.B, n, hidden, L.x, 1, L.w_q, q_true, nullptr, nullptr, gemm_ws[0],
                          SL.plan_single, stream, false, g0, g1);
      q_cur = sa::gemm_result(SL.plan_single, s.B, n, 1, 0, q_true, gemm_ws[0]);
    } else {
      e = sa::launch_gemm(s.B, n, hidden, L.x, 2, L.w_q, q_true, layers[i + 1].w_q, qp,
                          gemm_ws[0], SL.plan_dual, stream, false, g0, g1);
      q_cur = sa::gemm_result(SL.plan_dual, s.B, n, 2, 0, q_true, gemm_ws[0]);
      q_next = sa::gemm_result(SL.plan_dual, s.B, n, 2, 1, qp, gemm_ws[0]);
    }
    if (e != hipSuccess) { st = hip_fail(e, "GEMM kernel"); break; }
    // 2. the first layer selects with its own query (on `stream`: its attention needs it);
    //    the selection kernels also write the offloaded lists into the host mirrors
    if (i == 0) {
      st = after_recall(0, stream);
      if (st == SA_OK)
        st = run_select(s, minmax, q_cur, L.digests, seq_lens, top_k, L.block_table,
                      L.gpu_blocks, L.n_gpu, L.cpu_blocks, L.n_cpu, nullptr, mirror_blocks(0),
                      mirror_n(0), pages[0], sel_ws, stream);
      if (st == SA_OK && plan) st = spawn_host(0, q_cur, stream);
      if (st == SA_OK && side_stream) st = order(stream, side_stream);
      if (st != SA_OK) break;
    }
    // 3. layer-ahead work for layer i+1: with a side stream, the prediction GEMM (it needs
    //    only X^i), the selection and its hand-off run there, concurrently with layer i's
    //    GEMM, attention and merge on `stream` (layer 0 forked after its own selection)
    if (has_next) {
      const sa_layer& N = layers[i + 1];
      if (side_stream) {
        next_profile_events(&g0, &g1, SA_PROFILE_GEMM);
        e = sa::launch_gemm(s.B, n, hidden, L.x, 1, N.w_q, qp, nullptr, nullptr, gemm_ws[1],
                            SL.plan_single, side_stream, false, g0, g1);
        if (e != hipSuccess) st = hip_fail(e, "GEMM kernel");
        q_next = sa::gemm_result(SL.plan_single, s.B, n, 1, 0, qp, gemm_ws[1]);
      }
      if (st == SA_OK) st = after_recall(i + 1, sel_stream);
      if (st == SA_OK)
        st = run_select(s, minmax, q_next, N.digests, seq_lens, top_k, N.block_table,
                        N.gpu_blocks, N.n_gpu, N.cpu_blocks, N.n_cpu, nullptr,
                        mirror_blocks(i + 1), mirror_n(i + 1), pages[(i + 1) & 1], sel_ws,
                        sel_stream);
      // the next layer's attention needs its lists only: the event is recorded before the
      // host hand-off (query gather, signal), which then runs beside this layer's attention
      if (st == SA_OK && side_stream) {
        st = new_event(&sel_next);
        if (st == SA_OK && hipEventRecord(sel_next, side_stream) != hipSuccess)
          st = fail(SA_ERR_HIP, "hipEventRecord failed");
      }
      if (st == SA_OK && plan) st = spawn_host(i + 1, q_next, sel_stream);
      if (st != SA_OK) break;
    }
    // 4. layer i's lists were selected on the side stream one layer earlier
    if (i >= 1 && side_stream && hipStreamWaitEvent(stream, sel_done, 0) != hipSuccess) {
      st = fail(SA_ERR_HIP, "hipStreamWaitEvent failed");
      break;
    }
    sel_done = sel_next;
    // 5. GPU attention of layer i, merged with its host partial
    hipEvent_t e0, e1;
    next_profile_events(&e0, &e1);
    e = sa::launch_attention(s, SL.sel_layout.plan, q_cur, L.k_pool, L.v_pool, L.block_table,
                             seq_lens, L.gpu_blocks, pages[i & 1], L.n_gpu, top_k, scale,
                             parts, stream, e0, e1);
    if (e != hipSuccess) { st = hip_fail(e, "attention kernel"); break; }
    const float* ho = L.host_o;
    const float* hm = L.host_m;
    const float* hl = L.host_l;
    if (plan) {  // layer i's CPU side, spawned one layer earlier (layer 0: just now)
      if (flags) {
        e = sa::launch_wait(flags->flags() + num_layers + i, flags->flags() + i,
                            plan->wait_rounds, flags->flags() + 2 * num_layers, stream);
        if (e != hipSuccess) { st = hip_fail(e, "wait kernel"); break; }
      } else if (hipStreamWaitEvent(stream, host_done[i], 0) != hipSuccess) {
        st = fail(SA_ERR_HIP, "hipStreamWaitEvent failed");
        break;
      }
      ho = plan->layers[i].o_host;
      hm = plan->layers[i].m_host;
      hl = plan->layers[i].l_host;
    }
    e = sa::launch_reduce(s, SL.sel_layout.plan, L.n_gpu, parts, ho, hm, hl, L.n_cpu, L.out_o,
                          L.out_m, L.out_l, stream);
    if (e != hipSuccess) { st = hip_fail(e, "reduce kernel"); break; }
    // 6. periodic recall of layer i, off the critical path: nothing in this step reads layer
    //    i's table or pages any more, and the next step's use of them follows the final join.
    //    The layer's buffers are the caller's, writable when it has the plan recall.
    if (recalls && plan->recall[i].host_table_dev) {
      st = order(stream, recall_stream);
      if (st != SA_OK) break;
      const sa_host_layer& H = plan->layers[i];
      e = sa::launch_recall(s, top_k, plan->max_recall, seq_lens,
                            const_cast<int32_t*>(L.block_table), L.gpu_blocks, L.n_gpu,
                            L.cpu_blocks, L.n_cpu, H.k_host, H.v_host,
                            plan->recall[i].host_table_dev, H.host_pages,
                            const_cast<void*>(L.k_pool), const_cast<void*>(L.v_pool),
                            plan->recall[i].n_recalled, plan->recall_ws,
                            plan->recall_threshold, recall_stream);
      if (e != hipSuccess) { st = hip_fail(e, "recall kernels"); break; }
      if (overlap) {
        if (hipEventRecord(plan->recall_done[i], recall_stream) != hipSuccess) {
          st = fail(SA_ERR_HIP, "hipEventRecord failed");
          break;
        }
        plan->recall_pending[i] = 1;
      }
    }
  }
  // join the side stream and the host tasks back into `stream`
  if (side_stream) {
    sa_status j = order(side_stream, stream);
    if (st == SA_OK) st = j;
  }
  if (plan && !flags) {  // (with flags, each merge has already waited for its job)
    sa_status j = order(host_stream, stream);
    if (st == SA_OK) st = j;
  }
  if (recalls && !overlap) {
    sa_status j = order(recall_stream, stream);
    if (st == SA_OK) st = j;
  }
  return st == SA_OK ? ok() : st;
}

sa_status sa_decode_step(const sa_dims* dims, sa_digest_kind kind, int32_t hidden,
                         int32_t top_k, float scale, const int32_t* seq_lens,
                         int32_t num_layers, const sa_layer* layers, void* ws,
                         size_t ws_bytes, hipStream_t stream, hipStream_t side_stream) {
  return step_impl(dims, kind, hidden, top_k, scale, seq_lens, num_layers, layers, ws, ws_bytes,
                   stream, side_stream, nullptr, nullptr, nullptr);
}

sa_status sa_decode_step_offload(const sa_dims* dims, sa_digest_kind kind, int32_t hidden,
                                 int32_t top_k, float scale, const int32_t* seq_lens,
                                 int32_t num_layers, const sa_layer* layers, void* ws,
                                 size_t ws_bytes, hipStream_t stream, hipStream_t side_stream,
                                 sa_host_plan* plan, hipStream_t host_stream,
                                 hipStream_t recall_stream) {
  SA_NOT_NULL(plan);
  return step_impl(dims, kind, hidden, top_k, scale, seq_lens, num_layers, layers, ws, ws_bytes,
                   stream, side_stream, plan, host_stream, recall_stream);
}

}  // extern "C"
