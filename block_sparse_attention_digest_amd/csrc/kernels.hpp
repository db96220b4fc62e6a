// Host-side launchers of the gfx950 kernels (one per kernel family), called by the C ABI
// layer after it has validated every argument.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sa {

// Validated problem shape, in plain ints.
struct Shape {
  int B, Hq, Hkv, G, d, bs, max_blocks, P;
  bool bf16;  // KV dtype: bf16 (true) or float32 (false)
};

// ---- layout conversions (data movement only) ------------------------------------------------
// K pages [P][bs][d] -> chunk-major [P][d/x][bs][x], x = 16 bytes of elements.
hipError_t launch_pack_k(const Shape& s, const void* k_rows, void* k_pool, hipStream_t stream);
// V pages [P][bs][d] -> [P][bs/16][d][16] (each 16-token half channel-major).
hipError_t launch_pack_v(const Shape& s, const void* v_rows, void* v_pool, hipStream_t stream);
// W [n][k] bf16 -> [n/16][k/32][64][8] (one MFMA B operand per KiB); n % 16 == 0, k % 32 == 0.
hipError_t launch_pack_w(int n, int k, const void* w, void* w_packed, hipStream_t stream);

// ---- digests: one wave per block (chunk-major K pages) ------------------------------------
hipError_t launch_build_digests(const Shape& s, bool minmax, const void* k_pool,
                                const int32_t* block_table, const int32_t* seq_lens,
                                void* digests, hipStream_t stream);
// the digest of each (sequence, KV head)'s last block only, from its page (decode-time
// maintenance after a token append); bit-identical to launch_build_digests for that block
hipError_t launch_refresh_digests(const Shape& s, bool minmax, const void* k_pool,
                                  const int32_t* block_table, const int32_t* seq_lens,
                                  void* digests, hipStream_t stream);

// A float32 query [B][Hq][d] held as the sum of `parts` arrays (the k-slice partials of the
// query GEMM, or one plain array), summed by its consumer in part order.
struct QParts {
  const float* base;   // part 0, element (row 0, column 0)
  int parts;           // >= 1
  size_t part_stride;  // floats from one part to the next
  size_t row_stride;   // floats from one sequence row to the next (>= Hq * d)
};
inline QParts plain_query(const float* q, int n) { return QParts{q, 1, 0, (size_t)n}; }

// ---- skinny GEMM q[m][n] = x[m][k] . w[n][k]^T, for up to two weight matrices sharing x ---
// (weights in the launch_pack_w order)
struct GemmPlan {
  int ksplit;        // K slices (equal; k / ksplit is a multiple of 64)
  int kslice;        // columns of K per slice
  int tpw;           // 16-column tiles per workgroup and wave (divides n_total / 16)
  int kpw;           // waves per workgroup, each streaming 1/kpw of the k-slice
  size_t ws_bytes;   // float partials [ksplit][m][n_total] when ksplit > 1
};
// max_waves: waves per workgroup at most (1..5)
GemmPlan gemm_plan(int m, int n_total, int k, int max_waves = 4);
// sum_slices: also launch the slice sum into q0 / q1 (when ksplit > 1).  Without it the
// result of problem `prob` is left as gemm_result(...) describes, for a consumer to sum.
hipError_t launch_gemm(int m, int n, int k, const void* x, int nprob, const void* w0,
                       float* q0, const void* w1, float* q1, float* ws, const GemmPlan& plan,
                       hipStream_t stream, bool sum_slices = true,
                       hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
QParts gemm_result(const GemmPlan& plan, int m, int n, int nprob, int prob, const float* q,
                   const float* ws);
// ---- dense attention: the list of every resident block per pair ---------------------------
// lists [pairs][max_blocks] (ascending, unused entries untouched), counts [pairs]
hipError_t launch_dense_lists(const Shape& s, const int* seq_lens, const int* block_table,
                              int* lists, int* counts, hipStream_t stream);

// ---- periodic recall: the plan (one wave per pair), then one workgroup per copied block -----
// copies: [pairs][max_recall] int2 (pool page, host page); k_host/v_host device-addressable;
// threshold >= 0: nothing moves unless the layer's offloaded selected blocks exceed it
size_t recall_plan_lds_bytes(const Shape& s, int max_recall);
hipError_t launch_recall(const Shape& s, int list_stride, int max_recall, const int* seq_lens,
                         int* block_table, const int* gpu_blocks, const int* n_gpu,
                         const int* cpu_blocks, const int* n_cpu, const void* k_host,
                         const void* v_host, const int* host_table, int host_pages,
                         void* k_pool, void* v_pool, int* n_recalled, void* copies,
                         long threshold, hipStream_t stream);

// q_out[r][c] = the sum of the parts of q, for rows r < rows and columns c < n (n a multiple of
// 4); q_out may be device-addressable host memory.  With n_cpu ([rows][Hkv]), only the columns
// of KV heads h (columns [h * group_cols, (h + 1) * group_cols), a multiple of 4) whose
// n_cpu[r][h] > 0 are written.
hipError_t launch_gather_query(const QParts& q, int rows, int n, float* q_out, hipStream_t stream,
                               const int32_t* n_cpu = nullptr, int group_cols = 1, int Hkv = 1);

// ---- selection: scores, top-k and the resident split --------------------------------------
// Pairs [0, whole) get one workgroup each; the other `split` pairs are cut into nchunk
// chunks of `chunk` rows, one workgroup each, which hand their scores over through ws_bytes
// of workspace whose arrival counters must be zero before the first launch (every launch
// leaves them zero again).
struct SelectPlan {
  int whole;        // pairs of one workgroup each (full rounds of one per CU)
  int split;        // pairs cut into chunks (the rest)
  int chunk;        // rows per chunk workgroup
  int nchunk;       // chunks per split pair (of max_blocks rows)
  size_t ws_bytes;  // hand-over buffers; 0 when no pair is split
};
SelectPlan select_plan(const Shape& s, bool minmax);
// gpu_pages (optional, [pairs][top_k]): the page of each resident list entry, -1 past n_gpu.
hipError_t launch_select(const Shape& s, const SelectPlan& plan, bool minmax, const QParts& q,
                         const void* digests, const int32_t* seq_lens, int top_k,
                         const int32_t* block_table, int32_t* gpu_blocks, int32_t* n_gpu,
                         int32_t* cpu_blocks, int32_t* n_cpu, float* scores_or_null,
                         int32_t* cpu_blocks_host, int32_t* n_cpu_host,
                         int32_t* gpu_pages_or_null, void* ws, hipStream_t stream,
                         hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

// ---- attention: balanced waves write partials, then the reduction / merge per row -------
struct AttnPlan {
  int waves;         // W: waves in the grid; the resident selected blocks are split evenly
  int list_stride;   // entries per pair in the lists (bound of every per-pair count)
  size_t ws_bytes;   // pair prefix + one partial slot per (wave + pair) and head
};
AttnPlan attn_plan(const Shape& s, int list_stride);
hipError_t launch_attention(const Shape& s, const AttnPlan& plan, const QParts& q,
                            const void* k_pool, const void* v_pool,
                            const int32_t* block_table, const int32_t* seq_lens,
                            const int32_t* gpu_blocks, const int32_t* gpu_pages_or_null,
                            const int32_t* n_gpu, int list_stride, float scale,
                            float* partials, hipStream_t stream,
                            hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
// Combine the chunk partials of every (sequence, query head) row, optionally merged with a
// host partial (gated by n_cpu when given); writes normalised o and natural-unit m, l.
hipError_t launch_reduce(const Shape& s, const AttnPlan& plan, const int32_t* n_gpu,
                         const float* partials, const float* host_o, const float* host_m,
                         const float* host_l, const int32_t* n_cpu, float* o, float* m,
                         float* l, hipStream_t stream);

// ---- flags shared with the host (page-locked, coherent memory) -----------------------------
// *ready += 1 after everything before it on the stream (only the device writes *ready)
hipError_t launch_signal(uint32_t* ready, hipStream_t stream);
// holds the stream until *done == *ready (as read when the wait starts), for at most
// `rounds` polling rounds; on giving up it writes 1 to *timeouts and returns
hipError_t launch_wait(const uint32_t* done, const uint32_t* ready, uint32_t rounds,
                       uint32_t* timeouts, hipStream_t stream);
// polling rounds of launch_wait that last at least `ms` milliseconds
uint32_t wait_rounds(int ms);

// ---- merge of two normalised partials ------------------------------------------------------
hipError_t launch_merge(int rows, int d, const float* o_a, const float* m_a, const float* l_a,
                        const float* o_b, const float* m_b, const float* l_b, float* o,
                        float* m, float* l, hipStream_t stream);

}  // namespace sa
