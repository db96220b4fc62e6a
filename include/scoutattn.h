/*
 * scoutattn.h -- C ABI of libscoutattn.so, the MI355X (gfx950) GPU-side decode path of
 * ScoutAttention's GPU-CPU collaborative block-sparse attention.
 *
 * Source of every operation (cited by page title and section):
 *   "ScoutAttention: Efficient KV Cache Offloading via Layer-Ahead CPU Pre-computation for
 *   LLM Inference", arXiv:2603.27138 -- HTML full text ("[HTML Sec. n]"), and the
 *   papercache.org summary of the same paper, section 三, Algorithm 1 ("[Alg. 1]").
 *
 * Conventions shared by every call
 *   - Pointers named *_host are host memory; every other pointer is device memory owned by
 *     the caller.  The library keeps no pointer after a call returns and allocates no
 *     device memory: scratch space comes from the caller's workspace (`ws`, `ws_bytes`),
 *     whose required size the *_workspace_bytes() queries return.  (sa_decode_step keeps
 *     a per-thread pool of HIP events that order its two streams, reused across calls.)
 *   - Work is enqueued on the caller's `stream` and the call returns without waiting.
 *     Results are valid once the stream has reached that point.  Calls on different
 *     streams may run concurrently if they share no output or workspace.
 *   - Arguments are checked on the host before anything is launched: a failed check
 *     returns SA_ERR_INVALID_ARG / SA_ERR_UNSUPPORTED / SA_ERR_WORKSPACE and enqueues
 *     nothing.  A launch failure returns SA_ERR_HIP.  sa_last_error() then describes the
 *     failure (thread-local, valid until the next call on the same thread).  No C++
 *     exception crosses this interface.
 *   - Contents of device buffers (block-table entries, list entries and counts, sequence
 *     lengths) are NOT checked on the host: they must satisfy the ranges stated below,
 *     otherwise the results are unspecified.  The kernels clamp every index they take from
 *     these buffers, so no value in them makes a kernel access memory outside the buffers
 *     described here.
 *   - Layouts are row-major, innermost index last.  "KV dtype" is sa_dims.kv_dtype:
 *     SA_F32 (float) or SA_BF16 (bfloat16 bit patterns, uint16).
 *   - Alignment: every buffer is aligned to its element size, and the buffers the kernels
 *     move with 16-byte accesses to 16 bytes: the K/V pages and rows (k_pool, v_pool,
 *     k_rows, v_rows, k_host, v_host), digests, the GEMM's x, w and w_packed, the query q
 *     of the GEMM, selection and attention calls, and every workspace `ws`.  (hipMalloc and
 *     PyTorch allocations are 256-byte aligned.)  A call given one of these at another
 *     address returns SA_ERR_INVALID_ARG.
 *
 * Shapes: B sequences; Hq query heads; Hkv KV heads with G = Hq / Hkv query heads per KV
 * head (query head g uses KV head g / G); head dimension d; block size bs; P pages in the
 * paged K/V pool, one page holding bs tokens of one KV head.
 * block_table [B][Hkv][max_blocks] int32 maps block b of (sequence s, KV head h) to its
 * page, or holds -1 when that block is not resident in GPU memory.  Block b of sequence s
 * covers tokens [b*bs, min((b+1)*bs, seq_lens[s])); nb_s = ceil(seq_lens[s] / bs).
 *
 * Page layouts.  k_pool is chunk-major,
 * [P][d/x][bs][x] with x = 16 / (bytes per element) -- 8 for bf16, 4 for float32: the head
 * dimension is cut into 16-byte chunks and each chunk stores the page's bs tokens one after
 * another.  A 16-token slice of one chunk is then 256 contiguous bytes, which lets the
 * attention kernel load K straight into matrix-core operands with whole 128-byte cache
 * lines.  v_pool is [P][bs/16][d][16]: each 16-token half of a page stores its d channels
 * one after another, each channel's 16 tokens contiguous, so a 16-channel x 16-token tile
 * of V^T (a matrix-core operand) is 16*16 contiguous elements.  sa_pack_k_pages and
 * sa_pack_v_pages convert token-row pages [P][bs][d] into these layouts.
 */
#ifndef SCOUTATTN_H
#define SCOUTATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SA_ABI_VERSION 12

typedef enum {
  SA_OK = 0,
  SA_ERR_INVALID_ARG = -1,  /* null pointer, inconsistent or out-of-range argument   */
  SA_ERR_UNSUPPORTED = -2,  /* valid but not implemented: d, bs, dtype, G, GEMM shape */
  SA_ERR_WORKSPACE = -3,    /* ws_bytes smaller than the matching *_workspace_bytes() */
  SA_ERR_HIP = -4           /* a HIP runtime call or kernel launch failed             */
} sa_status;

typedef enum { SA_F32 = 0, SA_BF16 = 1 } sa_dtype;

/* Block digests [HTML Sec. 2.2]: MoBA-style mean pooling of K, or Quest-style channel-wise
 * min/max pooling of K. */
typedef enum { SA_DIGEST_MEAN = 0, SA_DIGEST_MINMAX = 1 } sa_digest_kind;

/* Problem shape.  Supported: head_dim in {64, 128}; block_size in {16, 32};
 * num_q_heads % num_kv_heads == 0 with G = num_q_heads / num_kv_heads in [1, 8];
 * 1 <= max_blocks <= 8192; batch * num_kv_heads <= 8192; num_pages >= 1; kv_dtype SA_F32
 * or SA_BF16. */
typedef struct {
  int32_t batch;         /* B                                                     */
  int32_t num_q_heads;   /* Hq                                                    */
  int32_t num_kv_heads;  /* Hkv                                                   */
  int32_t head_dim;      /* d                                                     */
  int32_t block_size;    /* bs, tokens per block and per page                    */
  int32_t max_blocks;    /* row length of block_table and of the digest arrays    */
  int32_t num_pages;     /* P, pages in k_pool / v_pool; table entries are < P    */
  sa_dtype kv_dtype;     /* dtype of k_pool, v_pool and the digests               */
} sa_dims;

/* ABI version of the loaded library (SA_ABI_VERSION when it matches this header). */
int sa_abi_version(void);

/* Description of the last failure on the calling thread ("" if none). */
const char* sa_last_error(void);

/* Name of a status code. */
const char* sa_status_string(sa_status status);

/* ---------------------------------------------------------------------------------------
 * sa_build_digests -- digest of every resident block [HTML Sec. 2.2].
 *   kind == SA_DIGEST_MEAN:   digests [B][Hkv][max_blocks][d]; entry b = mean of K over the
 *       block's valid tokens, accumulated exactly (float64) and rounded once,
 *       round-to-nearest-even, to the KV dtype.
 *   kind == SA_DIGEST_MINMAX: digests [B][Hkv][max_blocks][2][d]; [..][0][c] = minimum and
 *       [..][1][c] = maximum of K channel c over the block's valid tokens (exact).
 *   k_pool chunk-major (KV dtype); block_table [B][Hkv][max_blocks] (entries -1 or in
 *   [0, P)); seq_lens [B] (1 <= seq_lens[s] <= max_blocks*bs).  Entries of blocks that are
 *   not resident (table -1) or lie past the sequence end are left unchanged.
 * ------------------------------------------------------------------------------------- */
sa_status sa_build_digests(const sa_dims* dims, sa_digest_kind kind, const void* k_pool,
                           const int32_t* block_table, const int32_t* seq_lens,
                           void* digests, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * sa_refresh_last_digests -- digest maintenance during decode [HTML Sec. 2.2]: after the
 * token at position seq_lens[s] - 1 has been written into its page, the digest of the
 * block that holds it changes (its mean or min/max gains one token; a token that opens a
 * new block gives that block its first digest).  This recomputes, for every (sequence s,
 * KV head h), only the entry of block (seq_lens[s] - 1) / bs, from its page, with the same
 * arithmetic as sa_build_digests, so the entry is bit-identical to what a full rebuild
 * writes.  Arguments and layouts as for sa_build_digests; a pair whose last block is not
 * resident (table -1) is left unchanged.
 * ------------------------------------------------------------------------------------- */
sa_status sa_refresh_last_digests(const sa_dims* dims, sa_digest_kind kind,
                                  const void* k_pool, const int32_t* block_table,
                                  const int32_t* seq_lens, void* digests, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * sa_pack_k_pages -- layout conversion (no arithmetic): k_rows [P][bs][d] token-row pages
 * of K in the KV dtype -> k_pool [P][d/x][bs][x], the chunk-major K layout that every call
 * below reads (x = 16 / bytes per element).  Both device buffers hold P*bs*d elements and
 * must not overlap.
 * ------------------------------------------------------------------------------------- */
sa_status sa_pack_k_pages(const sa_dims* dims, const void* k_rows, void* k_pool,
                          hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * sa_pack_v_pages -- layout conversion (no arithmetic): v_rows [P][bs][d] token-row pages
 * of V in the KV dtype -> v_pool [P][bs/16][d][16], the layout every call below reads:
 * element (page, token t, channel c) goes to v_pool[page][t / 16][c][t % 16].  Both device
 * buffers hold P*bs*d elements and must not overlap.
 * ------------------------------------------------------------------------------------- */
sa_status sa_pack_v_pages(const sa_dims* dims, const void* v_rows, void* v_pool,
                          hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * sa_pack_weight -- layout conversion (no arithmetic) of a query-projection weight, done
 * once when the weights are loaded: w [n][k] bf16 (row j = output feature j, the
 * linear-layer layout) -> w_packed [n/16][k/32][64][8] bf16, the order in which
 * sa_predict_query streams it.  Tile (a, b) holds rows 16a..16a+15 and columns
 * 32b..32b+31; its element [l][e] is w[16a + l % 16][32b + 8 (l / 16) + e].  Both buffers
 * hold n*k elements and must not overlap.  Supported: n % 16 == 0, k % 32 == 0, n, k >= 32.
 * ------------------------------------------------------------------------------------- */
sa_status sa_pack_weight(int32_t n, int32_t k, const void* w, void* w_packed,
                         hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * sa_predict_query -- the layer-ahead query prediction Q_pred^{i+1} = W_Q^{i+1} X^i
 * ([Alg. 1]; [HTML Sec. 3.3]); the same call with W_Q^i gives the true query Q^i.
 *   x [m][k] bf16 (one row per sequence); w_packed: the weight w [n][k] bf16 (row j =
 *   output feature j) in the order written by sa_pack_weight; q [m][n] float32 = x w^T
 *   (bf16 products, float32 accumulation, not rounded further).
 *   Supported: 1 <= m <= 256, n % 64 == 0, k % 64 == 0, n, k >= 64.
 *   For attention, q is viewed as [m][Hq][d] (head j / d).
 *   ws: sa_predict_query_workspace_bytes(m, n, k) bytes (may be 0 -> ws may be NULL).
 * ------------------------------------------------------------------------------------- */
size_t sa_predict_query_workspace_bytes(int32_t m, int32_t n, int32_t k);
sa_status sa_predict_query(int32_t m, int32_t n, int32_t k, const void* x,
                           const void* w_packed, float* q, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * Workspace of sa_select_blocks + sa_sparse_decode (+ sa_decode_attend_merge) for a shape
 * and a top_k (a decode call uses list_stride == top_k).  Its first part holds the
 * selection's hand-over buffers and arrival counters: the caller fills the workspace with
 * zeros once, before its first use (hipMemset, or a zero-filled allocation), and every call
 * leaves the counters zero again.  Calls that share one workspace must not overlap in time
 * (same stream, or ordered with events).
 * ------------------------------------------------------------------------------------- */
size_t sa_workspace_bytes(const sa_dims* dims, int32_t top_k);

/* ---------------------------------------------------------------------------------------
 * sa_select_blocks -- B_pred = TopK(Q K_digest^T), B_cpu = B_pred \ B_gpu  ([Alg. 1];
 * [HTML Sec. 3.2]), once per (sequence s, KV head h):
 *   score sigma_b for every block b < nb_s, summed over the G query heads of the group:
 *     mean:   sigma_b = sum_g q_g . digest_b
 *     minmax: sigma_b = sum_g sum_c max(q_gc * min_bc, q_gc * max_bc)   (Quest's bound)
 *   select the k_s = min(top_k, nb_s) largest scores (equal scores: lower block index
 *   first), then split them by residency (block_table[s][h][b] >= 0).
 *   q [B][Hq][d] float32; digests as written by sa_build_digests; seq_lens [B] in
 *   [1, max_blocks*bs]; 1 <= top_k <= max_blocks.
 *   Outputs: gpu_blocks, cpu_blocks [B][Hkv][top_k] int32 -- the resident / offloaded
 *   selected block indices, ascending, padded with -1; n_gpu, n_cpu [B][Hkv] int32 (their
 *   counts, n_gpu + n_cpu = k_s).  scores [B][Hkv][max_blocks] float32 may be NULL; when
 *   given it receives sigma_b for b < nb_s.
 * ------------------------------------------------------------------------------------- */
sa_status sa_select_blocks(const sa_dims* dims, sa_digest_kind kind, const float* q,
                           const void* digests, const int32_t* seq_lens, int32_t top_k,
                           const int32_t* block_table, int32_t* gpu_blocks, int32_t* n_gpu,
                           int32_t* cpu_blocks, int32_t* n_cpu, float* scores, void* ws,
                           size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * sa_sparse_decode -- A_gpu = GPUATTN(Q, B_gpu) ([Alg. 1]; [HTML Sec. 3.2]): for every
 * query head g of sequence s, softmax attention over the valid tokens of the blocks listed
 * in gpu_blocks[s][g/G][0 .. n_gpu[s][g/G]) (each block read through block_table):
 *   z_t = scale * q_g . K_t,  m = max z,  l = sum exp(z - m),  o = sum exp(z - m) V_t / l.
 *   An empty list gives o = 0, m = -inf, l = 0.
 *   q [B][Hq][d] float32; k_pool (chunk-major), v_pool ([P][bs/16][d][16]) in the KV dtype;
 *   gpu_blocks [B][Hkv][list_stride] with
 *   entries in [0, nb_s) whose table entry is a page in [0, P); 0 <= n_gpu <= list_stride.
 *   Outputs o [B][Hq][d], m [B][Hq], l [B][Hq] float32 (m in natural-log units); m and l
 *   may be NULL when not wanted.
 *   ws: sa_workspace_bytes(dims, list_stride).
 * ------------------------------------------------------------------------------------- */
sa_status sa_sparse_decode(const sa_dims* dims, const float* q, const void* k_pool,
                           const void* v_pool, const int32_t* block_table,
                           const int32_t* seq_lens, const int32_t* gpu_blocks,
                           const int32_t* n_gpu, int32_t list_stride, float scale, float* o,
                           float* m, float* l, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * sa_merge -- A = MERGE(A_a, A_b), the FlashAttention combination of two partials over
 * disjoint token sets ([Alg. 1]; [HTML Sec. 3.2]), per row r < rows:
 *   M = max(m_a, m_b); w_x = l_x exp(m_x - M) (0 if m_x = -inf); l = w_a + w_b;
 *   o = (w_a o_a + w_b o_b) / l; m = M.  Two empty partials give (0, -inf, 0).
 *   o_* [rows][d], m_*, l_* [rows] float32, o normalised.  The outputs may alias a.
 *   Supported: rows >= 1, 1 <= d <= 1024.
 * ------------------------------------------------------------------------------------- */
sa_status sa_merge(int32_t rows, int32_t d, const float* o_a, const float* m_a,
                   const float* l_a, const float* o_b, const float* m_b, const float* l_b,
                   float* o, float* m, float* l, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * sa_decode_attend_merge -- GPUATTN followed by MERGE with the host partial in one
 * enqueue ([Alg. 1], the attention and merge steps of layer i): the result equals
 * sa_sparse_decode followed by sa_merge with (host_o, host_m, host_l) [B][Hq][d], [B][Hq],
 * except that when n_cpu is not NULL the host partial of every head of (s, h) with
 * n_cpu[s][h] == 0 is treated as empty (nothing was offloaded, so nothing came back).
 * Arguments as for sa_sparse_decode; ws: sa_workspace_bytes(dims, list_stride).
 * ------------------------------------------------------------------------------------- */
sa_status sa_decode_attend_merge(const sa_dims* dims, const float* q, const void* k_pool,
                                 const void* v_pool, const int32_t* block_table,
                                 const int32_t* seq_lens, const int32_t* gpu_blocks,
                                 const int32_t* n_gpu, int32_t list_stride, float scale,
                                 const float* host_o, const float* host_m,
                                 const float* host_l, const int32_t* n_cpu, float* o,
                                 float* m, float* l, void* ws, size_t ws_bytes,
                                 hipStream_t stream);

/*
 * sa_host_partial_attention -- A_cpu, the CPU side of the collaborative attention
 * ([Alg. 1]: the blocks of B_pred that are not resident on the GPU, B_cpu, are attended on
 * the CPU from host memory; [HTML Sec. 3.2, 3.3]).  HOST memory and host threads only: no
 * stream, no device pointer, and the call returns when the results are written.
 *
 * For every sequence s and query head qh (KV head h = qh / G): the partial (o, m, l) of
 * q[s][qh] over the valid tokens of blocks cpu_blocks_host[s][h][0 .. n_cpu_host[s][h]),
 * with scale `scale` (natural-log units: m is the largest scaled logit, l the sum of
 * exp(logit - m), o the normalised weighted sum of V rows) -- the form sa_merge and
 * sa_decode_attend_merge take as their host partial.  A pair with no block gives
 * (o = 0, m = -inf, l = 0).
 *
 *   dims: as for the device calls (num_pages is not used here); host_pages: pages in the
 *   host pool.  q_host [B][Hq][d] float32.  k_host, v_host [host_pages][bs][d], KV dtype,
 *   token rows (the layout blocks are offloaded in).  host_table [B][Hkv][max_blocks]
 *   int32: the host page of each block, or -1.  seq_lens_host [B].  cpu_blocks_host
 *   [B][Hkv][list_stride], n_cpu_host [B][Hkv]: the offloaded lists, as sa_select_blocks
 *   or sa_decode_step hand them over.  o_host [B][Hq][d], m_host, l_host [B][Hq] float32.
 *   num_threads: worker threads (0: the machine's hardware threads).
 * List entries outside [0, max_blocks), blocks without a host page and blocks past their
 * sequence are skipped.  The result does not depend on num_threads.
 */
sa_status sa_host_partial_attention(const sa_dims* dims, int32_t host_pages,
                                    const float* q_host, const void* k_host,
                                    const void* v_host, const int32_t* host_table,
                                    const int32_t* seq_lens_host,
                                    const int32_t* cpu_blocks_host, const int32_t* n_cpu_host,
                                    int32_t list_stride, float scale, float* o_host,
                                    float* m_host, float* l_host, int32_t num_threads);

/* ---------------------------------------------------------------------------------------
 * sa_decode_step -- one decode step over num_layers layers in the layer-ahead order of
 * Algorithm 1 ([Alg. 1]; [HTML Sec. 3.3]).  For layer i:
 *   1. Q^i = W_Q^i X^i and, for i < L-1, Q_pred^{i+1} = W_Q^{i+1} X^i (one GEMM launch);
 *   2. (layer 0 only) select B^0 with Q^0 -- the first layer has no predecessor;
 *   3. for i < L-1: select B_pred^{i+1} with Q_pred^{i+1} and layer i+1's digests and block
 *      table, writing layer i+1's lists; when a layer's host pointers are set, its selection
 *      kernel also writes n_cpu and cpu_blocks straight into them (the hand-off that spawns
 *      the CPU-side attention, with no copy).  They must be coherent page-locked host
 *      memory the device can address (hipHostMalloc with hipHostMallocCoherent); the values
 *      are complete once the stream that ran that selection has passed it;
 *   4. A_gpu^i over B_gpu^i with Q^i, merged with layer i's host partial (ignored for heads
 *      whose n_cpu is 0) into out_o/out_m/out_l.
 * With side_stream given, the prediction Q_pred^{i+1} and step 3 (the selection one layer
 * ahead) run on side_stream, concurrently with step 4 of layer i on `stream`; the two
 * touch disjoint buffers, and layer i+1's attention waits for its selection.  With
 * side_stream NULL (or equal to `stream`) every step runs in order on `stream`.  All layers share dims, digest kind, hidden, top_k, scale and seq_lens.  `layers`
 * is a host array of num_layers descriptors (read during the call only).  Before returning,
 * `stream` waits for everything enqueued on side_stream, so a graph captured from `stream`
 * is closed.  ws: sa_step_workspace_bytes(dims, hidden, top_k), zero-filled before its first
 * use (it holds the selection's arrival counters, which every step leaves zero again).
 * ------------------------------------------------------------------------------------- */
typedef struct {
  const void* x;            /* X^i [B][hidden] bf16                                       */
  const void* w_q;          /* W_Q^i [Hq*d][hidden] bf16, packed by sa_pack_weight       */
  const void* digests;      /* layer digests, sa_build_digests layout for the kind        */
  const int32_t* block_table; /* [B][Hkv][max_blocks]                                     */
  const void* k_pool;       /* chunk-major K pages, bf16                                  */
  const void* v_pool;       /* [P][bs/16][d][16] bf16 (sa_pack_v_pages)                   */
  const float* host_o;      /* A_cpu^i: [B][Hq][d], normalised                            */
  const float* host_m;      /* [B][Hq], natural-log units                                 */
  const float* host_l;      /* [B][Hq]                                                    */
  int32_t* gpu_blocks;      /* out: B_gpu^i list [B][Hkv][top_k]                          */
  int32_t* n_gpu;           /* out: [B][Hkv]                                              */
  int32_t* cpu_blocks;      /* out: B_cpu^i list [B][Hkv][top_k]                          */
  int32_t* n_cpu;           /* out: [B][Hkv]                                              */
  int32_t* cpu_blocks_host; /* optional host mirror of cpu_blocks (or NULL), coherent      */
  int32_t* n_cpu_host;      /* optional host mirror of n_cpu (or NULL), coherent           */
  float* out_o;             /* out: A^i [B][Hq][d]                                        */
  float* out_m;             /* out: [B][Hq] (may be NULL)                                 */
  float* out_l;             /* out: [B][Hq] (may be NULL)                                 */
} sa_layer;

size_t sa_step_workspace_bytes(const sa_dims* dims, int32_t hidden, int32_t top_k);
sa_status sa_decode_step(const sa_dims* dims, sa_digest_kind kind, int32_t hidden,
                         int32_t top_k, float scale, const int32_t* seq_lens,
                         int32_t num_layers, const sa_layer* layers, void* ws,
                         size_t ws_bytes, hipStream_t stream, hipStream_t side_stream);

/* ---------------------------------------------------------------------------------------
 * The CPU side of the step, run one layer ahead ([Alg. 1]: CPUAttn(B_cpu^{i+1}) is spawned
 * while layer i runs, and its result A_cpu^{i+1} is merged at layer i+1; [HTML Sec. 3.3]:
 * the CPU's window is the GPU's layer i).
 *
 * sa_host_layer -- one layer's host side.  The first three members may be ordinary host
 * memory (only host threads read them); the rest must be coherent page-locked host memory
 * the device can address (hipHostMalloc with hipHostMallocCoherent), as the device writes or
 * reads them.  All are owned by the caller and must stay valid while a plan that names
 * them exists.
 * ------------------------------------------------------------------------------------- */
typedef struct {
  const void* k_host;        /* the layer's offloaded keys [host_pages][bs][d], KV dtype,
                                token rows (the layout of sa_host_partial_attention)       */
  const void* v_host;        /* values, same layout                                         */
  const int32_t* host_table; /* [B][Hkv][max_blocks]: host page of each block, or -1        */
  int32_t host_pages;        /* pages in k_host / v_host                                    */
  float* q_host;             /* [B][Hq][d] float32, written by the step: the query the CPU
                                attends with (Q_pred^i; Q^0 for layer 0)                    */
  int32_t* cpu_blocks_host;  /* [B][Hkv][top_k], written by the step's selection: B_cpu^i   */
  int32_t* n_cpu_host;       /* [B][Hkv], written by the step's selection                   */
  float* o_host;             /* [B][Hq][d] float32: A_cpu^i, written by the host workers and
                                read by the step's merge of layer i                          */
  float* m_host;             /* [B][Hq], natural-log units                                  */
  float* l_host;             /* [B][Hq]                                                     */
} sa_host_layer;

/* sa_host_plan -- the host side of sa_decode_step_offload: the layers' host buffers, the
 * shape, and a pool of num_threads persistent worker threads (0: the machine's hardware
 * threads).  Creating it touches no device.  seq_lens_host [B] is read by the host work every
 * time it runs (not copied).  *plan receives the handle, or NULL on error.
 * sa_host_plan_destroy stops the workers; it must not be called while enqueued work (or a
 * HIP graph captured from sa_decode_step_offload) that uses the plan can still run.
 * sa_host_plan_stats: the number of layer tasks run so far and the host time they took
 * (seconds, wall clock inside the tasks); SA_ERR_HIP if a task failed (its partial is then
 * left as the empty partial).  Either output pointer may be NULL.
 * sa_host_plan_run: runs layer `layer`'s host task now, on the calling thread and the plan's
 * workers (what the step enqueues as a host function), from the layer's q_host and hand-off
 * lists as they are; returns when o_host/m_host/l_host are written.  For callers that drive
 * the CPU side themselves.  Not while the plan's tasks may run from a stream. */
typedef struct sa_host_plan sa_host_plan;
sa_status sa_host_plan_create(const sa_dims* dims, int32_t top_k, float scale,
                              const int32_t* seq_lens_host, int32_t num_layers,
                              const sa_host_layer* layers, int32_t num_threads,
                              sa_host_plan** plan);
sa_status sa_host_plan_run(sa_host_plan* plan, int32_t layer);

/* sa_host_plan_set_recall -- periodic recall inside the offload step ([HTML Sec. 3.4]: the
 * recall is issued after the layer's attention, off the critical path, and is needed only
 * at the same layer of the next step).  With it set, sa_decode_step_offload enqueues, after
 * each layer's merge, sa_recall_blocks for that layer on recall_stream, gated on the device:
 * nothing moves unless the layer's CPU compute ratio, sum of n_cpu over pairs / (pairs *
 * top_k), is above beta.  The plan's k_host / v_host must then be page-locked memory the
 * device reads (hipHostMalloc), and each layer's block_table, k_pool and v_pool in the
 * step's sa_layer are written (the step's own selection and attention of that layer are
 * over by then).  layers: num_layers entries (host array, copied): host_table_dev, the
 * layer's host_table in device memory (NULL: the layer is never recalled), and n_recalled
 * [B][Hkv] device int32, the blocks moved per pair at the layer's last step (0 when not
 * due).  ws: sa_recall_workspace_bytes(dims, max_recall) device bytes, used by one layer at a
 * time (the recalls run in order on recall_stream); it and the arrays must outlive the plan's
 * use.  max_recall in [1, 4096], beta >= 0.  layers == NULL turns recall off again.
 * overlap = 0: each step waits for its recalls before it returns.  overlap != 0: as in the
 * pages, a step leaves its recalls running and the next step's selection of layer i waits
 * for layer i's recall only; the caller synchronises recall_stream before it reads or writes
 * a layer's block table, pages or n_recalled itself, and such steps cannot be captured in a
 * graph (SA_ERR_INVALID_ARG).  The call waits for recalls still running, and creates the
 * events it needs on the current device. */
typedef struct {
  const int32_t* host_table_dev;
  int32_t* n_recalled;
} sa_recall_layer;
sa_status sa_host_plan_set_recall(sa_host_plan* plan, int32_t max_recall, float beta,
                                  const sa_recall_layer* layers, void* ws, size_t ws_bytes,
                                  int32_t overlap);
sa_status sa_host_plan_destroy(sa_host_plan* plan);
sa_status sa_host_plan_stats(const sa_host_plan* plan, int64_t* tasks, double* busy_seconds);

/* sa_host_plan_set_handoff -- how sa_decode_step_offload hands each layer's CPU side over
 * ([HTML Sec. 3.3]: the CPU attends layer i's offloaded blocks while the GPU works one layer
 * ahead; the GPU merges the two partials at layer i).
 *   SA_HANDOFF_HOST_FUNC (the default): a HIP host function per layer on host_stream, and an
 *     event the merge waits for.
 *   SA_HANDOFF_FLAGS: flags in memory both sides see.  flags: 2 * num_layers + 1 uint32
 *     words, page-locked and coherent (hipHostMalloc with hipHostMallocCoherent), owned by the
 *     caller and kept while the plan uses them; the call zeroes them.  Words [0, L) are the
 *     layers' ready counters, [L, 2L) their done flags, word 2L the GPU's timeout record.
 *     Per layer and step, a one-lane kernel advances ready[i] once the selection's lists and
 *     the gathered query are written; the plan's dispatcher thread, seeing ready[i] !=
 *     done[i], runs the layer's task and then sets done[i] = the ready value it served; a
 *     one-lane kernel before the merge holds `stream` until done[i] == ready[i].  Every
 *     ready value the dispatcher sees gets its done flag: after the task, after a failed
 *     task (partial empty), and, when the plan is destroyed or switched, for a layer raised
 *     but not served (partial empty).  The GPU wait gives up after about gpu_wait_ms (it then
 *     writes 1 to word 2L, the merge reads a partial that may be incomplete, and
 *     sa_host_plan_stats reports it), so no wait is left unresolved whatever the host does.
 *     gpu_wait_ms >= 1, well above the longest layer task.  No value comes from the host, so
 *     a step may be captured in a HIP graph and replayed.  host_stream is not used (it may be
 *     NULL).
 * Call it while no step of the plan is in flight.  With SA_HANDOFF_FLAGS, sa_host_plan_stats
 * first waits until every raised layer has been served (call it after the step's stream has
 * been synchronised), and fails (SA_ERR_HIP) if a GPU wait has timed out. */
typedef enum { SA_HANDOFF_HOST_FUNC = 0, SA_HANDOFF_FLAGS = 1 } sa_handoff;
sa_status sa_host_plan_set_handoff(sa_host_plan* plan, sa_handoff mode, uint32_t* flags,
                                   int32_t gpu_wait_ms);

/* sa_stream_signal / sa_stream_wait -- the two kernels of the flag hand-off, on their own.
 * counter, flag, timeouts: words in page-locked coherent host memory (or device memory).
 * sa_stream_signal: *counter += 1 once everything before it on `stream` has finished (only
 * the device may write *counter).  sa_stream_wait: holds `stream` until *flag equals
 * *counter (read when the wait starts), polling for at most about wait_ms milliseconds
 * (wait_ms >= 1); if they are still unequal then, it writes 1 to *timeouts and lets the
 * stream go on.  Its wave always ends. */
sa_status sa_stream_signal(uint32_t* counter, hipStream_t stream);
sa_status sa_stream_wait(const uint32_t* flag, const uint32_t* counter, int32_t wait_ms,
                         uint32_t* timeouts, hipStream_t stream);

/* sa_decode_step_offload -- sa_decode_step with the CPU side computed, not given.  The
 * arguments are those of sa_decode_step, with the plan's shape, top_k, scale and num_layers;
 * in `layers`, host_o/host_m/host_l and the host mirrors are not used (the plan's buffers
 * take their place).  For each layer i, once B^i is selected (layer 0 on `stream`, the
 * others one layer ahead on side_stream), the step writes the query the CPU attends with
 * into q_host (the query heads of the pairs with offloaded blocks; the other rows are left
 * as they are) and the lists into the plan's mirrors, then enqueues on host_stream a host
 * task that computes A_cpu^i with the plan's workers (as sa_host_partial_attention does)
 * into o_host/m_host/l_host; layer i's merge on `stream` waits for that task.  (With the
 * plan's SA_HANDOFF_FLAGS hand-off the task is run by the plan's dispatcher thread instead,
 * see sa_host_plan_set_handoff.)  host_stream
 * must be a stream of its own (not `stream`, not side_stream): each task holds it while it
 * runs.  Layer 0 has no layer before it, so its merge waits for its own CPU side.  Before
 * returning, `stream` waits for host_stream, side_stream and (unless the plan's recalls
 * overlap the next step) recall_stream.  recall_stream
 * (a stream of its own, or NULL) carries the recalls when the plan has them set
 * (sa_host_plan_set_recall); it is required then.  A HIP graph may be captured from
 * `stream`; its host tasks then run with the plan's buffers at every replay.
 * ------------------------------------------------------------------------------------- */
sa_status sa_decode_step_offload(const sa_dims* dims, sa_digest_kind kind, int32_t hidden,
                                 int32_t top_k, float scale, const int32_t* seq_lens,
                                 int32_t num_layers, const sa_layer* layers, void* ws,
                                 size_t ws_bytes, hipStream_t stream, hipStream_t side_stream,
                                 sa_host_plan* plan, hipStream_t host_stream,
                                 hipStream_t recall_stream);

/* ---------------------------------------------------------------------------------------
 * sa_dense_decode -- dense paged decode attention (FullKV, the pages' uncompressed baseline
 * [HTML Sec. 4]): for every query head g of sequence s, softmax attention over the valid
 * tokens of every block b < nb_s whose block_table entry is a page in [0, num_pages), in the
 * form of sa_sparse_decode's result (o normalised, m natural-log units, l; no block gives
 * o = 0, m = -inf, l = 0).  With every block resident this is plain attention over the whole
 * context.  Arguments as for sa_sparse_decode, with no lists; m and l may be NULL.
 * ws: sa_dense_workspace_bytes(dims) (the lists of every resident block, then the attention
 * partials).
 * ------------------------------------------------------------------------------------- */
size_t sa_dense_workspace_bytes(const sa_dims* dims);
sa_status sa_dense_decode(const sa_dims* dims, const float* q, const void* k_pool,
                          const void* v_pool, const int32_t* block_table,
                          const int32_t* seq_lens, float scale, float* o, float* m, float* l,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * sa_recall_blocks -- asynchronous periodic KV recall ([HTML Sec. 3.4]: at intervals,
 * important blocks are brought back from host memory into GPU memory, so that the share of
 * the budget the CPU attends stays below a threshold; the copy is issued after the layer's
 * attention and is needed only at the same layer of the next decode step).
 *
 * For every (sequence s, KV head h), from one layer's current selection lists:
 *   candidates: cpu_blocks[s][h][0 .. n_cpu) in list order, skipping entries outside the
 *     sequence, already resident (block_table >= 0) or without a host page;
 *   evictable: the resident blocks of the sequence (a page in [0, num_pages)) that are in
 *     neither gpu_blocks[s][h][0 .. n_gpu) nor the cpu list, in ascending block order;
 *   n = min(#candidates, #evictable, max_recall) blocks move: candidate t takes the page of
 *     evictable block t (block_table: evicted -> -1, candidate -> the page), and its keys and
 *     values are copied from the host store into that page, in the pool layouts
 *     (sa_pack_k_pages / sa_pack_v_pages).  n_recalled[s][h] = n.
 * Digests are not touched (a block's digest does not depend on where the block is held).
 *
 *   list_stride: the lists' row length (the selection's top_k).  seq_lens [B], block_table
 *   [B][Hkv][max_blocks] (updated in place), the lists, k_pool, v_pool, n_recalled [B][Hkv]:
 *   device memory.  k_host, v_host [host_pages][bs][d], KV dtype, token rows: page-locked
 *   host memory the device reads (hipHostMalloc).  host_table [B][Hkv][max_blocks]: host
 *   page of each block, or -1; device memory or page-locked host memory.
 *   ws: sa_recall_workspace_bytes(dims, max_recall) (the copy list).
 * Runs on `stream` (two launches); nothing else may read or write the layer's block table
 * or pool pages meanwhile -- issue it on the stream of the layer's attention, after it, or
 * order another stream after that attention and order the next use of the layer after it.
 * max_recall in [1, 4096].
 * ------------------------------------------------------------------------------------- */
size_t sa_recall_workspace_bytes(const sa_dims* dims, int32_t max_recall);
sa_status sa_recall_blocks(const sa_dims* dims, int32_t list_stride, int32_t max_recall,
                           const int32_t* seq_lens, int32_t* block_table,
                           const int32_t* gpu_blocks, const int32_t* n_gpu,
                           const int32_t* cpu_blocks, const int32_t* n_cpu, const void* k_host,
                           const void* v_host, const int32_t* host_table, int32_t host_pages,
                           void* k_pool, void* v_pool, int32_t* n_recalled, void* ws,
                           size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * sa_decode_attend_merge_noalloc -- sa_decode_attend_merge for callers that cannot allocate
 * (code under stream capture, tight serving loops, harnesses that forbid allocation): the
 * same arguments without the workspace, the same kernels and results.  The attention
 * partials go to a 16 MiB scratch array the library holds on every GPU it runs on, until
 * the process ends; the call itself allocates nothing.  A shape whose partials need more
 * (about (2048 + B*Hkv) * G * (d + 2) * 4 bytes) is refused with SA_ERR_WORKSPACE before
 * anything is launched.  All calls on one GPU share its scratch: calls that overlap in time
 * on one GPU (different streams, not ordered by events) race and give wrong results.
 * ------------------------------------------------------------------------------------- */
sa_status sa_decode_attend_merge_noalloc(const sa_dims* dims, const float* q,
                                         const void* k_pool, const void* v_pool,
                                         const int32_t* block_table, const int32_t* seq_lens,
                                         const int32_t* gpu_blocks, const int32_t* n_gpu,
                                         int32_t list_stride, float scale, const float* host_o,
                                         const float* host_m, const float* host_l,
                                         const int32_t* n_cpu, float* o, float* m, float* l,
                                         hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * sa_profile_kernels -- kernel timing of one stage: the attention kernel (GPUATTN), the
 * selection kernel (scoring + top-k + split) or the query GEMM kernel.  After this call the
 * next n launches of that stage's kernel made by the calling thread (from any call that
 * runs it, the decode step included) record start[i] when the i-th launch begins executing
 * and stop[i] when it ends, so hipEventElapsedTime(start[i], stop[i]) is that kernel's
 * duration (the GEMM's slice sum, a kernel of its own, is not included).  Events are
 * created by the caller and must stay valid until those launches have completed; the handle
 * arrays are copied.  Launches beyond n record nothing; n = 0 turns the hook off.  Not for
 * use while a stream is being captured.  sa_profile_attention(...) is
 * sa_profile_kernels(SA_PROFILE_ATTENTION, ...).
 * ------------------------------------------------------------------------------------- */
typedef enum {
  SA_PROFILE_ATTENTION = 0,
  SA_PROFILE_SELECT = 1,
  SA_PROFILE_GEMM = 2,
  SA_PROFILE_STAGES = 3
} sa_profile_stage;
sa_status sa_profile_kernels(sa_profile_stage stage, const hipEvent_t* start,
                             const hipEvent_t* stop, int32_t n);
sa_status sa_profile_attention(const hipEvent_t* start, const hipEvent_t* stop, int32_t n);

#ifdef __cplusplus
}
#endif

#endif /* SCOUTATTN_H */
