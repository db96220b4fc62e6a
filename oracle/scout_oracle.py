"""Plain float64 CPU oracle for the GPU-side decode path of ScoutAttention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or execute this
module: only the test suite, the smoke check and the benchmark's CPU-baseline leg use it.
It shares no code, helper, table or constant with the HIP kernels or their C ABI.

Sources (cited by title and section; no other material is used):
  [HTML]   "ScoutAttention: Efficient KV Cache Offloading via Layer-Ahead CPU Pre-computation
           for LLM Inference", arXiv:2603.27138, HTML full text.  Its section numbers are
           the ones the text itself cross-references (Sec. 2.2, 2.3, 3.2, 3.3, 3.4).
  [DIGEST] the papercache.org summary page of the same paper (same title), sections
           二 (background), 三 (method, with Algorithm 1 "layer-ahead CPU pre-computation").

What is computed (every stage is an exact definition, so this oracle is that definition
written out in float64, with no blocking, fusion or reordering beyond it):
  * Q_pred^{i+1} = W_Q^{i+1} X^i                      [DIGEST 三 eq. (Q_pred); HTML Sec. 3.3]
  * fixed-size KV blocks, each summarised by a digest: mean pooling of K (MoBA) or
    channel-wise min/max pooling of K (Quest)        [HTML Sec. 2.2; DIGEST 二]
  * block score = dot product of the query with the digest; top-k blocks
                                                      [HTML Sec. 2.2, Sec. 3.2; Algorithm 1]
  * B_cpu = B_pred \\ B_gpu                           [Algorithm 1; HTML Sec. 3.3]
  * GPU partial attention over the resident selected blocks, and a FlashAttention-style
    merge of the partials                             [HTML Sec. 3.2; Algorithm 1]
  * the layer-ahead order: layer i predicts and selects for layer i+1, then attends and
    merges layer i                                    [Algorithm 1; HTML Sec. 3.3]
  * the CPU side's partial over B_cpu, spawned one layer ahead and so computed with the
    predicted query                                   [Algorithm 1; HTML Sec. 3.3, 4]
  * periodic recall: offloaded selected blocks move into the pages of resident blocks
    that are no longer selected                       [HTML Sec. 3.4; DIGEST 三]

Readings taken where the pages are silent:
  R1 min/max score = sum_c max(q_c*min_c, q_c*max_c), Quest's upper bound on q.k.
  R2 one selection per (sequence, KV head): the scores of the G query heads that share
     the KV head are summed.
  R3 no scaling of the scores (top-k is invariant under a positive scale).
  R4 ties in the score: the lower block index wins.
  R5 k = budget_tokens / block_size; a sequence with fewer blocks selects all of them.
  R6 GPU attention covers only the selected resident blocks (S intersect R).
  R7 softmax scale 1/sqrt(d); m is the max of the scaled logits (natural-log units);
     o is normalised per partial.
  R8 the empty partial is (o = 0, m = -inf, l = 0), the identity of the merge.
  R9 a partial last block holds only its valid tokens: its mean divides by that count
     and attention ignores the rest.
  R10 the stored digest is the float64 value rounded once, round-to-nearest-even, to the
     KV dtype (mean); min/max are exact.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

NEG_INF = float("-inf")


# ----------------------------------------------------------------------------------------
# Storage rounding (reading R10)
# ----------------------------------------------------------------------------------------

def round_to_bf16(x) -> np.ndarray:
    """Round float64 values once, to nearest with ties to even, onto the bfloat16 grid.

    bfloat16 has an 8-bit significand (7 stored bits) and float32's exponent range.  For a
    value |x| in [2^e, 2^{e+1}) the grid spacing is 2^{e-7}; below 2^-126 the spacing stays
    2^-133 (subnormals).  The value is divided by the spacing (exact: a power of two),
    rounded half-to-even to an integer, and scaled back.  Results of magnitude 2^128 or
    more overflow to infinity.  Returns float64 arrays holding bfloat16 values.
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0.0)
    a = np.abs(x[fin])
    _, e2 = np.frexp(a)                    # a = f * 2^e2, f in [0.5, 1)
    e = np.maximum(e2 - 1, -126)           # floor(log2 a), clamped at the subnormal range
    spacing = np.ldexp(1.0, e - 7)
    r = np.rint(a / spacing) * spacing      # np.rint rounds half to even
    r = np.where(r >= 2.0 ** 128, np.inf, r)
    out[fin] = np.copysign(r, x[fin])
    return out


def round_to_f32(x) -> np.ndarray:
    """Round float64 values once (nearest, ties to even) to float32; returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def store_rounding(kv_dtype: str):
    """The single rounding a digest takes when stored in the KV dtype (reading R10)."""
    if kv_dtype == "bf16":
        return round_to_bf16
    if kv_dtype == "f32":
        return round_to_f32
    raise ValueError(f"unknown KV dtype {kv_dtype!r}")


# ----------------------------------------------------------------------------------------
# O1: layer-ahead query prediction  [DIGEST 三, the Q_pred equation; HTML Sec. 3.3]
# ----------------------------------------------------------------------------------------

def predict_query(X, W) -> np.ndarray:
    """Q_pred^{i+1} = W_Q^{i+1} X^i for a batch of rows.

    X is [M][hidden] (one row per sequence, the layer input X^i); W is [N][hidden], row n
    being output feature n (the usual linear-layer layout), so that W X for a column X is
    the row-major product X W^T.  Returns Q [M][N] in float64.  The same product with the
    layer's own W_Q^i gives the true query Q^i = W_Q^i X^i (Algorithm 1, true query step).
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    if X.ndim != 2 or W.ndim != 2 or X.shape[1] != W.shape[1]:
        raise ValueError("predict_query: X [M][hidden] and W [N][hidden] expected")
    return X @ W.T


def query_heads(Q_rows: np.ndarray, num_q_heads: int, head_dim: int) -> np.ndarray:
    """View the projection output [M][Hq*d] as per-head queries [M][Hq][d] (head = n div d)."""
    M, N = Q_rows.shape
    if N != num_q_heads * head_dim:
        raise ValueError("query_heads: width is not Hq*d")
    return Q_rows.reshape(M, num_q_heads, head_dim)


def gqa_group(h: int, group: int) -> range:
    """Query heads that share KV head h: the contiguous group h*G .. h*G+G-1 (reading R2)."""
    return range(h * group, (h + 1) * group)


# ----------------------------------------------------------------------------------------
# O2: fixed-size blocks  [HTML Sec. 2.2: the KV cache is cut into fixed-size blocks]
# ----------------------------------------------------------------------------------------

def num_blocks(seq_len: int, block_size: int) -> int:
    """Number of blocks covering seq_len tokens: ceil(seq_len / block_size)."""
    return -(-int(seq_len) // int(block_size))


def block_tokens(b: int, seq_len: int, block_size: int) -> range:
    """Token positions of block b: [b*bs, min((b+1)*bs, seq_len)) (reading R9)."""
    return range(b * block_size, min((b + 1) * block_size, seq_len))


# ----------------------------------------------------------------------------------------
# O3: digests  [HTML Sec. 2.2: MoBA mean pooling; Quest channel-wise min/max pooling]
# ----------------------------------------------------------------------------------------

def _block_view(K: np.ndarray, seq_len: int, block_size: int):
    """The full blocks of K as [nb_full][bs][d], and the valid rows of a partial last block
    (or None)."""
    nfull = int(seq_len) // int(block_size)
    full = K[:nfull * block_size].reshape(nfull, block_size, K.shape[1])
    tail = K[nfull * block_size:seq_len] if seq_len % block_size else None
    return full, tail


def digest_mean(K: np.ndarray, seq_len: int, block_size: int, kv_dtype: str) -> np.ndarray:
    """Mean-pooled digest of every block of one (sequence, KV head).

    K is the logical key sequence [T >= seq_len][d].  digest[b] = (1/n_b) * sum of K over
    block b's n_b valid tokens, computed in float64 and then rounded once to the KV dtype.
    Returns [nb][d] (float64 holding stored values).
    """
    K = np.asarray(K, dtype=np.float64)
    full, tail = _block_view(K, seq_len, block_size)
    rows = [full.sum(axis=1) / block_size]
    if tail is not None:
        rows.append(tail.sum(axis=0, keepdims=True) / tail.shape[0])
    return store_rounding(kv_dtype)(np.concatenate(rows, axis=0))


def digest_minmax(K: np.ndarray, seq_len: int, block_size: int) -> np.ndarray:
    """Channel-wise min/max digest of every block of one (sequence, KV head).

    Returns [nb][2][d]: [b][0] is the per-channel minimum of K over block b's valid tokens,
    [b][1] the maximum.  Both are exact (they are stored key values).
    """
    K = np.asarray(K, dtype=np.float64)
    full, tail = _block_view(K, seq_len, block_size)
    lo, hi = [full.min(axis=1)], [full.max(axis=1)]
    if tail is not None:
        lo.append(tail.min(axis=0, keepdims=True))
        hi.append(tail.max(axis=0, keepdims=True))
    return np.stack([np.concatenate(lo, axis=0), np.concatenate(hi, axis=0)], axis=1)


# ----------------------------------------------------------------------------------------
# O4: block scores  [HTML Sec. 2.2, Sec. 3.2: dot product of the query with each digest]
# ----------------------------------------------------------------------------------------

def score_mean(q_group: np.ndarray, digest: np.ndarray) -> np.ndarray:
    """sigma_b = sum over the group's query heads g of q_g . digest_b  (readings R2, R3).

    q_group [G][d]; digest [nb][d].  Returns [nb] float64.
    """
    q_group = np.asarray(q_group, dtype=np.float64)
    digest = np.asarray(digest, dtype=np.float64)
    sigma = np.zeros(digest.shape[0], dtype=np.float64)
    for g in range(q_group.shape[0]):
        sigma += digest @ q_group[g]
    return sigma


def score_minmax(q_group: np.ndarray, digest: np.ndarray) -> np.ndarray:
    """sigma_b = sum_g sum_c max(q_gc * min_bc, q_gc * max_bc)  (readings R1, R2, R3).

    q_group [G][d]; digest [nb][2][d] (min row, then max row).  Returns [nb] float64.
    """
    q_group = np.asarray(q_group, dtype=np.float64)
    digest = np.asarray(digest, dtype=np.float64)
    lo, hi = digest[:, 0, :], digest[:, 1, :]
    sigma = np.zeros(digest.shape[0], dtype=np.float64)
    for g in range(q_group.shape[0]):
        q = q_group[g]
        sigma += np.maximum(q * lo, q * hi).sum(axis=1)
    return sigma


def score_blocks(q_group, digest, kind: str) -> np.ndarray:
    if kind == "mean":
        return score_mean(q_group, digest)
    if kind == "minmax":
        return score_minmax(q_group, digest)
    raise ValueError(f"unknown digest kind {kind!r}")


# ----------------------------------------------------------------------------------------
# O5/O6: top-k and the resident / offloaded split  [Algorithm 1: B_pred = TopK(...),
#        B_cpu = B_pred \ B_gpu; HTML Sec. 3.2]
# ----------------------------------------------------------------------------------------

def select_topk(scores: np.ndarray, k: int) -> np.ndarray:
    """The min(k, nb) blocks with the largest score; equal scores go to the lower index
    (reading R4).  Returned as ascending block indices (int64)."""
    scores = np.asarray(scores, dtype=np.float64)
    n = scores.shape[0]
    ks = min(int(k), n)
    # lexsort: the last key is the primary one -> score descending, then index ascending
    order = np.lexsort((np.arange(n), -scores))
    return np.sort(order[:ks]).astype(np.int64)


def split_resident(selected: np.ndarray, resident: np.ndarray):
    """Split the selection into (S_gpu, S_cpu): selected blocks held in GPU memory and the
    rest.  `resident` is a boolean mask over blocks.  Both lists stay ascending."""
    selected = np.asarray(selected, dtype=np.int64)
    res = np.asarray(resident, dtype=bool)[selected]
    return selected[res], selected[~res]


def recall_pair(table_row, seq_len: int, block_size: int, gpu_blocks, cpu_blocks,
                host_pages_row, max_recall: int):
    """Periodic KV recall for one (sequence, KV head) [HTML Sec. 3.4; DIGEST 三, the
    asynchronous periodic recall]: blocks the CPU attends are brought back into GPU memory,
    refreshing the resident set towards the blocks that are important now.

    Readings (the pages name neither which blocks come back nor which make room):
      * recalled: the layer's current B_cpu in list order (ascending), skipping entries that
        are outside the sequence, already resident, or without a host page;
      * evicted: the resident blocks that are not in the current selection
        (B_gpu and B_cpu), in ascending block order; a recalled block takes the page of the
        evicted block paired with it;
      * n = min(#recalled candidates, #evictable, max_recall) blocks move.
    Returns (new table row, [(recalled block, page, host page), ...]).
    """
    table = np.array(table_row, dtype=np.int64)
    nb = min(num_blocks(seq_len, block_size), len(table))
    selected = set(int(b) for b in gpu_blocks) | set(int(b) for b in cpu_blocks)
    cands = [int(b) for b in cpu_blocks
             if 0 <= b < nb and table[b] < 0 and host_pages_row[b] >= 0]
    victims = [b for b in range(nb) if table[b] >= 0 and b not in selected]
    n = min(len(cands), len(victims), max_recall)
    moves = []
    for t in range(n):
        page = int(table[victims[t]])
        table[victims[t]] = -1
        table[cands[t]] = page
        moves.append((cands[t], page, int(host_pages_row[cands[t]])))
    return table, moves


def recall_due(n_cpu_per_pair, top_k: int, beta: float) -> bool:
    """Whether a layer is recalled [HTML Sec. 3.4]: its CPU compute ratio -- the share of the
    budget the CPU attends -- is above the threshold beta.  Reading: the ratio is counted in
    blocks, sum over pairs of |B_cpu| / (pairs * top_k), and tested after each selection (the
    pages set per-layer intervals offline so that the measured ratio stays under beta)."""
    n = np.asarray(n_cpu_per_pair, dtype=np.int64)
    return float(n.sum()) / (len(n) * top_k) > beta


# ----------------------------------------------------------------------------------------
# O7/O8: partial attention and the merge  [HTML Sec. 3.2: partials merged with the
#        FlashAttention algorithm; Algorithm 1: A_gpu = GPUATTN(Q, B_gpu),
#        A = MERGE(A_gpu, A_cpu)]
# ----------------------------------------------------------------------------------------

@dataclass
class Partial:
    """Attention over a token subset: normalised output o, max logit m, sum of exp l."""
    o: np.ndarray
    m: float
    l: float

    @property
    def lse(self) -> float:
        return self.m + math.log(self.l) if self.l > 0 else NEG_INF


def empty_partial(d: int) -> Partial:
    """The partial of an empty token set (reading R8)."""
    return Partial(np.zeros(d, dtype=np.float64), NEG_INF, 0.0)


def partial_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> Partial:
    """Softmax attention of one query over tokens K [T][d], V [T][d] (reading R7):
    z_t = scale * q.K_t, m = max z, l = sum exp(z - m), o = sum exp(z - m) V_t / l."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if K.shape[0] == 0:
        return empty_partial(q.shape[0])
    z = (K @ q) * scale
    m = float(z.max())
    p = np.exp(z - m)
    l = float(p.sum())
    return Partial((p @ V) / l, m, l)


def merge(a: Partial, b: Partial) -> Partial:
    """Combine two partials over disjoint token sets (online-softmax rescaling).

    m = max(m_a, m_b); w_i = l_i * exp(m_i - m) (0 for an empty partial); l = w_a + w_b;
    o = (w_a o_a + w_b o_b) / l.  Two empty partials give the empty partial.
    """
    m = max(a.m, b.m)
    if m == NEG_INF:
        return empty_partial(a.o.shape[0])
    wa = a.l * math.exp(a.m - m) if a.m != NEG_INF else 0.0
    wb = b.l * math.exp(b.m - m) if b.m != NEG_INF else 0.0
    l = wa + wb
    return Partial((wa * a.o + wb * b.o) / l, m, l)


def gather_tokens(X: np.ndarray, blocks, seq_len: int, block_size: int) -> np.ndarray:
    """Rows of the logical sequence X [T][d] that belong to the given blocks' valid tokens."""
    X = np.asarray(X, dtype=np.float64)
    parts = [np.arange(t.start, t.stop) for t in
             (block_tokens(int(b), seq_len, block_size) for b in blocks)]
    if not parts:
        return np.zeros((0, X.shape[1]), dtype=np.float64)
    return X[np.concatenate(parts)]


def attend_blocks(q, K, V, blocks, seq_len: int, block_size: int, scale: float) -> Partial:
    """Partial attention of q over the valid tokens of a set of blocks."""
    return partial_attention(q, gather_tokens(K, blocks, seq_len, block_size),
                             gather_tokens(V, blocks, seq_len, block_size), scale)


def dense_attention(q, K, V, seq_len: int, scale: float) -> Partial:
    """FullKV decode attention over the first seq_len tokens (the no-sparsity case)."""
    return partial_attention(q, np.asarray(K)[:seq_len], np.asarray(V)[:seq_len], scale)


# ----------------------------------------------------------------------------------------
# O9: one layer for one (sequence, KV head)  [HTML Sec. 3.2; Algorithm 1]
# ----------------------------------------------------------------------------------------

@dataclass
class PairResult:
    """Per (sequence, KV head) outcome of one layer."""
    scores: np.ndarray          # [nb]
    selected: np.ndarray        # B_pred, ascending
    gpu_blocks: np.ndarray      # S_gpu = selected and resident, ascending
    cpu_blocks: np.ndarray      # S_cpu = selected and not resident, ascending
    gpu: list                   # per query head of the group: Partial over S_gpu
    host: list                  # per query head: the host partial that was merged
    out: list                   # per query head: MERGE(gpu, host)


def select_pair(q_sel_group, digest, kind: str, top_k: int, resident):
    """Scores, B_pred and its split for one (sequence, KV head)."""
    sigma = score_blocks(q_sel_group, digest, kind)
    sel = select_topk(sigma, top_k)
    g_blocks, c_blocks = split_resident(sel, resident)
    return sigma, sel, g_blocks, c_blocks


def attend_selection(q_att_group, K, V, seq_len: int, block_size: int, sigma, selected,
                     resident, scale: float, host=None) -> PairResult:
    """Split a selection by residency, attend the resident part with q_att, and merge.

    `host` is None to compute the host partials here as the attention of q_att over the
    offloaded selected blocks (what the CPU side computes), or a list of one Partial per
    query head of the group to merge as given.  K/V need valid rows only for the blocks
    that are attended.
    """
    g_blocks, c_blocks = split_resident(selected, resident)
    gpu, hst, out = [], [], []
    for j in range(len(q_att_group)):
        pg = attend_blocks(q_att_group[j], K, V, g_blocks, seq_len, block_size, scale)
        if host is None:
            ph = attend_blocks(q_att_group[j], K, V, c_blocks, seq_len, block_size, scale)
        else:
            ph = host[j]
        gpu.append(pg)
        hst.append(ph)
        out.append(merge(pg, ph))
    return PairResult(sigma, np.asarray(selected), g_blocks, c_blocks, gpu, hst, out)


def forward_pair(q_sel_group, q_att_group, K, V, seq_len: int, block_size: int, digest,
                 kind: str, top_k: int, resident, scale: float, host=None) -> PairResult:
    """One layer for one (sequence, KV head): select with q_sel, attend with q_att, merge
    with the host partials (see attend_selection)."""
    sigma, sel, _, _ = select_pair(q_sel_group, digest, kind, top_k, resident)
    return attend_selection(q_att_group, K, V, seq_len, block_size, sigma, sel, resident,
                            scale, host)


# ----------------------------------------------------------------------------------------
# The layer-ahead decode step  [Algorithm 1; HTML Sec. 3.3]
# ----------------------------------------------------------------------------------------

def decode_step_pair(layers, s: int, h: int, group: int, head_dim: int, block_size: int,
                     top_k: int, scale: float, kind: str = "mean"):
    """Run Algorithm 1 over all layers for one (sequence s, KV head h).

    `layers` is a list of per-layer dicts with:
      X      [M][hidden]  layer input X^i (row s is used)
      W      [Hq*d][hidden] W_Q^i
      digest [nb][d] (or [nb][2][d]) digests of (s, h) at layer i
      resident  bool [nb]   B_gpu membership of (s, h) at layer i
      K, V   [T][d] logical keys/values of (s, h) at layer i (rows of resident blocks)
      seq_len  int
      host   list of Partial per query head of the group, merged when S_cpu is not empty;
             or, in place of `host`,
      K_host, V_host  [T][d] logical keys/values of (s, h) at layer i as the host holds
             them (rows of the offloaded blocks): the host partial is then computed here,
             as the CPU side does it, over S_cpu with the query the CPU has when layer i's
             work is spawned one layer ahead -- Q_pred^i (Q^0 for layer 0)
             [Algorithm 1: CPUAttn(B_cpu^{i+1}) is spawned while layer i runs, before Q^{i+1}
             exists; HTML Sec. 3.3 and the accuracy discussion of Sec. 4: the CPU side
             attends with the predicted query]
    Layer i selects for layer i+1 with Q_pred^{i+1} = W_Q^{i+1} X^i; layer 0 has no
    predecessor and selects with its own Q^0.  Layer i attends with Q^i = W_Q^i X^i.
    Returns a list of PairResult, one per layer.
    """
    heads = list(gqa_group(h, group))
    rows = [slice(g * head_dim, (g + 1) * head_dim) for g in heads]

    def q_of(X, W):
        x = np.asarray(X[s:s + 1], dtype=np.float64)
        Wg = np.concatenate([np.asarray(W[r], dtype=np.float64) for r in rows], axis=0)
        return predict_query(x, Wg).reshape(len(heads), head_dim)

    L = len(layers)
    q_sel = [None] * L
    q_sel[0] = q_of(layers[0]["X"], layers[0]["W"])
    results = []
    for i in range(L):
        Li = layers[i]
        q_true = q_of(Li["X"], Li["W"])
        if i + 1 < L:
            q_sel[i + 1] = q_of(Li["X"], layers[i + 1]["W"])
        sigma, sel, g_blocks, c_blocks = select_pair(q_sel[i], Li["digest"], kind, top_k,
                                                     Li["resident"])
        gpu, hst, out = [], [], []
        for j in range(len(heads)):
            pg = attend_blocks(q_true[j], Li["K"], Li["V"], g_blocks, Li["seq_len"],
                               block_size, scale)
            if len(c_blocks) == 0:
                ph = empty_partial(head_dim)
            elif "K_host" in Li:
                ph = attend_blocks(q_sel[i][j], Li["K_host"], Li["V_host"], c_blocks,
                                   Li["seq_len"], block_size, scale)
            else:
                ph = Li["host"][j]
            gpu.append(pg)
            hst.append(ph)
            out.append(merge(pg, ph))
        results.append(PairResult(sigma, sel, g_blocks, c_blocks, gpu, hst, out))
    return results
