"""Planted mistakes in the oracle must each make at least one pin fail.

Every mutation below is a plausible slip (a dropped term, a wrong sign or index, a
transposed operand, a double rounding).  The mutation is planted in the oracle module on
the CPU with monkeypatch; the pins are then run and at least one must raise.
"""

import math

import numpy as np
import pytest
import torch

import oracle_pins
from oracle import scout_oracle as so

_orig = {name: getattr(so, name) for name in dir(so) if callable(getattr(so, name))}


def _bf16_via_f32(x):
    x = np.asarray(x, dtype=np.float64)
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()


def _bf16_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0)
    a = np.abs(x[fin])
    _, e2 = np.frexp(a)
    sp = np.ldexp(1.0, np.maximum(e2 - 1, -126) - 7)
    out[fin] = np.copysign(np.floor(a / sp + 0.5) * sp, x[fin])
    return out


def _digest_mean_div_bs(K, seq_len, bs, kv_dtype):
    K = np.asarray(K, dtype=np.float64)
    nb = so.num_blocks(seq_len, bs)
    out = np.array([K[b * bs:min((b + 1) * bs, seq_len)].sum(0) / bs for b in range(nb)])
    return so.store_rounding(kv_dtype)(out)


def _digest_mean_unrounded(K, seq_len, bs, kv_dtype):
    K = np.asarray(K, dtype=np.float64)
    nb = so.num_blocks(seq_len, bs)
    return np.array([K[b * bs:min((b + 1) * bs, seq_len)].mean(0) for b in range(nb)])


def _minmax_swapped(K, seq_len, bs):
    return _orig["digest_minmax"](K, seq_len, bs)[:, ::-1, :]


def _score_minmax_min(q_group, digest):
    s = 0
    for q in np.asarray(q_group):
        s = s + np.minimum(q * digest[:, 0], q * digest[:, 1]).sum(1)
    return s


def _score_minmax_maxonly(q_group, digest):
    return sum((digest[:, 1] @ q) for q in np.asarray(q_group))


def _score_mean_first_head(q_group, digest):
    return np.asarray(digest) @ np.asarray(q_group)[0]


def _topk_ties_high(scores, k):
    n = len(scores)
    order = np.lexsort((-np.arange(n), -np.asarray(scores)))
    return np.sort(order[:min(k, n)])


def _topk_short(scores, k):
    return _orig["select_topk"](scores, k)[:-1] if min(k, len(scores)) > 1 else \
        _orig["select_topk"](scores, k)


def _topk_ascending(scores, k):
    n = len(scores)
    order = np.lexsort((np.arange(n), np.asarray(scores)))
    return np.sort(order[:min(k, n)])


def _split_inverted(selected, resident):
    g, c = _orig["split_resident"](selected, resident)
    return c, g


def _attn_no_scale(q, K, V, scale):
    return _orig["partial_attention"](q, K, V, 1.0)


def _attn_unnormalised(q, K, V, scale):
    p = _orig["partial_attention"](q, K, V, scale)
    return so.Partial(p.o * p.l, p.m, p.l)


def _attn_min_shift(q, K, V, scale):
    K = np.asarray(K, dtype=np.float64)
    if K.shape[0] == 0:
        return so.empty_partial(len(q))
    z = (K @ np.asarray(q)) * scale
    m = float(z.min())
    p = np.exp(z - m)
    return so.Partial((p @ np.asarray(V)) / p.sum(), m, float(p.sum()))


def _merge_no_rescale(a, b):
    if max(a.m, b.m) == -math.inf:
        return so.empty_partial(a.o.shape[0])
    l = a.l + b.l
    return so.Partial((a.l * a.o + b.l * b.o) / l, max(a.m, b.m), l)


def _merge_unnormalised(a, b):
    r = _orig["merge"](a, b)
    return so.Partial(r.o * r.l, r.m, r.l)


def _qpred_transposed(X, W):
    return np.asarray(X, dtype=np.float64) @ np.asarray(W, dtype=np.float64)


def _block_tokens_shifted(b, seq_len, bs):
    return range(b * bs + 1, min((b + 1) * bs + 1, seq_len))


def _step_selects_with_own_query(layers, *a, **k):
    return [_orig["decode_step_pair"]([L], *a, **k)[0] for L in layers]


def _step_always_merges_host(layers, s, h, group, head_dim, *a, **k):
    res = _orig["decode_step_pair"](layers, s, h, group, head_dim, *a, **k)
    for i, r in enumerate(res):
        r.out = [so.merge(r.gpu[j], layers[i]["host"][j]) for j in range(len(r.gpu))]
    return res


def _step_host_with_true_query(layers, s, h, group, head_dim, block_size, top_k, scale,
                               kind="mean"):
    """The CPU side attends with the layer's own Q^i instead of the query it has when its
    work is spawned (Q_pred^i)."""
    first = _orig["decode_step_pair"](layers, s, h, group, head_dim, block_size, top_k, scale,
                                      kind)
    heads = list(so.gqa_group(h, group))
    fixed = []
    for i, L in enumerate(layers):
        if "K_host" not in L:
            fixed.append(L)
            continue
        Q = np.asarray(L["X"][s], dtype=np.float64) @ np.asarray(L["W"], dtype=np.float64).T
        Q = Q.reshape(-1, head_dim)
        host = [so.attend_blocks(Q[g], L["K_host"], L["V_host"], first[i].cpu_blocks,
                                 L["seq_len"], block_size, scale) for g in heads]
        M = {key: v for key, v in L.items() if key not in ("K_host", "V_host")}
        M["host"] = host
        fixed.append(M)
    return _orig["decode_step_pair"](fixed, s, h, group, head_dim, block_size, top_k, scale,
                                     kind)


def _recall_evicts_descending(table_row, seq_len, block_size, gpu_blocks, cpu_blocks,
                              host_pages_row, max_recall):
    """Evicts the highest-indexed evictable blocks first."""
    table = np.array(table_row, dtype=np.int64)
    nb = min(so.num_blocks(seq_len, block_size), len(table))
    selected = set(int(b) for b in gpu_blocks) | set(int(b) for b in cpu_blocks)
    cands = [int(b) for b in cpu_blocks if 0 <= b < nb and table[b] < 0 and host_pages_row[b] >= 0]
    victims = [b for b in range(nb) if table[b] >= 0 and b not in selected][::-1]
    moves = []
    for t in range(min(len(cands), len(victims), max_recall)):
        page = int(table[victims[t]])
        table[victims[t]] = -1
        table[cands[t]] = page
        moves.append((cands[t], page, int(host_pages_row[cands[t]])))
    return table, moves


def _recall_evicts_selected(table_row, seq_len, block_size, gpu_blocks, cpu_blocks,
                            host_pages_row, max_recall):
    """Forgets B_gpu when choosing whom to evict."""
    return _orig["recall_pair"](table_row, seq_len, block_size, [], cpu_blocks, host_pages_row,
                                max_recall)


def _gqa_shifted(h, group):
    return range(h * group + 1, (h + 1) * group + 1)


def _f32_noop(x):
    return np.asarray(x, dtype=np.float64).copy()


def _f32_via_fp16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def _store_rounding_bf16_for_f32(kv_dtype):
    return _orig["round_to_bf16"] if kv_dtype in ("bf16", "f32") else _orig["store_rounding"](kv_dtype)


def _query_heads_channel_major(Q_rows, num_q_heads, head_dim):
    M, N = Q_rows.shape
    if N != num_q_heads * head_dim:
        raise ValueError("query_heads: width is not Hq*d")
    return np.ascontiguousarray(Q_rows.reshape(M, head_dim, num_q_heads).transpose(0, 2, 1))


def _score_blocks_minmax_as_mean_of_max(q_group, digest, kind):
    if kind == "minmax":
        return _orig["score_mean"](q_group, np.asarray(digest)[:, 1, :])
    return _orig["score_blocks"](q_group, digest, kind)


def _step_always_mean(layers, s, h, group, head_dim, block_size, top_k, scale, kind="mean"):
    return _orig["decode_step_pair"](layers, s, h, group, head_dim, block_size, top_k, scale,
                                     "mean")


def _block_view_drops_tail(K, seq_len, block_size):
    full, _ = _orig["_block_view"](K, seq_len, block_size)
    return full, None


def _block_view_tail_one_short(K, seq_len, block_size):
    full, tail = _orig["_block_view"](K, seq_len, block_size)
    return full, (tail[:-1] if tail is not None and len(tail) > 1 else tail)


def _gather_tokens_first_only(X, blocks, seq_len, block_size):
    return _orig["gather_tokens"](X, list(blocks)[:1], seq_len, block_size)


def _gather_tokens_drop_last_row(X, blocks, seq_len, block_size):
    rows = _orig["gather_tokens"](X, blocks, seq_len, block_size)
    return rows[:-1] if len(rows) > 1 else rows


def _attend_blocks_by_position(q, K, V, blocks, seq_len, block_size, scale):
    # attends the first len(blocks) blocks instead of the listed ones
    return _orig["attend_blocks"](q, K, V, list(range(len(list(blocks)))), seq_len, block_size,
                                  scale)


def _select_pair_swaps_split(q_sel_group, digest, kind, top_k, resident):
    sigma, sel, g, c = _orig["select_pair"](q_sel_group, digest, kind, top_k, resident)
    return sigma, sel, c, g


def _select_pair_unsorted_scores(q_sel_group, digest, kind, top_k, resident):
    sigma, sel, g, c = _orig["select_pair"](q_sel_group, digest, kind, top_k, resident)
    return sigma[::-1].copy(), sel, g, c


def _attend_selection_no_host(q_att_group, K, V, seq_len, block_size, sigma, selected,
                              resident, scale, host=None):
    r = _orig["attend_selection"](q_att_group, K, V, seq_len, block_size, sigma, selected,
                                  resident, scale, host)
    r.out = list(r.gpu)
    return r


def _attend_selection_all_on_gpu(q_att_group, K, V, seq_len, block_size, sigma, selected,
                                 resident, scale, host=None):
    every = np.ones(len(np.asarray(resident)), dtype=bool)
    return _orig["attend_selection"](q_att_group, K, V, seq_len, block_size, sigma, selected,
                                     every, scale, host)


def _dense_one_token_short(q, K, V, seq_len, scale):
    return _orig["dense_attention"](q, K, V, max(1, seq_len - 1), scale)


def _empty_partial_zero_max(d):
    return so.Partial(np.zeros(d, dtype=np.float64), 0.0, 0.0)


def _forward_pair_selects_with_q_att(q_sel_group, q_att_group, K, V, seq_len, block_size,
                                     digest, kind, top_k, resident, scale, host=None):
    return _orig["forward_pair"](q_att_group, q_att_group, K, V, seq_len, block_size, digest,
                                 kind, top_k, resident, scale, host)


def _num_blocks_floor(seq_len, block_size):
    return int(seq_len) // int(block_size)


def _recall_due_at_or_above(n_cpu_per_pair, top_k, beta):
    n = np.asarray(n_cpu_per_pair, dtype=np.int64)
    return float(n.sum()) / (len(n) * top_k) >= beta


def _recall_due_per_pair_max(n_cpu_per_pair, top_k, beta):
    return float(np.max(np.asarray(n_cpu_per_pair))) / top_k > beta


MUTATIONS = {
    "empty partial has running max 0": ("empty_partial", _empty_partial_zero_max),
    "one layer selects with the attention query": ("forward_pair", _forward_pair_selects_with_q_att),
    "block count rounds down": ("num_blocks", _num_blocks_floor),
    "recall due at the threshold itself": ("recall_due", _recall_due_at_or_above),
    "recall due on the worst pair's share": ("recall_due", _recall_due_per_pair_max),
    "block view drops the partial last block": ("_block_view", _block_view_drops_tail),
    "block view's partial last block one token short": ("_block_view", _block_view_tail_one_short),
    "gathered tokens of the first block only": ("gather_tokens", _gather_tokens_first_only),
    "gathered tokens miss the last row": ("gather_tokens", _gather_tokens_drop_last_row),
    "blocks attended by list position": ("attend_blocks", _attend_blocks_by_position),
    "selection returns the split swapped": ("select_pair", _select_pair_swaps_split),
    "selection returns the scores reversed": ("select_pair", _select_pair_unsorted_scores),
    "attention of a selection drops the host partial": ("attend_selection", _attend_selection_no_host),
    "attention of a selection ignores residency": ("attend_selection", _attend_selection_all_on_gpu),
    "dense attention one token short": ("dense_attention", _dense_one_token_short),
    "bf16 double rounding via f32": ("round_to_bf16", _bf16_via_f32),
    "bf16 ties away from zero": ("round_to_bf16", _bf16_ties_away),
    "Q_pred transposed operand": ("predict_query", _qpred_transposed),
    "mean digest divides by bs": ("digest_mean", _digest_mean_div_bs),
    "mean digest not rounded to the KV dtype": ("digest_mean", _digest_mean_unrounded),
    "min/max rows swapped": ("digest_minmax", _minmax_swapped),
    "min/max score takes the min": ("score_minmax", _score_minmax_min),
    "min/max score uses max only": ("score_minmax", _score_minmax_maxonly),
    "mean score drops the GQA sum": ("score_mean", _score_mean_first_head),
    "top-k ties go to the higher index": ("select_topk", _topk_ties_high),
    "top-k returns k-1 blocks": ("select_topk", _topk_short),
    "top-k picks the smallest scores": ("select_topk", _topk_ascending),
    "resident split inverted": ("split_resident", _split_inverted),
    "attention without 1/sqrt(d)": ("partial_attention", _attn_no_scale),
    "attention output not normalised": ("partial_attention", _attn_unnormalised),
    "attention shifted by the min logit": ("partial_attention", _attn_min_shift),
    "merge without exp rescale": ("merge", _merge_no_rescale),
    "merge output not normalised": ("merge", _merge_unnormalised),
    "block token range off by one": ("block_tokens", _block_tokens_shifted),
    "layer selects with its own query": ("decode_step_pair", _step_selects_with_own_query),
    "host partial merged when nothing offloaded": ("decode_step_pair", _step_always_merges_host),
    "GQA group off by one head": ("gqa_group", _gqa_shifted),
    "host side attends with the true query": ("decode_step_pair", _step_host_with_true_query),
    "recall evicts the highest blocks first": ("recall_pair", _recall_evicts_descending),
    "recall may evict selected resident blocks": ("recall_pair", _recall_evicts_selected),
    "f32 rounding is a no-op": ("round_to_f32", _f32_noop),
    "f32 rounding onto the fp16 grid": ("round_to_f32", _f32_via_fp16),
    "f32 digests stored with the bf16 rounding": ("store_rounding", _store_rounding_bf16_for_f32),
    "query heads read channel-major": ("query_heads", _query_heads_channel_major),
    "min/max dispatch scores the max row as a mean digest":
        ("score_blocks", _score_blocks_minmax_as_mean_of_max),
    "step ignores the digest kind": ("decode_step_pair", _step_always_mean),
}


@pytest.mark.parametrize("label", list(MUTATIONS))
def test_planted_mistake_is_caught(label, monkeypatch):
    name, fn = MUTATIONS[label]
    monkeypatch.setattr(so, name, fn)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except Exception as e:  # noqa: BLE001 -- any failure of a pin counts
            caught.append(f"{pin.__name__}: {type(e).__name__}")
    assert caught, f"no pin caught the planted mistake: {label}"
