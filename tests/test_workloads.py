"""The synthetic workload recipe against what the pages fix, and its layout plumbing."""

import json
import math
import os

import numpy as np
import torch

from block_sparse_attention_digest_amd import workloads as wk
from oracle import scout_oracle as so

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_qwen3_14b_kv_layout_matches_pages():
    """4 KB of KV per token per layer and 128 KB per 32-token page (HTML Sec. 2.3) are the
    Qwen3-14B layout the step workload uses: 8 KV heads x 128 x (K, V) x 2 bytes."""
    fix = json.load(open(os.path.join(GOLDEN, "pages_layout.json")))
    wl = wk.QWEN3_14B_STEP
    per_token = wl.num_kv_heads * wl.head_dim * 2 * torch.finfo(wl.torch_kv_dtype).bits // 8
    assert per_token == fix["bytes_per_token_per_layer"]
    assert wl.block_size == fix["page_tokens"]
    assert per_token * wl.block_size == fix["page_bytes"]


def test_layer_ahead_query_similarity_matches_table1():
    """The AR(1) layer inputs give cos(Q_pred^{i+1}, Q^{i+1}) near Table 1's Qwen3-8B 0.94."""
    fix = json.load(open(os.path.join(GOLDEN, "pages_table1.json")))
    wl = wk.QWEN3_14B_STEP.scaled(batch=8, layers=3)
    ins = wk.draw_layer_inputs(wl, "cpu")
    cos = []
    for i in range(wl.layers - 1):
        W = wk.f64(ins[i + 1]["W"])
        qp = so.predict_query(wk.f64(ins[i]["X"]), W)
        qt = so.predict_query(wk.f64(ins[i + 1]["X"]), W)
        cos += list((qp * qt).sum(1) / np.linalg.norm(qp, axis=1) / np.linalg.norm(qt, axis=1))
    assert abs(np.mean(cos) - fix["cosine_similarity"]["Qwen3-8B"]) < 0.02, np.mean(cos)


def test_generators_are_deterministic_and_distinct():
    wl = wk.TINY
    a = wk.draw_queries(wl, "cpu")["Q"]
    b = wk.draw_queries(wl, "cpu")["Q"]
    assert torch.equal(a, b)
    lens = wk.seq_lens(wl)
    kv = wk.draw_kv_pages(wl, lens, "cpu")
    assert not torch.equal(kv["K"][:4], kv["V"][:4])
    r = wk.seq_lens(wk.RAGGED)
    assert int(r.min()) >= 4096 and int(r.max()) <= 65536 and len(set(r.tolist())) > 40


def test_page_table_is_a_permutation_and_logical_view_gathers():
    wl = wk.RAGGED.scaled(batch=3, ctx_min=40, ctx_max=100)
    lens = wk.seq_lens(wl)
    kv = wk.draw_kv_pages(wl, lens, "cpu")
    t = kv["table"]
    used = t[t >= 0]
    assert sorted(used.tolist()) == list(range(kv["K"].shape[0]))
    for s in range(wl.batch):
        nb = -(-int(lens[s]) // wl.block_size)
        assert (t[s, :, :nb] >= 0).all() and (t[s, :, nb:] < 0).all()
        rows = wk.logical_rows(kv["K"], t[s, 1], int(lens[s]))
        b = nb - 1
        assert torch.equal(rows[b * wl.block_size], kv["K"][t[s, 1, b], 0])


def test_resident_sets_follow_the_recipe():
    wl = wk.QWEN3_14B_LAYER.scaled(batch=3, num_q_heads=10, num_kv_heads=2, context=4096)
    lens = wk.seq_lens(wl)
    sel = [[np.arange(0, 128, 2)[:64] for _ in range(2)] for _ in range(3)]
    R = wk.choose_resident(wl, sel, lens)
    for s in range(3):
        for h in range(2):
            inter = np.intersect1d(R[s][h], sel[s][h])
            assert len(inter) == math.floor(0.9 * 64 + 0.5) == 58
            assert len(R[s][h]) == 64 and len(np.unique(R[s][h])) == 64
    wl1 = wk.TINY
    sel1 = [[np.array([3, 5, 9, 12, 20, 33, 40, 63])] for _ in range(2)]
    R1 = wk.choose_resident(wl1, sel1, wk.seq_lens(wl1))
    assert np.intersect1d(R1[0][0], sel1[0][0]).tolist() == [3, 5, 9, 12]
    assert len(R1[0][0]) == 8


def test_pool_holds_the_resident_blocks():
    wl = wk.QWEN3_8B_LAYER.scaled(batch=2, num_q_heads=8, num_kv_heads=2, context=512)
    lens = wk.seq_lens(wl)
    kv = wk.draw_kv_pages(wl, lens, "cpu")
    R = [[np.array([0, 3, 7]), np.array([15])], [np.array([1, 2]), np.array([], dtype=np.int64)]]
    pool = wk.build_pool(wl, R, kv["K"], kv["V"], kv["table"], 4)
    bt = pool["block_table"]
    for s in range(2):
        for h in range(2):
            res = (bt[s, h] >= 0).nonzero().flatten().tolist()
            assert res == list(R[s][h])
            for b in res:
                assert torch.equal(pool["K"][bt[s, h, b]], kv["K"][kv["table"][s, h, b]])
                assert torch.equal(pool["V"][bt[s, h, b]], kv["V"][kv["table"][s, h, b]])


def test_step_pool_keys_carry_the_block_offsets():
    wl = wk.QWEN3_14B_STEP.scaled(batch=2, num_q_heads=10, num_kv_heads=2, context=512,
                                  layers=2, pool_blocks=4, hidden=256)
    off = wk.layer_offsets(wl, 1, "cpu")
    dig = wk.draw_layer_digests(wl, 1, off, "cpu")
    assert dig.dtype == torch.bfloat16 and dig.shape == (2, 2, 16, 128)
    sets = [[np.array([0, 5]), np.array([1, 2, 3])], [np.array([15]), np.array([4])]]
    pool = wk.draw_layer_pool(wl, 1, off, sets)
    bt = pool["block_table"]
    page = int(bt[0, 1, 2])
    k = pool["K"][page].float()
    # 32 unit-normal tokens around the offset: their mean is within ~5/sqrt(32) of it
    assert float((k.mean(0) - off[0, 1, 2]).abs().max()) < 5.0 / math.sqrt(32)
    hp = wk.draw_host_partials(wl, 0, "cpu")
    assert float(hp["l"].min()) >= 1.0 and float(hp["l"].max()) <= wl.block_size * wl.top_k


def test_largest_normal_moments_match_closed_forms_and_sampling():
    """The law the min/max stand-in digests draw from: the largest of n unit normals.  n = 1
    is N(0, 1); n = 2 has mean 1/sqrt(pi) and variance 1 - 1/pi; n = 32 against a seeded
    sample of 200,000 maxima."""
    m1, s1 = wk._largest_normal_moments(1)
    assert abs(m1) < 1e-9 and abs(s1 - 1.0) < 1e-6
    m2, s2 = wk._largest_normal_moments(2)
    assert abs(m2 - 1.0 / math.sqrt(math.pi)) < 1e-6
    assert abs(s2 - math.sqrt(1.0 - 1.0 / math.pi)) < 1e-6
    m32, s32 = wk._largest_normal_moments(32)
    mx = np.random.default_rng(5).standard_normal((200_000, 32)).max(axis=1)
    assert abs(m32 - mx.mean()) < 0.01 and abs(s32 - mx.std()) < 0.01


def test_minmax_stand_in_digests_bracket_the_offsets():
    """min/max stand-ins: [B][Hkv][max_blocks][2][d] in the KV dtype, minimum below the block's
    offset and maximum above it, each about E[max of bs unit normals] away."""
    wl = wk.QWEN3_14B_STEP.scaled(batch=2, num_q_heads=10, num_kv_heads=2, context=4096,
                                  layers=2, pool_blocks=4, hidden=256)
    off = wk.layer_offsets(wl, 1, "cpu")
    dig = wk.draw_layer_digests(wl, 1, off, "cpu", "minmax")
    assert dig.dtype == torch.bfloat16 and dig.shape == (2, 2, 128, 2, 128)
    lo, hi = dig[..., 0, :].float(), dig[..., 1, :].float()
    assert bool((lo < hi).all())
    mean, _ = wk._largest_normal_moments(wl.block_size)
    assert abs(float((hi - off).mean()) - mean) < 0.02
    assert abs(float((off - lo).mean()) - mean) < 0.02
    assert torch.equal(dig, wk.draw_layer_digests(wl, 1, off, "cpu", "minmax"))
