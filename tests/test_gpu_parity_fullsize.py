"""Full-size parity: the five workloads at their real sizes, through the same C-ABI calls and
launch configuration that bench.py times, against the CPU oracle.

At these sizes the oracle checks every (sequence, KV head) pair's digests (bit for bit),
scores and selection, and a seeded sample of pairs' attention outputs: the first and last
pair plus random ones, computed one by one.  The 40-layer step is checked on sampled pairs
through all 40 layers.  Inputs are generated on the GPU (each tensor from its own seeded
generator) and copied to the host for the oracle.
"""

import numpy as np
import pytest
import torch

import harness as H
from block_sparse_attention_digest_amd import binding as B
from block_sparse_attention_digest_amd import workloads as wk

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def sample_pairs(wl, n, seed):
    pairs = wl.batch * wl.num_kv_heads
    rng = np.random.default_rng(seed)
    picked = set(rng.choice(pairs, size=min(n, pairs), replace=False).tolist())
    return sorted(picked | {0, pairs - 1})


LAYER_CASES = [
    ("qwen3-8b-layer-b8-16k", wk.QWEN3_8B_LAYER, "mean"),
    ("qwen3-14b-layer-b40-32k-minmax", wk.QWEN3_14B_LAYER, "minmax"),
    ("ragged-b64-mean", wk.RAGGED, "mean"),
    ("ragged-b64-minmax", wk.RAGGED, "minmax"),
]


@pytest.mark.parametrize("name,wl,kind", LAYER_CASES, ids=[c[0] for c in LAYER_CASES])
def test_layer_fullsize(name, wl, kind):
    H.log(f"[case] full size {name}")
    r = H.run_layer(wl, kind, gen_device="cuda", pairs_to_check=sample_pairs(wl, 8, 11))
    assert r.n_pairs == wl.batch * wl.num_kv_heads


def test_step_fullsize():
    """The benchmark's 40-layer Qwen3-14B step (batch 40, 64K context, pool of 128 blocks),
    with the side stream and the host hand-off, sampled pairs through every layer."""
    wl = wk.QWEN3_14B_STEP
    H.log(f"[case] full size step {wl.name}")
    import harness_step as HS
    r = HS.run_step(wl, gen_device="cuda", handoff=True, pairs_to_check=sample_pairs(wl, 6, 5))
    assert 0.0 < r["cpu_ratio"] < 0.5


def test_step_fullsize_bs16():
    """The benchmark's step with blocks of 16 tokens, budget and pool kept in tokens (k = 128,
    a pool of 256 blocks, as bench.py --block-size 16): the selection ranks 4096 blocks a
    pair, so the step's GEMMs run five waves a workgroup; four layers, sampled pairs."""
    wl = wk.QWEN3_14B_STEP.scaled(block_size=16, top_k=128, pool_blocks=256, layers=4)
    H.log(f"[case] full size step {wl.name} bs16")
    import harness_step as HS
    r = HS.run_step(wl, gen_device="cuda", handoff=True, pairs_to_check=sample_pairs(wl, 4, 7))
    assert 0.0 < r["cpu_ratio"] < 0.5


def test_step_fullsize_minmax():
    """The benchmark's step shape with min/max digests (as bench.py --digest minmax), side
    stream and host hand-off; four layers, sampled pairs.  The pool holds 48 blocks, fewer
    than the budget of 64, so every pair offloads and the host mirrors carry real lists."""
    wl = wk.QWEN3_14B_STEP.scaled(layers=4, pool_blocks=48, digest_kinds=("minmax",))
    H.log(f"[case] full size step {wl.name} minmax")
    import harness_step as HS
    r = HS.run_step(wl, gen_device="cuda", handoff=True, kind="minmax",
                    pairs_to_check=sample_pairs(wl, 4, 13))
    assert 0.0 < r["cpu_ratio"] < 1.0


def test_step_offload_fullsize():
    """The benchmark's step with its CPU side computed by host tasks one layer ahead, from an
    aliased host store (as bench.py --offload), sampled pairs through every layer: the query
    handed over, the host partials and the merged outputs."""
    wl = wk.QWEN3_14B_STEP
    H.log(f"[case] full size offload step {wl.name}")
    import harness_step as HS
    r = HS.run_step(wl, gen_device="cuda", offload=True, store="aliased", host_threads=16,
                    pairs_to_check=sample_pairs(wl, 3, 9))
    assert 0.0 < r["cpu_ratio"] < 0.5


def test_dense_fullsize():
    """FullKV over one layer of the benchmark shape (40 sequences x 65536 tokens, every block
    resident, as bench.py --dense): sampled (sequence, query head) rows against the oracle's
    dense attention over the whole context."""
    from oracle import scout_oracle as so
    wl = wk.QWEN3_14B_STEP.scaled(layers=1)
    H.log(f"[case] full size dense {wl.name}")
    dev = "cuda"
    lens = wk.seq_lens(wl)
    kv = wk.draw_kv_pages(wl, lens, dev)
    P = kv["K"].shape[0]
    dims = H.dims_for(wl, P)
    q = wk.draw_queries(wl.scaled(hidden=0), dev)["Q"]
    k_pool = B.pack_k_pages(dims, kv["K"])
    v_pool = B.pack_v_pages(dims, kv["V"])
    o = torch.full((wl.batch, wl.num_q_heads, wl.head_dim), float("nan"), device=dev)
    m = torch.full((wl.batch, wl.num_q_heads), float("nan"), device=dev)
    l = torch.full_like(m, float("nan"))
    B.sa_dense_decode(dims, q, k_pool, v_pool, kv["table"], lens.to(dev), wl.scale, o, m, l)
    torch.cuda.synchronize()
    del k_pool, v_pool
    G = wl.group
    max_err = 0.0
    for p in sample_pairs(wl, 4, 13):
        s, h = divmod(p, wl.num_kv_heads)
        n = int(lens[s])
        K = wk.f64(wk.logical_rows(kv["K"], kv["table"][s, h], n))
        V = wk.f64(wk.logical_rows(kv["V"], kv["table"][s, h], n))
        for j in range(G):
            qh = h * G + j
            want = so.dense_attention(q[s, qh].double().cpu().numpy(), K, V, n, wl.scale)
            max_err = max(max_err, H.compare_partial(
                o[s, qh].double().cpu().numpy(), float(m[s, qh]), float(l[s, qh]), want,
                H.attn_tol(wl), f"seq {s} head {qh}"))
    H.log(f"  dense full size: max_err={max_err:.2e}")


def test_recall_fullsize():
    """One periodic recall of every layer after the benchmark's step (as bench.py --recall),
    sampled pairs bit for bit against the oracle's recall."""
    wl = wk.QWEN3_14B_STEP
    H.log(f"[case] full size recall {wl.name}")
    import harness_recall as HR
    moved = HR.run_recall_fullsize(wl, sample_pairs(wl, 6, 17))
    assert moved > 0
