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
