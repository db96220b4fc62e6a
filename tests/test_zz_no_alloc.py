"""The entry point that allocates nothing (sa_decode_attend_merge_noalloc) against the one
with a caller workspace (sa_decode_attend_merge), through the C ABI: two calls in a row,
the second with a smaller input, each bit-identical to the workspace call on the same
inputs (the same kernels run; only where their partials live differs).  Also: a shape whose
partials do not fit the scratch is refused before anything is launched."""

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


def case(wl, seed):
    """Pages, lists and host partials of one layer: for every (sequence, KV head) a random
    ascending set of resident blocks (up to top_k) is attended, and a random count of
    offloaded blocks gates the host partial."""
    dev = "cuda"
    lens = wk.seq_lens(wl)
    kv = wk.draw_kv_pages(wl, lens, dev)
    dims = H.dims_for(wl, kv["K"].shape[0])
    k = wl.top_k
    pairs = wl.batch * wl.num_kv_heads
    rng = np.random.default_rng(seed)
    gb = np.full((pairs, k), -1, np.int32)
    ng = np.zeros(pairs, np.int32)
    nc = np.zeros(pairs, np.int32)
    for p in range(pairs):
        nb = -(-int(lens[p // wl.num_kv_heads]) // wl.block_size)
        n = int(rng.integers(0, min(k, nb) + 1))
        gb[p, :n] = np.sort(rng.choice(nb, n, replace=False))
        ng[p] = n
        nc[p] = int(rng.integers(0, 3))
    rows = wl.batch * wl.num_q_heads
    q = torch.randn((wl.batch, wl.num_q_heads, wl.head_dim), device=dev,
                    generator=wk.generator(wl, f"noalloc_q{seed}", dev))
    hp = wk.draw_host_partials(wl, seed, dev)
    return dict(dims=dims, lens=lens.to(dev), K=B.pack_k_pages(dims, kv["K"]),
                V=B.pack_v_pages(dims, kv["V"]), table=kv["table"], q=q,
                gb=torch.from_numpy(gb).to(dev), ng=torch.from_numpy(ng).to(dev),
                nc=torch.from_numpy(nc).to(dev), host=hp, rows=rows, wl=wl)


def outputs(c, noalloc):
    wl, dev = c["wl"], "cuda"
    o = torch.full((c["rows"], wl.head_dim), float("nan"), device=dev)
    m = torch.full((c["rows"],), float("nan"), device=dev)
    l = torch.full((c["rows"],), float("nan"), device=dev)
    args = (c["dims"], c["q"], c["K"], c["V"], c["table"], c["lens"], c["gb"], c["ng"],
            wl.top_k, wl.scale, c["host"]["o"], c["host"]["m"], c["host"]["l"], c["nc"], o, m, l)
    if noalloc:
        B.sa_decode_attend_merge_noalloc(*args)
    else:
        ws = B.workspace(B.sa_workspace_bytes(c["dims"], wl.top_k))
        B.sa_decode_attend_merge(*args, ws=ws)
    torch.cuda.synchronize()
    return o, m, l


def test_noalloc_matches_workspace_call_twice_second_smaller():
    big = wk.RAGGED.scaled(batch=12, ctx_min=200, ctx_max=3000, top_k=48)
    small = wk.QWEN3_14B_LAYER.scaled(batch=2, num_q_heads=10, num_kv_heads=2, context=900,
                                      top_k=12, hidden=0)
    for name, wl, seed in (("first, larger", big, 1), ("second, smaller", small, 2)):
        H.log(f"[case] no-alloc call {name}: {wl.batch} sequences, top_k {wl.top_k}")
        c = case(wl, seed)
        got = outputs(c, True)
        want = outputs(c, False)
        for g, w, what in zip(got, want, ("o", "m", "l")):
            assert torch.equal(g, w), f"{name}: {what} differs from the workspace call"
        assert torch.isfinite(got[0]).all()


def test_noalloc_refuses_partials_beyond_scratch():
    """8192 (sequence, KV head) pairs of 8 query heads need about 42 MB of partials, more
    than the 16 MiB of scratch: refused on the host with SA_ERR_WORKSPACE."""
    dims = B.Dims(1024, 64, 8, 128, 32, 64, 1024, B.SA_BF16)
    dev = "cuda"
    rows = 1024 * 64
    t = torch.zeros(1, device=dev)
    big = torch.zeros(rows * 128, device=dev)
    i32 = torch.zeros(1024 * 8 * 64, dtype=torch.int32, device=dev)
    with pytest.raises(B.SaError) as e:
        B.sa_decode_attend_merge_noalloc(
            dims, big, torch.zeros(1024 * 32 * 128, dtype=torch.bfloat16, device=dev),
            torch.zeros(1024 * 32 * 128, dtype=torch.bfloat16, device=dev), i32,
            torch.full((1024,), 64, dtype=torch.int32, device=dev), i32, i32[:8192], 8, 0.1,
            big, big[:rows], big[:rows], i32[:8192], big, big[:rows], big[:rows])
    assert e.value.status == B.SA_ERR_WORKSPACE
    assert "scratch" in str(e.value)
    del t
