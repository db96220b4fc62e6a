"""HIP path against the CPU oracle, element by element, through the C ABI.

Small and scaled workloads (several tiles, ragged tails) plus edge cases.  The full-size
workloads live in test_gpu_parity_fullsize.py.
"""

import math

import numpy as np
import pytest
import torch

import harness as H
from block_sparse_attention_digest_amd import binding as B
from block_sparse_attention_digest_amd import workloads as wk
from oracle import scout_oracle as so

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


TINY = wk.TINY
CFG2_S = wk.QWEN3_8B_LAYER.scaled(batch=2, context=4096 - 19)
CFG3_S = wk.QWEN3_14B_LAYER.scaled(batch=2, context=8192 + 5)
CFG5_S = wk.RAGGED.scaled(batch=4, ctx_min=1, ctx_max=5000, top_k=64)

LAYER_CASES = [
    ("cfg1-tiny-fp32", TINY, "mean", {}),
    ("cfg1-tiny-minmax", TINY, "minmax", {}),
    ("cfg1-full-budget", TINY, "mean", dict(top_k=64)),
    ("cfg1-all-offloaded", TINY, "mean", dict(resident_override="none")),
    ("cfg1-all-resident-k1", TINY, "mean", dict(resident_override="all", top_k=1)),
    ("cfg2-scaled", CFG2_S, "mean", {}),
    ("cfg3-scaled-minmax", CFG3_S, "minmax", {}),
    ("cfg5-scaled-mean", CFG5_S, "mean", {}),
    # pairs too large to take whole (more than 192 KiB of digests each): each cut into pieces
    # whose top candidates are handed over; mean digests, ragged last block
    ("bf16-mean-pieces", wk.QWEN3_8B_LAYER.scaled(batch=2, context=30000 + 11), "mean", {}),
    ("cfg5-scaled-minmax", CFG5_S, "minmax", {}),
    ("bf16-g1-d64-bs16", wk.RAGGED.scaled(batch=2, num_q_heads=2, num_kv_heads=2, head_dim=64,
                                          ctx_min=300, ctx_max=900, top_k=12), "mean", {}),
    ("bf16-g8-d128-bs32", wk.QWEN3_14B_LAYER.scaled(batch=2, num_q_heads=16, num_kv_heads=2,
                                                    context=2000, top_k=20,
                                                    resident_frac=(0.5, 0.5)), "minmax", {}),
    ("bf16-g3-d64-bs32-full", wk.QWEN3_14B_LAYER.scaled(batch=2, num_q_heads=6, num_kv_heads=2,
                                                        head_dim=64, context=700, top_k=22),
     "mean", dict(resident_override="all")),
    ("f32-d128-bs32", wk.TINY.scaled(num_q_heads=10, num_kv_heads=2, head_dim=128,
                                     block_size=32, context=1000, top_k=6), "minmax", {}),
    ("bf16-short-seqs", wk.RAGGED.scaled(batch=5, ctx_min=1, ctx_max=40, top_k=3), "mean", {}),
    # few resident blocks (5-10 % of each selection): many more attention waves than blocks,
    # so waves with empty ranges, and reduce slots of covering waves that wrote nothing
    ("bf16-few-resident", wk.RAGGED.scaled(batch=4, ctx_min=2000, ctx_max=4000, top_k=64,
                                           resident_frac=(0.05, 0.1)), "mean", {}),
    # more than 512 (sequence, KV head) pairs: attention's workgroup-wide prefix scan, and
    # workgroup ranges that cross more pairs than it stages queries for
    ("bf16-many-pairs", wk.RAGGED.scaled(batch=72, ctx_min=1, ctx_max=300, top_k=4), "mean", {}),
    ("bf16-512-pairs", wk.RAGGED.scaled(batch=64, ctx_min=1, ctx_max=300, top_k=4), "mean", {}),
    # the most pairs the library takes (8192): the digest build's and attention's prefixes of
    # 8192 counts in LDS, and more selection workgroups than CUs
    ("bf16-8192-pairs", wk.RAGGED.scaled(batch=1024, ctx_min=1, ctx_max=48, top_k=2), "mean", {}),
    ("bf16-8192-pairs-minmax", wk.RAGGED.scaled(batch=1024, ctx_min=1, ctx_max=48, top_k=2,
                                                seed=1), "minmax", {}),
    # one block per pair and more blocks than waves: attention workgroups whose block ranges
    # cross more pairs than they stage queries for (those are summed from global memory)
    ("bf16-one-block-pairs", wk.RAGGED.scaled(batch=300, ctx_min=1, ctx_max=16, top_k=1), "mean",
     dict(resident_override="all")),
    # Algorithm 1 end to end: the host partial from the host worker over the GPU's hand-off
    # lists and host pages, merged on the GPU
    ("cfg1-host-worker", TINY, "mean", dict(host_worker=True)),
    ("cfg3-scaled-minmax-host-worker", CFG3_S, "minmax", dict(host_worker=True)),
    ("cfg5-scaled-mean-host-worker", CFG5_S, "mean", dict(host_worker=True)),
    # the unused rows of partly filled last pages hold NaN and infinities: no kernel (fp32 or
    # bf16 attention, digests, the host worker) may let them into a result.  Full budgets so
    # that every partly filled block is attended.
    ("f32-poisoned-tails", TINY.scaled(context=1000), "mean",
     dict(poison_tails=True, resident_override="all", top_k=63)),
    ("f32-poisoned-tails-sparse", TINY.scaled(context=1000), "minmax", dict(poison_tails=True)),
    ("f32-poisoned-tails-host-worker", TINY.scaled(context=1000), "mean",
     dict(poison_tails=True, resident_override="none", top_k=63, host_worker=True)),
    ("bf16-poisoned-tails", wk.RAGGED.scaled(batch=3, ctx_min=100, ctx_max=700, top_k=44),
     "minmax", dict(poison_tails=True, resident_override="all")),
    ("bf16-poisoned-tails-host-worker",
     wk.RAGGED.scaled(batch=3, ctx_min=100, ctx_max=700, top_k=44), "mean",
     dict(poison_tails=True, resident_override="none", host_worker=True)),
    # blocks of 64 tokens: four 16-token attention steps per block, digests of a page taken
    # in channel slabs, every dtype and head dimension, ragged tails
    ("bf16-d128-bs64", wk.QWEN3_8B_LAYER.scaled(batch=2, context=3000 + 7, block_size=64,
                                                top_k=32), "mean", {}),
    ("bf16-d128-bs64-minmax-ragged", wk.RAGGED.scaled(batch=4, ctx_min=1, ctx_max=3000,
                                                      block_size=64, top_k=16), "minmax", {}),
    ("bf16-d64-bs64-host-worker", wk.RAGGED.scaled(batch=3, num_q_heads=6, num_kv_heads=2,
                                                   head_dim=64, ctx_min=100, ctx_max=2500,
                                                   block_size=64, top_k=12), "mean",
     dict(host_worker=True)),
    ("f32-d128-bs64", wk.TINY.scaled(num_q_heads=10, num_kv_heads=2, head_dim=128,
                                     block_size=64, context=1000, top_k=6), "mean", {}),
    ("f32-d64-bs64-minmax", wk.TINY.scaled(block_size=64, context=1000 + 33, top_k=5,
                                           n_lowest=2), "minmax", {}),
    ("bf16-poisoned-tails-bs64", wk.RAGGED.scaled(batch=3, ctx_min=100, ctx_max=700,
                                                  block_size=64, top_k=11),
     "minmax", dict(poison_tails=True, resident_override="all")),
    ("f32-poisoned-tails-bs64", TINY.scaled(context=1000, block_size=64), "mean",
     dict(poison_tails=True, resident_override="all", top_k=16)),
]


@pytest.mark.parametrize("name,wl,kind,kw", LAYER_CASES, ids=[c[0] for c in LAYER_CASES])
def test_layer_parity(name, wl, kind, kw):
    H.log(f"[case] {name}")
    H.run_layer(wl, kind, gen_device="cpu", **kw)


@pytest.mark.parametrize("kv,d,bs", [("bf16", 128, 32), ("bf16", 64, 16), ("f32", 128, 16),
                                     ("f32", 64, 32), ("bf16", 128, 64), ("f32", 64, 64)])
def test_pack_v_pages_layout(kv, d, bs):
    """The V page layout, bit for bit: [P][bs][d] viewed as [P][bs/16][16][d] with the two
    inner axes swapped."""
    H.log(f"[case] pack V {kv} d{d} bs{bs}")
    P = 29
    g = torch.Generator().manual_seed(3 * d + bs)
    dt = torch.bfloat16 if kv == "bf16" else torch.float32
    rows = torch.randn(P, bs, d, generator=g).to(dt)
    want = rows.view(P, bs // 16, 16, d).permute(0, 1, 3, 2).contiguous()
    dims = B.Dims(1, 1, 1, d, bs, 1, P, B.SA_BF16 if kv == "bf16" else B.SA_F32)
    got = B.pack_v_pages(dims, rows.cuda()).cpu().view(P, bs // 16, d, 16)
    iv = torch.int16 if kv == "bf16" else torch.int32
    assert torch.equal(got.view(iv), want.view(iv))


@pytest.mark.parametrize("kv,d,bs", [("bf16", 128, 32), ("bf16", 64, 16), ("f32", 128, 16),
                                     ("f32", 64, 32), ("bf16", 128, 64), ("f32", 64, 64)])
def test_pack_k_pages_layout(kv, d, bs):
    """The chunk-major K layout, bit for bit: [P][bs][d] viewed as [P][bs][d/x][x] with the
    two middle axes swapped (x = 16 bytes of elements)."""
    H.log(f"[case] pack K {kv} d{d} bs{bs}")
    P = 37
    g = torch.Generator().manual_seed(d + bs)
    dt = torch.bfloat16 if kv == "bf16" else torch.float32
    x = 8 if kv == "bf16" else 4
    rows = torch.randn(P, bs, d, generator=g).to(dt)
    want = rows.view(P, bs, d // x, x).permute(0, 2, 1, 3).contiguous()
    dims = B.Dims(1, 1, 1, d, bs, 1, P, B.SA_BF16 if kv == "bf16" else B.SA_F32)
    got = B.pack_k_pages(dims, rows.cuda()).cpu().view(P, d // x, bs, x)
    iv = torch.int16 if kv == "bf16" else torch.int32
    assert torch.equal(got.view(iv), want.view(iv))


@pytest.mark.parametrize("n,k", [(64, 64), (48, 96), (5120, 5120)])
def test_pack_weight_layout(n, k):
    """The packed weight order, bit for bit: tile (a, b) = rows 16a.., columns 32b..; its
    element [16 q + r][e] is w[16 a + r][32 b + 8 q + e]."""
    H.log(f"[case] pack W {n}x{k}")
    g = torch.Generator().manual_seed(n + 3 * k)
    w = torch.randn(n, k, generator=g).to(torch.bfloat16)
    want = w.view(n // 16, 16, k // 32, 4, 8).permute(0, 2, 3, 1, 4).contiguous()
    got = B.pack_weight(w.cuda()).cpu()
    assert torch.equal(got.view(torch.int16).flatten(), want.view(torch.int16).flatten())


@pytest.mark.parametrize("m,n,k", [(1, 64, 64), (8, 4096, 4096), (40, 5120, 5120),
                                   (65, 256, 320), (256, 128, 1024), (40, 320, 640),
                                   (3, 960, 192), (17, 192, 8192), (64, 5120, 5120),
                                   (256, 640, 2560)])
def test_predict_query_parity(m, n, k):
    H.log(f"[case] gemm {m}x{n}x{k}")
    g = torch.Generator().manual_seed(m * 7 + n + k)
    X = torch.randn(m, k, generator=g).to(torch.bfloat16)
    W = (torch.randn(n, k, generator=g) / math.sqrt(k)).to(torch.bfloat16)
    want = so.predict_query(wk.f64(X), wk.f64(W))
    q = torch.empty(m, n, dtype=torch.float32, device="cuda")
    ws = B.workspace(B.sa_predict_query_workspace_bytes(m, n, k))
    B.sa_predict_query(X.cuda(), B.pack_weight(W.cuda()), q, ws)
    err = float(np.max(np.abs(q.cpu().double().numpy() - want)))
    assert err <= H.TOL_GEMM, err


def test_predict_query_shared_workspace():
    """One workspace, sized for the largest, serves GEMMs of several shapes in a row (k-split
    or not, the same shape again): every result matches the oracle, so nothing a call leaves
    in the workspace changes the next one's result."""
    shapes = [(40, 5120, 5120), (8, 4096, 4096), (1, 64, 64), (256, 640, 2560),
              (40, 5120, 5120), (17, 192, 8192), (3, 960, 192), (40, 5120, 5120)]
    ws = B.workspace(max(B.sa_predict_query_workspace_bytes(*s) for s in shapes))
    for i, (m, n, k) in enumerate(shapes):
        H.log(f"[case] shared workspace gemm {m}x{n}x{k} (call {i})")
        g = torch.Generator().manual_seed(1000 + i)
        X = torch.randn(m, k, generator=g).to(torch.bfloat16)
        W = (torch.randn(n, k, generator=g) / math.sqrt(k)).to(torch.bfloat16)
        want = so.predict_query(wk.f64(X), wk.f64(W))
        q = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
        B.sa_predict_query(X.cuda(), B.pack_weight(W.cuda()), q, ws)
        err = float(np.max(np.abs(q.cpu().double().numpy() - want)))
        assert err <= H.TOL_GEMM, (m, n, k, err)


@pytest.mark.parametrize("kind,kv,d,bs", [("mean", "bf16", 128, 32), ("minmax", "bf16", 64, 16),
                                          ("mean", "f32", 64, 16), ("minmax", "f32", 128, 32),
                                          ("mean", "bf16", 128, 64), ("minmax", "bf16", 64, 64),
                                          ("mean", "f32", 128, 64), ("minmax", "f32", 128, 64)])
def test_refresh_last_digests(kind, kv, d, bs):
    """Decode-time digest maintenance: after one more token per sequence, refreshing the
    last blocks gives exactly what a full rebuild gives (and what the oracle gives), for a
    partly filled block, a block that becomes full and a token that opens a new block."""
    H.log(f"[case] refresh digests {kind} {kv} d{d} bs{bs}")
    B_, Hq, Hkv, mb = 6, 4, 2, 5
    g = torch.Generator().manual_seed(d + bs + (kind == "minmax"))
    dt = torch.bfloat16 if kv == "bf16" else torch.float32
    P = B_ * Hkv * mb
    rows = torch.randn(P, bs, d, generator=g).to(dt)  # every block of every pair has a page
    table = torch.randperm(P, generator=g).to(torch.int32).view(B_, Hkv, mb)
    lens0 = torch.tensor([1, bs - 1, bs, bs + 1, 2 * bs - 1, 3 * bs], dtype=torch.int32)
    lens1 = lens0 + 1
    dims = B.Dims(B_, Hq, Hkv, d, bs, mb, P, B.SA_BF16 if kv == "bf16" else B.SA_F32)
    per = 2 if kind == "minmax" else 1
    kp = B.pack_k_pages(dims, rows.cuda())
    bt = table.cuda()
    def build(lens):
        dig = torch.zeros((B_, Hkv, mb, per, d), dtype=dt, device="cuda")
        B.sa_build_digests(dims, kind, kp, bt, lens.cuda(), dig)
        return dig
    dig = build(lens0)
    B.sa_refresh_last_digests(dims, kind, kp, bt, lens1.cuda(), dig)
    want = build(lens1)
    torch.cuda.synchronize()
    iv = torch.int16 if kv == "bf16" else torch.int32
    assert torch.equal(dig.cpu().view(iv), want.cpu().view(iv))
    # and the refreshed entries against the oracle
    for s in range(B_):
        n = int(lens1[s])
        b = (n - 1) // bs
        for h in range(Hkv):
            K = wk.f64(wk.logical_rows(rows, table[s, h], n))
            ref = (so.digest_mean(K, n, bs, kv) if kind == "mean" else
                   so.digest_minmax(K, n, bs))[b].reshape(per, d)
            got = wk.f64(dig[s, h, b].cpu())
            assert np.array_equal(got, ref), (s, h)


def test_merge_parity_and_aliasing():
    H.log("[case] merge")
    rows, d = 37, 128
    g = torch.Generator().manual_seed(5)
    o_a = torch.randn(rows, d, generator=g)
    o_b = torch.randn(rows, d, generator=g)
    m_a = torch.randn(rows, generator=g) * 3
    m_b = torch.randn(rows, generator=g) * 3
    l_a = torch.rand(rows, generator=g) * 50 + 1
    l_b = torch.rand(rows, generator=g) * 50 + 1
    # empty partials on either side, and on both
    for r, side in ((0, "a"), (1, "b"), (2, "ab")):
        if "a" in side:
            o_a[r], m_a[r], l_a[r] = 0, -math.inf, 0
        if "b" in side:
            o_b[r], m_b[r], l_b[r] = 0, -math.inf, 0
    want = [so.merge(so.Partial(wk.f64(o_a[r]), float(m_a[r]), float(l_a[r])),
                     so.Partial(wk.f64(o_b[r]), float(m_b[r]), float(l_b[r])))
            for r in range(rows)]
    dev = [t.cuda() for t in (o_a, m_a, l_a, o_b, m_b, l_b)]
    out = [torch.empty_like(dev[0]), torch.empty_like(dev[1]), torch.empty_like(dev[2])]
    B.sa_merge(*dev, *out)
    B.sa_merge(*dev, dev[0], dev[1], dev[2])  # outputs aliasing input a
    torch.cuda.synchronize()
    for o, m, l in (out, dev[:3]):
        o, m, l = o.cpu().double().numpy(), m.cpu().double().numpy(), l.cpu().double().numpy()
        for r in range(rows):
            H.compare_partial(o[r], m[r], l[r], want[r], 1e-5, f"merge row {r}")


def test_selection_ties_go_to_lower_index():
    """q = 0 makes every score 0 (+0 or -0): the lowest-indexed blocks are selected."""
    H.log("[case] ties")
    wl = wk.QWEN3_8B_LAYER.scaled(batch=2, context=1000, top_k=5)
    dims = H.dims_for(wl, 4)
    lens = torch.full((2,), 1000, dtype=torch.int32, device="cuda")
    q = torch.zeros(2, wl.num_q_heads, wl.head_dim, device="cuda")
    q[1, :, ::2] = -0.0
    dig = torch.randn(2, wl.num_kv_heads, wl.max_blocks, wl.head_dim).to(torch.bfloat16).cuda()
    bt = torch.full((2, wl.num_kv_heads, wl.max_blocks), -1, dtype=torch.int32, device="cuda")
    bt[:, :, 2] = 0
    pairs = 2 * wl.num_kv_heads
    gb = torch.empty(pairs, 5, dtype=torch.int32, device="cuda")
    cb, ng, nc = torch.empty_like(gb), torch.empty(pairs, dtype=torch.int32, device="cuda"), \
        torch.empty(pairs, dtype=torch.int32, device="cuda")
    ws = B.workspace(B.sa_workspace_bytes(dims, 5))
    B.sa_select_blocks(dims, "mean", q, dig, lens, 5, bt, gb, ng, cb, nc, None, ws)
    torch.cuda.synchronize()
    for p in range(pairs):
        assert gb[p].tolist() == [2, -1, -1, -1, -1] and ng[p] == 1
        assert cb[p].tolist() == [0, 1, 3, 4, -1] and nc[p] == 4


def test_step_parity():
    """Side stream and host hand-off; pools smaller than the budget, so every pair
    offloads blocks and the host mirrors carry real lists."""
    H.log("[case] step")
    import harness_step as HS
    r = HS.run_step(wk.QWEN3_14B_STEP.scaled(batch=3, num_q_heads=10, num_kv_heads=2,
                                             context=2000, layers=4, pool_blocks=6, hidden=512,
                                             top_k=8),
                    gen_device="cpu", handoff=True, side=True)
    assert r["cpu_ratio"] > 0.1


def test_step_parity_handoff_one_stream():
    H.log("[case] step hand-off, one stream")
    import harness_step as HS
    r = HS.run_step(wk.QWEN3_14B_STEP.scaled(batch=2, num_q_heads=8, num_kv_heads=2,
                                             context=1500, layers=3, pool_blocks=5, hidden=256,
                                             top_k=8),
                    gen_device="cpu", handoff=True, side=False)
    assert r["cpu_ratio"] > 0.1


def test_step_offload_parity():
    """The CPU side computed by host tasks one layer ahead (sa_decode_step_offload): the
    handed-over query, the host partials and the merged outputs against the oracle, which
    attends the offloaded blocks with Q_pred^i (Q^0 at layer 0)."""
    H.log("[case] step offload, side stream")
    import harness_step as HS
    r = HS.run_step(wk.QWEN3_14B_STEP.scaled(batch=3, num_q_heads=10, num_kv_heads=2,
                                             context=2000, layers=4, pool_blocks=6, hidden=512,
                                             top_k=8),
                    gen_device="cpu", side=True, offload=True)
    assert r["cpu_ratio"] > 0.1


def test_step_offload_parity_ragged():
    """Ragged lengths down to one token (k_s = min(k, nb_s)), bf16, bs 32."""
    H.log("[case] step offload, ragged")
    import harness_step as HS
    HS.run_step(wk.QWEN3_14B_STEP.scaled(batch=4, num_q_heads=10, num_kv_heads=2, context=0,
                                         ctx_min=1, ctx_max=2000, layers=3, pool_blocks=5,
                                         hidden=256, top_k=8),
                gen_device="cpu", side=True, offload=True, host_threads=3)


def test_step_offload_parity_one_stream_one_thread():
    H.log("[case] step offload, one stream, one host thread")
    import harness_step as HS
    r = HS.run_step(wk.QWEN3_14B_STEP.scaled(batch=2, num_q_heads=8, num_kv_heads=2,
                                             context=1500, layers=3, pool_blocks=5, hidden=256,
                                             top_k=8),
                    gen_device="cpu", side=False, offload=True, host_threads=1)
    assert r["cpu_ratio"] > 0.1


@pytest.mark.parametrize("pool,max_recall,ragged,bs", [(6, 64, False, 32), (12, 2, False, 32),
                                                        (12, 64, False, 32), (6, 64, True, 32),
                                                        (4, 64, True, 64)])
def test_recall_parity(pool, max_recall, ragged, bs):
    """Periodic recall of every layer after a step: tables, moved pages and untouched pages
    against the oracle bit for bit, then the next step over the new residency."""
    H.log(f"[case] recall pool={pool} max_recall={max_recall} ragged={ragged} bs={bs}")
    import harness_recall as HR
    wl = wk.QWEN3_14B_STEP.scaled(batch=3, num_q_heads=10, num_kv_heads=2, context=2000,
                                  layers=2, pool_blocks=pool, hidden=512, top_k=8 * 32 // bs,
                                  block_size=bs)
    if ragged:
        wl = wl.scaled(batch=4, context=0, ctx_min=1, ctx_max=2000)
    r = HR.run_recall(wl, max_recall)
    assert r["moved"] > 0


@pytest.mark.parametrize("beta", [0.0, 0.12, 1.0])
def test_step_with_recall_parity(beta):
    """Periodic recall inside the offload step, gated on the device by the CPU share against
    beta: due layers match the oracle's recall bit for bit, the others are untouched."""
    H.log(f"[case] step with in-step recall, beta={beta}")
    import harness_recall as HR
    r = HR.run_step_with_recall(wk.QWEN3_14B_STEP.scaled(batch=3, num_q_heads=10,
                                                         num_kv_heads=2, context=2000, layers=4,
                                                         pool_blocks=12, hidden=512, top_k=8),
                                beta, 64)
    if beta >= 1.0:
        assert r["due"] == 0 and r["moved"] == 0
    if beta == 0.0:
        assert r["moved"] > 0


def test_step_recall_overlap_matches_join():
    """Recalls left running into the next step (the next selection of a layer waits for that
    layer's recall only) give the same results as recalls joined at the end of their step."""
    H.log("[case] in-step recall, overlap vs join")
    import harness_recall as HR
    moved = HR.run_overlap_vs_join(wk.QWEN3_14B_STEP.scaled(batch=3, num_q_heads=10,
                                                            num_kv_heads=2, context=2000,
                                                            layers=4, pool_blocks=12, hidden=512,
                                                            top_k=8), 0.0)
    assert moved > 0


@pytest.mark.parametrize("side", [True, False])
def test_step_offload_parity_flag_handoff(side):
    """The offload step with its CPU side handed over through flags (a signal kernel per layer,
    the plan's dispatcher thread, a bounded wait kernel before each merge), three steps in a
    row: flags, host partials and merged outputs against the oracle."""
    H.log(f"[case] step offload, flag hand-off, side={side}")
    import harness_step as HS
    r = HS.run_step(wk.QWEN3_14B_STEP.scaled(batch=3, num_q_heads=10, num_kv_heads=2,
                                             context=0, ctx_min=1, ctx_max=2000, layers=4,
                                             pool_blocks=6, hidden=512, top_k=8),
                    gen_device="cpu", side=side, offload=True, flags=True, steps=3)
    assert r["cpu_ratio"] > 0.1


def test_stream_flags_signal_wait_and_bounded_timeout():
    """sa_stream_signal / sa_stream_wait on page-locked flags: a wait on a flag that already
    equals the counter passes without a timeout; a wait passes when the host sets the flag
    later; a wait on a flag nobody sets gives up after its bound, records the timeout, and
    its stream goes on."""
    import threading
    import time
    H.log("[case] stream flags")
    f = B.pinned_empty((4,), torch.int32).zero_()
    ctr, flag, tmo = f[0:1], f[1:2], f[3:4]
    s = torch.cuda.Stream()
    B.sa_stream_signal(ctr, s)  # counter 1
    s.synchronize()
    assert f[0].item() == 1
    flag.fill_(1)
    B.sa_stream_wait(flag, ctr, 1000, tmo, s)
    s.synchronize()
    assert f[3].item() == 0
    # the counter advances on the stream; the host sets the flag 50 ms later
    B.sa_stream_signal(ctr, s)  # counter 2
    B.sa_stream_wait(flag, ctr, 10000, tmo, s)
    t = threading.Timer(0.05, lambda: f.__setitem__(1, 2))
    t0 = time.monotonic()
    t.start()
    s.synchronize()
    t.join()
    assert f[0].item() == 2 and f[3].item() == 0 and time.monotonic() - t0 < 5
    # never set: the wait ends by itself after about 20 ms, and later work still runs
    B.sa_stream_signal(ctr, s)  # counter 3
    B.sa_stream_wait(flag, ctr, 20, tmo, s)
    B.sa_stream_signal(ctr, s)  # counter 4
    s.synchronize()
    assert f[3].item() == 1 and f[0].item() == 4 and f[1].item() == 2


def test_step_parity_selection_in_pieces():
    """The step with pairs large enough that the selection cuts them into pieces (the hand-over
    of each piece's candidates through device-coherent memory), side stream and host mirrors."""
    H.log("[case] step, selection in pieces")
    import harness_step as HS
    HS.run_step(wk.QWEN3_14B_STEP.scaled(batch=2, num_q_heads=8, num_kv_heads=2, context=26000,
                                         layers=2, pool_blocks=12, hidden=256, top_k=16),
                gen_device="cpu", handoff=True, side=True)


def test_step_offload_parity_bs64():
    """The offload step on blocks of 64 tokens, ragged, with the host worker."""
    H.log("[case] step offload bs64")
    import harness_step as HS
    HS.run_step(wk.QWEN3_14B_STEP.scaled(batch=3, num_q_heads=10, num_kv_heads=2, context=0,
                                         ctx_min=1, ctx_max=3000, layers=3, pool_blocks=6,
                                         hidden=512, top_k=5, block_size=64),
                gen_device="cpu", side=False, offload=True)


def test_step_parity_five_wave_gemm():
    """A selection over 4096 blocks a pair (64K tokens in blocks of 16): the step's GEMMs run
    five waves a workgroup, each over two of a k-slice's ten k-steps (hidden 5120 in 16
    slices); side stream and host hand-off.  One sequence, one KV head group, two layers."""
    H.log("[case] step, five-wave GEMM")
    import harness_step as HS
    HS.run_step(wk.QWEN3_14B_STEP.scaled(batch=1, num_q_heads=10, num_kv_heads=2,
                                         context=65536, layers=2, pool_blocks=6, hidden=5120,
                                         top_k=3, block_size=16),
                gen_device="cpu", handoff=True, side=True)


def test_step_parity_minmax_no_handoff():
    H.log("[case] step minmax")
    import harness_step as HS
    HS.run_step(wk.QWEN3_14B_STEP.scaled(batch=2, num_q_heads=8, num_kv_heads=2, context=1024,
                                         layers=3, pool_blocks=8, hidden=256, top_k=4,
                                         digest_kinds=("minmax",)),
                gen_device="cpu", handoff=False, side=False, kind="minmax")


@pytest.mark.parametrize("name,wl,drop", [
    ("f32-tiny", wk.TINY, 0.0),
    ("bf16-ragged-bs16", wk.RAGGED.scaled(batch=6, ctx_min=1, ctx_max=2500), 0.0),
    ("bf16-ragged-bs32", wk.RAGGED.scaled(batch=4, ctx_min=40, ctx_max=3000, block_size=32,
                                          top_k=64), 0.0),
    ("bf16-some-blocks-without-page", wk.RAGGED.scaled(batch=5, ctx_min=1, ctx_max=1500), 0.3),
    ("bf16-ragged-bs64", wk.RAGGED.scaled(batch=4, ctx_min=1, ctx_max=3000, block_size=64,
                                          top_k=32), 0.1),
    ("f32-bs64", wk.TINY.scaled(block_size=64, context=1000 + 9), 0.0),
])
def test_dense_parity(name, wl, drop):
    """FullKV (sa_dense_decode) against the oracle's dense attention over the whole context;
    with blocks left without a page, against attention over the blocks that have one."""
    H.log(f"[case] dense {name}")
    lens = wk.seq_lens(wl)
    kv = wk.draw_kv_pages(wl, lens, "cpu")
    table = kv["table"].clone()
    if drop:
        g = wk.generator(wl, "dense_drop", "cpu")
        gone = (torch.rand(table.shape, generator=g) < drop) & (table >= 0)
        table[gone] = -1
        table[0, 0, :] = -1  # one pair with nothing: the empty partial
    q = wk.draw_queries(wl, "cpu")["Q"]
    P = kv["K"].shape[0]
    dims = H.dims_for(wl, P)
    dev = "cuda"
    o = torch.full((wl.batch, wl.num_q_heads, wl.head_dim), float("nan"), device=dev)
    m = torch.full((wl.batch, wl.num_q_heads), float("nan"), device=dev)
    l = torch.full_like(m, float("nan"))
    B.sa_dense_decode(dims, q.to(dev), B.pack_k_pages(dims, kv["K"].to(dev)),
                      B.pack_v_pages(dims, kv["V"].to(dev)), table.to(dev), lens.to(dev),
                      wl.scale, o, m, l)
    torch.cuda.synchronize()
    o, m, l = o.cpu().double().numpy(), m.cpu().double().numpy(), l.cpu().double().numpy()
    G, bs = wl.group, wl.block_size
    max_err = 0.0
    for s in range(wl.batch):
        n = int(lens[s])
        for h in range(wl.num_kv_heads):
            K = wk.f64(wk.logical_rows(kv["K"], kv["table"][s, h], n))
            V = wk.f64(wk.logical_rows(kv["V"], kv["table"][s, h], n))
            blocks = [b for b in range(so.num_blocks(n, bs)) if int(table[s, h, b]) >= 0]
            for j in range(G):
                qh = h * G + j
                qv = q[s, qh].double().numpy()
                if drop:
                    want = so.attend_blocks(qv, K, V, blocks, n, bs, wl.scale)
                else:
                    want = so.dense_attention(qv, K, V, n, wl.scale)
                max_err = max(max_err, H.compare_partial(o[s, qh], m[s, qh], l[s, qh], want,
                                                         H.attn_tol(wl), f"seq {s} head {qh}"))
    H.log(f"  dense {name}: max_err={max_err:.2e}")
