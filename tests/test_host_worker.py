"""The host-side partial attention (A_cpu over the offloaded blocks) against the oracle.

CPU only: sa_host_partial_attention runs on host threads over host memory, so these tests
need the built library but no GPU.  The oracle's partial over a set of blocks is
`attend_blocks` (float64); the worker accumulates in float32, so the tolerances below are
those of float32 sums over a few hundred tokens.
"""

import math
import os

import numpy as np
import pytest
import torch

from block_sparse_attention_digest_amd import binding as B
from oracle import scout_oracle as so


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from block_sparse_attention_digest_amd import build
        build.build()
    return B.lib()


def make_problem(kv: str, seed: int, B_=3, Hq=8, Hkv=2, d=64, bs=16, max_blocks=8,
                 lens=(100, 128, 37), top=5):
    """Logical K/V per (sequence, KV head), scattered over host pages in a random order, and
    offloaded lists of random ascending blocks (pair 1 offloads nothing)."""
    g = torch.Generator().manual_seed(seed)
    dt = torch.bfloat16 if kv == "bf16" else torch.float32
    L = max_blocks * bs
    K = torch.randn(B_, Hkv, L, d, generator=g).to(dt)
    V = torch.randn(B_, Hkv, L, d, generator=g).to(dt)
    q = torch.randn(B_, Hq, d, generator=g)
    pairs = B_ * Hkv
    perm = torch.randperm(pairs * max_blocks, generator=g)
    table = perm.to(torch.int32).view(B_, Hkv, max_blocks).clone()
    k_host = torch.full((pairs * max_blocks, bs, d), float("nan")).to(dt)
    v_host = torch.full_like(k_host, float("nan"))
    for s in range(B_):
        for h in range(Hkv):
            for b in range(so.num_blocks(lens[s], bs)):
                n = min(bs, lens[s] - b * bs)
                p = int(table[s, h, b])
                k_host[p, :n] = K[s, h, b * bs:b * bs + n]  # rows past the end stay NaN
                v_host[p, :n] = V[s, h, b * bs:b * bs + n]
    cpu = torch.full((pairs, top), -1, dtype=torch.int32)
    n_cpu = torch.zeros(pairs, dtype=torch.int32)
    for p in range(pairs):
        if p == 1:
            continue
        nb = so.num_blocks(lens[p // Hkv], bs)
        pick = sorted(torch.randperm(nb, generator=g)[:min(top, nb - 1)].tolist())
        cpu[p, :len(pick)] = torch.tensor(pick, dtype=torch.int32)
        n_cpu[p] = len(pick)
    dims = B.Dims(B_, Hq, Hkv, d, bs, max_blocks, 1, B.SA_BF16 if kv == "bf16" else B.SA_F32)
    return dict(dims=dims, q=q, K=K, V=V, k_host=k_host, v_host=v_host, table=table,
                lens=torch.tensor(lens, dtype=torch.int32), cpu=cpu, n_cpu=n_cpu, top=top,
                scale=1.0 / math.sqrt(d))


def run_worker(P, threads):
    dims = P["dims"]
    rows = dims.batch * dims.num_q_heads
    o = torch.empty(rows, dims.head_dim)
    m = torch.empty(rows)
    l = torch.empty(rows)
    B.sa_host_partial_attention(dims, P["q"], P["k_host"], P["v_host"], P["table"], P["lens"],
                                P["cpu"], P["n_cpu"], P["top"], P["scale"], o, m, l, threads)
    return o.numpy().astype(np.float64), m.numpy().astype(np.float64), l.numpy().astype(np.float64)


@pytest.mark.parametrize("kv", ["f32", "bf16"])
def test_host_partial_matches_oracle(lib, kv):
    P = make_problem(kv, seed=11 if kv == "f32" else 12)
    dims = P["dims"]
    o, m, l = run_worker(P, threads=3)
    G = dims.num_q_heads // dims.num_kv_heads
    K = P["K"].double().numpy()
    V = P["V"].double().numpy()
    q = P["q"].double().numpy()
    for s in range(dims.batch):
        for qh in range(dims.num_q_heads):
            h = qh // G
            p = s * dims.num_kv_heads + h
            blocks = P["cpu"][p, :int(P["n_cpu"][p])].tolist()
            want = so.attend_blocks(q[s, qh], K[s, h], V[s, h], blocks, int(P["lens"][s]),
                                    dims.block_size, P["scale"])
            row = s * dims.num_q_heads + qh
            if not blocks:  # the empty partial
                assert m[row] == -math.inf and l[row] == 0.0 and not np.any(o[row])
                continue
            assert np.max(np.abs(o[row] - want.o)) <= 1e-5, (s, qh)
            assert abs(m[row] - want.m) <= 1e-5 * max(1.0, abs(want.m)), (s, qh)
            lse = m[row] + math.log(l[row])
            assert abs(lse - want.lse) <= 1e-5 * max(1.0, abs(want.lse)), (s, qh)


def test_host_partial_is_independent_of_thread_count(lib):
    P = make_problem("bf16", seed=21)
    ref = run_worker(P, threads=1)
    for t in (2, 5, 0):
        got = run_worker(P, threads=t)
        for a, b in zip(ref, got):
            assert np.array_equal(a, b, equal_nan=True)


def test_host_partial_skips_bad_entries(lib):
    """Entries outside the table, blocks without a host page and blocks past the sequence
    are skipped: the result is the partial over the remaining blocks."""
    P = make_problem("f32", seed=31, top=8)  # sequence 0 (7 blocks) offloads 6: room for 2
    good = run_worker(P, threads=2)
    Q = dict(P)
    Q["cpu"] = P["cpu"].clone()
    Q["n_cpu"] = P["n_cpu"].clone()
    Q["table"] = P["table"].clone()
    p = 0
    n = int(Q["n_cpu"][p])
    Q["cpu"][p, n] = 7                        # past sequence 0's 7 blocks
    Q["cpu"][p, n + 1] = 1000                 # outside the table
    Q["n_cpu"][p] = n + 2
    assert P["top"] >= n + 2
    bad = run_worker(Q, threads=2)
    for a, b in zip(good, bad):
        assert np.array_equal(a, b, equal_nan=True)
    # a block whose host page is -1 counts as not offloaded
    Q2 = dict(P)
    Q2["table"] = P["table"].clone()
    first = int(P["cpu"][p, 0])
    Q2["table"][0, 0, first] = -1
    dims = P["dims"]
    o, m, l = run_worker(Q2, threads=2)
    G = dims.num_q_heads // dims.num_kv_heads
    rest = P["cpu"][p, 1:int(P["n_cpu"][p])].tolist()
    want = so.attend_blocks(P["q"].double().numpy()[0, 0], P["K"].double().numpy()[0, 0],
                            P["V"].double().numpy()[0, 0], rest, int(P["lens"][0]),
                            dims.block_size, P["scale"])
    assert G >= 1 and np.max(np.abs(o[0] - want.o)) <= 1e-5


def test_host_partial_rejects_bad_arguments(lib):
    P = make_problem("f32", seed=41)
    dims = P["dims"]
    rows = dims.batch * dims.num_q_heads
    o, m, l = torch.empty(rows, dims.head_dim), torch.empty(rows), torch.empty(rows)
    args = [dims, P["q"], P["k_host"], P["v_host"], P["table"], P["lens"], P["cpu"],
            P["n_cpu"], P["top"], P["scale"], o, m, l]
    with pytest.raises(B.SaError):  # list stride 0
        B.sa_host_partial_attention(*args[:8], 0, *args[9:])
    with pytest.raises(B.SaError):  # scale not positive
        B.sa_host_partial_attention(*args[:9], -1.0, *args[10:])
    with pytest.raises(B.SaError):  # negative thread count
        B.sa_host_partial_attention(*args, -2)
    h = lib.sa_host_partial_attention
    st = h(ctypes_dims(dims), 1, None, None, None, None, None, None, None, 1, 0.1, None, None,
           None, 0)
    assert st == B.SA_ERR_INVALID_ARG


def ctypes_dims(dims):
    import ctypes
    return ctypes.byref(dims.c())


def plan_layer(P):
    """A host-plan layer over a make_problem instance (plain CPU tensors: nothing on the
    device reads them here)."""
    dims = P["dims"]
    rows = dims.batch * dims.num_q_heads
    return dict(k_host=P["k_host"], v_host=P["v_host"], host_table=P["table"],
                q_host=P["q"].clone(), cpu_blocks_host=P["cpu"].clone(),
                n_cpu_host=P["n_cpu"].clone(),
                o_host=torch.full((rows, dims.head_dim), float("nan")),
                m_host=torch.full((rows,), float("nan")), l_host=torch.full((rows,), float("nan")))


@pytest.mark.parametrize("threads", [1, 3])
def test_host_plan_run_matches_the_worker(lib, threads):
    """A plan's layer task (persistent workers that spin, then sleep, between jobs) gives
    exactly what sa_host_partial_attention gives for the same layer, run after run."""
    import time
    Ps = [make_problem("bf16", seed=51), make_problem("bf16", seed=52)]
    for P in Ps[1:]:  # one shape for the plan: same dims, lengths and list stride
        P["lens"] = Ps[0]["lens"]
    layers = [plan_layer(P) for P in Ps]
    dims = Ps[0]["dims"]
    plan = B.HostPlan(dims, Ps[0]["top"], Ps[0]["scale"], Ps[0]["lens"], layers, threads=threads)
    try:
        for rep in range(3):
            for i in (1, 0):
                layers[i]["o_host"].fill_(float("nan"))
                plan.run(i)
                want = run_worker(Ps[i], threads=2)
                got = (layers[i]["o_host"].numpy().astype(np.float64),
                       layers[i]["m_host"].numpy().astype(np.float64),
                       layers[i]["l_host"].numpy().astype(np.float64))
                for a, b in zip(got, want):
                    assert np.array_equal(a, b, equal_nan=True), (rep, i)
            time.sleep(0.002 * rep)  # past the spin: the workers sleep and are woken
        n, secs = plan.stats()
        assert n == 6 and secs > 0
        with pytest.raises(B.SaError):
            plan.run(2)
    finally:
        plan.close()


@pytest.mark.parametrize("isa", ["base", "avx2"])
def test_host_partial_narrower_builds(isa, tmp_path):
    """The SSE and AVX2 builds of the block routine (the widest one the CPU runs is what the
    other tests see) against the oracle and against the widest build, in a fresh process
    with SCOUTATTN_HOST_ISA set (it is read once per process)."""
    import subprocess
    import sys
    code = (
        "import sys, numpy as np; sys.path.insert(0, 'tests'); "
        "import test_host_worker as T; from block_sparse_attention_digest_amd import binding as B; "
        "B.lib(); P = T.make_problem('bf16', seed=12); o, m, l = T.run_worker(P, threads=2); "
        "np.save(sys.argv[1], np.concatenate([o.ravel(), m.ravel(), l.ravel()]))")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    outs = {}
    for name, env_isa in (("narrow", isa), ("widest", "")):
        path = str(tmp_path / f"{name}.npy")
        env = dict(os.environ, SCOUTATTN_HOST_ISA=env_isa)
        r = subprocess.run([sys.executable, "-c", code, path], cwd=root, env=env,
                           capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stderr
        outs[name] = np.load(path)
    a, b = outs["narrow"], outs["widest"]
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin)
    assert np.max(np.abs(a[fin] - b[fin])) <= 1e-5 * max(1.0, float(np.max(np.abs(b[fin]))))


def test_host_plan_many_jobs_with_random_pauses(lib):
    """200 jobs on one plan, with pauses from none to well past the workers' spin (so they are
    caught spinning, falling asleep and asleep): every result is identical to the first."""
    import time
    P = make_problem("f32", seed=71)
    layers = [plan_layer(P)]
    plan = B.HostPlan(P["dims"], P["top"], P["scale"], P["lens"], layers, threads=4)
    rng = np.random.default_rng(5)
    try:
        plan.run(0)
        ref = [layers[0][n].clone() for n in ("o_host", "m_host", "l_host")]
        for it in range(200):
            pause = float(rng.choice([0.0, 0.0001, 0.0003, 0.002]))
            if pause:
                time.sleep(pause)
            layers[0]["o_host"].fill_(float("nan"))
            plan.run(0)
            for r, n in zip(ref, ("o_host", "m_host", "l_host")):
                assert torch.equal(layers[0][n], r), (it, n)
        assert plan.stats()[0] == 201
    finally:
        plan.close()
