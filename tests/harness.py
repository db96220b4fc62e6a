"""Parity harness: one workload run through the HIP library (via the C ABI) and through
the CPU oracle, on the same seeded inputs, with every stage compared.

The oracle only ever sees generator outputs (or values it computed itself): it never
reads anything the HIP path produced.  Selections are compared as sets, allowing a block
in the symmetric difference only if its oracle score is within 1e-6 relative of the
oracle's k-th score.  Outputs are compared with the oracle's attention over the GPU's
selection: the oracle's own where the two agree, and otherwise (a tie) the oracle's
attention over the GPU's selection once it has passed that check.
"""

from __future__ import annotations

import math
import sys
from dataclasses import dataclass, field

import numpy as np
import torch

from block_sparse_attention_digest_amd import binding as B
from block_sparse_attention_digest_amd import workloads as wk
from oracle import scout_oracle as so

TIE_REL = 1e-6          # selection: allowed |sigma(b) - sigma_(k)| / |sigma_(k)|
TOL_F32 = 2e-3          # attention / merge, float32 KV, max abs
TOL_BF16 = 1e-2         # attention / merge, bf16 KV with float32 accumulation, max abs
TOL_GEMM = 1e-3         # Q_pred against float64, max abs


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dims_for(wl: wk.Workload, num_pages: int) -> B.Dims:
    return B.Dims(wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size,
                  wl.max_blocks, num_pages, B.SA_BF16 if wl.kv_dtype == "bf16" else B.SA_F32)


def attn_tol(wl):
    return TOL_BF16 if wl.kv_dtype == "bf16" else TOL_F32


def selection_matches(sel_gpu, sel_oracle, sigma_oracle, k_s):
    """True if identical; otherwise every differing block must be a tie within TIE_REL of
    the oracle's k-th largest score (else AssertionError)."""
    a, b = set(int(x) for x in sel_gpu), set(int(x) for x in sel_oracle)
    assert len(a) == len(b) == k_s, (len(a), len(b), k_s)
    if a == b:
        return True
    kth = np.sort(sigma_oracle)[::-1][k_s - 1]
    for blk in a ^ b:
        assert abs(sigma_oracle[blk] - kth) <= TIE_REL * abs(kth), \
            f"block {blk}: score {sigma_oracle[blk]} vs k-th {kth}"
    return False


def compare_partial(o_g, m_g, l_g, p: so.Partial, tol, what):
    """GPU (o, m, l) against an oracle Partial: o max-abs, lse, and -inf exactly."""
    if p.m == -math.inf:
        assert m_g == -math.inf and l_g == 0.0 and not np.any(o_g), f"{what}: expected empty"
        return 0.0
    assert np.isfinite(m_g) and l_g > 0, f"{what}: GPU partial empty or invalid ({m_g}, {l_g})"
    err_o = float(np.max(np.abs(o_g - p.o)))
    err_lse = abs((m_g + math.log(l_g)) - p.lse)
    assert err_o <= tol, f"{what}: o max abs err {err_o} > {tol}"
    assert err_lse <= tol, f"{what}: lse err {err_lse} > {tol}"
    return max(err_o, err_lse)


@dataclass
class LayerRun:
    """Results of one single-layer case."""
    n_pairs: int = 0
    ties: int = 0
    max_err_attn: float = 0.0
    max_err_final: float = 0.0
    max_err_q: float = 0.0
    max_rel_score: float = 0.0
    digest_mismatch: int = 0
    notes: list = field(default_factory=list)


def oracle_query(wl, qin):
    if "Q" in qin:
        return wk.f64(qin["Q"])
    X, W = wk.f64(qin["X"]), wk.f64(qin["W"])
    return so.query_heads(so.predict_query(X, W), wl.num_q_heads, wl.head_dim)


def poison_page_tails(kv: dict, lens, block_size: int):
    """Rows past each sequence's end inside its last page are no token of any block: fill
    them with NaN keys and infinite values (alternating signs), which the kernels must never
    let into a result."""
    table = kv["table"].cpu()
    bad_k = torch.tensor([float("nan"), float("-inf")])
    bad_v = torch.tensor([float("inf"), float("nan")])
    n_rows = 0
    for s in range(table.shape[0]):
        n = int(lens[s])
        used = n % block_size
        if used == 0:
            continue
        last = (n - 1) // block_size
        for h in range(table.shape[1]):
            page = int(table[s, h, last])
            for t in range(used, block_size):
                kv["K"][page, t] = bad_k[t % 2].to(kv["K"].dtype)
                kv["V"][page, t] = bad_v[t % 2].to(kv["V"].dtype)
                n_rows += 1
    return n_rows


def run_layer(wl: wk.Workload, kind: str, gen_device: str = "cpu", top_k: int | None = None,
              resident_override=None, pairs_to_check=None, host_worker=False,
              poison_tails=False) -> LayerRun:
    """Run one single-layer workload (configs 1, 2, 3, 5 and their scaled variants).

    resident_override: None (the workload recipe), "all" or "none".
    pairs_to_check: None (all pairs) or a list of pair indices for the output comparison.
    host_worker: the host partial comes from the library's host worker over the GPU's own
    offloaded lists and the token-row pages in host memory (Algorithm 1 end to end), instead
    of from the oracle.
    poison_tails: the unused rows of partly filled last pages hold NaN and infinities.
    """
    dev = "cuda"
    res = LayerRun()
    k = wl.top_k if top_k is None else top_k
    B_, Hkv, G, d, bs = wl.batch, wl.num_kv_heads, wl.group, wl.head_dim, wl.block_size
    lens = wk.seq_lens(wl)
    kv = wk.draw_kv_pages(wl, lens, gen_device)
    if poison_tails:
        res.notes.append(f"poisoned tail rows: {poison_page_tails(kv, lens, bs)}")
    qin = wk.draw_queries(wl, gen_device)
    P_full = kv["K"].shape[0]

    # ---------------- oracle: query, digests, selection (from generator outputs only)
    Qo = oracle_query(wl, qin)
    table_g = kv["table"]

    def logical(s, h, which):
        n = int(lens[s])
        return wk.f64(wk.logical_rows(kv[which], table_g[s, h], n))

    sel_o, sig_o, dig_o = {}, {}, {}
    pairs = B_ * Hkv
    check = set(range(pairs)) if pairs_to_check is None else set(pairs_to_check)
    for s in range(B_):
        n = int(lens[s])
        if s % 16 == 15:
            log(f"  oracle digests/selection: {s + 1}/{B_} sequences")
        for h in range(Hkv):
            Kl = logical(s, h, "K")
            dig = so.digest_mean(Kl, n, bs, wl.kv_dtype) if kind == "mean" else \
                so.digest_minmax(Kl, n, bs)
            dig_o[(s, h)] = dig  # the stored values, held in float64
            qg = Qo[s, h * G:(h + 1) * G]
            sig = so.score_blocks(qg, dig, kind)
            sig_o[(s, h)] = sig
            sel_o[(s, h)] = so.select_topk(sig, k)
    sel_lists = [[sel_o[(s, h)] for h in range(Hkv)] for s in range(B_)]
    if resident_override is None:
        R = wk.choose_resident(wl, sel_lists, lens)
    else:
        R = [[np.arange(so.num_blocks(int(lens[s]), bs)) if resident_override == "all"
              else np.zeros(0, np.int64) for h in range(Hkv)] for s in range(B_)]
    cap = max(1, max(len(R[s][h]) for s in range(B_) for h in range(Hkv)))
    pool = wk.build_pool(wl, R, kv["K"], kv["V"], kv["table"], cap)
    P_pool = pool["K"].shape[0]
    bt_cpu = pool["block_table"].cpu()

    # oracle layer result per checked pair; host partial = attention over S_cpu (same
    # query).  Unchecked pairs get an empty host partial: their outputs are not compared.
    out_o = {}
    host_o = np.zeros((B_, wl.num_q_heads, d))
    host_m = np.full((B_, wl.num_q_heads), -np.inf)
    host_l = np.zeros((B_, wl.num_q_heads))
    for s in range(B_):
        n = int(lens[s])
        for h in range(Hkv):
            if s * Hkv + h not in check:
                continue
            resident = (bt_cpu[s, h, :so.num_blocks(n, bs)] >= 0).numpy()
            qg = Qo[s, h * G:(h + 1) * G]
            r = so.attend_selection(qg, logical(s, h, "K"), logical(s, h, "V"), n, bs,
                                    sig_o[(s, h)], sel_o[(s, h)], resident, wl.scale)
            out_o[(s, h)] = r
            for j in range(G):
                host_o[s, h * G + j] = r.host[j].o
                host_m[s, h * G + j] = r.host[j].m
                host_l[s, h * G + j] = r.host[j].l
    log(f"  oracle done: {B_ * Hkv} pairs selected, {len(check)} attended")

    # ---------------- HIP path through the C ABI
    f32, i32 = torch.float32, torch.int32
    lens_d = lens.to(dev)
    if "Q" in qin:
        Qg = qin["Q"].to(dev).contiguous()
    else:
        X, W = qin["X"].to(dev), qin["W"].to(dev)
        Qg = torch.empty((B_, wl.num_q_heads * d), dtype=f32, device=dev)
        gws = B.workspace(B.sa_predict_query_workspace_bytes(B_, W.shape[0], X.shape[1]))
        B.sa_predict_query(X, B.pack_weight(W), Qg, gws)
        Qg = Qg.view(B_, wl.num_q_heads, d)
    dims_full = dims_for(wl, P_full)
    per = 2 if kind == "minmax" else 1
    dig_g = torch.zeros((B_, Hkv, wl.max_blocks, per, d), dtype=wl.torch_kv_dtype, device=dev)
    K_full = B.pack_k_pages(dims_full, kv["K"].to(dev))
    B.sa_build_digests(dims_full, kind, K_full, kv["table"].to(dev), lens_d, dig_g)
    del K_full
    dims = dims_for(wl, P_pool)
    gb = torch.empty((pairs, k), dtype=i32, device=dev)
    cb = torch.empty_like(gb)
    ng = torch.empty(pairs, dtype=i32, device=dev)
    nc = torch.empty_like(ng)
    scores = torch.zeros((pairs, wl.max_blocks), dtype=f32, device=dev)
    ws = B.workspace(B.sa_workspace_bytes(dims, k))
    bt = pool["block_table"].to(dev)
    B.sa_select_blocks(dims, kind, Qg, dig_g, lens_d, k, bt, gb, ng, cb, nc, scores, ws)
    Kp, Vp = B.pack_k_pages(dims, pool["K"].to(dev)), B.pack_v_pages(dims, pool["V"].to(dev))
    rows = B_ * wl.num_q_heads
    o_gpu = torch.empty((rows, d), dtype=f32, device=dev)
    m_gpu = torch.empty(rows, dtype=f32, device=dev)
    l_gpu = torch.empty(rows, dtype=f32, device=dev)
    B.sa_sparse_decode(dims, Qg, Kp, Vp, bt, lens_d, gb, ng, k, wl.scale, o_gpu, m_gpu, l_gpu, ws)
    if host_worker:  # A_cpu on host threads, from the hand-off lists and host pages
        torch.cuda.synchronize()
        ho = torch.empty((rows, d), dtype=f32)
        hm = torch.empty(rows, dtype=f32)
        hl = torch.empty(rows, dtype=f32)
        B.sa_host_partial_attention(dims_full, Qg.cpu().contiguous(), kv["K"].cpu().contiguous(),
                                    kv["V"].cpu().contiguous(),
                                    kv["table"].cpu().to(i32).contiguous(), lens.cpu().to(i32),
                                    cb.cpu(), nc.cpu(), k, wl.scale, ho, hm, hl, 8)
        hto, htm, htl = ho.to(dev), hm.to(dev), hl.to(dev)
        log("  host worker done")
    else:
        hto = torch.from_numpy(host_o).to(f32).to(dev).contiguous()
        htm = torch.from_numpy(host_m).to(f32).to(dev).contiguous()
        htl = torch.from_numpy(host_l).to(f32).to(dev).contiguous()
    o_fin = torch.empty_like(o_gpu)
    m_fin = torch.empty_like(m_gpu)
    l_fin = torch.empty_like(l_gpu)
    B.sa_decode_attend_merge(dims, Qg, Kp, Vp, bt, lens_d, gb, ng, k, wl.scale, hto, htm, htl,
                             nc, o_fin, m_fin, l_fin, ws)
    # the separate merge call must agree with the fused one
    o_mrg = torch.empty_like(o_gpu)
    m_mrg = torch.empty_like(m_gpu)
    l_mrg = torch.empty_like(l_gpu)
    B.sa_merge(o_gpu, m_gpu, l_gpu, hto, htm, htl, o_mrg, m_mrg, l_mrg)
    torch.cuda.synchronize()
    log("  HIP path done")

    # ---------------- compare
    if "X" in qin:
        res.max_err_q = float(np.max(np.abs(Qg.cpu().double().numpy() - Qo)))
        assert res.max_err_q <= TOL_GEMM, f"Q_pred max abs err {res.max_err_q}"
    dg = dig_g.cpu()
    gb_c, cb_c, ng_c, nc_c = gb.cpu().numpy(), cb.cpu().numpy(), ng.cpu().numpy(), nc.cpu().numpy()
    sc_c = scores.cpu().double().numpy()
    o_g, m_g, l_g = o_gpu.cpu().double().numpy(), m_gpu.cpu().double().numpy(), l_gpu.cpu().double().numpy()
    o_f, m_f, l_f = o_fin.cpu().double().numpy(), m_fin.cpu().double().numpy(), l_fin.cpu().double().numpy()
    o_m2, m_m2, l_m2 = o_mrg.cpu().double().numpy(), m_mrg.cpu().double().numpy(), l_mrg.cpu().double().numpy()
    tol = attn_tol(wl)
    for s in range(B_):
        n = int(lens[s])
        nb = so.num_blocks(n, bs)
        for h in range(Hkv):
            p = s * Hkv + h
            # digests: bit-exact (exact float64 sums, one rounding on both sides)
            dgp = wk.f64(dg[s, h, :nb].reshape(nb, per, d))
            want = dig_o[(s, h)].reshape(nb, per, d)
            res.digest_mismatch += int(np.sum(dgp != want))
            # scores (informative) and selection
            sig = sig_o[(s, h)]
            rel = np.abs(sc_c[p, :nb] - sig) / max(1e-30, np.max(np.abs(sig)))
            res.max_rel_score = max(res.max_rel_score, float(rel.max()))
            k_s = min(k, nb)
            sel_g = np.sort(np.concatenate([gb_c[p, :ng_c[p]], cb_c[p, :nc_c[p]]]))
            assert ng_c[p] + nc_c[p] == k_s, (p, ng_c[p], nc_c[p], k_s)
            assert np.all(gb_c[p, ng_c[p]:] == -1) and np.all(cb_c[p, nc_c[p]:] == -1)
            assert np.all(np.diff(gb_c[p, :ng_c[p]]) > 0) and np.all(np.diff(cb_c[p, :nc_c[p]]) > 0)
            resident = (bt_cpu[s, h, :nb] >= 0).numpy()
            assert np.all(resident[gb_c[p, :ng_c[p]]]) and not np.any(resident[cb_c[p, :nc_c[p]]])
            same = selection_matches(sel_g, sel_o[(s, h)], sig, k_s)
            res.n_pairs += 1
            res.ties += not same
            if p not in check:
                continue
            r = out_o[(s, h)]
            if not same:
                # a valid tie-alternative selection: the oracle's attention over the GPU's
                # own selection, merged with the host partial the GPU was given
                qg = Qo[s, h * G:(h + 1) * G]
                r = so.attend_selection(qg, logical(s, h, "K"), logical(s, h, "V"), n, bs, sig,
                                        sel_g, resident, wl.scale,
                                        None if host_worker else r.host)
            for j in range(G):
                row = s * wl.num_q_heads + h * G + j
                e1 = compare_partial(o_g[row], m_g[row], l_g[row], r.gpu[j], tol, f"gpu part row {row}")
                e2 = compare_partial(o_f[row], m_f[row], l_f[row], r.out[j], tol, f"final row {row}")
                e3 = compare_partial(o_m2[row], m_m2[row], l_m2[row], r.out[j], tol, f"merge row {row}")
                res.max_err_attn = max(res.max_err_attn, e1)
                res.max_err_final = max(res.max_err_final, e2, e3)
    assert res.digest_mismatch == 0, f"{res.digest_mismatch} digest elements differ"
    assert res.ties <= max(1, res.n_pairs // 100), f"too many tie-differing pairs: {res.ties}"
    log(f"  {wl.name}/{kind}: pairs={res.n_pairs} ties={res.ties} "
        f"attn_err={res.max_err_attn:.2e} final_err={res.max_err_final:.2e} "
        f"q_err={res.max_err_q:.2e} score_rel={res.max_rel_score:.2e}")
    return res
