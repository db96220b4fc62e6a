"""Parity harness for periodic recall (sa_recall_blocks) inside a multi-layer step.

A step runs once (sa_decode_step, host partials given); its selection lists and outputs are
first checked against the oracle's Algorithm 1, and only then drive the recall of every
layer.  The recall is checked against the oracle's recall_pair, bit for
bit: the new block tables, the number of blocks moved, the recalled pages' keys and values
(unpacked from the pool layouts in numpy and compared with the host store they were drawn
into), and every page that did not move.  The step then runs again: its CPU share must
fall, and its outputs must match the oracle's step over the new residency, whose keys and
values come from the generators (the host store for recalled blocks, the pool draw for the
rest), never from the device.
"""

from __future__ import annotations

import numpy as np
import torch

import harness as H
import harness_step as HS
from block_sparse_attention_digest_amd import binding as B
from block_sparse_attention_digest_amd import workloads as wk
from oracle import scout_oracle as so


def unpack_k(pool_page: torch.Tensor, bs: int, d: int) -> torch.Tensor:
    """Chunk-major [d/x][bs][x] -> token rows [bs][d] (x = 16 bytes of elements)."""
    x = 16 // pool_page.element_size()
    return pool_page.reshape(d // x, bs, x).permute(1, 0, 2).reshape(bs, d)


def unpack_v(pool_page: torch.Tensor, bs: int, d: int) -> torch.Tensor:
    """[bs/16][d][16] -> token rows [bs][d]."""
    return pool_page.reshape(bs // 16, d, 16).permute(0, 2, 1).reshape(bs, d)


def run_recall(wl: wk.Workload, max_recall: int):
    dev = "cuda"
    B_, Hkv, Hq, G, d, bs, k = (wl.batch, wl.num_kv_heads, wl.num_q_heads, wl.group,
                                wl.head_dim, wl.block_size, wl.top_k)
    pairs = B_ * Hkv
    i32, f32 = torch.int32, torch.float32
    data = HS.prepare_step(wl, "cpu")
    lens = wk.seq_lens(wl)
    lens_d = lens.to(dev)
    P = data[0]["pool"]["K"].shape[0]
    dims = H.dims_for(wl, P)
    dev_layers, stores = [], []
    for i, Ld in enumerate(data):
        dig = Ld["dig"].to(dev).contiguous()
        k_pool = B.pack_k_pages(dims, Ld["pool"]["K"].to(dev))
        B.sa_build_digests(dims, "mean", k_pool, Ld["pool"]["block_table"].to(dev), lens_d, dig)
        dev_layers.append(dict(
            x=Ld["X"].to(dev), w_q=B.pack_weight(Ld["W"].to(dev)), digests=dig,
            block_table=Ld["pool"]["block_table"].to(dev).to(i32).contiguous(), k_pool=k_pool,
            v_pool=B.pack_v_pages(dims, Ld["pool"]["V"].to(dev)),
            host_o=Ld["host"]["o"].to(dev).contiguous(), host_m=Ld["host"]["m"].to(dev).contiguous(),
            host_l=Ld["host"]["l"].to(dev).contiguous(),
            gpu_blocks=torch.full((pairs, k), -7, dtype=i32, device=dev),
            n_gpu=torch.full((pairs,), -7, dtype=i32, device=dev),
            cpu_blocks=torch.full((pairs, k), -7, dtype=i32, device=dev),
            n_cpu=torch.full((pairs,), -7, dtype=i32, device=dev),
            out_o=torch.empty((B_, Hq, d), dtype=f32, device=dev),
            out_m=torch.empty((B_, Hq), dtype=f32, device=dev),
            out_l=torch.empty((B_, Hq), dtype=f32, device=dev)))
        st = wk.draw_host_store(wl, i, Ld["off"])
        kh = B.pinned_empty(tuple(st["K"].shape), st["K"].dtype)
        vh = B.pinned_empty(tuple(st["V"].shape), st["V"].dtype)
        kh.copy_(st["K"])
        vh.copy_(st["V"])
        stores.append(dict(K=kh, V=vh, table=st["table"], table_d=st["table"].to(dev)))
    ws = B.workspace(B.sa_step_workspace_bytes(dims, wl.hidden, k))
    side = torch.cuda.Stream()
    B.sa_decode_step(dims, "mean", wl.hidden, k, wl.scale, lens_d, dev_layers, ws, side_stream=side)
    torch.cuda.synchronize()
    first = HS.check_step(wl, data, dev_layers, lens)
    H.log(f"  first step done, lists and outputs match the oracle (ties {first['ties']})")
    n_cpu_before = sum(int(e["n_cpu"].sum()) for e in dev_layers)

    # ---------------- recall every layer, then check it against the oracle
    tables_before = [e["block_table"].cpu().clone() for e in dev_layers]
    kp_before = [e["k_pool"].cpu().clone() for e in dev_layers]
    vp_before = [e["v_pool"].cpu().clone() for e in dev_layers]
    rws = B.workspace(B.sa_recall_workspace_bytes(dims, max_recall))
    moved_total = 0
    new_tables = []
    for i, e in enumerate(dev_layers):
        n_rec = torch.full((pairs,), -7, dtype=i32, device=dev)
        B.sa_recall_blocks(dims, k, max_recall, lens_d, e["block_table"], e["gpu_blocks"],
                           e["n_gpu"], e["cpu_blocks"], e["n_cpu"], stores[i]["K"],
                           stores[i]["V"], stores[i]["table_d"], e["k_pool"], e["v_pool"],
                           n_rec, rws)
        torch.cuda.synchronize()
        tab = e["block_table"].cpu().view(pairs, -1)
        tb0 = tables_before[i].view(pairs, -1)
        kp, vp = e["k_pool"].cpu(), e["v_pool"].cpu()
        moved_pages = set()
        oracle_tab = torch.empty_like(tb0)
        gl, cl = e["gpu_blocks"].cpu(), e["cpu_blocks"].cpu()
        ngl, ncl = e["n_gpu"].cpu(), e["n_cpu"].cpu()
        for p in range(pairs):
            s, h = divmod(p, Hkv)
            want_tab, moves = so.recall_pair(
                tb0[p].numpy(), int(lens[s]), bs, gl[p, :int(ngl[p])].numpy(),
                cl[p, :int(ncl[p])].numpy(), stores[i]["table"][s, h].numpy(), max_recall)
            assert np.array_equal(tab[p].numpy(), want_tab), f"layer {i} pair {p}: table"
            oracle_tab[p] = torch.from_numpy(want_tab.astype(np.int32))
            assert int(n_rec[p]) == len(moves), f"layer {i} pair {p}: n_recalled"
            for b, page, hp in moves:
                assert torch.equal(unpack_k(kp[page], bs, d), stores[i]["K"][hp]), (i, p, b)
                assert torch.equal(unpack_v(vp[page], bs, d), stores[i]["V"][hp]), (i, p, b)
                moved_pages.add(page)
            moved_total += len(moves)
        keep = torch.tensor([pg not in moved_pages for pg in range(P)])
        assert torch.equal(kp[keep], kp_before[i][keep]) and torch.equal(vp[keep], vp_before[i][keep])
        new_tables.append(oracle_tab.view(B_, Hkv, -1))  # (equal to the device's, checked)
    H.log(f"  recall: {moved_total} blocks moved, tables and pages match the oracle")

    # ---------------- the step again, over the new residency
    B.sa_decode_step(dims, "mean", wl.hidden, k, wl.scale, lens_d, dev_layers, ws, side_stream=side)
    torch.cuda.synchronize()
    n_cpu_after = sum(int(e["n_cpu"].sum()) for e in dev_layers)
    H.log(f"  second step: offloaded selected blocks {n_cpu_before} -> {n_cpu_after}")
    # the inputs are unchanged, so the selection is too: every recalled block is now a
    # resident selected block, and no evicted block was selected
    assert n_cpu_after == n_cpu_before - moved_total

    max_err, ties = 0.0, 0
    for p in range(pairs):
        s, h = divmod(p, Hkv)
        n = int(lens[s])
        nb = so.num_blocks(n, bs)
        olayers = []
        for i, Ld in enumerate(data):
            bt0 = tables_before[i].view(B_, Hkv, -1)[s, h]
            bt1 = new_tables[i][s, h]
            resident = (bt1[:nb] >= 0).numpy()
            Kl = np.zeros((nb * bs, d))
            Vl = np.zeros((nb * bs, d))
            for b in np.nonzero(resident)[0]:
                if int(bt0[b]) == int(bt1[b]):  # stayed: the pool draw
                    Kl[b * bs:(b + 1) * bs] = wk.f64(Ld["pool"]["K"][int(bt0[b])])
                    Vl[b * bs:(b + 1) * bs] = wk.f64(Ld["pool"]["V"][int(bt0[b])])
                else:                            # recalled: the host store's copy
                    hp = int(stores[i]["table"][s, h, b])
                    Kl[b * bs:(b + 1) * bs] = wk.f64(stores[i]["K"][hp])
                    Vl[b * bs:(b + 1) * bs] = wk.f64(stores[i]["V"][hp])
            # digests: the pool blocks' digests were rebuilt from the pool keys before the
            # recall and the recall does not touch them
            dig = wk.f64(Ld["dig"][s, h, :nb])
            res0 = (bt0[:nb] >= 0).numpy()
            K0 = np.zeros((nb * bs, d))
            for b in np.nonzero(res0)[0]:
                K0[b * bs:(b + 1) * bs] = wk.f64(Ld["pool"]["K"][int(bt0[b])])
            full = so.digest_mean(K0, n, bs, wl.kv_dtype)
            dig[np.nonzero(res0)[0]] = full[np.nonzero(res0)[0]]
            host = [so.Partial(wk.f64(Ld["host"]["o"][s, h * G + j]),
                               float(Ld["host"]["m"][s, h * G + j]),
                               float(Ld["host"]["l"][s, h * G + j])) for j in range(G)]
            olayers.append(dict(X=wk.f64(Ld["X"]), W=wk.f64(Ld["W"]), digest=dig,
                                resident=resident, K=Kl, V=Vl, seq_len=n, host=host))
        want = so.decode_step_pair(olayers, s, h, G, d, bs, k, wl.scale, "mean")
        for i, e in enumerate(dev_layers):
            ng, nc = int(e["n_gpu"][p]), int(e["n_cpu"][p])
            gbl = e["gpu_blocks"][p].cpu().numpy()
            cbl = e["cpu_blocks"][p].cpu().numpy()
            sel = np.sort(np.concatenate([gbl[:ng], cbl[:nc]]))
            if not H.selection_matches(sel, want[i].selected, want[i].scores, min(k, nb)):
                ties += 1
                continue
            assert np.array_equal(gbl[:ng], want[i].gpu_blocks)
            o = e["out_o"][s, h * G:(h + 1) * G].cpu().double().numpy()
            m = e["out_m"][s, h * G:(h + 1) * G].cpu().double().numpy()
            l = e["out_l"][s, h * G:(h + 1) * G].cpu().double().numpy()
            for j in range(G):
                max_err = max(max_err, H.compare_partial(o[j], m[j], l[j], want[i].out[j],
                                                         H.attn_tol(wl), f"layer {i} pair {p}"))
    assert ties <= max(1, pairs * len(data) // 100)
    H.log(f"  second step matches the oracle: max_err={max_err:.2e} ties={ties}")
    return dict(moved=moved_total, n_cpu_before=n_cpu_before, n_cpu_after=n_cpu_after)


def run_step_with_recall(wl: wk.Workload, beta: float, max_recall: int):
    """The offload step with periodic recall inside it (sa_host_plan_set_recall): after each
    layer's merge the step recalls that layer on a fourth stream when its CPU share (in
    blocks) is above beta.  Checked against the oracle's recall_due and recall_pair on the
    step's own lists, bit for bit (tables, counts, moved pages); layers not due must be
    untouched.  Then the next step's CPU share must not be higher."""
    dev = "cuda"
    B_, Hkv, d, bs, k = wl.batch, wl.num_kv_heads, wl.head_dim, wl.block_size, wl.top_k
    pairs = B_ * Hkv
    data = HS.prepare_step(wl, "cpu")
    lens = wk.seq_lens(wl)
    lens_d = lens.to(dev)
    P = data[0]["pool"]["K"].shape[0]
    dims = H.dims_for(wl, P)
    layers = HS.device_layers(wl, data, dims, lens_d, "mean", handoff=False)
    stores, host_layers = HS.host_side(wl, data)
    for h in host_layers:  # the recall reads the host store from the device: page-locked
        for n in ("k_host", "v_host"):
            pinned = B.pinned_empty(tuple(h[n].shape), h[n].dtype)
            pinned.copy_(h[n])
            h[n] = pinned
    plan = B.HostPlan(dims, k, wl.scale, lens.clone(), host_layers, threads=3)
    rec = [dict(host_table_dev=st["table"].to(dev),
                n_recalled=torch.full((pairs,), -7, dtype=torch.int32, device=dev))
           for st in stores]
    plan.set_recall(dims, max_recall, beta, rec)
    ws = B.workspace(B.sa_step_workspace_bytes(dims, wl.hidden, k))
    side, host, recall = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    tables0 = [L["block_table"].cpu().clone() for L in layers]
    kp0 = [L["k_pool"].cpu().clone() for L in layers]
    try:
        B.sa_decode_step_offload(dims, "mean", wl.hidden, k, wl.scale, lens_d, layers, ws, plan,
                                 host, side_stream=side, recall_stream=recall)
        torch.cuda.synchronize()
        # the lists the recall reads are the step's: checked against the oracle first
        HS.check_step(wl, data, layers, lens, None, "mean", offload=True, stores=stores,
                      host_layers=host_layers)
        due_layers, moved = 0, 0
        share0 = sum(int(L["n_cpu"].sum()) for L in layers)
        for i, L in enumerate(layers):
            ncl = L["n_cpu"].cpu()
            # beta crosses the C ABI as a float32: the oracle takes the same value
            due = so.recall_due(ncl.numpy(), k, float(np.float32(beta)))
            tab = L["block_table"].cpu().view(pairs, -1)
            nrec = rec[i]["n_recalled"].cpu()
            if not due:
                assert torch.equal(tab, tables0[i].view(pairs, -1)), f"layer {i} not due, changed"
                assert torch.equal(L["k_pool"].cpu(), kp0[i]), f"layer {i} not due, pages changed"
                assert int(nrec.abs().sum()) == 0, f"layer {i}: n_recalled {nrec.tolist()}"
                continue
            due_layers += 1
            gl, cl, ngl = L["gpu_blocks"].cpu(), L["cpu_blocks"].cpu(), L["n_gpu"].cpu()
            kp, vp = L["k_pool"].cpu(), L["v_pool"].cpu()
            for p in range(pairs):
                s, h = divmod(p, Hkv)
                want, moves = so.recall_pair(
                    tables0[i].view(pairs, -1)[p].numpy(), int(lens[s]), bs,
                    gl[p, :int(ngl[p])].numpy(), cl[p, :int(ncl[p])].numpy(),
                    stores[i]["table"][s, h].numpy(), max_recall)
                assert np.array_equal(tab[p].numpy(), want), f"layer {i} pair {p}: table"
                assert int(nrec[p]) == len(moves), f"layer {i} pair {p}: n_recalled"
                for b, page, hp in moves:
                    assert torch.equal(unpack_k(kp[page], bs, d), stores[i]["K"][hp])
                    assert torch.equal(unpack_v(vp[page], bs, d), stores[i]["V"][hp])
                moved += len(moves)
        # the next step, over the new residency
        B.sa_decode_step_offload(dims, "mean", wl.hidden, k, wl.scale, lens_d, layers, ws, plan,
                                 host, side_stream=side, recall_stream=recall)
        torch.cuda.synchronize()
        share1 = sum(int(L["n_cpu"].sum()) for L in layers)
    finally:
        torch.cuda.synchronize()
        plan.close()
    assert share1 <= share0 - moved, (share0, share1, moved)
    H.log(f"  in-step recall beta={beta}: {due_layers}/{len(layers)} layers due, {moved} blocks "
          f"moved, offloaded selected blocks {share0} -> {share1}")
    return dict(due=due_layers, moved=moved, share0=share0, share1=share1)


def _offload_setup(wl, beta, overlap, max_recall=64):
    dev = "cuda"
    pairs = wl.batch * wl.num_kv_heads
    data = HS.prepare_step(wl, "cpu")
    lens = wk.seq_lens(wl)
    lens_d = lens.to(dev)
    dims = H.dims_for(wl, data[0]["pool"]["K"].shape[0])
    layers = HS.device_layers(wl, data, dims, lens_d, "mean", handoff=False)
    stores, host_layers = HS.host_side(wl, data)
    for h in host_layers:
        for n in ("k_host", "v_host"):
            pinned = B.pinned_empty(tuple(h[n].shape), h[n].dtype)
            pinned.copy_(h[n])
            h[n] = pinned
    plan = B.HostPlan(dims, wl.top_k, wl.scale, lens.clone(), host_layers, threads=2)
    rec = [dict(host_table_dev=st["table"].to(dev),
                n_recalled=torch.full((pairs,), -7, dtype=torch.int32, device=dev))
           for st in stores]
    plan.set_recall(dims, max_recall, beta, rec, overlap=overlap)
    ws = B.workspace(B.sa_step_workspace_bytes(dims, wl.hidden, wl.top_k))
    streams = dict(side_stream=torch.cuda.Stream(), recall_stream=torch.cuda.Stream())
    host = torch.cuda.Stream()

    def step():
        B.sa_decode_step_offload(dims, "mean", wl.hidden, wl.top_k, wl.scale, lens_d, layers, ws,
                                 plan, host, **streams)

    return dict(layers=layers, rec=rec, plan=plan, step=step, host_layers=host_layers)


def state(S):
    out = []
    for L in S["layers"]:
        out += [L[n].clone() for n in ("out_o", "out_m", "out_l", "gpu_blocks", "n_gpu",
                                       "cpu_blocks", "n_cpu", "block_table", "k_pool", "v_pool")]
    out += [r["n_recalled"].clone() for r in S["rec"]]
    return out


def run_overlap_vs_join(wl, beta, steps=3):
    """Steps whose recalls overlap the next step against steps that join their recalls: the
    same computations in another order, so every output, list, table and page must be the
    same bit for bit after each step.  Also: an overlapping step refuses graph capture."""
    A = _offload_setup(wl, beta, overlap=False)
    Bv = _offload_setup(wl, beta, overlap=True)
    moved = 0
    try:
        for t in range(steps):
            A["step"]()
            Bv["step"]()
            torch.cuda.synchronize()
            sa, sb = state(A), state(Bv)
            assert all(torch.equal(x, y) for x, y in zip(sa, sb)), f"step {t}"
            moved += sum(int(r["n_recalled"].sum()) for r in A["rec"])
        import warnings
        g = torch.cuda.CUDAGraph()
        refused = False
        with warnings.catch_warnings():
            warnings.simplefilter("ignore")  # the refused capture leaves the graph empty
            try:
                with torch.cuda.graph(g):
                    try:
                        Bv["step"]()
                    except B.SaError:
                        refused = True
            except Exception:  # noqa: BLE001 -- an empty capture may itself complain
                pass
        assert refused, "an overlapping step was captured"
        torch.cuda.synchronize()
    finally:
        torch.cuda.synchronize()
        A["plan"].close()
        Bv["plan"].close()
    H.log(f"  overlap vs join: {steps} steps identical, {moved} blocks moved")
    return moved


def run_recall_fullsize(wl, pairs_to_check, host_pages=32768, max_recall=64):
    """The benchmark-sized step, then one recall of every layer from an aliased page-locked
    host store (as bench.py --recall), checked on sampled pairs against the oracle's
    recall_pair bit for bit: tables, counts and the moved pages."""
    dev = "cuda"
    Hkv, d, bs, k = wl.num_kv_heads, wl.head_dim, wl.block_size, wl.top_k
    pairs = wl.batch * Hkv
    data = HS.prepare_step(wl, dev)
    lens = wk.seq_lens(wl)
    lens_d = lens.to(dev)
    dims = H.dims_for(wl, data[0]["pool"]["K"].shape[0])
    layers = HS.device_layers(wl, data, dims, lens_d, "mean", handoff=False)
    ws = B.workspace(B.sa_step_workspace_bytes(dims, wl.hidden, k))
    B.sa_decode_step(dims, "mean", wl.hidden, k, wl.scale, lens_d, layers, ws,
                     side_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    # the sampled pairs' lists (which the recall reads) against the oracle first
    HS.check_step(wl, data, layers, lens, pairs_to_check)
    del data
    st = wk.draw_host_store_aliased(wl, host_pages)
    K = B.pinned_empty(tuple(st["K"].shape), st["K"].dtype)
    V = B.pinned_empty(tuple(st["V"].shape), st["V"].dtype)
    K.copy_(st["K"])
    V.copy_(st["V"])
    table_d = st["table"].to(dev)
    rws = B.workspace(B.sa_recall_workspace_bytes(dims, max_recall))
    moved = 0
    for i, L in enumerate(layers):
        t0 = L["block_table"].view(pairs, -1)[pairs_to_check].cpu()
        lists = {n: L[n].cpu() for n in ("gpu_blocks", "n_gpu", "cpu_blocks", "n_cpu")}
        n_rec = torch.full((pairs,), -7, dtype=torch.int32, device=dev)
        B.sa_recall_blocks(dims, k, max_recall, lens_d, L["block_table"], L["gpu_blocks"],
                           L["n_gpu"], L["cpu_blocks"], L["n_cpu"], K, V, table_d, L["k_pool"],
                           L["v_pool"], n_rec, rws)
        torch.cuda.synchronize()
        tab = L["block_table"].view(pairs, -1)
        for j, p in enumerate(pairs_to_check):
            s, h = divmod(p, Hkv)
            gl = lists["gpu_blocks"][p, :int(lists["n_gpu"][p])].numpy()
            cl = lists["cpu_blocks"][p, :int(lists["n_cpu"][p])].numpy()
            want, moves = so.recall_pair(t0[j].numpy(), int(lens[s]), bs, gl, cl,
                                         st["table"][s, h].numpy(), max_recall)
            assert np.array_equal(tab[p].cpu().numpy(), want), f"layer {i} pair {p}: table"
            assert int(n_rec[p]) == len(moves), f"layer {i} pair {p}: n_recalled"
            for b, page, hp in moves:
                assert torch.equal(unpack_k(L["k_pool"][page].cpu(), bs, d), st["K"][hp])
                assert torch.equal(unpack_v(L["v_pool"][page].cpu(), bs, d), st["V"][hp])
            moved += len(moves)
    H.log(f"  full-size recall: {moved} blocks moved on {len(pairs_to_check)} sampled pairs x "
          f"{len(layers)} layers, all matching the oracle")
    return moved
