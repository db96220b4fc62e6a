"""Parity harness for the layer-ahead decode step (Algorithm 1) over several layers.

Inputs come from the generators; the resident pool of every layer is the top
`pool_blocks` blocks under the true query Q^i = W_Q^i X^i on the drawn digests, chosen by
the ORACLE (the stand-in for "important blocks found in earlier steps").  Pool-block
digests are then recomputed from the pool keys on both sides.  The HIP step runs through
sa_decode_step; the oracle runs decode_step_pair for the checked pairs.
"""

from __future__ import annotations

import numpy as np
import torch

import harness as H
from block_sparse_attention_digest_amd import binding as B
from block_sparse_attention_digest_amd import workloads as wk
from oracle import scout_oracle as so


def oracle_pool_sets(wl, X64, W64, dig64, kind="mean"):
    """Top pool_blocks blocks per (seq, KV head) under the true query of one layer."""
    Q = so.query_heads(so.predict_query(X64, W64), wl.num_q_heads, wl.head_dim)
    G = wl.group
    sets = []
    for s in range(wl.batch):
        row = []
        for h in range(wl.num_kv_heads):
            sig = so.score_blocks(Q[s, h * G:(h + 1) * G], dig64[s, h], kind)
            row.append(so.select_topk(sig, wl.pool_blocks))
        sets.append(row)
    return sets


def prepare_step(wl, gen_device, kind="mean"):
    """Generate every layer and choose the pools with the oracle.  Returns (layers, oracle
    layer dicts builder data)."""
    dev = "cuda"
    ins = wk.draw_layer_inputs(wl, gen_device)
    layers = []
    for i in range(wl.layers):
        off = wk.layer_offsets(wl, i, gen_device)
        dig = wk.draw_layer_digests(wl, i, off, gen_device)
        if kind == "minmax":
            # stand-in min/max digests around the drawn centre: centre -+ |N(0, 1)| spread
            spread = torch.randn(dig.shape, generator=wk.generator(wl, f"spread{i}", gen_device),
                                 device=gen_device).abs().to(dig.dtype)
            dig = torch.stack([(dig.float() - spread.float()).to(dig.dtype),
                               (dig.float() + spread.float()).to(dig.dtype)], dim=3)
        X64, W64 = wk.f64(ins[i]["X"]), wk.f64(ins[i]["W"])
        sets = oracle_pool_sets(wl, X64, W64, wk.f64(dig), kind)
        pool = wk.draw_layer_pool(wl, i, off, sets)
        hp = wk.draw_host_partials(wl, i, gen_device)
        layers.append(dict(X=ins[i]["X"], W=ins[i]["W"], dig=dig, pool=pool, host=hp, sets=sets,
                           off=off))
    return layers


def device_layers(wl, data, dims, lens_d, kind="mean", handoff=True):
    """The step's per-layer device buffers (sa_layer fields): pool pages packed, pool-block
    digests rebuilt from the pool keys, lists and outputs allocated (lists poisoned with -7)."""
    dev = "cuda"
    B_, Hkv, Hq, d, k = wl.batch, wl.num_kv_heads, wl.num_q_heads, wl.head_dim, wl.top_k
    pairs = B_ * Hkv
    i32, f32 = torch.int32, torch.float32
    out = []
    for Ld in data:
        dig = Ld["dig"].to(dev).contiguous()
        k_pool = B.pack_k_pages(dims, Ld["pool"]["K"].to(dev))
        B.sa_build_digests(dims, kind, k_pool, Ld["pool"]["block_table"].to(dev), lens_d, dig)
        e = dict(x=Ld["X"].to(dev), w_q=B.pack_weight(Ld["W"].to(dev)), digests=dig,
                 block_table=Ld["pool"]["block_table"].to(dev), k_pool=k_pool,
                 v_pool=B.pack_v_pages(dims, Ld["pool"]["V"].to(dev)),
                 host_o=Ld["host"]["o"].to(dev).contiguous(),
                 host_m=Ld["host"]["m"].to(dev).contiguous(),
                 host_l=Ld["host"]["l"].to(dev).contiguous(),
                 gpu_blocks=torch.full((pairs, k), -7, dtype=i32, device=dev),
                 n_gpu=torch.full((pairs,), -7, dtype=i32, device=dev),
                 cpu_blocks=torch.full((pairs, k), -7, dtype=i32, device=dev),
                 n_cpu=torch.full((pairs,), -7, dtype=i32, device=dev),
                 out_o=torch.empty((B_, Hq, d), dtype=f32, device=dev),
                 out_m=torch.empty((B_, Hq), dtype=f32, device=dev),
                 out_l=torch.empty((B_, Hq), dtype=f32, device=dev))
        if handoff:
            e["cpu_blocks_host"] = B.pinned_empty((pairs, k)).zero_()
            e["n_cpu_host"] = B.pinned_empty((pairs,)).zero_()
        out.append(e)
    return out


def host_side(wl, data, store="full", host_pages=32768):
    """Host stores and the host-plan layers (pinned hand-off buffers, poisoned)."""
    B_, Hkv, Hq, d, k = wl.batch, wl.num_kv_heads, wl.num_q_heads, wl.head_dim, wl.top_k
    pairs = B_ * Hkv
    f32 = torch.float32
    if store == "aliased":
        shared = wk.draw_host_store_aliased(wl, host_pages)
        stores = [shared] * len(data)
    else:
        stores = [wk.draw_host_store(wl, i, Ld["off"]) for i, Ld in enumerate(data)]
    host_layers = []
    for st in stores:
        host_layers.append(dict(
            k_host=st["K"], v_host=st["V"], host_table=st["table"],
            q_host=B.pinned_empty((B_, Hq, d), f32).fill_(float("nan")),
            cpu_blocks_host=B.pinned_empty((pairs, k)).fill_(-7),
            n_cpu_host=B.pinned_empty((pairs,)).fill_(-7),
            o_host=B.pinned_empty((B_, Hq, d), f32).fill_(float("nan")),
            m_host=B.pinned_empty((B_, Hq), f32).fill_(float("nan")),
            l_host=B.pinned_empty((B_, Hq), f32).fill_(float("nan"))))
    return stores, host_layers


def run_step(wl: wk.Workload, gen_device="cpu", handoff=True, kind="mean", pairs_to_check=None,
             side=True, offload=False, host_threads=4, store="full", host_pages=32768,
             flags=False, steps=1):
    """handoff: give every layer host mirrors of its offloaded lists; side: run the
    layer-ahead work on a side stream; offload: compute the CPU side with host tasks
    (sa_decode_step_offload) from a host store of every block, instead of merging the
    drawn host partials.  store: "full" gives every block its own host page
    (draw_host_store); "aliased" maps every block into one pool of host_pages pages shared by
    all layers (draw_host_store_aliased), for shapes whose offloaded KV would not fit.
    flags: the offload step hands its CPU side over with flags (SA_HANDOFF_FLAGS) instead of
    HIP host functions; steps: how many times the step runs before the check (same inputs)."""
    dev = "cuda"
    B_, Hkv, Hq, G, d, bs, k = (wl.batch, wl.num_kv_heads, wl.num_q_heads, wl.group,
                                wl.head_dim, wl.block_size, wl.top_k)
    L = wl.layers
    data = prepare_step(wl, gen_device, kind)
    lens = wk.seq_lens(wl)
    lens_d = lens.to(dev)
    P = data[0]["pool"]["K"].shape[0]
    dims = H.dims_for(wl, P)
    pairs = B_ * Hkv
    i32, f32 = torch.int32, torch.float32

    # ---------------- HIP path: pool digests rebuilt from the pool keys, then the step
    dev_layers = device_layers(wl, data, dims, lens_d, kind, handoff)
    ws = B.workspace(B.sa_step_workspace_bytes(dims, wl.hidden, k))
    side_stream = torch.cuda.Stream() if side else None
    stores = host_layers = None
    if offload:
        stores, host_layers = host_side(wl, data, store, host_pages)
        plan = B.HostPlan(dims, k, wl.scale, lens.clone(), host_layers, threads=host_threads)
        host_stream = None
        if flags:
            plan.set_handoff("flags", gpu_wait_ms=30000)
        else:
            host_stream = torch.cuda.Stream()
        for rep in range(steps):
            if rep:  # the host partials are written again by the next step's tasks
                for hl in host_layers:
                    hl["o_host"].fill_(float("nan"))
            B.sa_decode_step_offload(dims, kind, wl.hidden, k, wl.scale, lens_d, dev_layers, ws,
                                     plan, host_stream, side_stream=side_stream)
            torch.cuda.synchronize()
        tasks, secs = plan.stats()
        if flags:
            fl = plan.flags.view(torch.int32)
            assert fl[:2 * L].tolist() == [steps] * (2 * L) and fl[2 * L].item() == 0, fl
        plan.close()
        assert tasks == L * steps, (tasks, L, steps)
        H.log(f"  HIP step with host tasks done ({tasks} tasks, {secs * 1e3:.2f} ms on the host)")
    else:
        B.sa_decode_step(dims, kind, wl.hidden, k, wl.scale, lens_d, dev_layers, ws,
                         side_stream=side_stream)
        torch.cuda.synchronize()
        H.log("  HIP step done")

    r = check_step(wl, data, dev_layers, lens, pairs_to_check, kind, offload, stores,
                   host_layers, handoff)
    cpu_ratio = np.mean([float(e["n_cpu"].sum()) * bs / (pairs * k * bs) for e in dev_layers])
    H.log(f"  step {wl.name}: checked={r['checked']} ties={r['ties']} max_err={r['max_err']:.2e} "
          f"cpu_ratio={cpu_ratio:.3f}")
    return dict(max_err=r["max_err"], ties=r["ties"], cpu_ratio=cpu_ratio)


def _oracle_layer(wl, data, i, s, h, OL, offload, sel=None):
    """The oracle's layer i for pair (s, h) over a given selection (a valid tie-alternative
    the GPU made): GPU part with Q^i over the resident selected blocks, host part over the
    offloaded ones (with Q_pred^i, Q^0 at layer 0, from the host's copy when computed; as
    given otherwise; empty when nothing is offloaded), merged."""
    G, d, bs = wl.group, wl.head_dim, wl.block_size
    n = OL["seq_len"]
    rows = slice(h * G * d, (h + 1) * G * d)
    x = wk.f64(data[i]["X"])[s:s + 1]
    q_true = so.predict_query(x, wk.f64(data[i]["W"])[rows]).reshape(G, d)
    _, c_blocks = so.split_resident(sel, OL["resident"])
    if len(c_blocks) == 0:
        host = [so.empty_partial(d)] * G
    elif offload:
        xs = wk.f64(data[i - 1]["X"] if i > 0 else data[0]["X"])[s:s + 1]
        q_sel = so.predict_query(xs, wk.f64(data[i]["W"])[rows]).reshape(G, d)
        host = [so.attend_blocks(q_sel[j], OL["K_host"], OL["V_host"], c_blocks, n, bs, wl.scale)
                for j in range(G)]
    else:
        host = OL["host"]
    return so.attend_selection(q_true, OL["K"], OL["V"], n, bs, None, sel, OL["resident"],
                               wl.scale, host)


def check_step(wl, data, dev_layers, lens, pairs_to_check=None, kind="mean", offload=False,
               stores=None, host_layers=None, handoff=False):
    """The step's lists and outputs (dev_layers, after the step ran) against the oracle's
    Algorithm 1 for the checked pairs: selections identical up to ties; outputs (and, with
    offload, the handed-over query and the host partials) within the attention tolerance of
    the oracle over the GPU's selection.  Returns {max_err, ties, checked}."""
    B_, Hkv, G, d, bs, k = (wl.batch, wl.num_kv_heads, wl.group, wl.head_dim, wl.block_size,
                            wl.top_k)
    L = len(data)
    pairs = B_ * Hkv
    check = range(pairs) if pairs_to_check is None else pairs_to_check
    ties = 0
    max_err = 0.0
    for p in check:
        s, h = divmod(p, Hkv)
        n = int(lens[s])
        nb = so.num_blocks(n, bs)
        olayers = []
        for i, Ld in enumerate(data):
            bt = Ld["pool"]["block_table"][s, h].cpu()
            resident = (bt[:nb] >= 0).numpy()
            Kl = np.zeros((nb * bs, d))
            Vl = np.zeros((nb * bs, d))
            Kp, Vp = Ld["pool"]["K"], Ld["pool"]["V"]
            for b in np.nonzero(resident)[0]:
                Kl[b * bs:(b + 1) * bs] = wk.f64(Kp[int(bt[b])])
                Vl[b * bs:(b + 1) * bs] = wk.f64(Vp[int(bt[b])])
            dig = wk.f64(Ld["dig"][s, h, :nb])
            res_blocks = np.nonzero(resident)[0]
            if kind == "mean":
                full = so.digest_mean(Kl, n, bs, wl.kv_dtype)
            else:
                full = so.digest_minmax(Kl, n, bs)
            dig[res_blocks] = full[res_blocks]
            OL = dict(X=wk.f64(Ld["X"]), W=wk.f64(Ld["W"]), digest=dig, resident=resident,
                      K=Kl, V=Vl, seq_len=n)
            if offload:  # the host's copy of the blocks; the oracle attends the offloaded ones
                st = stores[i]
                Kh = np.zeros((nb * bs, d))
                Vh = np.zeros((nb * bs, d))
                # rows of the blocks the step handed to the CPU (the oracle's own offloaded
                # blocks differ from these only on a tie, and then the GPU's are attended)
                e = dev_layers[i]
                nc_ = int(e["n_cpu"][p])
                for b in e["cpu_blocks"][p, :nc_].cpu().tolist():
                    hp = int(st["table"][s, h, b])
                    Kh[b * bs:(b + 1) * bs] = wk.f64(st["K"][hp])
                    Vh[b * bs:(b + 1) * bs] = wk.f64(st["V"][hp])
                OL["K_host"] = Kh
                OL["V_host"] = Vh
            else:
                OL["host"] = [so.Partial(wk.f64(Ld["host"]["o"][s, h * G + j]),
                                         float(Ld["host"]["m"][s, h * G + j]),
                                         float(Ld["host"]["l"][s, h * G + j]))
                              for j in range(G)]
            olayers.append(OL)
        want = so.decode_step_pair(olayers, s, h, G, d, bs, k, wl.scale, kind)
        for i in range(L):
            e = dev_layers[i]
            ng, nc = int(e["n_gpu"][p]), int(e["n_cpu"][p])
            gbl = e["gpu_blocks"][p].cpu().numpy()
            cbl = e["cpu_blocks"][p].cpu().numpy()
            assert np.all(gbl[ng:] == -1) and np.all(cbl[nc:] == -1)
            if offload:
                hl_ = host_layers[i]
                assert int(hl_["n_cpu_host"][p]) == nc
                assert np.array_equal(hl_["cpu_blocks_host"][p].numpy(), cbl)
            elif handoff:
                assert int(e["n_cpu_host"][p]) == nc
                assert np.array_equal(e["cpu_blocks_host"][p].numpy(), cbl)
            sel = np.sort(np.concatenate([gbl[:ng], cbl[:nc]]))
            same = H.selection_matches(sel, want[i].selected, want[i].scores, min(k, nb))
            r = want[i]
            if same:
                assert np.array_equal(gbl[:ng], r.gpu_blocks)
            else:
                ties += 1
                resident = olayers[i]["resident"]
                assert np.all(resident[gbl[:ng]]) and not np.any(resident[cbl[:nc]])
                r = _oracle_layer(wl, data, i, s, h, olayers[i], offload, sel)
            if offload:
                # the query handed to the CPU (Q_pred^i; Q^0 at layer 0) and the CPU's partial
                X64 = wk.f64(data[i - 1]["X"] if i > 0 else data[0]["X"])[s:s + 1]
                W64 = wk.f64(data[i]["W"])[h * G * d:(h + 1) * G * d]
                q_want = so.predict_query(X64, W64).reshape(G, d)
                q_got = host_layers[i]["q_host"][s, h * G:(h + 1) * G].double().numpy()
                if nc > 0:  # (handed over only where something is offloaded)
                    assert np.max(np.abs(q_got - q_want)) <= \
                        1e-3 * max(1.0, np.max(np.abs(q_want)))
                hl_ = host_layers[i]
                for j in range(G):  # (the empty partial where nothing is offloaded)
                    max_err = max(max_err, H.compare_partial(
                        hl_["o_host"][s, h * G + j].double().numpy(),
                        float(hl_["m_host"][s, h * G + j]), float(hl_["l_host"][s, h * G + j]),
                        r.host[j], H.attn_tol(wl), f"host partial layer {i} pair {p}"))
            o = e["out_o"][s, h * G:(h + 1) * G].cpu().double().numpy()
            m = e["out_m"][s, h * G:(h + 1) * G].cpu().double().numpy()
            l = e["out_l"][s, h * G:(h + 1) * G].cpu().double().numpy()
            for j in range(G):
                max_err = max(max_err, H.compare_partial(o[j], m[j], l[j], r.out[j],
                                                         H.attn_tol(wl), f"layer {i} pair {p}"))
    n_checked = len(list(check)) * L
    assert ties <= max(1, n_checked // 100), f"too many tie-differing selections: {ties}"
    return dict(max_err=max_err, ties=ties, checked=n_checked)
