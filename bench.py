#!/usr/bin/env python3
"""Decode-step benchmark of the GPU-side ScoutAttention path on one MI355X.

Workload: the Qwen3-14B-shaped 40-layer decode step, batch 40, context 65536 (2048 blocks
of 32 per sequence and KV head), budget 2048 tokens (64 blocks), bf16 KV with mean
digests, a resident pool of 128 blocks per (sequence, KV head) per layer.  One step runs
Algorithm 1 over all 40 layers: the Q^i GEMM, and on a side stream the Q_pred^{i+1} GEMM
with digest scoring + top-k + split for layer i+1 (the offloaded lists written straight
into host mirrors), then block-sparse attention over the resident blocks of layer i and
the merge with layer i's host partial.  Inputs are synthetic (seeded) and resident in HBM
before timing.

Prints one JSON line: seq-layers/s (= batch * layers / step time) over K replays of the
step captured as a HIP graph; the attention kernel's achieved HBM bandwidth against the
8 TB/s peak, from HIP events recorded at each attention launch's own start and end, both
inside eager steps (sharing the GPU with the side stream) and launched alone; and the CPU
oracle timed on a bounded sample of the same workload.  In the timed step the host partials
are given (seeded); with --offload the line also carries "offload": the same step with
its CPU side computed by host threads one layer ahead (sa_decode_step_offload) from an
aliased host KV store, and the share of that step the GPU spends waiting for it; with
--recall, "recall": one periodic recall of every layer (sa_recall_blocks) over the host
link, the CPU share before and after, and (with --offload) the offload step again; with
--dense, "dense": FullKV attention over one layer's whole 64K context (sa_dense_decode).

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-graph] [--offload] [--recall]
                    [--dense] [--drift-steps S]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0  # dense bf16 MFMA


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# The single-layer workloads timed after the step (name -> workload, digest kind).
LEGS = {
    "qwen3-8b-layer-mean": ("QWEN3_8B_LAYER", "mean"),
    "qwen3-14b-layer-minmax": ("QWEN3_14B_LAYER", "minmax"),
    "ragged-mean": ("RAGGED", "mean"),
    "ragged-minmax": ("RAGGED", "minmax"),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager steps instead of replays of the step captured as a graph")
    ap.add_argument("--profile-steps", type=int, default=3,
                    help="eager steps (at least 1) after the timed region whose attention, "
                         "selection and GEMM launches are timed with kernel-precise HIP "
                         "events")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--leg", choices=sorted(LEGS), default=None,
                    help="run only this single-layer workload (no step, no oracle baseline) "
                         "and print its figures as the JSON line: the unit a per-workload "
                         "profile covers")
    ap.add_argument("--no-legs", action="store_true",
                    help="skip the single-layer workloads (the Qwen3-8B and Qwen3-14B layers "
                         "and the ragged batch), each kernel timed after a cache flush")
    ap.add_argument("--offload", action="store_true",
                    help="after the GPU path, also time the step with its CPU side computed "
                         "by host tasks (sa_decode_step_offload), reported as \"offload\"")
    ap.add_argument("--offload-steps", type=int, default=5)
    ap.add_argument("--host-threads", type=int, default=16,
                    help="host worker threads of the offload step (at most the CPUs present)")
    ap.add_argument("--host-pages", type=int, default=32768,
                    help="pages of the aliased host KV store of the offload step")
    ap.add_argument("--recall", action="store_true",
                    help="after the GPU path (and --offload), recall every layer's offloaded "
                         "selected blocks from the host store (sa_recall_blocks), reported as "
                         "\"recall\"; with --offload the offload step is timed again after it")
    ap.add_argument("--dense", action="store_true",
                    help="also time dense (FullKV) attention over one layer of the workload's "
                         "whole context (sa_dense_decode), reported as \"dense\"")
    ap.add_argument("--drift-steps", type=int, default=0,
                    help="decode steps of a drift study: each step's layer inputs move "
                         "(X <- rho X + sqrt(1 - rho^2) Z), once without recall and once "
                         "recalling every layer whose CPU share exceeds --beta, reported as "
                         "\"drift\"")
    ap.add_argument("--drift-rho", type=float, default=0.97)
    ap.add_argument("--beta", type=float, default=0.12)
    ap.add_argument("--block-size", type=int, default=None, choices=(16, 32, 64),
                    help="KV block size instead of the workload's 32, with the token budget "
                         "and the resident pool kept in tokens (a study of the digest "
                         "granularity; not the headline workload)")
    ap.add_argument("--digest", choices=("mean", "minmax"), default="mean",
                    help="digests of the 40-layer step: mean keys (the default) or Quest's "
                         "per-channel min/max (the GPU step only)")
    ap.add_argument("--pool-blocks", type=int, default=None,
                    help="resident pool blocks per (sequence, KV head) instead of the "
                         "workload's 128 (a study of the CPU share; not the headline workload)")
    args = ap.parse_args()
    if args.profile_steps < 1:
        ap.error("--profile-steps must be at least 1 (the roofline figures come from them)")
    return args


def source_hash(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def measured_traffic(wl, kind, kernel):
    """HBM bytes per launch of `kernel` from the committed PMC measurement of this workload
    (rocprofv3 FETCH_SIZE and WRITE_SIZE, scaled by a plain copy's counts), or None when the
    measurement is of another workload or the kernel's source has changed since."""
    path = os.path.join(ROOT, "profiles", "kernel_traffic.json")
    if not os.path.exists(path):
        return None
    t = json.load(open(path))
    w = t.get("workload", {})
    if (w.get("name"), w.get("block_size"), w.get("resident_pool_blocks"), w.get("digest")) != \
            (wl.name, wl.block_size, wl.pool_blocks, kind):
        return None
    for name, k in t.get("kernels", {}).items():
        if name.startswith(kernel + "<") and \
                k.get("source_sha256_16") == source_hash(os.path.join(ROOT, k["source"])):
            return k["hbm_bytes_per_launch"]
    return None


# ---------------------------------------------------------------------------------------
# workload setup (untimed)
# ---------------------------------------------------------------------------------------

def setup(wl, torch, B, wk, kind="mean"):
    dev = "cuda"
    L, Bsz, Hkv, Hq, d, k = (wl.layers, wl.batch, wl.num_kv_heads, wl.num_q_heads,
                             wl.head_dim, wl.top_k)
    pairs = Bsz * Hkv
    lens = wk.seq_lens(wl).to(dev)
    P = pairs * wl.pool_blocks
    dims = B.Dims(Bsz, Hq, Hkv, d, wl.block_size, wl.max_blocks, P, B.SA_BF16)
    ins = wk.draw_layer_inputs(wl, dev)
    # the pool of each layer: the top pool_blocks blocks under the layer's true query
    # Q^i = W_Q^i X^i on the drawn digests (blocks found important in earlier steps)
    table_none = torch.full((Bsz, Hkv, wl.max_blocks), -1, dtype=torch.int32, device=dev)
    kp = wl.pool_blocks
    sel_ws = B.workspace(B.sa_workspace_bytes(dims, kp))
    gemm_ws = B.workspace(B.sa_predict_query_workspace_bytes(Bsz, Hq * d, wl.hidden))
    q = torch.empty((Bsz, Hq * d), dtype=torch.float32, device=dev)
    gb = torch.empty((pairs, kp), dtype=torch.int32, device=dev)
    cb, ng, nc = torch.empty_like(gb), torch.empty(pairs, dtype=torch.int32, device=dev), \
        torch.empty(pairs, dtype=torch.int32, device=dev)
    layers = []
    t0 = time.time()
    for i in range(L):
        off = wk.layer_offsets(wl, i, dev)
        dig = wk.draw_layer_digests(wl, i, off, dev, kind)
        w_packed = B.pack_weight(ins[i]["W"])  # once, at weight load
        B.sa_predict_query(ins[i]["X"], w_packed, q, gemm_ws)
        B.sa_select_blocks(dims, kind, q, dig, lens, kp, table_none, gb, ng, cb, nc, None,
                           sel_ws)
        sets = [[None] * Hkv for _ in range(Bsz)]
        cbh = cb.cpu().numpy()
        for p in range(pairs):
            sets[p // Hkv][p % Hkv] = cbh[p]
        pool = wk.draw_layer_pool(wl, i, off, sets)
        k_pool = B.pack_k_pages(dims, pool["K"])  # K pages in the chunk-major layout
        v_pool = B.pack_v_pages(dims, pool["V"])  # V pages as [P][bs/16][d][16]
        del pool["K"], pool["V"]
        B.sa_build_digests(dims, kind, k_pool, pool["block_table"], lens, dig)
        hp = wk.draw_host_partials(wl, i, dev)
        del off
        layers.append(dict(
            x=ins[i]["X"], w_q=w_packed, digests=dig, block_table=pool["block_table"],
            k_pool=k_pool, v_pool=v_pool, host_o=hp["o"], host_m=hp["m"],
            host_l=hp["l"],
            gpu_blocks=torch.empty((pairs, k), dtype=torch.int32, device=dev),
            n_gpu=torch.empty(pairs, dtype=torch.int32, device=dev),
            cpu_blocks=torch.empty((pairs, k), dtype=torch.int32, device=dev),
            n_cpu=torch.empty(pairs, dtype=torch.int32, device=dev),
            cpu_blocks_host=B.pinned_empty((pairs, k)).zero_(),
            n_cpu_host=B.pinned_empty((pairs,)).zero_(),
            out_o=torch.empty((Bsz, Hq, d), dtype=torch.float32, device=dev),
            out_m=torch.empty((Bsz, Hq), dtype=torch.float32, device=dev),
            out_l=torch.empty((Bsz, Hq), dtype=torch.float32, device=dev)))
        if i % 8 == 7 or i == L - 1:
            torch.cuda.synchronize()
            log(f"setup: {i + 1}/{L} layers ({time.time() - t0:.1f} s)")
    ws = B.workspace(B.sa_step_workspace_bytes(dims, wl.hidden, k))
    return dims, lens, layers, ws


# ---------------------------------------------------------------------------------------
# algorithmic bytes
# ---------------------------------------------------------------------------------------

def attention_bytes(wl, n_gpu_sum):
    """GPUATTN of one layer: the selected resident K and V rows, q, and the (o, m, l) result."""
    kv = n_gpu_sum * wl.block_size * wl.head_dim * 2 * 2
    q = wl.batch * wl.num_q_heads * wl.head_dim * 4
    out = wl.batch * wl.num_q_heads * (wl.head_dim + 2) * 4
    return kv + q + out


def select_bytes(wl, kind="mean", lens=None):
    """Scoring + top-k + split of one layer: every valid digest row, the query, the block
    table entries of the valid blocks, and the two lists with their counts."""
    import math as _m
    Bsz, Hkv, Hq, d, k, bs = (wl.batch, wl.num_kv_heads, wl.num_q_heads, wl.head_dim,
                              wl.top_k, wl.block_size)
    el = 2 if wl.kv_dtype == "bf16" else 4
    per = 2 if kind == "minmax" else 1
    nbs = ([_m.ceil(int(n) / bs) for n in lens] if lens is not None
           else [wl.max_blocks] * Bsz)
    rows = Hkv * sum(nbs)
    return rows * (per * d * el + 4) + Bsz * Hq * d * 4 + Bsz * Hkv * 2 * (k + 1) * 4


def gemm_bytes(m, n, k):
    """Q = X W^T: W and X read once, Q written once (float32)."""
    return n * k * 2 + m * k * 2 + m * n * 4


def spread(ms):
    """Median, p10, p90 and mean of a list of kernel times (ms), in microseconds."""
    v = sorted(ms)
    q = lambda f: v[min(len(v) - 1, max(0, int(round(f * (len(v) - 1)))))]
    return {"median_us": round(q(0.5) * 1e3, 2), "p10_us": round(q(0.1) * 1e3, 2),
            "p90_us": round(q(0.9) * 1e3, 2), "mean_us": round(sum(v) / len(v) * 1e3, 2),
            "launches": len(v)}


def step_bytes(wl, n_gpu_sums, kind="mean"):
    """Algorithmic bytes of one whole step (every stage of every layer)."""
    Bsz, Hkv, Hq, d, k, L = (wl.batch, wl.num_kv_heads, wl.num_q_heads, wl.head_dim,
                             wl.top_k, wl.layers)
    n, hid = Hq * d, wl.hidden
    gemm = lambda: n * hid * 2 + Bsz * hid * 2 + Bsz * n * 4
    per = 2 if kind == "minmax" else 1  # digest rows per block
    score = (Bsz * Hkv * wl.max_blocks * per * d * 2 + Bsz * Hq * d * 4 +
             Bsz * Hkv * (2 * k + 2) * 4)
    merge = 3 * Bsz * Hq * (d + 2) * 4
    total = 0
    for i in range(L):
        total += gemm() * (2 if i + 1 < L else 1)
        total += score * (2 if i == 0 else (1 if i + 1 < L else 0))
        total += attention_bytes(wl, n_gpu_sums[i]) + merge
    return total


# ---------------------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the same workload
# ---------------------------------------------------------------------------------------

def cpu_baseline(wl_full, budget_s, kind="mean"):
    import numpy as np
    from threadpoolctl import threadpool_info

    from block_sparse_attention_digest_amd import workloads as wk
    from oracle import scout_oracle as so

    nseq = 1
    wl = wl_full.scaled(batch=nseq, layers=2)
    ins = wk.draw_layer_inputs(wl, "cpu")
    G, d, bs = wl.group, wl.head_dim, wl.block_size
    nb = wl.max_blocks
    olayers_by_pair = {(0, h): [] for h in range(wl.num_kv_heads)}
    for i in range(wl.layers):
        off = wk.layer_offsets(wl, i, "cpu")
        dig = wk.draw_layer_digests(wl, i, off, "cpu", kind)
        X64 = ins[i]["X"].float().numpy().astype(np.float64)
        W32 = ins[i]["W"].float().numpy()
        Q = so.query_heads(so.predict_query(X64, W32), wl.num_q_heads, d)
        dig64 = dig.float().numpy().astype(np.float64)
        sets = [[so.select_topk(so.score_blocks(Q[0, h * G:(h + 1) * G], dig64[0, h], kind),
                                wl.pool_blocks) for h in range(wl.num_kv_heads)]]
        pool = wk.draw_layer_pool(wl, i, off, sets)
        hp = wk.draw_host_partials(wl, i, "cpu")
        for h in range(wl.num_kv_heads):
            bt = pool["block_table"][0, h]
            resident = (bt >= 0).numpy()
            Kl = np.zeros((nb * bs, d))
            Vl = np.zeros((nb * bs, d))
            for b in np.nonzero(resident)[0]:
                Kl[b * bs:(b + 1) * bs] = pool["K"][int(bt[b])].float().numpy()
                Vl[b * bs:(b + 1) * bs] = pool["V"][int(bt[b])].float().numpy()
            digh = dig64[0, h].copy()
            res_b = np.nonzero(resident)[0]
            built = (so.digest_minmax(Kl, nb * bs, bs) if kind == "minmax"
                     else so.digest_mean(Kl, nb * bs, bs, "bf16"))
            digh[res_b] = built[res_b]
            host = [so.Partial(hp["o"][0, h * G + j].double().numpy(), float(hp["m"][0, h * G + j]),
                               float(hp["l"][0, h * G + j])) for j in range(G)]
            olayers_by_pair[(0, h)].append(dict(X=X64, W=W32, digest=digh, resident=resident,
                                                K=Kl, V=Vl, seq_len=nb * bs, host=host))
    # time whole (sequence, layer) units: all KV heads of the sequence through one layer
    def run(seconds):
        done = 0
        t0 = time.perf_counter()
        while True:
            for h in range(wl.num_kv_heads):
                so.decode_step_pair(olayers_by_pair[(0, h)], 0, h, G, d, bs, wl.top_k, wl.scale,
                                    kind=kind)
            done += wl.layers
            el = time.perf_counter() - t0
            if el >= seconds:
                return done, el

    done, el = run(budget_s)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        done1, el1 = run(budget_s / 2)
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": done / el, "unit": "seq-layers/s", "cores": threads, "kind": "oracle",
            "cpu_model": model, "os_cpu_count": os.cpu_count(),
            "one_thread": {"value": done1 / el1, "unit": "seq-layers/s", "cores": 1,
                           "sample": f"{done1} seq-layers in {el1:.1f} s"},
            "sample": f"{done} seq-layers: 1 sequence x {wl.layers} layers of the step "
                      f"(all {wl.num_kv_heads} KV heads, Algorithm 1 end to end in float64, "
                      f"{kind} digests), "
                      f"repeated for {el:.1f} s; same shapes and recipe as the GPU workload"}


# ---------------------------------------------------------------------------------------

def host_store(wl, args, B, wk):
    """The aliased host KV store (draw_host_store_aliased) in page-locked memory, which the
    host workers read and the recall kernels read over the host link."""
    t0 = time.time()
    st = wk.draw_host_store_aliased(wl, args.host_pages)
    K = B.pinned_empty(tuple(st["K"].shape), st["K"].dtype)
    V = B.pinned_empty(tuple(st["V"].shape), st["V"].dtype)
    K.copy_(st["K"])
    V.copy_(st["V"])
    log(f"host store of {args.host_pages} pages ready ({time.time() - t0:.1f} s)")
    return {"K": K, "V": V, "table": st["table"]}


def recall_measure(wl, dims, lens, layers, store, torch, B):
    """Periodic recall (sa_recall_blocks) of every layer, from the lists of the last step:
    each layer's offloaded selected blocks move into pages of resident blocks no longer
    selected, read from the page-locked host store over the host link.  Timed per layer with
    HIP events; then one step shows the CPU share that is left."""
    Bsz, Hkv, bs, d, k = wl.batch, wl.num_kv_heads, wl.block_size, wl.head_dim, wl.top_k
    pairs = Bsz * Hkv
    table_d = store["table"].to("cuda")
    rws = B.workspace(B.sa_recall_workspace_bytes(dims, k))
    n_rec = torch.empty(pairs, dtype=torch.int32, device="cuda")
    share0 = sum(int(L["n_cpu"].sum()) for L in layers) / (wl.layers * pairs * k)
    torch.cuda.synchronize()
    ms, moved = [], 0
    for L in layers:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        B.sa_recall_blocks(dims, k, k, lens, L["block_table"], L["gpu_blocks"], L["n_gpu"],
                           L["cpu_blocks"], L["n_cpu"], store["K"], store["V"], table_d,
                           L["k_pool"], L["v_pool"], n_rec, rws)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
        moved += int(n_rec.sum())
    el = 2 if wl.kv_dtype == "bf16" else 4
    nbytes = moved * 2 * bs * d * el
    total_ms = sum(ms)
    log(f"recall: {moved} blocks, {nbytes / 1e6:.1f} MB in {total_ms:.2f} ms "
        f"({nbytes / (total_ms * 1e-3) / 1e9:.1f} GB/s)")
    return {"blocks_moved": moved, "bytes_moved": nbytes,
            "ms_per_layer": round(total_ms / len(ms), 4),
            "host_link_gbs": round(nbytes / (total_ms * 1e-3) / 1e9, 2),
            "cpu_share_before": round(share0, 4)}


def gemm_measure(wl, layers, torch, B, n=40):
    """The query GEMM (a1) alone: Q = X W^T for one layer (M = batch rows, N = Hq * d, K =
    hidden), the stand-alone call with its slice sum, timed with HIP events over n launches.
    Its flops per byte of W are M, so at the HBM peak it could reach M * 8 TB/s of flops, a
    small share of the bf16 MFMA peak; both fractions are reported."""
    M, N, K = wl.batch, wl.num_q_heads * wl.head_dim, wl.hidden
    q = torch.empty((M, N), dtype=torch.float32, device="cuda")
    gws = B.workspace(B.sa_predict_query_workspace_bytes(M, N, K))
    L = len(layers)

    def calls():  # each layer's own W once per pass (no W stays cached)
        for i in range(n):
            B.sa_predict_query(layers[i % L]["x"], layers[i % L]["w_q"], q, gws)
    calls()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    calls()
    e1.record()
    torch.cuda.synchronize()
    call_us = e0.elapsed_time(e1) / n * 1e3
    kern = spread(timed_multi(torch, B, {"gemm": n}, calls)["gemm"])
    us = kern["median_us"]
    flops = 2.0 * M * N * K
    tflops = flops / (us * 1e-6) / 1e12
    ceiling = M * PEAK_HBM_GBS / 1e3  # TFLOP/s at the HBM peak (M flops per W byte)
    gbs = gemm_bytes(M, N, K) / (us * 1e-6) / 1e9
    log(f"query GEMM alone: kernel {us:.1f} us median ({tflops:.0f} TFLOP/s, {gbs:.0f} GB/s); "
        f"call with its slice sum {call_us:.1f} us")
    return {"kernel": "gemm_kernel (Q_pred / Q)", "m": M, "n": N, "k": K,
            "kernel_time": kern, "achieved": round(tflops, 1), "unit": "TFLOP/s",
            "peak": PEAK_BF16_TFLOPS, "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "hbm_ceiling": round(ceiling, 1), "frac_of_hbm_ceiling": round(tflops / ceiling, 4),
            "hbm_gbs": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "avg_call_us_with_slice_sum": round(call_us, 2)}


def dense_measure(wl, args, torch, B, wk, sparse_us):
    """FullKV attention of one layer of the workload (every block of the 64K context
    resident, 10.7 GB of K and V) with sa_dense_decode, next to the sparse path's attention
    of the same layer.  Keys and values are drawn on the device (N(0, 1), bf16)."""
    dev = "cuda"
    Bsz, Hq, Hkv, d, bs = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size
    nb = wl.max_blocks
    P = Bsz * Hkv * nb
    dims = B.Dims(Bsz, Hq, Hkv, d, bs, nb, P, B.SA_BF16)
    g = torch.Generator(device=dev)
    g.manual_seed(20240)
    t0 = time.time()

    def pool(pack):
        rows = torch.empty((P, bs, d), dtype=torch.bfloat16, device=dev)
        step = 1 << 15
        for p0 in range(0, P, step):
            p1 = min(P, p0 + step)
            rows[p0:p1] = torch.randn((p1 - p0, bs, d), generator=g, device=dev).to(torch.bfloat16)
        out = pack(dims, rows)
        del rows
        return out

    k_pool = pool(B.pack_k_pages)
    v_pool = pool(B.pack_v_pages)
    perm = torch.randperm(P, generator=g, device=dev).to(torch.int32)
    table = perm.view(Bsz, Hkv, nb).contiguous()
    lens = torch.full((Bsz,), wl.context, dtype=torch.int32, device=dev)
    q = torch.randn((Bsz, Hq, d), generator=g, device=dev)
    o = torch.empty((Bsz, Hq, d), device=dev)
    m = torch.empty((Bsz, Hq), device=dev)
    l = torch.empty_like(m)
    ws = B.workspace(B.sa_dense_workspace_bytes(dims))
    torch.cuda.synchronize()
    log(f"dense: one layer's full KV ready ({time.time() - t0:.1f} s)")

    def run():
        B.sa_dense_decode(dims, q, k_pool, v_pool, table, lens, wl.scale, o, m, l, ws)

    for _ in range(2):
        run()
    torch.cuda.synchronize()
    n = max(3, args.steps // 2)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    kv_bytes = 2 * Bsz * Hkv * wl.context * d * 2
    io_bytes = Bsz * Hq * d * 4 + Bsz * Hq * (d + 2) * 4
    gbs = (kv_bytes + io_bytes) / (ms * 1e-3) / 1e9
    log(f"dense: {ms:.3f} ms per layer, {gbs:.0f} GB/s")
    out = {"ms_per_layer": round(ms, 4), "hbm_gbs": round(gbs, 1),
           "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4), "kv_bytes": kv_bytes,
           "sparse_attention_us_alone": round(sparse_us, 2),
           "dense_over_sparse_attention": round(ms * 1e3 / sparse_us, 1),
           "note": "one layer, 40 sequences x 65536 tokens, every block resident; the "
                   "sparse figure is the same layer's block-sparse attention launched alone"}
    del k_pool, v_pool
    torch.cuda.empty_cache()
    return out


def drift_measure(wl, dims, lens, layers, ws, side_stream, store, args, torch, B):  # noqa: C901
    """The CPU share over decode steps whose inputs drift, without and with periodic recall.

    Each step moves every layer's input, X^i <- rho X^i + sqrt(1 - rho^2) Z (Z ~ N(0, 1),
    seeded per step), so the queries, and with them the selections, drift away from the
    resident pools, which were chosen for the first step's queries.  Run once without recall
    and once with it; in the second run a layer whose CPU share (offloaded selected blocks
    over the budget) exceeds beta after a step is recalled from that step's lists
    (sa_recall_blocks) before the next step -- an online stand-in for the pages' per-layer
    intervals chosen offline to keep the share under beta.  The pools change in the second
    run only, so it goes last."""
    import math as _m
    Bsz, Hkv, k = wl.batch, wl.num_kv_heads, wl.top_k
    pairs = Bsz * Hkv
    x0 = [L["x"].clone() for L in layers]
    table_d = store["table"].to("cuda")
    rws = B.workspace(B.sa_recall_workspace_bytes(dims, k))
    n_rec = torch.empty(pairs, dtype=torch.int32, device="cuda")
    c = _m.sqrt(1.0 - args.drift_rho ** 2)

    def run(recall):
        for L, x in zip(layers, x0):
            L["x"].copy_(x)
        g = torch.Generator(device="cuda")
        g.manual_seed(4242)
        shares, recalls, moved, rec_ms = [], 0, 0, 0.0
        for _ in range(args.drift_steps):
            for L in layers:
                z = torch.randn(L["x"].shape, generator=g, device="cuda")
                L["x"].copy_((args.drift_rho * L["x"].float() + c * z).to(torch.bfloat16))
            B.sa_decode_step(dims, "mean", wl.hidden, k, wl.scale, lens, layers, ws,
                             side_stream=side_stream)
            torch.cuda.synchronize()
            per_layer = [int(L["n_cpu"].sum()) / (pairs * k) for L in layers]
            shares.append(round(sum(per_layer) / len(per_layer), 4))
            if recall:
                for L, sh in zip(layers, per_layer):
                    if sh <= args.beta:
                        continue
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    B.sa_recall_blocks(dims, k, k, lens, L["block_table"], L["gpu_blocks"],
                                       L["n_gpu"], L["cpu_blocks"], L["n_cpu"], store["K"],
                                       store["V"], table_d, L["k_pool"], L["v_pool"], n_rec, rws)
                    e1.record()
                    torch.cuda.synchronize()
                    rec_ms += e0.elapsed_time(e1)
                    recalls += 1
                    moved += int(n_rec.sum())
        return shares, recalls, moved, rec_ms

    def run_offload(recall):
        """The whole system: the CPU side as host tasks one layer ahead, and (recall) periodic
        recall inside the step, gated on the device by beta; per-step time and share."""
        for L, x in zip(layers, x0):
            L["x"].copy_(x)
        f32 = torch.float32
        hls = [dict(k_host=store["K"], v_host=store["V"], host_table=store["table"],
                    q_host=B.pinned_empty((Bsz, wl.num_q_heads, wl.head_dim), f32),
                    cpu_blocks_host=B.pinned_empty((pairs, k)),
                    n_cpu_host=B.pinned_empty((pairs,)),
                    o_host=B.pinned_empty((Bsz, wl.num_q_heads, wl.head_dim), f32),
                    m_host=B.pinned_empty((Bsz, wl.num_q_heads), f32),
                    l_host=B.pinned_empty((Bsz, wl.num_q_heads), f32)) for _ in layers]
        threads = max(1, min(args.host_threads, os.cpu_count() or 1))
        plan = B.HostPlan(dims, k, wl.scale, lens.cpu().contiguous(), hls, threads=threads)
        host_stream, recall_stream = torch.cuda.Stream(), torch.cuda.Stream()
        nrec = [torch.zeros(pairs, dtype=torch.int32, device="cuda") for _ in layers]
        if recall:  # recalls overlap the next step, as in the pages
            plan.set_recall(dims, k, args.beta,
                            [dict(host_table_dev=table_d, n_recalled=n) for n in nrec], rws,
                            overlap=True)
        g = torch.Generator(device="cuda")
        g.manual_seed(4242)
        shares, ms, moved = [], [], 0
        try:
            for _ in range(args.drift_steps):
                for L in layers:
                    z = torch.randn(L["x"].shape, generator=g, device="cuda")
                    L["x"].copy_((args.drift_rho * L["x"].float() + c * z).to(torch.bfloat16))
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                B.sa_decode_step_offload(dims, "mean", wl.hidden, k, wl.scale, lens, layers, ws,
                                         plan, host_stream, side_stream=side_stream,
                                         recall_stream=recall_stream if recall else None)
                e1.record()
                e1.synchronize()  # the step's own streams; a recall may still be running
                ms.append(round(e0.elapsed_time(e1), 3))
                shares.append(round(sum(int(L["n_cpu"].sum()) for L in layers)
                                    / (len(layers) * pairs * k), 4))
            torch.cuda.synchronize()
            if recall:
                moved = sum(int(n.sum()) for n in nrec)  # (the last step's recalls)
        finally:
            torch.cuda.synchronize()
            plan.close()
        return shares, ms, moved

    t0 = time.time()
    s0, _, _, _ = run(False)
    out = {"steps": args.drift_steps, "rho": args.drift_rho, "beta": args.beta,
           "cpu_share_no_recall": s0, "mean_no_recall": round(sum(s0) / len(s0), 4),
           "layers": wl.layers,
           "note": "CPU share = offloaded selected blocks / budget, averaged over the layers "
                   "after each step; a layer is recalled when its share exceeds beta"}
    if args.offload:
        # the whole system; the run with recall changes the pools, so it goes last
        so0, ms0, _ = run_offload(False)
        so1, ms1, moved = run_offload(True)
        assert so0 == s0, "the offload step selects as the GPU-only step does"
        out.update({"cpu_share_with_recall": so1, "mean_with_recall": round(sum(so1) / len(so1), 4),
                    "blocks_moved_last_step": moved,
                    "recall": "inside the offload step (4th stream), overlapping the next step",
                    "offload_ms_per_step_no_recall": ms0,
                    "offload_ms_per_step_with_recall": ms1,
                    "mean_offload_ms_no_recall": round(sum(ms0) / len(ms0), 3),
                    "mean_offload_ms_with_recall": round(sum(ms1) / len(ms1), 3),
                    "launch": "eager"})
        log(f"drift: offload step {out['mean_offload_ms_no_recall']} ms without recall, "
            f"{out['mean_offload_ms_with_recall']} ms with in-step recall; mean CPU share "
            f"{out['mean_no_recall']} -> {out['mean_with_recall']}")
    else:
        s1, recalls, moved, rec_ms = run(True)
        out.update({"cpu_share_with_recall": s1, "mean_with_recall": round(sum(s1) / len(s1), 4),
                    "layer_recalls": recalls, "blocks_moved": moved,
                    "recall_ms_total": round(rec_ms, 2), "recall": "between steps"})
        log(f"drift: mean CPU share {out['mean_no_recall']:.3f} without recall, "
            f"{out['mean_with_recall']:.3f} with ({recalls} layer recalls)")
    log(f"drift: done in {time.time() - t0:.1f} s")
    return out


def offload_measure(wl, dims, lens, layers, ws, side_stream, ms_gpu, args, torch, B, wk,
                    store=None):
    """The same step with its CPU side computed, not given: sa_decode_step_offload runs each
    layer's host partial on host threads one layer ahead (Algorithm 1) and makes the merge
    wait for it.  The host KV is an aliased store (draw_host_store_aliased): the 64K-token
    offloaded KV of 40 layers would not fit in host memory, so every block maps into one
    pool of host pages.  Not the headline figure: the GPU path is."""
    Bsz, Hq, Hkv, d, k = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.top_k
    pairs = Bsz * Hkv
    f32 = torch.float32
    threads = max(1, min(args.host_threads, os.cpu_count() or 1))
    t0 = time.time()
    if store is None:
        store = wk.draw_host_store_aliased(wl, args.host_pages)
    hls = [dict(k_host=store["K"], v_host=store["V"], host_table=store["table"],
                q_host=B.pinned_empty((Bsz, Hq, d), f32),
                cpu_blocks_host=B.pinned_empty((pairs, k)), n_cpu_host=B.pinned_empty((pairs,)),
                o_host=B.pinned_empty((Bsz, Hq, d), f32), m_host=B.pinned_empty((Bsz, Hq), f32),
                l_host=B.pinned_empty((Bsz, Hq), f32)) for _ in range(wl.layers)]
    plan = B.HostPlan(dims, k, wl.scale, lens.cpu().contiguous(), hls, threads=threads)
    host_stream = torch.cuda.Stream()
    log(f"offload: host store of {args.host_pages} pages ready ({time.time() - t0:.1f} s), "
        f"{threads} host threads")

    handoff = "host_func"

    def step():
        B.sa_decode_step_offload(dims, "mean", wl.hidden, k, wl.scale, lens, layers, ws, plan,
                                 host_stream if handoff == "host_func" else None,
                                 side_stream=side_stream)

    def timed(run, n):
        torch.cuda.synchronize()
        n0, b0 = plan.stats()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            run()
        e1.record()
        torch.cuda.synchronize()
        n1, b1 = plan.stats()
        return e0.elapsed_time(e1) / n, (b1 - b0) / max(1, n1 - n0) * 1e3

    out = {}
    try:
        for _ in range(2):
            step()
        torch.cuda.synchronize()
        ms_eager, host_ms = timed(step, args.offload_steps)
        log(f"offload step (eager): {ms_eager:.2f} ms/step, host {host_ms:.3f} ms per layer")
        out = {"ms_per_step_eager": round(ms_eager, 3)}
        ms_off, mode = ms_eager, "eager"
        graph = None
        try:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                step()
            torch.cuda.synchronize()
            ms_graph, host_ms = timed(graph.replay, args.offload_steps)
            log(f"offload step (hip-graph): {ms_graph:.2f} ms/step")
            out["ms_per_step_graph"] = round(ms_graph, 3)
            if ms_graph < ms_off:
                ms_off, mode = ms_graph, "hip-graph"
        except Exception as e:  # noqa: BLE001
            log(f"offload step: graph capture unavailable ({e})")
        torch.cuda.synchronize()
        del graph
        # the same step with the flag hand-off (the plan's dispatcher thread and bounded GPU
        # waits on flags in page-locked memory), eager and replayed from a graph
        handoff = "flags"
        plan.set_handoff("flags", gpu_wait_ms=30000)
        for _ in range(2):
            step()
        torch.cuda.synchronize()
        ms_flags, host_ms_f = timed(step, args.offload_steps)
        log(f"offload step (flag hand-off, eager): {ms_flags:.2f} ms/step")
        out["ms_per_step_flags_eager"] = round(ms_flags, 3)
        if ms_flags < ms_off:
            ms_off, mode, host_ms = ms_flags, "eager, flag hand-off", host_ms_f
        graph = None
        try:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                step()
            torch.cuda.synchronize()
            ms_fg, host_ms_fg = timed(graph.replay, args.offload_steps)
            log(f"offload step (flag hand-off, hip-graph): {ms_fg:.2f} ms/step")
            out["ms_per_step_flags_graph"] = round(ms_fg, 3)
            if ms_fg < ms_off:
                ms_off, mode, host_ms = ms_fg, "hip-graph, flag hand-off", host_ms_fg
        except Exception as e:  # noqa: BLE001
            log(f"offload step (flag hand-off): graph capture unavailable ({e})")
        torch.cuda.synchronize()
        del graph
        plan.set_handoff("host_func")
        out.update({
            "ms_per_step": round(ms_off, 3), "launch": mode,
            "seq_layers_per_s": round(wl.batch * wl.layers / (ms_off * 1e-3), 1),
            "gpu_only_ms_per_step": round(ms_gpu, 4),
            "gpu_wait_frac": round(max(0.0, 1.0 - ms_gpu / ms_off), 4),
            "host_ms_per_layer": round(host_ms, 3), "host_threads": threads,
            "host_store": f"aliased pool of {args.host_pages} pages ({wl.kv_dtype})",
            "note": "gpu_wait_frac = 1 - (step time without the CPU side) / (step time with "
                    "it): the share of the step the GPU spends waiting for host partials"})
    finally:
        torch.cuda.synchronize()
        plan.close()
    return out


def timed_multi(torch, B, counts, fn):
    """Run fn() with the next counts[stage] launches of each stage's kernel timed from the
    kernel's own start to its end (sa_profile_kernels); returns {stage: [ms, ...]}."""
    ev = {}
    for stage, n in counts.items():
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        stops = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in starts + stops:
            e.record()
        ev[stage] = (starts, stops)
    torch.cuda.synchronize()
    for stage, (starts, stops) in ev.items():
        B.sa_profile_kernels(stage, starts, stops)
    fn()
    torch.cuda.synchronize()
    for stage in ev:
        B.sa_profile_kernels(stage, [], [])
    return {stage: [a.elapsed_time(b) for a, b in zip(*ev[stage])] for stage in ev}


def attention_bytes_exact(wl, lens, gb, ng):
    """GPUATTN bytes of one layer with ragged lengths: the valid K and V rows of every
    resident selected block, q, and the (o, m, l) result."""
    import numpy as np
    bs, d = wl.block_size, wl.head_dim
    el = 2 if wl.kv_dtype == "bf16" else 4
    g, n = gb.cpu().numpy(), ng.cpu().numpy()
    L = lens.cpu().numpy().astype(np.int64)
    tokens = 0
    for p in range(g.shape[0]):
        blocks = g[p, :max(0, int(n[p]))].astype(np.int64)
        tokens += int(np.minimum(bs, L[p // wl.num_kv_heads] - blocks * bs).sum())
    Hq = wl.num_q_heads
    return tokens * d * 2 * el + wl.batch * Hq * d * 4 + wl.batch * Hq * (d + 2) * 4


def evict(flush):
    """Read a 1 GiB buffer: it displaces the L2 caches and the 256 MB last-level cache with
    clean lines (a write would leave dirty lines that the timed kernel then has to write
    back while it reads)."""
    return flush.amax()


def layer_leg(wl, kind, torch, B, wk, flush, reps=20):
    """One single-layer workload end to end on the GPU -- digests built from the full key
    cache (a0), the query (a1: W_Q X, or drawn), the selection (a3 + a4), and the attention
    (a5) over the resident selected blocks -- with residency chosen from the GPU's own
    selection by the workload recipe.  Each kernel is timed per repetition from its own
    start to its end, after a 1 GiB read that evicts the L2 caches and the 256 MB
    last-level cache, so every byte comes from HBM."""
    import numpy as np
    dev = "cuda"
    Bsz, Hq, Hkv, d, bs, k, mb = (wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                  wl.block_size, wl.top_k, wl.max_blocks)
    pairs = Bsz * Hkv
    el = 2 if wl.kv_dtype == "bf16" else 4
    lens = wk.seq_lens(wl)
    lens_d = lens.to(dev)
    kv = wk.draw_kv_pages(wl, lens, dev)
    P_full = kv["K"].shape[0]
    SAK = B.SA_BF16 if wl.kv_dtype == "bf16" else B.SA_F32
    dims_full = B.Dims(Bsz, Hq, Hkv, d, bs, mb, P_full, SAK)
    k_full = B.pack_k_pages(dims_full, kv["K"])
    per = 2 if kind == "minmax" else 1
    dig = torch.zeros((Bsz, Hkv, mb, per, d), dtype=wl.torch_kv_dtype, device=dev)

    def each(stage, fn, n=reps):
        out = []
        for _ in range(n):
            evict(flush)
            out += timed_multi(torch, B, {stage: 1}, fn)[stage]
        return out

    # a0: the digest build (one launch; timed with events around the call)
    dig_ms = []
    for _ in range(5):
        evict(flush)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        B.sa_build_digests(dims_full, kind, k_full, kv["table"], lens_d, dig)
        e1.record()
        torch.cuda.synchronize()
        dig_ms.append(e0.elapsed_time(e1))
    ntok = int(lens.sum()) * Hkv
    nblk = sum(wk.blocks_of(lens, bs)) * Hkv
    dig_bytes = ntok * d * el + nblk * per * d * el
    del k_full
    out = {"workload": wl.name, "digest": kind}
    st = spread(dig_ms)
    out["digest_build"] = dict(time=st, bytes=dig_bytes, gbs=round(dig_bytes / (st["median_us"] * 1e-6) / 1e9, 1),
                               frac=round(dig_bytes / (st["median_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4))
    # a1: the query
    if wl.hidden:
        qin = wk.draw_queries(wl, dev)
        w_packed = B.pack_weight(qin["W"])
        q = torch.empty((Bsz, Hq * d), dtype=torch.float32, device=dev)
        gws = B.workspace(B.sa_predict_query_workspace_bytes(Bsz, Hq * d, wl.hidden))
        B.sa_predict_query(qin["X"], w_packed, q, gws)
        g_ms = each("gemm", lambda: B.sa_predict_query(qin["X"], w_packed, q, gws))
        st = spread(g_ms)
        gb_ = gemm_bytes(Bsz, Hq * d, wl.hidden)
        flops = 2.0 * Bsz * Hq * d * wl.hidden
        out["gemm"] = dict(time=st, bytes=gb_, gbs=round(gb_ / (st["median_us"] * 1e-6) / 1e9, 1),
                           frac=round(gb_ / (st["median_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                           tflops=round(flops / (st["median_us"] * 1e-6) / 1e12, 1))
        q = q.view(Bsz, Hq, d)
    else:
        q = wk.draw_queries(wl, dev)["Q"].contiguous()
    # residency from the GPU's own selection over every block, by the workload recipe
    gb = torch.empty((pairs, k), dtype=torch.int32, device=dev)
    cb, ng, nc = torch.empty_like(gb), torch.empty(pairs, dtype=torch.int32, device=dev), \
        torch.empty(pairs, dtype=torch.int32, device=dev)
    ws = B.workspace(B.sa_workspace_bytes(dims_full, k))
    B.sa_select_blocks(dims_full, kind, q, dig, lens_d, k, kv["table"], gb, ng, cb, nc, None, ws)
    g, n = gb.cpu().numpy(), ng.cpu().numpy()
    sel = [[np.sort(g[s * Hkv + h, :n[s * Hkv + h]]) for h in range(Hkv)] for s in range(Bsz)]
    R = wk.choose_resident(wl, sel, lens)
    pool = wk.build_pool(wl, R, kv["K"], kv["V"], kv["table"], k)
    del kv
    dims = B.Dims(Bsz, Hq, Hkv, d, bs, mb, pool["K"].shape[0], SAK)
    kp, vp = B.pack_k_pages(dims, pool["K"]), B.pack_v_pages(dims, pool["V"])
    bt = pool["block_table"]
    del pool
    ws = B.workspace(B.sa_workspace_bytes(dims, k))
    run_sel = lambda: B.sa_select_blocks(dims, kind, q, dig, lens_d, k, bt, gb, ng, cb, nc,
                                         None, ws)
    run_sel()
    s_ms = each("select", run_sel)
    st = spread(s_ms)
    sb = select_bytes(wl, kind, lens)
    out["select"] = dict(time=st, bytes=sb, gbs=round(sb / (st["median_us"] * 1e-6) / 1e9, 1),
                         frac=round(sb / (st["median_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4))
    torch.cuda.synchronize()
    o = torch.empty((Bsz * Hq, d), dtype=torch.float32, device=dev)
    hp = wk.draw_host_partials(wl, 0, dev)
    run_att = lambda: B.sa_decode_attend_merge(dims, q, kp, vp, bt, lens_d, gb, ng, k, wl.scale,
                                               hp["o"], hp["m"], hp["l"], nc, o, ws=ws)
    run_att()
    a_ms = each("attention", run_att)
    st = spread(a_ms)
    ab = attention_bytes_exact(wl, lens, gb, ng)
    out["attention"] = dict(time=st, bytes=ab, gbs=round(ab / (st["median_us"] * 1e-6) / 1e9, 1),
                            frac=round(ab / (st["median_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4))
    out["resident_selected_blocks"] = int(ng.sum())
    out["offloaded_selected_blocks"] = int(nc.sum())
    log(f"leg {wl.name}/{kind}: select {out['select']['time']['median_us']:.1f} us "
        f"({out['select']['frac']:.2f}), attention {out['attention']['time']['median_us']:.1f} us "
        f"({out['attention']['frac']:.2f})" +
        (f", GEMM {out['gemm']['time']['median_us']:.1f} us" if "gemm" in out else ""))
    del kp, vp, dig
    torch.cuda.empty_cache()
    return out


def copy_ceiling(torch, n_bytes=1 << 30, reps=10):
    """A plain device-to-device copy of 1 GiB (read once, written once), timed with events:
    the bandwidth a streaming kernel can reach on this machine."""
    a = torch.empty(n_bytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    st = spread(ms)
    gbs = 2 * n_bytes / (st["median_us"] * 1e-6) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return {"bytes_moved": 2 * n_bytes, "time": st, "gbs": round(gbs, 1),
            "frac": round(gbs / PEAK_HBM_GBS, 4)}


def select_alone(wl, dims, lens, layers, kind, torch, B, passes=2):
    """The selection kernel (scoring + top-k + split) launched by itself for every layer,
    each with the query the step selects it with (Q_pred^i = W_Q^i X^{i-1}; Q^0 for layer
    0), so each launch reads that layer's own digests (about 168 MB, and 40 layers' worth
    between two reads of the same ones: nothing stays in the 256 MB last-level cache)."""
    Bsz, Hq, Hkv, d, k = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.top_k
    n, pairs = Hq * d, Bsz * Hkv
    gws = B.workspace(B.sa_predict_query_workspace_bytes(Bsz, n, wl.hidden))
    qs = []
    for i, L in enumerate(layers):
        q = torch.empty((Bsz, n), dtype=torch.float32, device="cuda")
        B.sa_predict_query(layers[max(i - 1, 0)]["x"], L["w_q"], q, gws)
        qs.append(q)
    ws = B.workspace(B.sa_workspace_bytes(dims, k))
    gb = torch.empty((pairs, k), dtype=torch.int32, device="cuda")
    cb = torch.empty_like(gb)
    ng = torch.empty(pairs, dtype=torch.int32, device="cuda")
    nc = torch.empty_like(ng)

    def run():
        for i, L in enumerate(layers):
            B.sa_select_blocks(dims, kind, qs[i], L["digests"], lens, k, L["block_table"], gb,
                               ng, cb, nc, None, ws)
    run()
    ms = timed_multi(torch, B, {"select": passes * len(layers)},
                     lambda: [run() for _ in range(passes)])["select"]
    st = spread(ms)
    nbytes = select_bytes(wl, kind)
    gbs = nbytes / (st["median_us"] * 1e-6) / 1e9
    log(f"selection alone: {st['median_us']:.1f} us median (p10 {st['p10_us']:.1f}, p90 "
        f"{st['p90_us']:.1f}), {gbs:.0f} GB/s")
    return dict(st, achieved=round(gbs, 1), bytes=nbytes)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: this decode path has no multi-GPU mode; "
              "it would shard over sequences or KV heads with no exchange on the path.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from block_sparse_attention_digest_amd import binding as B
    from block_sparse_attention_digest_amd import workloads as wk
    if not os.path.exists(B.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    B.lib()
    torch.cuda.set_device(0)

    if args.leg is not None:
        name, kd = LEGS[args.leg]
        flush = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        out = layer_leg(getattr(wk, name), kd, torch, B, wk, flush)
        print(json.dumps({"leg": args.leg, **out}), flush=True)
        return

    wl = wk.QWEN3_14B_STEP
    if args.pool_blocks is not None:
        wl = wl.scaled(pool_blocks=args.pool_blocks)
    if args.block_size is not None and args.block_size != wl.block_size:
        bs0, bs1 = wl.block_size, args.block_size  # budget and pool kept in tokens
        wl = wl.scaled(block_size=bs1, top_k=wl.top_k * bs0 // bs1,
                       pool_blocks=wl.pool_blocks * bs0 // bs1)
    kind = args.digest
    if kind != "mean" and (args.offload or args.recall or args.drift_steps):
        print("--digest minmax times the GPU step (and the single-layer workloads); the "
              "offload, recall and drift studies run with mean digests", file=sys.stderr)
        sys.exit(2)
    log(f"workload {wl.name}: setup ({kind} digests)")
    dims, lens, layers, ws = setup(wl, torch, B, wk, kind)
    side_stream = torch.cuda.Stream()

    def step():
        B.sa_decode_step(dims, kind, wl.hidden, wl.top_k, wl.scale, lens, layers, ws,
                         side_stream=side_stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ref_out = layers[-1]["out_o"].clone()
    n_gpu_sums = [int(L["n_gpu"].sum()) for L in layers]
    n_cpu_sums = [int(L["n_cpu"].sum()) for L in layers]
    log("warmup done")

    # The timed region: K replays of the step captured as a HIP graph (the way a serving
    # loop runs it), each checked first to reproduce the eager result; eager steps if the
    # capture is unavailable.
    mode, graph = "eager", None
    if not args.no_graph:
        try:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                step()
            torch.cuda.synchronize()
            same = True
            for _ in range(3):
                layers[-1]["out_o"].zero_()
                graph.replay()
                torch.cuda.synchronize()
                same &= bool(torch.equal(layers[-1]["out_o"], ref_out))
            if same:
                mode = "hip-graph"
            else:
                log("graph replay differs from eager launches: timing eager steps")
                graph = None
        except Exception as e:  # noqa: BLE001
            log(f"graph capture unavailable ({e}): timing eager steps")
            graph = None
    run = graph.replay if graph is not None else step
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / args.steps
    log(f"timed {args.steps} steps ({mode}): {ms_step:.3f} ms/step (wall {wall:.3f} s)")

    # Kernel launches timed with HIP events recorded at the kernel's own start and end on
    # its stream (sa_profile_kernels; a graph cannot hold such events, and they slow the step
    # down by about a tenth, so they are taken outside the timed region):
    #  (1) inside eager steps, sharing the GPU with the other stream as in the step: every
    #      attention, selection and query-GEMM launch of those steps;
    #  (2) alone: each layer's attention and selection launched by themselves.
    L_ = wl.layers
    nprof = args.profile_steps * L_
    n_sel, n_gemm = nprof, args.profile_steps * (2 * L_ - 1)
    in_step = timed_multi(torch, B, {"attention": nprof, "select": n_sel, "gemm": n_gemm},
                          lambda: [step() for _ in range(args.profile_steps)])
    attn_ms = in_step["attention"]
    attn_avg_ms = sum(attn_ms) / len(attn_ms)
    attn_bytes_avg = sum(attention_bytes(wl, n_gpu_sums[j % wl.layers])
                         for j in range(nprof)) / nprof
    achieved = attn_bytes_avg / (attn_avg_ms * 1e-3) / 1e9
    log(f"attention in the step: {attn_avg_ms * 1e3:.1f} us avg, {achieved:.0f} GB/s")
    sbytes = select_bytes(wl, kind)
    sel_step = spread(in_step["select"])
    gemm_step = spread(in_step["gemm"])
    log(f"selection in the step: {sel_step['mean_us']:.1f} us mean (median "
        f"{sel_step['median_us']:.1f}); query GEMM in the step: "
        f"{gemm_step['median_us']:.1f} us median")

    rows = wl.batch * wl.num_q_heads
    o_iso = torch.empty((rows, wl.head_dim), dtype=torch.float32, device="cuda")
    sel_ws = B.workspace(B.sa_workspace_bytes(dims, wl.top_k))
    q_iso = torch.randn((wl.batch, wl.num_q_heads, wl.head_dim), device="cuda",
                        generator=wk.generator(wl, "bench_q", "cuda"))

    def alone():
        for L in layers:
            B.sa_sparse_decode(dims, q_iso, L["k_pool"], L["v_pool"], L["block_table"], lens,
                               L["gpu_blocks"], L["n_gpu"], wl.top_k, wl.scale, o_iso, ws=sel_ws)
    alone()
    iso_ms = timed_multi(torch, B, {"attention": 2 * wl.layers},
                         lambda: [alone() for _ in range(2)])["attention"]
    iso_avg_ms = sum(iso_ms) / len(iso_ms)
    iso_bytes_avg = sum(attention_bytes(wl, n) for n in n_gpu_sums) / wl.layers
    iso_achieved = iso_bytes_avg / (iso_avg_ms * 1e-3) / 1e9
    log(f"attention alone: {iso_avg_ms * 1e3:.1f} us avg, {iso_achieved:.0f} GB/s")
    sel_alone = select_alone(wl, dims, lens, layers, kind, torch, B)
    total_bytes = step_bytes(wl, n_gpu_sums, kind)
    log(f"attention: {attn_avg_ms * 1e3:.1f} us avg, {achieved:.0f} GB/s algorithmic")

    traffic = measured_traffic(wl, kind, "attn_bf16_kernel")
    sel_traffic = measured_traffic(wl, kind, "select_kernel")

    value = wl.batch * wl.layers / (ms_step * 1e-3)
    result = {
        "metric": "decode-attn seq-layers/s + achieved HBM GB/s (%peak), Qwen3-14B shape 64K ctx",
        "value": round(value, 1),
        "unit": "seq-layers/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": wl.layers, "batch": wl.batch,
                   "context": wl.context, "block_size": wl.block_size,
                   "budget_tokens": wl.top_k * wl.block_size, "q_heads": wl.num_q_heads,
                   "kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim, "hidden": wl.hidden,
                   "digest": kind, "resident_pool_blocks": wl.pool_blocks,
                   "launch": mode + ", two streams", "parallelism": "single-gpu"},
        "step_hbm_gbs": round(total_bytes / (ms_step * 1e-3) / 1e9, 1),
        "step_frac_of_peak": round(total_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "cpu_ratio": round(sum(n_cpu_sums) / (wl.layers * wl.batch * wl.num_kv_heads * wl.top_k), 4),
        "roofline": {"kernel": "attn_bf16_kernel (GPUATTN)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "avg_launch_us": round(attn_avg_ms * 1e3, 2),
                     "algorithmic_bytes_per_launch": int(attn_bytes_avg),
                     "measured": f"{nprof} launches in {args.profile_steps} eager steps "
                                 "after the timed region, HIP events at each kernel's start "
                                 "and end",
                     "shares_hbm_with": "the next layer's selection on the side stream, "
                                        "which streams its digests during most of the "
                                        "launch (step_hbm_gbs covers both)"},
        "roofline_isolated": {"kernel": "attn_bf16_kernel (GPUATTN), launched alone",
                              "bound": "hbm", "achieved": round(iso_achieved, 1),
                              "peak": PEAK_HBM_GBS, "unit": "GB/s",
                              "frac": round(iso_achieved / PEAK_HBM_GBS, 4),
                              "avg_launch_us": round(iso_avg_ms * 1e3, 2),
                              "time": spread(iso_ms),
                              "algorithmic_bytes_per_launch": int(iso_bytes_avg)},
        "roofline_select": {
            "kernel": "select_kernel (digest scoring + top-k + resident split), in the step",
            "bound": "hbm",
            "achieved": round(sbytes / (sel_step["mean_us"] * 1e-6) / 1e9, 1),
            "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(sbytes / (sel_step["mean_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "traffic": sel_traffic, "time": sel_step, "algorithmic_bytes_per_launch": sbytes,
            "measured": f"{n_sel} launches in {args.profile_steps} eager steps, HIP events at "
                        "each kernel's start and end; mean (in these eager steps a launch "
                        "either overlaps the attention beside it, about 80 us, or runs after "
                        "it, about 40 us, so the median jumps between the two)",
            "shares_hbm_with": "the previous layer's attention on the main stream"},
        "roofline_select_isolated": {
            "kernel": "select_kernel, launched alone (each layer's digests once per pass)",
            "bound": "hbm", "achieved": sel_alone["achieved"], "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(sel_alone["achieved"] / PEAK_HBM_GBS, 4),
            "time": {k_: v for k_, v in sel_alone.items() if k_ not in ("achieved", "bytes")},
            "algorithmic_bytes_per_launch": sbytes},
        "attention_in_step_time": spread(attn_ms),
    }
    result["gemm"] = gemm_measure(wl, layers, torch, B)
    result["gemm"]["in_step_kernel"] = gemm_step
    result["copy_ceiling"] = copy_ceiling(torch)
    log(f"copy ceiling: {result['copy_ceiling']['gbs']:.0f} GB/s")
    if args.dense:
        result["dense"] = dense_measure(wl, args, torch, B, wk, iso_avg_ms * 1e3)
    store = host_store(wl, args, B, wk) if (args.recall or args.drift_steps) else None
    if args.offload:
        result["offload"] = offload_measure(wl, dims, lens, layers, ws, side_stream, ms_step,
                                            args, torch, B, wk, store)
    if args.recall:
        rec = recall_measure(wl, dims, lens, layers, store, torch, B)
        step()  # the next step over the new residency
        torch.cuda.synchronize()
        rec["cpu_share_after"] = round(
            sum(int(L["n_cpu"].sum()) for L in layers) / (wl.layers * wl.batch * wl.num_kv_heads
                                                          * wl.top_k), 4)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        rec["gpu_only_ms_per_step_after"] = round(e0.elapsed_time(e1) / args.steps, 4)
        rec["after_launch"] = "eager"
        rec["note"] = ("one recall of every layer from the last step's lists; the inputs do "
                       "not change between steps here, so the selection does not drift and "
                       "the CPU share after the recall is what the pool's free pages allow")
        if args.offload:
            ms_after = rec["gpu_only_ms_per_step_after"]
            rec["offload_after"] = offload_measure(wl, dims, lens, layers, ws, side_stream,
                                                   ms_after, args, torch, B, wk, store)
        result["recall"] = rec
    if args.drift_steps:
        result["drift"] = drift_measure(wl, dims, lens, layers, ws, side_stream, store, args,
                                        torch, B)
    if not args.no_legs:
        # the single-layer workloads, after the step's buffers are released
        del layers, ws, store
        graph = run = None
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        flush = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        result["layer_workloads"] = [layer_leg(getattr(wk, name), kd, torch, B, wk, flush)
                                     for name, kd in LEGS.values()]
        del flush
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, kind)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
