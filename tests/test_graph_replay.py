"""HIP graphs of the decode step.

The step, and the step with its CPU side as host tasks, are each captured once and replayed
several times.  Between replays the outputs are poisoned and an eager step runs.  Every
replay and every eager step must reproduce the first eager result bit for bit: the same
kernels and the same host tasks run on the same inputs.
"""

import pytest
import torch

import harness as H
import harness_step as HS
from block_sparse_attention_digest_amd import binding as B
from block_sparse_attention_digest_amd import workloads as wk

pytestmark = pytest.mark.gpu

WL = wk.QWEN3_14B_STEP.scaled(batch=3, num_q_heads=10, num_kv_heads=2, context=2000, layers=4,
                              pool_blocks=6, hidden=512, top_k=8)


@pytest.fixture(scope="module", autouse=True)
def gpu_lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def snapshot(layers, host_layers):
    out = []
    for L in layers:
        out += [L[n].clone() for n in ("out_o", "out_m", "out_l", "gpu_blocks", "n_gpu",
                                       "cpu_blocks", "n_cpu")]
    for h in host_layers or []:
        out += [h[n].clone() for n in ("q_host", "o_host", "m_host", "l_host", "n_cpu_host",
                                       "cpu_blocks_host")]
    return out


def poison(layers, host_layers):
    for L in layers:
        for n in ("out_o", "out_m", "out_l"):
            L[n].fill_(float("nan"))
        for n in ("gpu_blocks", "n_gpu", "cpu_blocks", "n_cpu"):
            L[n].fill_(-7)
    for h in host_layers or []:
        for n in ("q_host", "o_host", "m_host", "l_host"):
            h[n].fill_(float("nan"))


def same(a, b):
    """Bit for bit, NaN matching NaN (query rows of pairs with nothing offloaded are not
    handed over, so they keep the poison)."""
    def eq(x, y):
        if x.is_floating_point():
            return x.shape == y.shape and torch.equal(x.isnan(), y.isnan()) and \
                torch.equal(x.nan_to_num(0.0).view(torch.int32), y.nan_to_num(0.0).view(torch.int32))
        return torch.equal(x, y)
    return all(eq(x, y) for x, y in zip(a, b)) and len(a) == len(b)


@pytest.mark.parametrize("offload,recall,flags",
                         [(False, False, False), (True, False, False), (True, True, False),
                          (True, False, True)],
                         ids=["step", "step-with-host-tasks", "step-with-host-tasks-and-recall",
                              "step-with-flag-handoff"])
def test_step_graph_replays_match_eager(offload, recall, flags):
    """With recall (beta 0), the first eager step recalls every offloaded selected block it
    can, and the state is then stable: later steps find nothing due, on the device, inside
    the graph as well.  With the flag hand-off, every replay advances each layer's counter
    once and the plan's dispatcher serves it."""
    H.log(f"[case] graph replay, offload={offload} recall={recall} flags={flags}")
    data = HS.prepare_step(WL, "cpu")
    lens = wk.seq_lens(WL)
    lens_d = lens.to("cuda")
    dims = H.dims_for(WL, data[0]["pool"]["K"].shape[0])
    layers = HS.device_layers(WL, data, dims, lens_d, "mean", handoff=not offload)
    ws = B.workspace(B.sa_step_workspace_bytes(dims, WL.hidden, WL.top_k))
    side = torch.cuda.Stream()
    host_layers = plan = None
    recall_stream = None
    if offload:
        stores, host_layers = HS.host_side(WL, data)
        if recall:  # the recall reads the host store from the device: page-locked
            for h in host_layers:
                for n in ("k_host", "v_host"):
                    pinned = B.pinned_empty(tuple(h[n].shape), h[n].dtype)
                    pinned.copy_(h[n])
                    h[n] = pinned
        plan = B.HostPlan(dims, WL.top_k, WL.scale, lens.clone(), host_layers, threads=3)
        host_stream = torch.cuda.Stream()
        if flags:
            plan.set_handoff("flags", gpu_wait_ms=30000)
            host_stream = None
        if recall:
            pairs = WL.batch * WL.num_kv_heads
            plan.set_recall(dims, 64, 0.0, [
                dict(host_table_dev=st["table"].to("cuda"),
                     n_recalled=torch.zeros(pairs, dtype=torch.int32, device="cuda"))
                for st in stores])
            recall_stream = torch.cuda.Stream()

    def step():
        if offload:
            B.sa_decode_step_offload(dims, "mean", WL.hidden, WL.top_k, WL.scale, lens_d, layers,
                                     ws, plan, host_stream, side_stream=side,
                                     recall_stream=recall_stream)
        else:
            B.sa_decode_step(dims, "mean", WL.hidden, WL.top_k, WL.scale, lens_d, layers, ws,
                             side_stream=side)

    try:
        step()
        torch.cuda.synchronize()
        if recall:  # the first step recalled; from here on the state is stable
            moved = sum(int(L["n_cpu"].sum()) for L in layers)
            step()
            torch.cuda.synchronize()
            assert sum(int(L["n_cpu"].sum()) for L in layers) < moved
        ref = snapshot(layers, host_layers)
        if recall:
            ref += [L["block_table"].clone() for L in layers]
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        for rep in range(3):
            poison(layers, host_layers)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            got = snapshot(layers, host_layers)
            if recall:
                got += [L["block_table"].clone() for L in layers]
            assert same(got, ref), f"replay {rep}"
            poison(layers, host_layers)
            step()  # eager work between the replays
            torch.cuda.synchronize()
            got = snapshot(layers, host_layers)
            if recall:
                got += [L["block_table"].clone() for L in layers]
            assert same(got, ref), f"eager step after replay {rep}"
        del graph
        torch.cuda.synchronize()
        if offload:
            tasks, _ = plan.stats()
            # the capture enqueues no task; each eager step and each replay runs one per layer
            assert tasks == WL.layers * (8 if recall else 7), tasks
            if flags:  # ready and done of every layer: 7 steps, no GPU timeout
                fl = plan.flags.view(torch.int32).tolist()
                assert fl == [7] * (2 * WL.layers) + [0], fl
    finally:
        if plan is not None:
            torch.cuda.synchronize()
            plan.close()
