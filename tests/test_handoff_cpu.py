"""The host half of the offload step's flag hand-off (sa_host_plan_set_handoff with
SA_HANDOFF_FLAGS), on the CPU: the test plays the GPU, advancing ready counters in a plain
int32 array and reading the done flags.  The guarantee under test: every ready value the
plan's dispatcher sees gets its done flag -- after the layer's task, and, when the plan is
switched or destroyed, for a layer raised but not yet served (with an empty partial) -- so a
GPU wait on a done flag ends as soon as the host has answered.  ScoutAttention, HTML
Sec. 3.3 (the CPU's partial of layer i is computed while the GPU works one layer ahead and
merged at layer i)."""

import time

import numpy as np
import pytest
import torch

from block_sparse_attention_digest_amd import binding as B
from test_host_worker import lib, make_problem, plan_layer, run_worker  # noqa: F401


def wait_until(pred, seconds):
    end = time.monotonic() + seconds
    while time.monotonic() < end:
        if pred():
            return True
        time.sleep(0.0005)
    return pred()


def two_layer_plan(threads=2):
    Ps = [make_problem("bf16", seed=71), make_problem("bf16", seed=72)]
    Ps[1]["lens"] = Ps[0]["lens"]
    layers = [plan_layer(P) for P in Ps]
    plan = B.HostPlan(Ps[0]["dims"], Ps[0]["top"], Ps[0]["scale"], Ps[0]["lens"], layers,
                      threads=threads)
    return Ps, layers, plan


def partial(layer):
    return tuple(layer[k].numpy().astype(np.float64) for k in ("o_host", "m_host", "l_host"))


def raise_ready(flags, layer):
    flags[layer] += 1
    return flags[layer].item()


def test_raised_layers_are_served_then_marked_done(lib):
    Ps, layers, plan = two_layer_plan()
    try:
        flags = torch.full((5,), 77, dtype=torch.int32)
        plan.set_handoff("flags", flags, gpu_wait_ms=10000)
        assert flags.tolist() == [0] * 5  # zeroed by the call
        for step in range(3):
            time.sleep(0.002)  # nothing raised: nothing may be done
            assert flags[2].item() == step and flags[3].item() == step
            for i in (0, 1):
                layers[i]["o_host"].fill_(float("nan"))
            v0 = raise_ready(flags, 0)  # the "GPU" raises layer 0
            assert wait_until(lambda: flags[2].item() == v0, 5)
            v1 = raise_ready(flags, 1)
            assert wait_until(lambda: flags[3].item() == v1, 5)
            for i in (0, 1):
                want = run_worker(Ps[i], threads=2)
                for a, b in zip(partial(layers[i]), want):
                    assert np.array_equal(a, b, equal_nan=True), (step, i)
        n, secs = plan.stats()
        assert n == 6 and flags.tolist() == [3, 3, 3, 3, 0]
    finally:
        plan.close()


def test_layers_raised_together_or_out_of_order_are_all_served(lib):
    Ps, layers, plan = two_layer_plan()
    try:
        flags = torch.zeros(5, dtype=torch.int32)
        plan.set_handoff("flags", flags, gpu_wait_ms=10000)
        raise_ready(flags, 1)  # layer 1 before layer 0
        raise_ready(flags, 0)
        assert wait_until(lambda: flags[2:4].tolist() == [1, 1], 5)
        # a layer raised twice before it is answered (the GPU gave up on the first): the
        # dispatcher answers the latest value
        flags[0] = 3
        assert wait_until(lambda: flags[2].item() == 3, 5)
        n, _ = plan.stats()
        assert n >= 3
    finally:
        plan.close()


def test_stats_waits_for_every_raised_layer(lib):
    Ps, layers, plan = two_layer_plan()
    try:
        flags = torch.zeros(5, dtype=torch.int32)
        plan.set_handoff("flags", flags, gpu_wait_ms=10000)
        for _ in range(20):
            raise_ready(flags, 0)
            raise_ready(flags, 1)
            plan.stats()  # returns only once both are answered
            assert flags[2].item() == flags[0].item() and flags[3].item() == flags[1].item()
    finally:
        plan.close()


def test_destroy_and_switch_close_raised_layers(lib):
    """A layer raised while the dispatcher is stopping is answered (served, or closed with an
    empty partial) before the call returns: no done flag is left behind."""
    for how in ("close", "switch"):
        for _ in range(5):
            Ps, layers, plan = two_layer_plan()
            flags = torch.zeros(5, dtype=torch.int32)
            try:
                plan.set_handoff("flags", flags, gpu_wait_ms=10000)
                raise_ready(flags, 0)
                raise_ready(flags, 1)
                if how == "close":
                    plan.close()
                else:
                    plan.set_handoff("host_func")
                assert flags[2].item() == 1 and flags[3].item() == 1, how
                for L in layers:  # either the task's result or the empty partial
                    o, m, l = partial(L)
                    assert not np.isnan(o).any() and not np.isnan(m).any(), how
            finally:
                plan.close()


def test_gpu_timeout_record_is_reported(lib):
    Ps, layers, plan = two_layer_plan()
    try:
        flags = torch.zeros(5, dtype=torch.int32)
        plan.set_handoff("flags", flags, gpu_wait_ms=10000)
        plan.stats()
        flags[4] = 1  # what the GPU's wait writes when it gives up
        with pytest.raises(B.SaError, match="GPU wait"):
            plan.stats()
    finally:
        plan.close()


def test_idle_dispatcher_answers_after_a_pause(lib):
    """After an idle spell (the dispatcher sleeping between polls) a raised layer is still
    answered, well within a GPU wait's bound."""
    Ps, layers, plan = two_layer_plan()
    try:
        flags = torch.zeros(5, dtype=torch.int32)
        plan.set_handoff("flags", flags, gpu_wait_ms=10000)
        time.sleep(0.05)
        t0 = time.monotonic()
        v = raise_ready(flags, 1)
        assert wait_until(lambda: flags[3].item() == v, 5)
        assert time.monotonic() - t0 < 1.0
    finally:
        plan.close()


def test_handoff_argument_checks(lib):
    Ps, layers, plan = two_layer_plan()
    try:
        h = plan.handle
        L = B.lib()
        flags = torch.zeros(5, dtype=torch.int32)
        p = flags.data_ptr()
        assert L.sa_host_plan_set_handoff(h, 1, None, 10) == B.SA_ERR_INVALID_ARG
        assert L.sa_host_plan_set_handoff(h, 1, p, 0) == B.SA_ERR_INVALID_ARG
        assert L.sa_host_plan_set_handoff(h, 1, p + 2, 10) == B.SA_ERR_INVALID_ARG
        assert L.sa_host_plan_set_handoff(h, 7, p, 10) == B.SA_ERR_INVALID_ARG
        assert L.sa_host_plan_set_handoff(None, 1, p, 10) == B.SA_ERR_INVALID_ARG
        assert L.sa_stream_wait(None, p, 10, p, None) == B.SA_ERR_INVALID_ARG
        assert L.sa_stream_wait(p, p, 0, p, None) == B.SA_ERR_INVALID_ARG
        assert L.sa_stream_wait(p, p + 2, 10, p, None) == B.SA_ERR_INVALID_ARG
        assert L.sa_stream_signal(None, None) == B.SA_ERR_INVALID_ARG
        assert L.sa_stream_signal(p + 1, None) == B.SA_ERR_INVALID_ARG
    finally:
        plan.close()
