"""The C-ABI library without a GPU: it loads, exports every symbol the header declares,
and rejects bad arguments on the host before launching anything."""

import ctypes
import os
import re

import pytest
import torch

from block_sparse_attention_digest_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "scoutattn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from block_sparse_attention_digest_amd import build
        build.build()
    return B.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_path(lib):
    names = declared_functions()
    for n in ("sa_pack_k_pages", "sa_pack_v_pages", "sa_pack_weight", "sa_build_digests",
              "sa_predict_query",
              "sa_select_blocks", "sa_sparse_decode", "sa_merge", "sa_decode_attend_merge",
              "sa_decode_step", "sa_host_partial_attention", "sa_refresh_last_digests",
              "sa_host_plan_create", "sa_host_plan_destroy", "sa_host_plan_stats",
              "sa_host_plan_run", "sa_recall_blocks", "sa_recall_workspace_bytes",
              "sa_dense_decode", "sa_dense_workspace_bytes",
              "sa_decode_step_offload", "sa_host_plan_set_recall"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(declared_functions()) <= set(B.SIGNATURES)


def test_abi_version(lib):
    assert lib.sa_abi_version() == B.ABI_VERSION == 12
    assert lib.sa_status_string(B.SA_ERR_WORKSPACE) == b"SA_ERR_WORKSPACE"


def test_workspace_holds_the_selection_handover(lib):
    """With several chunk workgroups per pair, the workspace starts with the selection's
    hand-over buffers: a score and a table entry per (pair, block), and a counter per pair."""
    big = dims(batch=40, num_q_heads=40, num_kv_heads=8, max_blocks=2048, num_pages=40960)
    pairs = 40 * 8
    assert lib.sa_workspace_bytes(ctypes.byref(big), 64) >= pairs * (2 * 2048 + 1) * 4
    # one chunk per pair (a tiny shape): no hand-over region beyond the attention partials
    tiny = dims(batch=1, num_q_heads=4, num_kv_heads=1, max_blocks=8, num_pages=8)
    assert lib.sa_workspace_bytes(ctypes.byref(tiny), 4) < 64 * 1024


def test_profile_hook_validation(lib):
    assert lib.sa_profile_kernels(7, None, None, 0) == B.SA_ERR_INVALID_ARG
    assert lib.sa_profile_kernels(1, None, None, -1) == B.SA_ERR_INVALID_ARG
    assert lib.sa_profile_kernels(2, None, None, 3) == B.SA_ERR_INVALID_ARG
    for stage in range(3):
        assert lib.sa_profile_kernels(stage, None, None, 0) == B.SA_OK


# The calls below must all fail validation; on a machine with a GPU they are skipped so
# that a validation bug can never launch a kernel on dummy pointers.
no_gpu = pytest.mark.skipif(torch.cuda.is_available(), reason="host-only checks (no GPU)")
FAKE = 0x1000


def dims(**kw):
    base = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=32,
                max_blocks=64, num_pages=128, kv_dtype=B.SA_BF16)
    base.update(kw)
    return B.sa_dims(**base)


def select(lib, d, top_k=8, ws_bytes=1 << 30, q=FAKE, kind=0):
    return lib.sa_select_blocks(ctypes.byref(d), kind, q, FAKE, FAKE, top_k, FAKE, FAKE, FAKE,
                                FAKE, FAKE, None, FAKE, ws_bytes, None)


@no_gpu
def test_noalloc_refuses_partials_beyond_scratch(lib):
    """8192 pairs of 8 query heads need about 42 MB of attention partials, more than the
    16 MiB of per-GPU scratch of sa_decode_attend_merge_noalloc: refused on the host."""
    d = dims(batch=1024, num_q_heads=64, num_kv_heads=8, max_blocks=64, num_pages=1024)
    st = lib.sa_decode_attend_merge_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE,
                                            FAKE, FAKE, 8, 0.1, FAKE, FAKE, FAKE, FAKE, FAKE,
                                            None, None, None)
    assert st == B.SA_ERR_WORKSPACE
    assert b"scratch" in lib.sa_last_error()
    assert lib.sa_decode_attend_merge_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE,
                                              FAKE, FAKE, 8, 0.1, None, FAKE, FAKE, FAKE,
                                              FAKE, None, None, None) == B.SA_ERR_INVALID_ARG


@no_gpu
def test_dims_validation(lib):
    assert select(lib, dims(head_dim=96)) == B.SA_ERR_UNSUPPORTED
    assert b"head_dim" in lib.sa_last_error()
    assert select(lib, dims(block_size=8)) == B.SA_ERR_UNSUPPORTED
    assert select(lib, dims(num_q_heads=7)) == B.SA_ERR_INVALID_ARG
    assert select(lib, dims(num_q_heads=18, num_kv_heads=2)) == B.SA_ERR_UNSUPPORTED  # G = 9
    assert select(lib, dims(kv_dtype=7)) == B.SA_ERR_UNSUPPORTED
    assert select(lib, dims(batch=0)) == B.SA_ERR_INVALID_ARG
    assert select(lib, dims(max_blocks=9000)) == B.SA_ERR_UNSUPPORTED
    assert lib.sa_select_blocks(None, 0, FAKE, FAKE, FAKE, 8, FAKE, FAKE, FAKE, FAKE, FAKE,
                                None, FAKE, 1 << 30, None) == B.SA_ERR_INVALID_ARG


@no_gpu
def test_select_validation(lib):
    d = dims()
    assert select(lib, d, q=None) == B.SA_ERR_INVALID_ARG
    assert b"q is NULL" in lib.sa_last_error()
    assert select(lib, d, top_k=0) == B.SA_ERR_INVALID_ARG
    assert select(lib, d, top_k=65) == B.SA_ERR_INVALID_ARG
    assert select(lib, d, kind=5) == B.SA_ERR_INVALID_ARG
    need = lib.sa_workspace_bytes(ctypes.byref(d), 8)
    assert need > 0
    assert select(lib, d, ws_bytes=need - 1) == B.SA_ERR_WORKSPACE
    assert lib.sa_workspace_bytes(ctypes.byref(dims(head_dim=96)), 8) == 0


@no_gpu
def test_decode_and_merge_validation(lib):
    d = dims()
    ws = lib.sa_workspace_bytes(ctypes.byref(d), 8)
    args = [ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 0.088, FAKE, FAKE,
            FAKE, FAKE, ws, None]
    bad_scale = list(args)
    bad_scale[9] = float("nan")
    assert lib.sa_sparse_decode(*bad_scale) == B.SA_ERR_INVALID_ARG
    bad_scale[9] = 0.0
    assert lib.sa_sparse_decode(*bad_scale) == B.SA_ERR_INVALID_ARG
    bad = list(args)
    bad[8] = 65
    assert lib.sa_sparse_decode(*bad) == B.SA_ERR_INVALID_ARG
    bad = list(args)
    bad[14] = ws - 1
    assert lib.sa_sparse_decode(*bad) == B.SA_ERR_WORKSPACE
    bad = list(args)
    bad[10] = None  # o
    assert lib.sa_sparse_decode(*bad) == B.SA_ERR_INVALID_ARG
    assert lib.sa_decode_attend_merge(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      8, 0.088, None, FAKE, FAKE, None, FAKE, None, None, FAKE,
                                      ws, None) == B.SA_ERR_INVALID_ARG
    assert lib.sa_merge(0, 128, *([FAKE] * 9), None) == B.SA_ERR_INVALID_ARG
    assert lib.sa_merge(4, 2000, *([FAKE] * 9), None) == B.SA_ERR_INVALID_ARG
    assert lib.sa_merge(4, 128, FAKE, None, *([FAKE] * 7), None) == B.SA_ERR_INVALID_ARG


@no_gpu
def test_gemm_validation(lib):
    assert lib.sa_predict_query(0, 64, 64, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == B.SA_ERR_INVALID_ARG
    assert lib.sa_predict_query(300, 64, 64, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == B.SA_ERR_UNSUPPORTED
    assert lib.sa_predict_query(8, 100, 64, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == B.SA_ERR_UNSUPPORTED
    assert lib.sa_predict_query(8, 64, 96, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == B.SA_ERR_UNSUPPORTED
    assert lib.sa_predict_query(8, 64, 64, None, FAKE, FAKE, FAKE, 1 << 30, None) == B.SA_ERR_INVALID_ARG
    need = lib.sa_predict_query_workspace_bytes(40, 5120, 5120)
    assert need > 0
    assert lib.sa_predict_query(40, 5120, 5120, FAKE, FAKE, FAKE, FAKE, need - 1,
                                None) == B.SA_ERR_WORKSPACE
    assert lib.sa_predict_query_workspace_bytes(40, 100, 5120) == 0


@no_gpu
def test_gemm_split_plan(lib):
    """The GEMM's k-split, seen through its workspace (ksplit float32 partials of m x n): the
    fewest equal slices (a divisor of k / 64, at most 16) that give about one workgroup per
    CU, with 5 column tiles of 16 a workgroup where they divide the tiles, else 4."""
    def ws(m, n, k):
        return lib.sa_predict_query_workspace_bytes(m, n, k)
    # 320 tiles -> 64 groups of 5: 4 slices fill 256 CUs
    assert ws(40, 5120, 5120) == 4 * 40 * 5120 * 4
    # 64 rows still one row group of 64
    assert ws(64, 5120, 5120) == 4 * 64 * 5120 * 4
    # 256 tiles -> 64 groups of 4
    assert ws(8, 4096, 4096) == 4 * 8 * 4096 * 4
    # 40 tiles -> 8 groups of 5, 4 row groups of 64: 8 slices
    assert ws(256, 640, 2560) == 8 * 256 * 640 * 4
    # 12 tiles -> 3 groups of 4: 16 slices at most (k / 64 = 128 has the divisor 16)
    assert ws(17, 192, 8192) == 16 * 17 * 192 * 4
    # k / 64 = 5: the divisors are 1 and 5
    assert ws(3, 960, 320) == 5 * 3 * 960 * 4
    # 1024 tiles -> 256 groups of 4: one slice, no partials
    assert ws(8, 16384, 4096) == 0
    # k / 64 = 1: nothing to split
    assert ws(1, 64, 64) == 0


@no_gpu
def test_alignment_validation(lib):
    """Buffers the kernels move with 16-byte accesses are refused on the host when they are
    not 16-byte aligned (the rest of each call's arguments valid)."""
    d = dims()
    odd = FAKE + 8

    def refused(status, name):
        assert status == B.SA_ERR_INVALID_ARG, name
        assert b"16-byte aligned" in lib.sa_last_error(), name

    need = lib.sa_predict_query_workspace_bytes(40, 5120, 5120)
    refused(lib.sa_predict_query(40, 5120, 5120, odd, FAKE, FAKE, FAKE, need, None), "x")
    refused(lib.sa_predict_query(40, 5120, 5120, FAKE, odd, FAKE, FAKE, need, None), "w_packed")
    refused(lib.sa_predict_query(40, 5120, 5120, FAKE, FAKE, odd, FAKE, need, None), "q")
    refused(lib.sa_predict_query(40, 5120, 5120, FAKE, FAKE, FAKE, odd, need, None), "ws")
    refused(lib.sa_pack_weight(64, 64, odd, FAKE + 65536, None), "w")
    refused(lib.sa_pack_k_pages(ctypes.byref(d), odd, FAKE + (1 << 30), None), "k_rows")
    refused(lib.sa_pack_v_pages(ctypes.byref(d), FAKE, FAKE + (1 << 30) + 8, None), "v_pool")
    refused(lib.sa_build_digests(ctypes.byref(d), 0, odd, FAKE, FAKE, FAKE, None), "k_pool")
    refused(lib.sa_build_digests(ctypes.byref(d), 0, FAKE, FAKE, FAKE, odd, None), "digests")
    assert select(lib, d, q=odd) == B.SA_ERR_INVALID_ARG
    assert b"16-byte aligned" in lib.sa_last_error()
    ws = lib.sa_workspace_bytes(ctypes.byref(d), 8)
    args = [ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 0.088, FAKE, FAKE,
            FAKE, FAKE, ws, None]
    for i, name in ((1, "q"), (2, "k_pool"), (3, "v_pool"), (13, "ws")):
        bad = list(args)
        bad[i] = odd
        refused(lib.sa_sparse_decode(*bad), name)
    dw = lib.sa_dense_workspace_bytes(ctypes.byref(d))
    refused(lib.sa_dense_decode(ctypes.byref(d), FAKE, odd, FAKE, FAKE, FAKE, 0.088, FAKE, None,
                                None, FAKE, dw, None), "dense k_pool")
    # the same buffers at aligned addresses pass these checks (and fail later, on the size)
    assert lib.sa_predict_query(40, 5120, 5120, FAKE, FAKE, FAKE, FAKE, need - 1,
                                None) == B.SA_ERR_WORKSPACE


@no_gpu
def test_pack_validation(lib):
    d = dims()
    nbytes = 128 * 32 * 128 * 2
    assert lib.sa_pack_k_pages(ctypes.byref(d), None, FAKE, None) == B.SA_ERR_INVALID_ARG
    assert lib.sa_pack_k_pages(ctypes.byref(d), FAKE, None, None) == B.SA_ERR_INVALID_ARG
    # in-place or overlapping conversion is refused
    assert lib.sa_pack_k_pages(ctypes.byref(d), FAKE, FAKE, None) == B.SA_ERR_INVALID_ARG
    assert lib.sa_pack_k_pages(ctypes.byref(d), FAKE, FAKE + nbytes - 16, None) == B.SA_ERR_INVALID_ARG
    assert lib.sa_pack_k_pages(ctypes.byref(dims(head_dim=96)), FAKE, FAKE + nbytes,
                               None) == B.SA_ERR_UNSUPPORTED
    assert lib.sa_pack_v_pages(ctypes.byref(d), None, FAKE, None) == B.SA_ERR_INVALID_ARG
    assert lib.sa_pack_v_pages(ctypes.byref(d), FAKE, None, None) == B.SA_ERR_INVALID_ARG
    assert lib.sa_pack_v_pages(ctypes.byref(d), FAKE, FAKE + nbytes - 2, None) == B.SA_ERR_INVALID_ARG
    assert lib.sa_pack_v_pages(ctypes.byref(dims(head_dim=96)), FAKE, FAKE + nbytes,
                               None) == B.SA_ERR_UNSUPPORTED
    assert lib.sa_pack_weight(16, 64, FAKE, FAKE + 4096, None) == B.SA_ERR_INVALID_ARG
    assert lib.sa_pack_weight(40, 64, FAKE, FAKE + 8192, None) == B.SA_ERR_UNSUPPORTED
    assert lib.sa_pack_weight(64, 48, FAKE, FAKE + 8192, None) == B.SA_ERR_UNSUPPORTED
    assert lib.sa_pack_weight(64, 64, FAKE, FAKE + 100, None) == B.SA_ERR_INVALID_ARG
    assert lib.sa_pack_weight(64, 64, None, FAKE, None) == B.SA_ERR_INVALID_ARG


@no_gpu
def test_step_validation(lib):
    d = dims()
    ws = lib.sa_step_workspace_bytes(ctypes.byref(d), 1024, 8)
    assert ws > 0
    layers = (B.sa_layer * 2)()
    for L in layers:
        for name, _ in B.sa_layer._fields_:
            setattr(L, name, FAKE)
    layers[1].out_o = None
    assert lib.sa_decode_step(ctypes.byref(d), 0, 1024, 8, 0.088, FAKE, 2, layers, FAKE, ws,
                              None, None) == B.SA_ERR_INVALID_ARG
    assert b"layer 1" in lib.sa_last_error()
    layers[1].out_o = FAKE
    layers[0].n_cpu_host = None
    assert lib.sa_decode_step(ctypes.byref(d), 0, 1024, 8, 0.088, FAKE, 2, layers, FAKE, ws,
                              None, None) == B.SA_ERR_INVALID_ARG
    layers[0].n_cpu_host = FAKE
    assert lib.sa_decode_step(ctypes.byref(d), 0, 1000, 8, 0.088, FAKE, 2, layers, FAKE, ws,
                              None, None) == B.SA_ERR_UNSUPPORTED
    assert lib.sa_decode_step(ctypes.byref(d), 0, 1024, 8, 0.088, FAKE, 0, layers, FAKE, ws,
                              None, None) == B.SA_ERR_INVALID_ARG
    assert lib.sa_decode_step(ctypes.byref(d), 0, 1024, 8, 0.088, FAKE, 2, layers, FAKE,
                              ws - 1, None, None) == B.SA_ERR_WORKSPACE


def host_layers(n):
    arr = (B.sa_host_layer * n)()
    for L in arr:
        for name, _ in B.sa_host_layer._fields_:
            setattr(L, name, 4 if name == "host_pages" else FAKE)
    return arr


def test_host_plan_lifecycle(lib):
    """Creating a plan starts its workers and touches no device; nothing runs until a step
    enqueues its tasks, so the fake pointers are never read."""
    d = dims()
    plan = ctypes.c_void_p()
    assert lib.sa_host_plan_create(ctypes.byref(d), 8, 0.088, FAKE, 3, host_layers(3), 4,
                                   ctypes.byref(plan)) == B.SA_OK
    assert plan.value
    n, t = ctypes.c_int64(-1), ctypes.c_double(-1.0)
    assert lib.sa_host_plan_stats(plan, ctypes.byref(n), ctypes.byref(t)) == B.SA_OK
    assert n.value == 0 and t.value == 0.0
    assert lib.sa_host_plan_destroy(plan) == B.SA_OK
    assert lib.sa_host_plan_destroy(None) == B.SA_OK  # like free(NULL)


def test_host_plan_rejects_bad_arguments(lib):
    d = dims()
    plan = ctypes.c_void_p(FAKE)

    def create(top_k=8, scale=0.088, lens=FAKE, n=2, layers=None, threads=0, out=True):
        layers = host_layers(max(n, 1)) if layers is None else layers
        return lib.sa_host_plan_create(ctypes.byref(d), top_k, scale, lens, n, layers, threads,
                                       ctypes.byref(plan) if out else None)

    assert create(top_k=0) == B.SA_ERR_INVALID_ARG and plan.value is None
    assert create(top_k=65) == B.SA_ERR_INVALID_ARG
    assert create(scale=0.0) == B.SA_ERR_INVALID_ARG
    assert create(lens=None) == B.SA_ERR_INVALID_ARG
    assert create(n=0) == B.SA_ERR_INVALID_ARG
    assert create(threads=-1) == B.SA_ERR_INVALID_ARG
    assert create(out=False) == B.SA_ERR_INVALID_ARG
    bad = host_layers(2)
    bad[1].host_pages = 0
    assert create(layers=bad) == B.SA_ERR_INVALID_ARG and b"host layer 1" in lib.sa_last_error()
    bad = host_layers(2)
    bad[0].o_host = None
    assert create(layers=bad) == B.SA_ERR_INVALID_ARG and b"host layer 0" in lib.sa_last_error()


@no_gpu
def test_offload_step_validation(lib):
    """The plan must match the step's dims, top_k, scale and layer count, and host_stream
    must be a stream of its own; all checked before anything is enqueued."""
    d = dims()
    plan = ctypes.c_void_p()
    assert lib.sa_host_plan_create(ctypes.byref(d), 8, 0.088, FAKE, 2, host_layers(2), 2,
                                   ctypes.byref(plan)) == B.SA_OK
    try:
        ws = lib.sa_step_workspace_bytes(ctypes.byref(d), 1024, 8)
        layers = (B.sa_layer * 2)()
        for L in layers:
            for name, _ in B.sa_layer._fields_:
                setattr(L, name, FAKE)
            L.host_o = L.host_m = L.host_l = L.cpu_blocks_host = L.n_cpu_host = None

        def step(dd=d, top_k=8, scale=0.088, n=2, p=plan, host=FAKE + 3, side=FAKE + 2,
                 rec=None):
            return lib.sa_decode_step_offload(ctypes.byref(dd), 0, 1024, top_k, scale, FAKE, n,
                                              layers, FAKE, ws, FAKE + 1, side, p, host, rec)

        assert step(p=None) == B.SA_ERR_INVALID_ARG
        assert step(dd=dims(batch=3)) == B.SA_ERR_INVALID_ARG
        assert b"other dims" in lib.sa_last_error()
        assert step(top_k=4) == B.SA_ERR_INVALID_ARG
        assert step(scale=0.1) == B.SA_ERR_INVALID_ARG
        assert step(n=1) == B.SA_ERR_INVALID_ARG
        assert step(host=None) == B.SA_ERR_INVALID_ARG
        assert step(host=FAKE + 1) == B.SA_ERR_INVALID_ARG  # the main stream
        assert step(host=FAKE + 2) == B.SA_ERR_INVALID_ARG  # the side stream
        assert b"stream of its own" in lib.sa_last_error()
        # with recall set, a recall stream of its own is required
        rl = (B.sa_recall_layer * 2)()
        for r in rl:
            r.host_table_dev, r.n_recalled = FAKE, FAKE
        rws = lib.sa_recall_workspace_bytes(ctypes.byref(d), 8)
        assert lib.sa_host_plan_set_recall(plan, 8, 0.12, rl, FAKE, rws - 1, 0) == B.SA_ERR_WORKSPACE
        assert lib.sa_host_plan_set_recall(plan, 0, 0.12, rl, FAKE, rws, 0) == B.SA_ERR_INVALID_ARG
        assert lib.sa_host_plan_set_recall(plan, 8, -1.0, rl, FAKE, rws, 0) == B.SA_ERR_INVALID_ARG
        rl[1].n_recalled = None
        assert lib.sa_host_plan_set_recall(plan, 8, 0.12, rl, FAKE, rws, 0) == B.SA_ERR_INVALID_ARG
        rl[1].n_recalled = FAKE
        assert lib.sa_host_plan_set_recall(plan, 8, 0.12, rl, FAKE, rws, 0) == B.SA_OK
        assert step(rec=None) == B.SA_ERR_INVALID_ARG
        assert step(rec=FAKE + 3) == B.SA_ERR_INVALID_ARG  # the host stream
        assert b"recall_stream" in lib.sa_last_error()
        assert lib.sa_host_plan_set_recall(plan, 0, 0.0, None, None, 0, 0) == B.SA_OK  # off
        # without a plan the same layers lack their host partials
        assert lib.sa_decode_step(ctypes.byref(d), 0, 1024, 8, 0.088, FAKE, 2, layers, FAKE,
                                  ws, None, None) == B.SA_ERR_INVALID_ARG
    finally:
        assert lib.sa_host_plan_destroy(plan) == B.SA_OK


@no_gpu
def test_recall_validation(lib):
    d = dims()
    ws = lib.sa_recall_workspace_bytes(ctypes.byref(d), 8)
    assert ws >= 2 * 2 * 8 * 4
    assert lib.sa_recall_workspace_bytes(ctypes.byref(d), 0) == 0
    assert lib.sa_recall_workspace_bytes(ctypes.byref(d), 5000) == 0

    def call(stride=8, maxr=8, hp=16, ws_=ws, **null):
        args = dict(seq_lens=FAKE, block_table=FAKE, gpu_blocks=FAKE, n_gpu=FAKE,
                    cpu_blocks=FAKE, n_cpu=FAKE, k_host=FAKE, v_host=FAKE, host_table=FAKE,
                    k_pool=FAKE, v_pool=FAKE, n_recalled=FAKE)
        args.update(null)
        a = args
        return lib.sa_recall_blocks(ctypes.byref(d), stride, maxr, a["seq_lens"],
                                    a["block_table"], a["gpu_blocks"], a["n_gpu"],
                                    a["cpu_blocks"], a["n_cpu"], a["k_host"], a["v_host"],
                                    a["host_table"], hp, a["k_pool"], a["v_pool"],
                                    a["n_recalled"], FAKE, ws_, None)

    assert call(stride=0) == B.SA_ERR_INVALID_ARG
    assert call(stride=65) == B.SA_ERR_INVALID_ARG
    assert call(maxr=0) == B.SA_ERR_INVALID_ARG
    assert call(hp=0) == B.SA_ERR_INVALID_ARG
    assert call(ws_=ws - 1) == B.SA_ERR_WORKSPACE
    for name in ("seq_lens", "block_table", "cpu_blocks", "k_host", "host_table", "v_pool",
                 "n_recalled"):
        assert call(**{name: None}) == B.SA_ERR_INVALID_ARG, name


def test_binding_requires_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        B.lib()
