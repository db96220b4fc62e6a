"""ctypes binding of libscoutattn.so (C ABI in include/scoutattn.h).

Argument marshalling only: every function takes torch tensors (device memory), checks
their dtype / device / size against what the C call will read or write, and passes raw
pointers and the current HIP stream.  All computation happens in the library's kernels.
A failing call raises SaError with the library's message.  The library is loaded on first
use; if it has not been built, that is an error (there is no fallback).
"""

from __future__ import annotations

import ctypes
import weakref
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libscoutattn.so")

SA_OK, SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED, SA_ERR_WORKSPACE, SA_ERR_HIP = 0, -1, -2, -3, -4
SA_F32, SA_BF16 = 0, 1
SA_DIGEST_MEAN, SA_DIGEST_MINMAX = 0, 1
ABI_VERSION = 12

KIND = {"mean": SA_DIGEST_MEAN, "minmax": SA_DIGEST_MINMAX}


class SaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{status}: {msg}")
        self.status = status


class sa_dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("kv_dtype", ctypes.c_int32)]


class sa_layer(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "x", "w_q", "digests", "block_table", "k_pool", "v_pool", "host_o", "host_m", "host_l",
        "gpu_blocks", "n_gpu", "cpu_blocks", "n_cpu", "cpu_blocks_host", "n_cpu_host",
        "out_o", "out_m", "out_l")]


class sa_host_layer(ctypes.Structure):
    _fields_ = [("k_host", ctypes.c_void_p), ("v_host", ctypes.c_void_p),
                ("host_table", ctypes.c_void_p), ("host_pages", ctypes.c_int32)] + [
        (n, ctypes.c_void_p) for n in ("q_host", "cpu_blocks_host", "n_cpu_host", "o_host",
                                       "m_host", "l_host")]


class sa_recall_layer(ctypes.Structure):
    _fields_ = [("host_table_dev", ctypes.c_void_p), ("n_recalled", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float
_Z = ctypes.c_size_t
_D = ctypes.POINTER(sa_dims)

SIGNATURES = {
    "sa_abi_version": (ctypes.c_int, []),
    "sa_last_error": (ctypes.c_char_p, []),
    "sa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "sa_pack_k_pages": (ctypes.c_int, [_D, _P, _P, _P]),
    "sa_pack_v_pages": (ctypes.c_int, [_D, _P, _P, _P]),
    "sa_pack_weight": (ctypes.c_int, [_I, _I, _P, _P, _P]),
    "sa_build_digests": (ctypes.c_int, [_D, ctypes.c_int, _P, _P, _P, _P, _P]),
    "sa_refresh_last_digests": (ctypes.c_int, [_D, ctypes.c_int, _P, _P, _P, _P, _P]),
    "sa_predict_query_workspace_bytes": (_Z, [_I, _I, _I]),
    "sa_predict_query": (ctypes.c_int, [_I, _I, _I, _P, _P, _P, _P, _Z, _P]),
    "sa_workspace_bytes": (_Z, [_D, _I]),
    "sa_select_blocks": (ctypes.c_int, [_D, ctypes.c_int, _P, _P, _P, _I, _P, _P, _P, _P, _P,
                                        _P, _P, _Z, _P]),
    "sa_sparse_decode": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _P, _P, _I, _F, _P, _P, _P,
                                        _P, _Z, _P]),
    "sa_merge": (ctypes.c_int, [_I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "sa_decode_attend_merge": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _P, _P, _I, _F, _P, _P,
                                              _P, _P, _P, _P, _P, _P, _Z, _P]),
    "sa_decode_attend_merge_noalloc": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _P, _P, _I, _F,
                                                      _P, _P, _P, _P, _P, _P, _P, _P]),
    "sa_step_workspace_bytes": (_Z, [_D, _I, _I]),
    "sa_decode_step": (ctypes.c_int, [_D, ctypes.c_int, _I, _I, _F, _P, _I,
                                      ctypes.POINTER(sa_layer), _P, _Z, _P, _P]),
    "sa_profile_attention": (ctypes.c_int, [ctypes.POINTER(_P), ctypes.POINTER(_P), _I]),
    "sa_profile_kernels": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(_P), ctypes.POINTER(_P),
                                          _I]),
    "sa_dense_workspace_bytes": (_Z, [_D]),
    "sa_dense_decode": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _F, _P, _P, _P, _P, _Z, _P]),
    "sa_recall_workspace_bytes": (_Z, [_D, _I]),
    "sa_recall_blocks": (ctypes.c_int, [_D, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P,
                                        _P, _P, _P, _Z, _P]),
    "sa_host_plan_create": (ctypes.c_int, [_D, _I, _F, _P, _I, ctypes.POINTER(sa_host_layer), _I,
                                           ctypes.POINTER(_P)]),
    "sa_host_plan_destroy": (ctypes.c_int, [_P]),
    "sa_host_plan_run": (ctypes.c_int, [_P, _I]),
    "sa_host_plan_stats": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_int64),
                                          ctypes.POINTER(ctypes.c_double)]),
    "sa_decode_step_offload": (ctypes.c_int, [_D, ctypes.c_int, _I, _I, _F, _P, _I,
                                              ctypes.POINTER(sa_layer), _P, _Z, _P, _P, _P, _P,
                                              _P]),
    "sa_host_plan_set_recall": (ctypes.c_int, [_P, _I, _F, ctypes.POINTER(sa_recall_layer), _P,
                                               _Z, _I]),
    "sa_host_partial_attention": (ctypes.c_int, [_D, _I, _P, _P, _P, _P, _P, _P, _P, _I, _F,
                                                 _P, _P, _P, _I]),
    "sa_host_plan_set_handoff": (ctypes.c_int, [_P, ctypes.c_int, _P, _I]),
    "sa_stream_signal": (ctypes.c_int, [_P, _P]),
    "sa_stream_wait": (ctypes.c_int, [_P, _P, _I, _P, _P]),
}

HANDOFF = {"host_func": 0, "flags": 1}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_sparse_attention_digest_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        if h.sa_abi_version() != ABI_VERSION:
            raise RuntimeError(f"libscoutattn ABI {h.sa_abi_version()} != {ABI_VERSION}")
        _lib = h
    return _lib


def _check(status: int):
    if status != SA_OK:
        raise SaError(status, lib().sa_last_error().decode())


def _ptr(t, dtype=None, numel=None, name="tensor", device=True):
    """Pointer of a contiguous tensor (None -> NULL) on the GPU (device=True) or the host,
    with marshalling checks."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if device and not t.is_cuda:
        raise ValueError(f"{name}: expected a GPU tensor")
    if not device and t.is_cuda:
        raise ValueError(f"{name}: expected a host (CPU) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name}: {t.numel()} elements < {numel} required")
    return t.data_ptr()


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream if hasattr(s, "cuda_stream") else int(s)


@dataclass(frozen=True)
class Dims:
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    max_blocks: int
    num_pages: int
    kv_dtype: int  # SA_F32 | SA_BF16

    def c(self) -> sa_dims:
        return sa_dims(self.batch, self.num_q_heads, self.num_kv_heads, self.head_dim,
                       self.block_size, self.max_blocks, self.num_pages, self.kv_dtype)

    @property
    def kv_torch(self):
        return torch.bfloat16 if self.kv_dtype == SA_BF16 else torch.float32


_hip = None
# Page-locked buffers whose tensors have died.  They are released (hipHostFree, which waits
# for the device) at the next pinned_empty call or by release_pinned(), never from inside a
# garbage-collection pass, which could land in the middle of a stream capture.
_PENDING_FREE = []


HIP_HOST_MALLOC_COHERENT = 0x40000000


def pinned_empty(shape, dtype=torch.int32) -> torch.Tensor:
    """A CPU tensor in coherent page-locked memory (hipHostMalloc with
    hipHostMallocCoherent), for the host mirrors of the hand-off (cpu_blocks_host,
    n_cpu_host), which the selection kernel writes directly."""
    global _hip
    if _hip is None:
        lib()  # loads libamdhip64 as a dependency of the library
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipHostMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t,
                                       ctypes.c_uint]
        _hip.hipHostFree.argtypes = [ctypes.c_void_p]
    release_pinned()
    n = 1
    for v in (shape if isinstance(shape, (tuple, list)) else (shape,)):
        n *= int(v)
    nbytes = max(1, n) * torch.empty((), dtype=dtype).element_size()
    ptr = ctypes.c_void_p()
    if _hip.hipHostMalloc(ctypes.byref(ptr), nbytes, HIP_HOST_MALLOC_COHERENT) != 0 or not ptr.value:
        raise RuntimeError(f"hipHostMalloc of {nbytes} bytes failed")
    buf = (ctypes.c_char * nbytes).from_address(ptr.value)
    # the tensor (and every view of it) holds buf; once the last one dies, the memory is
    # queued for release
    weakref.finalize(buf, _PENDING_FREE.append, ptr.value)
    return torch.frombuffer(buf, dtype=dtype, count=n).view(shape)


def release_pinned() -> int:
    """Free the page-locked buffers whose tensors have died; returns how many.  Not to be
    called while a stream is being captured (hipHostFree waits for the device)."""
    freed = 0
    if _PENDING_FREE and torch.cuda.is_initialized():
        torch.cuda.synchronize()  # no queued work may still read or write them
    while _PENDING_FREE:
        if _hip.hipHostFree(ctypes.c_void_p(_PENDING_FREE.pop())) != 0:
            raise RuntimeError("hipHostFree failed")
        freed += 1
    return freed


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A zero-filled device byte buffer of at least nbytes (at least 256 so it is never
    empty).  Zero is what the selection's arrival counters must hold before their first
    use; the calls leave them zero again."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ---- calls (same names as the C ABI) -----------------------------------------------------

def sa_abi_version() -> int:
    return lib().sa_abi_version()


def sa_workspace_bytes(dims: Dims, top_k: int) -> int:
    return lib().sa_workspace_bytes(ctypes.byref(dims.c()), top_k)


def sa_predict_query_workspace_bytes(m: int, n: int, k: int) -> int:
    return lib().sa_predict_query_workspace_bytes(m, n, k)


def sa_step_workspace_bytes(dims: Dims, hidden: int, top_k: int) -> int:
    return lib().sa_step_workspace_bytes(ctypes.byref(dims.c()), hidden, top_k)


def sa_pack_k_pages(dims: Dims, k_rows, k_pool, stream=None):
    """k_rows [P][bs][d] token-row pages -> k_pool, the chunk-major K layout."""
    n = dims.num_pages * dims.block_size * dims.head_dim
    _check(lib().sa_pack_k_pages(
        ctypes.byref(dims.c()), _ptr(k_rows, dims.kv_torch, n, "k_rows"),
        _ptr(k_pool, dims.kv_torch, n, "k_pool"), _stream(stream)))


def pack_k_pages(dims: Dims, k_rows, stream=None):
    """Allocate a chunk-major K pool of k_rows' size and fill it with sa_pack_k_pages."""
    out = torch.empty_like(k_rows)
    sa_pack_k_pages(dims, k_rows, out, stream)
    return out


def sa_pack_v_pages(dims: Dims, v_rows, v_pool, stream=None):
    """v_rows [P][bs][d] token-row pages -> v_pool [P][bs/16][d][16]."""
    n = dims.num_pages * dims.block_size * dims.head_dim
    _check(lib().sa_pack_v_pages(
        ctypes.byref(dims.c()), _ptr(v_rows, dims.kv_torch, n, "v_rows"),
        _ptr(v_pool, dims.kv_torch, n, "v_pool"), _stream(stream)))


def pack_v_pages(dims: Dims, v_rows, stream=None):
    """Allocate a V pool of v_rows' size and fill it with sa_pack_v_pages."""
    out = torch.empty_like(v_rows)
    sa_pack_v_pages(dims, v_rows, out, stream)
    return out


def sa_pack_weight(w, w_packed, stream=None):
    """w [n][k] bf16 -> w_packed (n*k bf16), the order sa_predict_query streams."""
    n, k = w.shape
    _check(lib().sa_pack_weight(n, k, _ptr(w, torch.bfloat16, n * k, "w"),
                                _ptr(w_packed, torch.bfloat16, n * k, "w_packed"),
                                _stream(stream)))


def pack_weight(w, stream=None):
    """Allocate a packed copy of w [n][k] bf16 (same shape, packed order)."""
    out = torch.empty_like(w)
    sa_pack_weight(w, out, stream)
    return out


def sa_build_digests(dims: Dims, kind: str, k_pool, block_table, seq_lens, digests,
                     stream=None):
    per = 2 if kind == "minmax" else 1
    n_dig = dims.batch * dims.num_kv_heads * dims.max_blocks * per * dims.head_dim
    _check(lib().sa_build_digests(
        ctypes.byref(dims.c()), KIND[kind],
        _ptr(k_pool, dims.kv_torch, dims.num_pages * dims.block_size * dims.head_dim, "k_pool"),
        _ptr(block_table, torch.int32, dims.batch * dims.num_kv_heads * dims.max_blocks,
             "block_table"),
        _ptr(seq_lens, torch.int32, dims.batch, "seq_lens"),
        _ptr(digests, dims.kv_torch, n_dig, "digests"), _stream(stream)))


def sa_refresh_last_digests(dims: Dims, kind: str, k_pool, block_table, seq_lens, digests,
                            stream=None):
    per = 2 if kind == "minmax" else 1
    n_dig = dims.batch * dims.num_kv_heads * dims.max_blocks * per * dims.head_dim
    _check(lib().sa_refresh_last_digests(
        ctypes.byref(dims.c()), KIND[kind],
        _ptr(k_pool, dims.kv_torch, dims.num_pages * dims.block_size * dims.head_dim, "k_pool"),
        _ptr(block_table, torch.int32, dims.batch * dims.num_kv_heads * dims.max_blocks,
             "block_table"),
        _ptr(seq_lens, torch.int32, dims.batch, "seq_lens"),
        _ptr(digests, dims.kv_torch, n_dig, "digests"), _stream(stream)))


def sa_predict_query(x, w_packed, q, ws=None, stream=None):
    """q [m][n] = x [m][k] w^T, w given packed by sa_pack_weight (n*k elements)."""
    m, k = x.shape
    n = q.numel() // m
    if q.numel() != m * n or w_packed.numel() != n * k:
        raise ValueError("sa_predict_query: shapes x [m][k], w_packed n*k, q [m][n] expected")
    _check(lib().sa_predict_query(
        m, n, k, _ptr(x, torch.bfloat16, m * k, "x"),
        _ptr(w_packed, torch.bfloat16, n * k, "w_packed"),
        _ptr(q, torch.float32, m * n, "q"), _ptr(ws, torch.uint8, name="ws"),
        0 if ws is None else ws.numel(), _stream(stream)))


def sa_select_blocks(dims: Dims, kind: str, q, digests, seq_lens, top_k: int, block_table,
                     gpu_blocks, n_gpu, cpu_blocks, n_cpu, scores=None, ws=None, stream=None):
    pairs = dims.batch * dims.num_kv_heads
    _check(lib().sa_select_blocks(
        ctypes.byref(dims.c()), KIND[kind],
        _ptr(q, torch.float32, dims.batch * dims.num_q_heads * dims.head_dim, "q"),
        _ptr(digests, dims.kv_torch, name="digests"),
        _ptr(seq_lens, torch.int32, dims.batch, "seq_lens"), top_k,
        _ptr(block_table, torch.int32, pairs * dims.max_blocks, "block_table"),
        _ptr(gpu_blocks, torch.int32, pairs * top_k, "gpu_blocks"),
        _ptr(n_gpu, torch.int32, pairs, "n_gpu"),
        _ptr(cpu_blocks, torch.int32, pairs * top_k, "cpu_blocks"),
        _ptr(n_cpu, torch.int32, pairs, "n_cpu"),
        _ptr(scores, torch.float32, pairs * dims.max_blocks, "scores"),
        _ptr(ws, torch.uint8, name="ws"), 0 if ws is None else ws.numel(), _stream(stream)))


def sa_sparse_decode(dims: Dims, q, k_pool, v_pool, block_table, seq_lens, gpu_blocks, n_gpu,
                     list_stride: int, scale: float, o, m=None, l=None, ws=None, stream=None):
    rows = dims.batch * dims.num_q_heads
    _check(lib().sa_sparse_decode(
        ctypes.byref(dims.c()), _ptr(q, torch.float32, rows * dims.head_dim, "q"),
        _ptr(k_pool, dims.kv_torch, name="k_pool"), _ptr(v_pool, dims.kv_torch, name="v_pool"),
        _ptr(block_table, torch.int32, name="block_table"),
        _ptr(seq_lens, torch.int32, dims.batch, "seq_lens"),
        _ptr(gpu_blocks, torch.int32, name="gpu_blocks"), _ptr(n_gpu, torch.int32, name="n_gpu"),
        list_stride, scale, _ptr(o, torch.float32, rows * dims.head_dim, "o"),
        _ptr(m, torch.float32, rows, "m"), _ptr(l, torch.float32, rows, "l"),
        _ptr(ws, torch.uint8, name="ws"), 0 if ws is None else ws.numel(), _stream(stream)))


def sa_decode_attend_merge(dims: Dims, q, k_pool, v_pool, block_table, seq_lens, gpu_blocks,
                           n_gpu, list_stride: int, scale: float, host_o, host_m, host_l,
                           n_cpu, o, m=None, l=None, ws=None, stream=None):
    rows = dims.batch * dims.num_q_heads
    _check(lib().sa_decode_attend_merge(
        ctypes.byref(dims.c()), _ptr(q, torch.float32, rows * dims.head_dim, "q"),
        _ptr(k_pool, dims.kv_torch, name="k_pool"), _ptr(v_pool, dims.kv_torch, name="v_pool"),
        _ptr(block_table, torch.int32, name="block_table"),
        _ptr(seq_lens, torch.int32, dims.batch, "seq_lens"),
        _ptr(gpu_blocks, torch.int32, name="gpu_blocks"), _ptr(n_gpu, torch.int32, name="n_gpu"),
        list_stride, scale, _ptr(host_o, torch.float32, rows * dims.head_dim, "host_o"),
        _ptr(host_m, torch.float32, rows, "host_m"), _ptr(host_l, torch.float32, rows, "host_l"),
        _ptr(n_cpu, torch.int32, name="n_cpu"),
        _ptr(o, torch.float32, rows * dims.head_dim, "o"),
        _ptr(m, torch.float32, rows, "m"), _ptr(l, torch.float32, rows, "l"),
        _ptr(ws, torch.uint8, name="ws"), 0 if ws is None else ws.numel(), _stream(stream)))


def sa_decode_attend_merge_noalloc(dims: Dims, q, k_pool, v_pool, block_table, seq_lens,
                                   gpu_blocks, n_gpu, list_stride: int, scale: float, host_o,
                                   host_m, host_l, n_cpu, o, m=None, l=None, stream=None):
    """sa_decode_attend_merge with its attention partials in the library's per-GPU scratch
    instead of a caller workspace (no allocation anywhere in the call)."""
    rows = dims.batch * dims.num_q_heads
    _check(lib().sa_decode_attend_merge_noalloc(
        ctypes.byref(dims.c()), _ptr(q, torch.float32, rows * dims.head_dim, "q"),
        _ptr(k_pool, dims.kv_torch, name="k_pool"), _ptr(v_pool, dims.kv_torch, name="v_pool"),
        _ptr(block_table, torch.int32, name="block_table"),
        _ptr(seq_lens, torch.int32, dims.batch, "seq_lens"),
        _ptr(gpu_blocks, torch.int32, name="gpu_blocks"), _ptr(n_gpu, torch.int32, name="n_gpu"),
        list_stride, scale, _ptr(host_o, torch.float32, rows * dims.head_dim, "host_o"),
        _ptr(host_m, torch.float32, rows, "host_m"), _ptr(host_l, torch.float32, rows, "host_l"),
        _ptr(n_cpu, torch.int32, name="n_cpu"),
        _ptr(o, torch.float32, rows * dims.head_dim, "o"),
        _ptr(m, torch.float32, rows, "m"), _ptr(l, torch.float32, rows, "l"), _stream(stream)))


def sa_merge(o_a, m_a, l_a, o_b, m_b, l_b, o, m, l, stream=None):
    rows, d = o_a.shape[0], o_a.shape[-1]
    rows = o_a.numel() // d
    f = torch.float32
    _check(lib().sa_merge(rows, d, _ptr(o_a, f, rows * d, "o_a"), _ptr(m_a, f, rows, "m_a"),
                          _ptr(l_a, f, rows, "l_a"), _ptr(o_b, f, rows * d, "o_b"),
                          _ptr(m_b, f, rows, "m_b"), _ptr(l_b, f, rows, "l_b"),
                          _ptr(o, f, rows * d, "o"), _ptr(m, f, rows, "m"),
                          _ptr(l, f, rows, "l"), _stream(stream)))


def sa_host_partial_attention(dims: Dims, q, k_host, v_host, host_table, seq_lens, cpu_blocks,
                              n_cpu, list_stride: int, scale: float, o, m, l, threads: int = 0):
    """A_cpu on host threads: every argument is a CPU tensor (k_host, v_host [pages][bs][d])."""
    rows = dims.batch * dims.num_q_heads
    pairs = dims.batch * dims.num_kv_heads
    pages = k_host.shape[0]
    per_page = dims.block_size * dims.head_dim
    i32, f32 = torch.int32, torch.float32
    _check(lib().sa_host_partial_attention(
        ctypes.byref(dims.c()), pages,
        _ptr(q, f32, rows * dims.head_dim, "q", device=False),
        _ptr(k_host, dims.kv_torch, pages * per_page, "k_host", device=False),
        _ptr(v_host, dims.kv_torch, pages * per_page, "v_host", device=False),
        _ptr(host_table, i32, pairs * dims.max_blocks, "host_table", device=False),
        _ptr(seq_lens, i32, dims.batch, "seq_lens", device=False),
        _ptr(cpu_blocks, i32, pairs * list_stride, "cpu_blocks", device=False),
        _ptr(n_cpu, i32, pairs, "n_cpu", device=False), list_stride, scale,
        _ptr(o, f32, rows * dims.head_dim, "o", device=False),
        _ptr(m, f32, rows, "m", device=False), _ptr(l, f32, rows, "l", device=False), threads))


def sa_decode_step(dims: Dims, kind: str, hidden: int, top_k: int, scale: float, seq_lens,
                   layers: list, ws, stream=None, side_stream=None):
    """`layers` is a list of dicts with the sa_layer field names (tensors; the *_host ones
    pinned CPU tensors or None)."""
    arr = (sa_layer * len(layers))()
    for i, L in enumerate(layers):
        for name, _ in sa_layer._fields_:
            t = L.get(name)
            host = name.endswith("_host")
            setattr(arr[i], name, _ptr(t, name=f"layers[{i}].{name}", device=not host))
    _check(lib().sa_decode_step(
        ctypes.byref(dims.c()), KIND[kind], hidden, top_k, scale,
        _ptr(seq_lens, torch.int32, dims.batch, "seq_lens"), len(layers), arr,
        _ptr(ws, torch.uint8, name="ws"), ws.numel(), _stream(stream),
        None if side_stream is None else _stream(side_stream)))


def sa_dense_workspace_bytes(dims: Dims) -> int:
    return lib().sa_dense_workspace_bytes(ctypes.byref(dims.c()))


def sa_dense_decode(dims: Dims, q, k_pool, v_pool, block_table, seq_lens, scale: float, o,
                    m=None, l=None, ws=None, stream=None):
    """FullKV attention over every resident block (GPU tensors)."""
    B_, Hq, Hkv, d = dims.batch, dims.num_q_heads, dims.num_kv_heads, dims.head_dim
    f32, i32 = torch.float32, torch.int32
    n = dims.num_pages * dims.block_size * d
    if ws is None:
        ws = workspace(sa_dense_workspace_bytes(dims))
    _check(lib().sa_dense_decode(
        ctypes.byref(dims.c()), _ptr(q, f32, B_ * Hq * d, "q"),
        _ptr(k_pool, dims.kv_torch, n, "k_pool"), _ptr(v_pool, dims.kv_torch, n, "v_pool"),
        _ptr(block_table, i32, B_ * Hkv * dims.max_blocks, "block_table"),
        _ptr(seq_lens, i32, B_, "seq_lens"), scale, _ptr(o, f32, B_ * Hq * d, "o"),
        _ptr(m, f32, B_ * Hq, "m"), _ptr(l, f32, B_ * Hq, "l"), _ptr(ws, torch.uint8, name="ws"),
        ws.numel(), _stream(stream)))


def sa_recall_blocks(dims: Dims, list_stride: int, max_recall: int, seq_lens, block_table,
                     gpu_blocks, n_gpu, cpu_blocks, n_cpu, k_host, v_host, host_table,
                     k_pool, v_pool, n_recalled, ws=None, stream=None):
    """Periodic recall for one layer.  k_host, v_host: pinned CPU tensors (pinned_empty)
    [pages][bs][d]; host_table: a GPU tensor or a pinned CPU tensor; the rest GPU tensors.
    block_table, k_pool, v_pool and n_recalled are written."""
    i32 = torch.int32
    B_, Hkv, mb = dims.batch, dims.num_kv_heads, dims.max_blocks
    pairs = B_ * Hkv
    pages = k_host.shape[0]
    per_page = dims.block_size * dims.head_dim
    if ws is None:
        ws = workspace(sa_recall_workspace_bytes(dims, max_recall))
    _check(lib().sa_recall_blocks(
        ctypes.byref(dims.c()), list_stride, max_recall,
        _ptr(seq_lens, i32, B_, "seq_lens"), _ptr(block_table, i32, pairs * mb, "block_table"),
        _ptr(gpu_blocks, i32, pairs * list_stride, "gpu_blocks"),
        _ptr(n_gpu, i32, pairs, "n_gpu"), _ptr(cpu_blocks, i32, pairs * list_stride, "cpu_blocks"),
        _ptr(n_cpu, i32, pairs, "n_cpu"),
        _ptr(k_host, dims.kv_torch, pages * per_page, "k_host", device=False),
        _ptr(v_host, dims.kv_torch, pages * per_page, "v_host", device=False),
        _ptr(host_table, i32, pairs * mb, "host_table", device=host_table.is_cuda), pages,
        _ptr(k_pool, dims.kv_torch, dims.num_pages * per_page, "k_pool"),
        _ptr(v_pool, dims.kv_torch, dims.num_pages * per_page, "v_pool"),
        _ptr(n_recalled, i32, pairs, "n_recalled"), _ptr(ws, torch.uint8, name="ws"),
        ws.numel(), _stream(stream)))


def sa_recall_workspace_bytes(dims: Dims, max_recall: int) -> int:
    return lib().sa_recall_workspace_bytes(ctypes.byref(dims.c()), max_recall)


class HostPlan:
    """The host side of sa_decode_step_offload (sa_host_plan_create): per layer a dict with
    k_host, v_host [pages][bs][d] and host_table [B][Hkv][max_blocks] (CPU tensors), and the
    pinned buffers (pinned_empty) q_host [B][Hq][d], cpu_blocks_host [B][Hkv][top_k],
    n_cpu_host [B][Hkv], o_host [B][Hq][d], m_host, l_host [B][Hq].  Keeps the tensors alive;
    close() stops the workers (not while enqueued work or a captured graph may still use
    the plan)."""

    def __init__(self, dims: Dims, top_k: int, scale: float, seq_lens_host, layers: list,
                 threads: int = 0):
        i32, f32 = torch.int32, torch.float32
        B, Hq, Hkv, d = dims.batch, dims.num_q_heads, dims.num_kv_heads, dims.head_dim
        per_page = dims.block_size * d
        arr = (sa_host_layer * len(layers))()
        for i, L in enumerate(layers):
            pages = L["k_host"].shape[0]
            if L["v_host"].shape[0] != pages:
                raise ValueError(f"layers[{i}]: k_host and v_host differ in pages")
            a = arr[i]
            a.k_host = _ptr(L["k_host"], dims.kv_torch, pages * per_page, f"[{i}].k_host", False)
            a.v_host = _ptr(L["v_host"], dims.kv_torch, pages * per_page, f"[{i}].v_host", False)
            a.host_table = _ptr(L["host_table"], i32, B * Hkv * dims.max_blocks,
                                f"[{i}].host_table", False)
            a.host_pages = pages
            a.q_host = _ptr(L["q_host"], f32, B * Hq * d, f"[{i}].q_host", False)
            a.cpu_blocks_host = _ptr(L["cpu_blocks_host"], i32, B * Hkv * top_k,
                                     f"[{i}].cpu_blocks_host", False)
            a.n_cpu_host = _ptr(L["n_cpu_host"], i32, B * Hkv, f"[{i}].n_cpu_host", False)
            a.o_host = _ptr(L["o_host"], f32, B * Hq * d, f"[{i}].o_host", False)
            a.m_host = _ptr(L["m_host"], f32, B * Hq, f"[{i}].m_host", False)
            a.l_host = _ptr(L["l_host"], f32, B * Hq, f"[{i}].l_host", False)
        self.layers = layers
        self.seq_lens = seq_lens_host
        self.handle = _P()
        _check(lib().sa_host_plan_create(
            ctypes.byref(dims.c()), top_k, scale,
            _ptr(seq_lens_host, i32, B, "seq_lens_host", device=False), len(layers), arr,
            threads, ctypes.byref(self.handle)))

    def stats(self):
        """(host tasks run, seconds they took)."""
        n = ctypes.c_int64()
        t = ctypes.c_double()
        _check(lib().sa_host_plan_stats(self.handle, ctypes.byref(n), ctypes.byref(t)))
        return n.value, t.value

    def set_recall(self, dims: Dims, max_recall: int, beta: float, layers, ws=None,
                   overlap: bool = False):
        """Periodic recall inside the offload step (sa_host_plan_set_recall): `layers` is a
        list of dicts with host_table_dev (GPU int32 [B][Hkv][max_blocks], or None) and
        n_recalled (GPU int32 [B][Hkv]); None turns recall off."""
        if layers is None:
            _check(lib().sa_host_plan_set_recall(self.handle, 0, 0.0, None, None, 0, 0))
            self._recall = None
            return
        pairs = dims.batch * dims.num_kv_heads
        if ws is None:
            ws = workspace(sa_recall_workspace_bytes(dims, max_recall))
        arr = (sa_recall_layer * len(layers))()
        for i, L in enumerate(layers):
            arr[i].host_table_dev = _ptr(L.get("host_table_dev"), torch.int32,
                                         pairs * dims.max_blocks, f"[{i}].host_table_dev")
            arr[i].n_recalled = _ptr(L.get("n_recalled"), torch.int32, pairs,
                                     f"[{i}].n_recalled")
        self._recall = (layers, ws)
        _check(lib().sa_host_plan_set_recall(self.handle, max_recall, beta, arr,
                                             _ptr(ws, torch.uint8, name="ws"), ws.numel(),
                                             1 if overlap else 0))

    def set_handoff(self, mode: str, flags=None, gpu_wait_ms: int = 30000):
        """sa_host_plan_set_handoff: "host_func" (HIP host functions, the default) or
        "flags" (a dispatcher thread and flags in memory both sides see).  flags: an int32
        CPU tensor of 2 * layers + 1 words (default: a new page-locked coherent one),
        zeroed by the call and kept alive here."""
        if mode == "flags" and flags is None:
            flags = pinned_empty((2 * len(self.layers) + 1,), torch.int32)
        ptr = None
        if mode == "flags":
            ptr = _ptr(flags, torch.int32, 2 * len(self.layers) + 1, "flags", device=False)
        _check(lib().sa_host_plan_set_handoff(self.handle, HANDOFF[mode], ptr, gpu_wait_ms))
        self.flags = flags if mode == "flags" else None

    def run(self, layer: int):
        """Layer `layer`'s host task now, on this thread and the plan's workers."""
        _check(lib().sa_host_plan_run(self.handle, layer))

    def close(self):
        if self.handle:
            _check(lib().sa_host_plan_destroy(self.handle))
            self.handle = _P()


def sa_decode_step_offload(dims: Dims, kind: str, hidden: int, top_k: int, scale: float,
                           seq_lens, layers: list, ws, plan: HostPlan, host_stream,
                           stream=None, side_stream=None, recall_stream=None):
    """sa_decode_step with the CPU side computed by `plan` on `host_stream` (a stream of its
    own); host_o/m/l and the host mirrors of `layers` are not used."""
    arr = (sa_layer * len(layers))()
    for i, L in enumerate(layers):
        for name, _ in sa_layer._fields_:
            if name.endswith("_host") or name in ("host_o", "host_m", "host_l"):
                continue
            setattr(arr[i], name, _ptr(L.get(name), name=f"layers[{i}].{name}"))
    _check(lib().sa_decode_step_offload(
        ctypes.byref(dims.c()), KIND[kind], hidden, top_k, scale,
        _ptr(seq_lens, torch.int32, dims.batch, "seq_lens"), len(layers), arr,
        _ptr(ws, torch.uint8, name="ws"), ws.numel(), _stream(stream),
        None if side_stream is None else _stream(side_stream), plan.handle,
        None if host_stream is None else _stream(host_stream),
        None if recall_stream is None else _stream(recall_stream)))


def _word(t, name):
    return _ptr(t, torch.int32, 1, name, device=t.is_cuda)


def sa_stream_signal(counter, stream=None):
    """*counter += 1 once the stream's earlier work is done (counter: a one-element int32
    tensor in page-locked host memory or on the GPU)."""
    _check(lib().sa_stream_signal(_word(counter, "counter"), _stream(stream)))


def sa_stream_wait(flag, counter, wait_ms: int, timeouts, stream=None):
    """Hold the stream until *flag == *counter, for at most about wait_ms ms; on giving up,
    *timeouts = 1."""
    _check(lib().sa_stream_wait(_word(flag, "flag"), _word(counter, "counter"), wait_ms,
                                _word(timeouts, "timeouts"), _stream(stream)))


PROFILE_STAGE = {"attention": 0, "select": 1, "gemm": 2}


def sa_profile_kernels(stage: str, starts, stops):
    """Time the next len(starts) launches of one stage's kernel ("attention", "select" or
    "gemm") on this thread: `starts` and `stops` are torch.cuda.Event(enable_timing=True)
    objects (already recorded once, so that they exist).  Read durations with
    starts[i].elapsed_time(stops[i])."""
    n = len(starts)
    a = (_P * max(1, n))(*[e.cuda_event for e in starts])
    b = (_P * max(1, n))(*[e.cuda_event for e in stops])
    _check(lib().sa_profile_kernels(PROFILE_STAGE[stage], a, b, n))


def sa_profile_attention(starts, stops):
    """Time the next len(starts) attention-kernel launches of this thread: `starts` and
    `stops` are torch.cuda.Event(enable_timing=True) objects (already recorded once, so
    that they exist).  Read durations with starts[i].elapsed_time(stops[i])."""
    n = len(starts)
    a = (_P * max(1, n))(*[e.cuda_event for e in starts])
    b = (_P * max(1, n))(*[e.cuda_event for e in stops])
    _check(lib().sa_profile_attention(a, b, n))
