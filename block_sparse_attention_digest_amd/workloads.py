"""Seeded synthetic inputs for the block-sparse decode path.

This module draws random tensors and lays them out (page permutations, block tables,
gathers into a page pool).  It holds none of the method's arithmetic: no projection, no
digest, no score, no selection, no attention.  Where a layout depends on which blocks the
method selects (the resident sets), the selection is passed in by the caller.

Both the HIP path and the CPU oracle consume exactly the tensors made here.  Every tensor
comes from its own torch.Generator, seeded from (workload seed, config id, tensor name), so
that draws do not depend on call order.  A CPU generator and a GPU generator produce
different (but each reproducible) streams; small cases are drawn on the CPU.

The workloads are stand-ins for the pages' model shapes (Qwen3-8B / Qwen3-14B attention
layouts) with synthetic values; the pages' own evaluation data (LongBench) is not used.
"""

from __future__ import annotations

import dataclasses
import math
import zlib
from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    """Shape and value recipe of one synthetic decode workload."""
    name: str
    cfg_id: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    top_k: int                          # blocks per selection = budget tokens / block size
    kv_dtype: str                       # "f32" | "bf16"
    digest_kinds: tuple = ("mean",)
    context: int = 0                    # fixed context length; 0 means ragged
    ctx_min: int = 0                    # ragged: lengths uniform in [ctx_min, ctx_max]
    ctx_max: int = 0
    hidden: int = 0                     # >0: queries are W_Q X products; 0: drawn directly
    resident: str = "fraction"          # "lowest" | "fraction" | "pool"
    resident_frac: tuple = (0.75, 0.75)  # per-sequence fraction ~ U[lo, hi]
    n_lowest: int = 0                   # "lowest": this many lowest-indexed selected blocks
    layers: int = 1
    pool_blocks: int = 0                # "pool": resident pool size per (seq, KV head)
    offset_std: float = 0.5             # per-block key offset ~ N(0, offset_std^2 I)
    ar_rho: float = 0.94                # "pool": X^i = rho X^{i-1} + sqrt(1-rho^2) Z
    seed: int = 0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_len(self) -> int:
        return self.context if self.context else self.ctx_max

    @property
    def max_blocks(self) -> int:
        return -(-self.max_len // self.block_size)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def torch_kv_dtype(self):
        return torch.bfloat16 if self.kv_dtype == "bf16" else torch.float32

    def scaled(self, **kw) -> "Workload":
        """A smaller copy with the same recipe (for tests the oracle finishes quickly)."""
        return dataclasses.replace(self, **kw)


# The five workloads: shapes of the Qwen3-8B / Qwen3-14B attention layers, budget 2048
# tokens in blocks of 32 (4096 tokens in blocks of 16 for the ragged batch).
TINY = Workload("tiny-fp32-gqa4", 1, batch=2, num_q_heads=4, num_kv_heads=1, head_dim=64,
                block_size=16, top_k=8, kv_dtype="f32", context=1024, resident="lowest",
                n_lowest=4)
QWEN3_8B_LAYER = Workload("qwen3-8b-layer-b8-16k", 2, batch=8, num_q_heads=32,
                          num_kv_heads=8, head_dim=128, block_size=32, top_k=64,
                          kv_dtype="bf16", context=16384, hidden=4096,
                          resident_frac=(0.75, 0.75))
QWEN3_14B_LAYER = Workload("qwen3-14b-layer-b40-32k-minmax", 3, batch=40, num_q_heads=40,
                           num_kv_heads=8, head_dim=128, block_size=32, top_k=64,
                           kv_dtype="bf16", digest_kinds=("minmax",), context=32768,
                           hidden=5120, resident_frac=(0.9, 0.9))
QWEN3_14B_STEP = Workload("qwen3-14b-40layer-step-b40-64k", 4, batch=40, num_q_heads=40,
                          num_kv_heads=8, head_dim=128, block_size=32, top_k=64,
                          kv_dtype="bf16", context=65536, hidden=5120, resident="pool",
                          layers=40, pool_blocks=128)
RAGGED = Workload("ragged-b64-4k..64k-bs16", 5, batch=64, num_q_heads=40, num_kv_heads=8,
                  head_dim=128, block_size=16, top_k=256, kv_dtype="bf16",
                  digest_kinds=("mean", "minmax"), ctx_min=4096, ctx_max=65536,
                  resident_frac=(0.5, 1.0))

WORKLOADS = {w.cfg_id: w for w in (TINY, QWEN3_8B_LAYER, QWEN3_14B_LAYER, QWEN3_14B_STEP,
                                   RAGGED)}


# ----------------------------------------------------------------------------------------
# generators
# ----------------------------------------------------------------------------------------

def generator(wl: Workload, name: str, device) -> torch.Generator:
    """A torch.Generator on `device` seeded from (seed, config id, tensor name)."""
    key = zlib.crc32(f"{wl.seed}/{wl.cfg_id}/{name}".encode())
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(key)
    return g


def _normal(shape, gen, device, std=1.0, chunk_rows=1 << 16):
    """N(0, std^2) float32, drawn in fixed chunks along dim 0 (bounds peak memory)."""
    out = torch.empty(shape, dtype=torch.float32, device=device)
    rows = shape[0]
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        out[r0:r1].normal_(0.0, std, generator=gen)
    return out


def seq_lens(wl: Workload) -> torch.Tensor:
    """Context length of every sequence (int32, on the CPU)."""
    if wl.context:
        return torch.full((wl.batch,), wl.context, dtype=torch.int32)
    g = generator(wl, "seq_lens", "cpu")
    return torch.randint(wl.ctx_min, wl.ctx_max + 1, (wl.batch,), generator=g,
                         dtype=torch.int64).to(torch.int32)


def blocks_of(lens: torch.Tensor, block_size: int) -> list:
    return [-(-int(n) // block_size) for n in lens.tolist()]


def draw_queries(wl: Workload, device, layer: int = 0) -> dict:
    """Query inputs: {"X" [B][hidden] bf16, "W" [Hq*d][hidden] bf16} when the query is a
    projection W_Q X, else {"Q" [B][Hq][d] float32 ~ N(0, 1)}."""
    if wl.hidden:
        X = _normal((wl.batch, wl.hidden), generator(wl, f"X{layer}", device), device)
        W = _normal((wl.num_q_heads * wl.head_dim, wl.hidden),
                    generator(wl, f"W{layer}", device), device, std=1.0 / math.sqrt(wl.hidden))
        return {"X": X.to(torch.bfloat16), "W": W.to(torch.bfloat16)}
    Q = _normal((wl.batch, wl.num_q_heads, wl.head_dim), generator(wl, "Q", device), device)
    return {"Q": Q}


def draw_kv_pages(wl: Workload, lens: torch.Tensor, device) -> dict:
    """The full key/value cache of one layer, paged.

    Every valid block (s, h, b) owns one page of a pool [P][bs][d]; pages are assigned by a
    random permutation.  K = N(0, 1) + a per-block offset ~ N(0, offset_std^2 I) shared by
    the block's tokens; V = N(0, 1).  Tokens past a sequence's end inside its last page are
    drawn too but never belong to any block.  Returns {"K", "V" [P][bs][d] in the KV dtype,
    "table" [B][Hkv][max_blocks] int32 (page of every block, -1 past the end)}.
    """
    nbs = blocks_of(lens, wl.block_size)
    B, H, mb, bs, d = wl.batch, wl.num_kv_heads, wl.max_blocks, wl.block_size, wl.head_dim
    P = H * sum(nbs)
    perm = torch.randperm(P, generator=generator(wl, "page_perm", "cpu")).to(torch.int32)
    table = torch.full((B, H, mb), -1, dtype=torch.int32)
    pos = 0
    for s in range(B):
        for h in range(H):
            table[s, h, :nbs[s]] = perm[pos:pos + nbs[s]]
            pos += nbs[s]
    K = _normal((P, bs, d), generator(wl, "K", device), device)
    off = _normal((P, 1, d), generator(wl, "K_offset", device), device, std=wl.offset_std)
    K += off
    del off
    K = K.to(wl.torch_kv_dtype)
    V = _normal((P, bs, d), generator(wl, "V", device), device).to(wl.torch_kv_dtype)
    return {"K": K, "V": V, "table": table.to(device)}


def logical_rows(pages: torch.Tensor, table_row: torch.Tensor, seq_len: int) -> torch.Tensor:
    """The logical sequence [seq_len][d] of one (seq, KV head), gathered from its pages."""
    nb = -(-seq_len // pages.shape[1])
    idx = table_row[:nb].to(device=pages.device, dtype=torch.int64)
    return pages[idx].reshape(-1, pages.shape[2])[:seq_len]


def choose_resident(wl: Workload, selected, lens: torch.Tensor) -> list:
    """The resident block set R of every (seq, KV head), given the method's selection.

    `selected[s][h]` lists the selected blocks (ascending).  R holds n_res of them plus
    "filler" blocks that are resident but not selected, up to the pool capacity k_s:
      "lowest":   n_res = n_lowest, the lowest-indexed selected blocks;
      "fraction": n_res = floor(f_s * k_s + 0.5), a random subset, with f_s ~ U[lo, hi]
                  drawn once per sequence.
    Fillers are drawn at random from the unselected blocks.  Returns R[s][h] as sorted
    int64 numpy arrays.
    """
    g = generator(wl, "resident", "cpu")
    nbs = blocks_of(lens, wl.block_size)
    lo, hi = wl.resident_frac
    R = []
    for s in range(wl.batch):
        f = lo + (hi - lo) * float(torch.rand((), generator=g))
        row = []
        for h in range(wl.num_kv_heads):
            sel = np.asarray(selected[s][h], dtype=np.int64)
            ks = len(sel)
            if wl.resident == "lowest":
                keep = sel[:min(wl.n_lowest, ks)]
            else:
                n_res = int(math.floor(f * ks + 0.5))
                pick = torch.randperm(ks, generator=g)[:n_res].numpy()
                keep = sel[pick]
            unsel = np.setdiff1d(np.arange(nbs[s], dtype=np.int64), sel)
            n_fill = min(ks - len(keep), len(unsel))
            fill = unsel[torch.randperm(len(unsel), generator=g)[:n_fill].numpy()]
            row.append(np.sort(np.concatenate([keep, fill])))
        R.append(row)
    return R


def build_pool(wl: Workload, R, src_K: torch.Tensor, src_V: torch.Tensor,
               src_table: torch.Tensor, capacity_per_pair: int, name: str = "pool") -> dict:
    """Copy the resident blocks R[s][h] into a paged pool with a permuted block table.

    The pool has B * Hkv * capacity_per_pair pages; pair (s, h) gets a random set of them.
    Returns {"K", "V" [P][bs][d], "block_table" [B][Hkv][max_blocks] int32 with -1 for a
    block that is not resident}.  src_* are a paged cache and its table (draw_kv_pages).
    """
    B, H, mb = wl.batch, wl.num_kv_heads, wl.max_blocks
    cap = B * H * capacity_per_pair
    perm = torch.randperm(cap, generator=generator(wl, f"{name}_perm", "cpu"))
    table = torch.full((B, H, mb), -1, dtype=torch.int64)
    src_idx, dst_idx = [], []
    src_table_cpu = src_table.cpu().to(torch.int64)
    for s in range(B):
        for h in range(H):
            r = torch.as_tensor(R[s][h], dtype=torch.int64)
            if len(r) > capacity_per_pair:
                raise ValueError("resident set larger than the pool capacity")
            base = (s * H + h) * capacity_per_pair
            pages = perm[base:base + len(r)]
            table[s, h, r] = pages
            dst_idx.append(pages)
            src_idx.append(src_table_cpu[s, h, r])
    dev = src_K.device
    dst = torch.cat(dst_idx).to(dev) if dst_idx else torch.zeros(0, dtype=torch.int64)
    src = torch.cat(src_idx).to(dev) if src_idx else torch.zeros(0, dtype=torch.int64)
    K = torch.zeros((cap,) + tuple(src_K.shape[1:]), dtype=src_K.dtype, device=dev)
    V = torch.zeros_like(K)
    K[dst] = src_K[src]
    V[dst] = src_V[src]
    return {"K": K, "V": V, "block_table": table.to(torch.int32).to(dev)}


# ----------------------------------------------------------------------------------------
# the 40-layer step workload ("pool" residency)
# ----------------------------------------------------------------------------------------

def draw_layer_inputs(wl: Workload, device) -> list:
    """Per-layer X^i (AR(1) across layers, N(0,1) marginals, bf16) and W_Q^i ~ N(0, 1/hidden)
    (bf16).  Returns a list of {"X", "W"}."""
    out = []
    rho = wl.ar_rho
    x = None
    for i in range(wl.layers):
        z = _normal((wl.batch, wl.hidden), generator(wl, f"Z{i}", device), device)
        x = z if x is None else rho * x + math.sqrt(1.0 - rho * rho) * z
        W = _normal((wl.num_q_heads * wl.head_dim, wl.hidden),
                    generator(wl, f"W{i}", device), device, std=1.0 / math.sqrt(wl.hidden))
        out.append({"X": x.to(torch.bfloat16), "W": W.to(torch.bfloat16)})
    return out


def layer_offsets(wl: Workload, layer: int, device) -> torch.Tensor:
    """Per-block key offsets of one layer, [B][Hkv][max_blocks][d] float32 (regenerable)."""
    return _normal((wl.batch, wl.num_kv_heads, wl.max_blocks, wl.head_dim),
                   generator(wl, f"offset{layer}", device), device, std=wl.offset_std)


def _largest_normal_moments(n: int):
    """Mean and standard deviation of the largest of n independent N(0, 1) draws, by
    quadrature of its density n phi(x) Phi(x)^(n-1) over [-8, 8]."""
    x = np.linspace(-8.0, 8.0, 16001)
    phi = np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)
    cdf = 0.5 * (1.0 + np.array([math.erf(v / math.sqrt(2.0)) for v in x]))
    pdf = n * phi * cdf ** (n - 1)
    dx = x[1] - x[0]
    mean = float(np.sum(x * pdf) * dx)
    return mean, math.sqrt(float(np.sum((x - mean) ** 2 * pdf) * dx))


def draw_layer_digests(wl: Workload, layer: int, offsets: torch.Tensor, device,
                       kind: str = "mean") -> torch.Tensor:
    """Stand-in digests for blocks whose keys are never materialised, stored in the KV dtype.

    mean: offset + N(0, 1/bs), the law of the mean of bs unit-normal keys around the offset;
    [B][Hkv][max_blocks][d].
    minmax: [B][Hkv][max_blocks][2][d], [..][0] = offset - E1 and [..][1] = offset + E2,
    where E1, E2 are drawn from the normal law with the mean and spread of the largest of bs
    unit normals (the per-channel extremes of bs keys around the offset, taken apart)."""
    if kind == "mean":
        noise = _normal(tuple(offsets.shape), generator(wl, f"digest_noise{layer}", device),
                        device, std=1.0 / math.sqrt(wl.block_size))
        return (offsets + noise).to(wl.torch_kv_dtype)
    if kind != "minmax":
        raise ValueError(f"digest kind {kind!r}")
    mean, sd = _largest_normal_moments(wl.block_size)
    shape = tuple(offsets.shape)
    lo = offsets - (_normal(shape, generator(wl, f"digest_lo{layer}", device), device, std=sd)
                    + mean)
    hi = offsets + (_normal(shape, generator(wl, f"digest_hi{layer}", device), device, std=sd)
                    + mean)
    return torch.stack([lo, hi], dim=3).to(wl.torch_kv_dtype)


def draw_layer_pool(wl: Workload, layer: int, offsets: torch.Tensor, pool_sets) -> dict:
    """Keys and values of the resident pool of one layer.

    pool_sets[s][h] lists the resident blocks (at most pool_blocks).  Their keys are
    offset + N(0, 1) per token and their values N(0, 1); pages are assigned by a random
    permutation.  Returns {"K", "V" [P][bs][d], "block_table" [B][Hkv][max_blocks]}.
    """
    B, H, bs, d = wl.batch, wl.num_kv_heads, wl.block_size, wl.head_dim
    cap = wl.pool_blocks
    dev = offsets.device
    P = B * H * cap
    perm = torch.randperm(P, generator=generator(wl, f"pool_perm{layer}", "cpu"))
    table = torch.full((B, H, wl.max_blocks), -1, dtype=torch.int64)
    blk_of_page = torch.full((P,), -1, dtype=torch.int64)
    for s in range(B):
        for h in range(H):
            r = torch.as_tensor(np.asarray(pool_sets[s][h]), dtype=torch.int64)
            if len(r) > cap:
                raise ValueError("pool set larger than the pool capacity")
            pages = perm[(s * H + h) * cap:(s * H + h) * cap + len(r)]
            table[s, h, r] = pages
            blk_of_page[pages] = (s * H + h) * wl.max_blocks + r
    K = _normal((P, bs, d), generator(wl, f"poolK{layer}", dev), dev)
    used = blk_of_page >= 0
    flat_off = offsets.reshape(-1, d)
    page_off = torch.zeros((P, d), dtype=torch.float32, device=dev)
    page_off[used.to(dev)] = flat_off[blk_of_page[used].to(dev)]
    K += page_off[:, None, :]
    V = _normal((P, bs, d), generator(wl, f"poolV{layer}", dev), dev)
    return {"K": K.to(wl.torch_kv_dtype), "V": V.to(wl.torch_kv_dtype),
            "block_table": table.to(torch.int32).to(dev)}


def draw_host_store(wl: Workload, layer: int, offsets: torch.Tensor) -> dict:
    """The host's copy of one layer's KV, from which the CPU side reads offloaded blocks:
    every block of every (sequence, KV head) has a host page (a seeded permutation); keys are
    offset + N(0, 1) per token, values N(0, 1), in the KV dtype, on the CPU.  Returns
    {"K", "V" [P][bs][d], "table" [B][Hkv][max_blocks] int32}."""
    B, H, bs, d, mb = wl.batch, wl.num_kv_heads, wl.block_size, wl.head_dim, wl.max_blocks
    P = B * H * mb
    perm = torch.randperm(P, generator=generator(wl, f"host_perm{layer}", "cpu"))
    table = perm.to(torch.int32).view(B, H, mb).clone()
    noise = _normal((P, bs, d), generator(wl, f"host_k{layer}", "cpu"), "cpu")
    k_log = offsets.cpu().reshape(P, 1, d) + noise      # logical order (s, h, b)
    v_log = _normal((P, bs, d), generator(wl, f"host_v{layer}", "cpu"), "cpu")
    K = torch.empty_like(k_log)
    V = torch.empty_like(v_log)
    K[perm] = k_log
    V[perm] = v_log
    return {"K": K.to(wl.torch_kv_dtype), "V": V.to(wl.torch_kv_dtype), "table": table}


def draw_host_store_aliased(wl: Workload, host_pages: int) -> dict:
    """A host store for shapes whose whole offloaded KV would not fit in host memory: a pool
    of host_pages pages (keys and values N(0, 1) in the KV dtype) that every (sequence, KV
    head, block) maps into through a seeded random table, so any selection reads the bytes a
    distinct-page store would.  Returns {"K", "V" [host_pages][bs][d], "table" [B][Hkv]
    [max_blocks] int32}, on the CPU."""
    bs, d = wl.block_size, wl.head_dim
    g = generator(wl, "host_alias", "cpu")
    K = torch.empty((host_pages, bs, d), dtype=wl.torch_kv_dtype)
    V = torch.empty_like(K)
    step = max(1, (1 << 22) // (bs * d))  # pages per chunk: 4M values at a time
    for p0 in range(0, host_pages, step):
        p1 = min(host_pages, p0 + step)
        K[p0:p1] = torch.randn((p1 - p0, bs, d), generator=g).to(wl.torch_kv_dtype)
        V[p0:p1] = torch.randn((p1 - p0, bs, d), generator=g).to(wl.torch_kv_dtype)
    table = torch.randint(0, host_pages, (wl.batch, wl.num_kv_heads, wl.max_blocks),
                          generator=g, dtype=torch.int32)
    return {"K": K, "V": V, "table": table}


def draw_host_partials(wl: Workload, layer: int, device) -> dict:
    """Stand-in partials of the offloaded blocks (what the CPU side returns): o ~ N(0, 1)^d,
    m ~ N(0, 1), l ~ U[1, bs * k].  float32, [B][Hq][d] and [B][Hq]."""
    B, Hq, d = wl.batch, wl.num_q_heads, wl.head_dim
    o = _normal((B, Hq, d), generator(wl, f"host_o{layer}", device), device)
    m = _normal((B, Hq), generator(wl, f"host_m{layer}", device), device)
    u = torch.rand((B, Hq), generator=generator(wl, f"host_l{layer}", device), device=device)
    l = 1.0 + (wl.block_size * wl.top_k - 1.0) * u
    return {"o": o, "m": m, "l": l}


# ----------------------------------------------------------------------------------------
# conversions for the oracle (exact widening only)
# ----------------------------------------------------------------------------------------

def f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a float32 / bfloat16 tensor to a float64 numpy array on the host."""
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)
