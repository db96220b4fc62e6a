"""Host replay of the kernels' index arithmetic on adversarial buffer contents.

The attention, reduce, selection and digest kernels take counts, list entries, pages and
lengths from caller memory.  Each such value is clamped before it forms an address (counts
into [0, list stride], entries into [0, max_blocks), pages into [0, P), lengths folded into
the block count), so bad contents give wrong numbers but never an access outside a buffer.
This test re-traces, in plain Python, every address those kernels form from such values --
the same formulas, lane by lane and wave by wave -- over random, deliberately bad contents
(negative counts and entries, counts past the list stride, entries past the table, pages
past the pool, negative and huge lengths), and asserts that each lies inside its buffer.
It runs on the CPU only; the kernels' own source is the reference for each formula (named
in each function's docstring).
"""

import random

WAVE = 64


def clamp(v, lo, hi):
    return min(max(v, lo), hi)


def wave_start(w, T, W):
    return (w * T) // W


def wave_of(g, T, W):
    return ((g + 1) * W + T - 1) // T - 1


def pair_prefix(n_gpu, cap):
    """attention.hip pair_prefix / wave_prefix: exclusive prefix of the clamped counts."""
    pfx = [0]
    for n in n_gpu:
        pfx.append(pfx[-1] + clamp(n, 0, cap))
    return pfx


def pair_of(pfx, npairs, g):
    lo, hi = 0, npairs - 1
    while lo < hi:
        mid = (lo + hi + 1) >> 1
        if pfx[mid] <= g:
            lo = mid
        else:
            hi = mid - 1
    return lo


def trace_attention(c, waves_per_wg, check):
    """attn_bf16_kernel: the query staging, each window's lookup (list entry, page list or
    block table, sequence length), the K/V page reads of every step, and the partial slots.
    check(buffer, index) asserts 0 <= index < size of buffer."""
    npairs, stride, G, D, BS = c["npairs"], c["stride"], c["G"], c["D"], c["BS"]
    W, P, mb, Hkv = c["W"], c["P"], c["max_blocks"], c["Hkv"]
    pfx = pair_prefix(c["n_gpu"], stride)
    for p in range(npairs):
        check("n_gpu", p)
    T = pfx[npairs]
    if T == 0:
        return
    kq_stage, per_pair = 4, G * D // 4
    for wg in range(W // waves_per_wg):
        lo = wave_start(wg * waves_per_wg, T, W)
        hi = wave_start((wg + 1) * waves_per_wg, T, W)
        q_lo = q_n = 0
        if lo < hi:
            q_lo = pair_of(pfx, npairs, lo)
            q_n = min(kq_stage, pair_of(pfx, npairs, hi - 1) - q_lo + 1)
        total = max(q_n, 1) * per_pair
        for t in range(0, 256 * ((kq_stage * per_pair + 255) // 256)):
            i = min(t, total - 1)
            pair = q_lo + i // per_pair
            check("q", (pair // Hkv) * c["row_stride"] + (pair % Hkv) * G * D + 4 * (i % per_pair))
        for wv in range(waves_per_wg):
            gw = wg * waves_per_wg + wv
            b0, b1 = wave_start(gw, T, W), wave_start(gw + 1, T, W)
            gfirst = min(b0, T - 1)
            p = pair_of(pfx, npairs, gfirst)
            windows = [(gfirst, min(WAVE, b1 - b0) if b0 < b1 else 1)]
            windows += [(wb, min(WAVE, b1 - wb)) for wb in range(b0 + WAVE, b1, WAVE)]
            for wb, nw in windows:
                for lane in range(WAVE):
                    g = wb + min(lane, nw - 1)
                    pj = p
                    while pfx[pj + 1] <= g:
                        pj += 1
                        check("pfx", pj + 1)
                    idx = pj * stride + (g - pfx[pj])
                    check("gpu_blocks", idx)
                    blk = clamp(c["gpu_blocks"][idx], 0, mb - 1)
                    check("seq_lens", pj // Hkv)
                    if c["use_pages"]:
                        check("gpu_pages", idx)
                        page = c["gpu_pages"][idx]
                    else:
                        check("table", pj * mb + blk)
                        page = c["table"][pj * mb + blk]
                    page = clamp(page, 0, P - 1)
                    for hh in range(BS // 16):
                        for kq in range(4):
                            for c16 in (0, 15):
                                for ks in range(D // 32):
                                    e = page * BS * D + (kq * BS + 16 * hh + c16) * 8 + ks * 4 * BS * 8
                                    check("k_pool", e + 7)
                                for cg in range(D // 16):
                                    e = ((page * (BS // 16) + hh) * D * 16 + c16 * 16 + 4 * kq
                                         + cg * 16 * 16)
                                    check("v_pool", e + 3)
                p = pair_of(pfx, npairs, min(wb + nw - 1, T - 1))
            # every pair the range touches gets a partial in slot gw + pair
            if b0 < b1:
                for pair in range(pair_of(pfx, npairs, b0), pair_of(pfx, npairs, b1 - 1) + 1):
                    if pfx[pair + 1] <= pfx[pair]:
                        continue  # (no block of the pair in the range)
                    written = c.setdefault("written", {})
                    assert gw + pair not in written, (gw, pair)  # one partial per slot
                    written[gw + pair] = pair
                    for g in range(G):
                        check("partial_o", ((gw + pair) * G + g) * D + D - 1)
                        check("partial_ml", ((gw + pair) * G + g) * 2 + 1)


def trace_reduce(c, check):
    """reduce_kernel: the covering waves' slots of every row, with the count clamped and the
    preloaded o vectors' slot index clamped into the covering range.  Beyond the addresses,
    the partials it combines (the covering slots of live waves) are exactly those the
    attention waves wrote for the pair."""
    npairs, stride, G, D, W = c["npairs"], c["stride"], c["G"], c["D"], c["W"]
    pfx = pair_prefix(c["n_gpu"], stride)
    T = pfx[npairs]
    kpre = 16
    written = c.get("written", {})
    for pair in range(npairs):
        check("n_gpu", pair)
        ng = clamp(c["n_gpu"][pair], 0, stride)
        w_lo = nslot = 0
        if ng > 0:
            w_lo = wave_of(pfx[pair], T, W)
            nslot = wave_of(pfx[pair] + ng - 1, T, W) - w_lo + 1
        for g in range(G):
            for j in range(kpre):  # the preload, indexes clamped
                jj = max(0, min(j, nslot - 1))
                check("partial_o", ((w_lo + jj + pair) * G + g) * D + D - 1)
            for j in range(nslot):  # (m, l) of the covering slots, then their o vectors
                check("partial_ml", ((w_lo + j + pair) * G + g) * 2 + 1)
                check("partial_o", ((w_lo + j + pair) * G + g) * D + D - 1)
        # a covering wave with an empty range (possible when W > T) wrote nothing
        live = {w_lo + j + pair for j in range(nslot)
                if W <= T or wave_start(w_lo + j, T, W) < wave_start(w_lo + j + 1, T, W)}
        want = {slot for slot, p in written.items() if p == pair}
        assert live == want, (pair, sorted(live), sorted(want))


def trace_select(c, check, waves=8, threads=512, batch=8, tbl_run=8):
    """select_kernel: the block count from the length, each wave's digest rows (clamped into
    its range), the block-table reads, the query parts, and the list writes."""
    B, Hkv, G, D, bs, mb, k = c["B"], c["Hkv"], c["G"], c["D"], c["BS"], c["max_blocks"], c["k"]
    row = c["per"] * D
    vec = 8
    lpr = D // vec
    bpi = WAVE // lpr
    lpb = c["per"]
    bpb = batch // lpb * bpi
    for pair in range(B * Hkv):
        s, h = divmod(pair, Hkv)
        check("seq_lens", s)
        L = c["seq_lens"][s]
        nb = min(max(int((L + bs - 1) / bs), 0), mb)      # C division truncates toward 0
        ks = min(k, nb)
        per_wave = (nb + waves - 1) // waves
        for wave in range(waves):
            wb0 = min(nb, wave * per_wave)
            wb1 = min(nb, wb0 + per_wave)
            firsts = [wb0] + [min(b + off, wb1 - 1) for b in range(wb0, wb1, 2 * bpb)
                              for off in (bpb, 2 * bpb)]
            for bf in firsts:
                for u in range(batch // lpb):
                    for bi in range(bpi):
                        b = max(min(bf + u * bpi + bi, wb1 - 1), 0)
                        for r in range(lpb):
                            check("digests", (pair * mb + b) * row + r * D + (lpr - 1) * vec + vec - 1)
        for tid in range(0, threads, 97):
            for u in range(tbl_run):
                check("table", pair * mb + max(min(tid + u * threads, nb - 1), 0))
            for part in range(c["parts"]):
                q_own = tid < G * D // 4
                check("q", s * c["row_stride"] + h * G * D + 4 * (tid if q_own else 0)
                      + part * c["part_stride"] + 3)
        for j in range(ks):
            check("lists", pair * k + j)


def trace_digest(c, check):
    """digest.hip block_count_prefix + digest_kernel: the pairs' block counts from the
    (clamped) lengths, each wave's balanced range of blocks, each lane's pair by a forward
    scan, its table entry and length, and the page reads and digest writes of resident
    blocks only (a page outside [0, P) is not resident)."""
    Hkv, mb, P, BS, D = c["Hkv"], c["max_blocks"], c["P"], c["BS"], c["D"]
    npairs = c["B"] * Hkv
    lens = c["seq_lens"]
    pfx = [0]
    for p in range(npairs):
        check("seq_lens", p // Hkv)
        L = clamp(lens[p // Hkv], 0, mb * BS)
        pfx.append(pfx[-1] + (L + BS - 1) // BS)
    Nb = pfx[npairs]
    W = c["digest_waves"]
    for gw in range(W):
        i0, i1 = gw * Nb // W, (gw + 1) * Nb // W
        if i0 >= i1:
            continue
        p = pair_of(pfx, npairs, i0)
        for w0 in range(i0, i1, WAVE):
            last_pj = p
            for lane in range(WAVE):
                g = min(w0 + lane, i1 - 1)
                pj = p
                while pfx[pj + 1] <= g:
                    pj += 1
                    assert pj < npairs
                b = g - pfx[pj]
                assert 0 <= b < mb
                slot = pj * mb + b
                check("table", slot)
                check("seq_lens", pj // Hkv)
                page = c["table"][slot]
                L = lens[pj // Hkv]
                assert min(BS, L - b * BS) >= 1
                if w0 + lane < i1 and 0 <= page < P:
                    check("k_pool", page * BS * D)
                    check("k_pool", page * BS * D + BS * D - 1)
                    check("digests", slot * c["per"] * D + c["per"] * D - 1)
                last_pj = pj
            p = last_pj


def bad_int(rng, lo, hi):
    """A value of any kind: in range, negative, just past the end, or far past it."""
    r = rng.random()
    if r < 0.5:
        return rng.randint(lo, max(lo, hi - 1))
    if r < 0.65:
        return -rng.randint(1, 1 << 20)
    if r < 0.8:
        return hi + rng.randint(0, 3)
    return rng.randint(hi, 1 << 30)


def random_case(rng, long_lists=False):
    """long_lists: few pairs with long, mostly full lists, so that a pair's blocks span
    more waves than the reduce preloads, both with more waves than blocks and with fewer."""
    Hkv = rng.choice([1, 2, 8]) if not long_lists else 1
    G = rng.choice([1, 3, 5, 8])
    D = rng.choice([64, 128])
    BS = rng.choice([16, 32, 64])
    B = rng.randint(1, 6) if not long_lists else rng.randint(1, 3)
    mb = rng.randint(1, 40) if not long_lists else rng.randint(60, 100)
    stride = rng.randint(1, 20) if not long_lists else rng.randint(40, mb)
    P = rng.randint(1, 60)
    npairs = B * Hkv
    waves_per_wg = 4
    W = waves_per_wg * rng.randint(1, 12) if not long_lists else waves_per_wg * rng.randint(8, 40)
    c = dict(B=B, Hkv=Hkv, G=G, D=D, BS=BS, max_blocks=mb, stride=stride, P=P, npairs=npairs,
             W=W, k=stride, per=rng.choice([1, 2]), parts=rng.randint(1, 5),
             digest_waves=rng.randint(1, 40), use_pages=rng.random() < 0.5)
    c["row_stride"] = Hkv * G * D
    c["part_stride"] = B * c["row_stride"]
    c["n_gpu"] = [bad_int(rng, 0, stride + 1) if not long_lists or rng.random() < 0.2
                  else rng.randint(stride // 2, stride) for _ in range(npairs)]
    c["gpu_blocks"] = [bad_int(rng, -1, mb) for _ in range(npairs * stride)]
    c["gpu_pages"] = [bad_int(rng, -1, P) for _ in range(npairs * stride)]
    c["table"] = [bad_int(rng, -1, P) for _ in range(npairs * mb)]
    c["seq_lens"] = [bad_int(rng, 0, mb * BS + 1) for _ in range(B)]
    sizes = dict(
        n_gpu=npairs, pfx=npairs + 1, gpu_blocks=npairs * stride, gpu_pages=npairs * stride,
        table=npairs * mb, seq_lens=B, k_pool=P * BS * D, v_pool=P * BS * D,
        q=c["parts"] * c["part_stride"], lists=npairs * stride,
        partial_o=(W + npairs) * G * D, partial_ml=(W + npairs) * G * 2,
        digests=npairs * mb * c["per"] * D)
    return c, sizes, waves_per_wg


def test_kernel_addresses_stay_in_bounds_on_bad_contents():
    rng = random.Random(2024)
    bad = []
    for trial in range(120):
        c, sizes, wpg = random_case(rng)

        def check(buf, i, c=c, trial=trial):
            if not 0 <= i < sizes[buf]:
                bad.append((trial, buf, i, sizes[buf]))

        trace_attention(c, wpg, check)
        trace_reduce(c, check)
        trace_select(c, check)
        trace_digest(c, check)
        assert not bad, bad[:5]


def test_pairs_spanning_many_waves_stay_in_bounds_and_match():
    """Long lists: pairs whose blocks span more than 16 waves (the reduce's preload), with
    more waves than blocks (empty waves among the covering ones) and with fewer."""
    rng = random.Random(77)
    bad = []
    seen = dict(ge=0, lt=0)
    for trial in range(60):
        c, sizes, wpg = random_case(rng, long_lists=True)
        pfx = pair_prefix(c["n_gpu"], c["stride"])
        T, W = pfx[-1], c["W"]
        for p in range(c["npairs"]):
            ng = pfx[p + 1] - pfx[p]
            if ng and T:
                n = wave_of(pfx[p] + ng - 1, T, W) - wave_of(pfx[p], T, W) + 1
                if n > 16:
                    seen["ge" if W >= T else "lt"] += 1

        def check(buf, i, c=c, trial=trial):
            if not 0 <= i < sizes[buf]:
                bad.append((trial, buf, i, sizes[buf]))

        trace_attention(c, wpg, check)
        trace_reduce(c, check)
        assert not bad, bad[:5]
    assert seen["ge"] > 0 and seen["lt"] > 0, seen


def test_bad_contents_exercise_the_clamps():
    """The random cases do reach the clamps: counts past the stride, entries and pages out
    of range, and lengths that would give a negative or oversize block count."""
    rng = random.Random(2024)
    seen = dict(count_hi=0, count_neg=0, entry=0, page=0, len_neg=0, len_hi=0)
    for _ in range(120):
        c, _, _ = random_case(rng)
        seen["count_hi"] += sum(n > c["stride"] for n in c["n_gpu"])
        seen["count_neg"] += sum(n < 0 for n in c["n_gpu"])
        seen["entry"] += sum(not 0 <= e < c["max_blocks"] for e in c["gpu_blocks"])
        seen["page"] += sum(not 0 <= p < c["P"] for p in c["gpu_pages"] + c["table"])
        seen["len_neg"] += sum(n < 0 for n in c["seq_lens"])
        seen["len_hi"] += sum(n > c["max_blocks"] * c["BS"] for n in c["seq_lens"])
    assert all(v > 0 for v in seen.values()), seen
