"""Host-side check of the balanced work split the attention kernels use.

The resident selected blocks of all (sequence, KV head) pairs are laid end to end (T in
all); wave w of W owns [floor(w T / W), floor((w + 1) T / W)).  The reduction finds the
waves that covered pair p as the non-empty waves between wave_of(first block) and
wave_of(last block), and reads the partial of wave w for pair p from slot w + p.  This test
checks, by brute force over random layouts (empty pairs, W above and below T), that those
waves are exactly the owners of p's blocks and that the slots never collide.
"""

import random


def start(w, T, W):
    return (w * T) // W


def wave_of(g, T, W):
    return ((g + 1) * W + T - 1) // T - 1


def test_balanced_split_bookkeeping():
    rng = random.Random(1)
    for _ in range(3000):
        npairs, W = rng.randint(1, 40), rng.randint(1, 300)
        n = [rng.choice([0, 0, 1, 2, 5, 17, 64]) for _ in range(npairs)]
        pfx = [0]
        for x in n:
            pfx.append(pfx[-1] + x)
        T = pfx[-1]
        if T == 0:
            continue
        owner = {}
        for w in range(W):
            for g in range(start(w, T, W), start(w + 1, T, W)):
                owner[g] = w
        assert len(owner) == T
        slots = set()
        for p in range(npairs):
            if n[p] == 0:
                continue
            lo, hi = wave_of(pfx[p], T, W), wave_of(pfx[p] + n[p] - 1, T, W)
            owners = {owner[g] for g in range(pfx[p], pfx[p] + n[p])}
            covering = {w for w in range(lo, hi + 1) if start(w, T, W) < start(w + 1, T, W)}
            assert owners == covering
            for w in owners:
                assert w + p not in slots
                slots.add(w + p)
