"""Pins of the CPU oracle against facts fixed outside it.

Each pin checks the oracle against a closed form, an invariant, brute force on a tiny
input, a hand-derived special case or an independent library routine -- never against a
retyped copy of its own formula.  The pins are plain functions raising AssertionError so
that test_oracle_pins.py runs them and test_oracle_mutations.py checks that a planted
mistake in the oracle makes at least one of them fail.

Sources: "ScoutAttention: Efficient KV Cache Offloading via Layer-Ahead CPU Pre-computation
for LLM Inference" (arXiv:2603.27138), HTML full text, cited as [HTML Sec. n]; Algorithm 1
is the layer-ahead pre-computation listing of the paper (papercache.org summary, 三).
"""

from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import torch

from oracle import scout_oracle as so

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert a.shape == b.shape and err <= tol, f"{what}: max abs err {err} > {tol}"


# ---------------------------------------------------------------- storage rounding (R10)

def pin_bf16_hand_cases():
    """Round-to-nearest-even onto the bf16 grid, worked by hand (spacing 2^-7 on [1, 2))."""
    cases = [
        (1.0 + 2.0 ** -8, 1.0),                          # tie -> even significand
        (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6),          # tie -> even (up)
        (1.0 + 2.0 ** -8 + 2.0 ** -40, 1.0 + 2.0 ** -7),  # above the tie: ONE rounding
        (-2.5, -2.5),
        ((2 - 2.0 ** -7) * 2.0 ** 127, (2 - 2.0 ** -7) * 2.0 ** 127),  # largest finite
        ((2 - 2.0 ** -8) * 2.0 ** 127, math.inf),        # tie above the largest -> inf
        (2.0 ** -133, 2.0 ** -133),                      # smallest subnormal
        (2.0 ** -134, 0.0),                              # tie to even (zero)
        (3 * 2.0 ** -134, 2.0 ** -132),                  # tie to even (up)
        (0.1, 0.10009765625),                            # 0.1 = 1.6 * 2^-4 -> 205/2048
    ]
    x = np.array([c[0] for c in cases])
    want = np.array([c[1] for c in cases])
    got = so.round_to_bf16(x)
    assert np.array_equal(got, want), f"bf16 RNE: got {got}, want {want}"


def pin_f32_hand_cases():
    """Round-to-nearest-even onto the float32 grid, worked by hand (spacing 2^-23 on [1, 2),
    so the ties sit at odd multiples of 2^-24)."""
    cases = [
        (1.0 + 2.0 ** -24, 1.0),                              # tie -> even significand
        (1.0 + 3 * 2.0 ** -24, 1.0 + 2.0 ** -22),             # tie -> even (up)
        (1.0 + 2.0 ** -24 + 2.0 ** -50, 1.0 + 2.0 ** -23),    # just above the tie: up
        (1.0 + 2.0 ** -24 - 2.0 ** -50, 1.0),                 # just below the tie: down
        (1.0 + 2.0 ** -22, 1.0 + 2.0 ** -22),                 # on the grid, not on bf16's
        (-3.0, -3.0),
        ((2 - 2.0 ** -23) * 2.0 ** 127, (2 - 2.0 ** -23) * 2.0 ** 127),  # largest finite
        ((2 - 2.0 ** -24) * 2.0 ** 127, math.inf),            # tie above the largest -> inf
        (2.0 ** -149, 2.0 ** -149),                           # smallest subnormal
        (2.0 ** -150, 0.0),                                   # tie to even (zero)
        (3 * 2.0 ** -150, 2.0 ** -148),                       # tie to even (up)
        # 0.1 = 1.6 * 2^-4: 1.6 * 2^23 = 13421772.8 rounds to 13421773
        (0.1, 13421773 * 2.0 ** -27),
    ]
    x = np.array([c[0] for c in cases])
    want = np.array([c[1] for c in cases])
    with np.errstate(over="ignore"):        # the overflow case is meant to overflow
        got = so.round_to_f32(x)
    assert np.array_equal(got, want), f"f32 RNE: got {got.tolist()}, want {want.tolist()}"


def pin_bf16_matches_library_on_float32():
    """On float32 inputs a single RNE to bf16 is what torch's float32->bfloat16 cast does."""
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        rng.standard_normal(2000)]).astype(np.float32)
    lib = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = so.round_to_bf16(x.astype(np.float64))
    assert np.array_equal(got, lib), "bf16 RNE disagrees with torch's cast on float32 inputs"


# ---------------------------------------------------------------- O1: Q_pred = W_Q X

def pin_predict_query_hand():
    """W_Q X for a column X is X W^T in row-major rows: a 2x3 by (2 features x 3) case
    worked by hand, non-square so that a transposed operand cannot pass."""
    X = np.array([[1.0, 2.0, 3.0], [4.0, 5.0, 6.0]])
    W = np.array([[1.0, 1.0, 1.0], [1.0, 0.0, -1.0]])
    want = np.array([[6.0, -2.0], [15.0, -2.0]])
    assert np.array_equal(so.predict_query(X, W), want)
    # a square case where W != W^T
    X2 = np.array([[1.0, 0.0], [0.0, 1.0], [2.0, 3.0]])
    W2 = np.array([[1.0, 2.0], [3.0, 4.0]])       # feature 0 = x0 + 2 x1; feature 1 = 3x0 + 4x1
    want2 = np.array([[1.0, 3.0], [2.0, 4.0], [8.0, 18.0]])
    assert np.array_equal(so.predict_query(X2, W2), want2)


def pin_query_heads_layout():
    """The projection output [M][Hq*d] viewed per head: element n of a row belongs to head
    n div d, channel n mod d.  A non-square case (Hq = 3, d = 4) worked by hand, so that a
    channel-major reading (head n mod Hq) cannot pass."""
    M, Hq, d = 2, 3, 4
    rows = np.arange(M * Hq * d, dtype=np.float64).reshape(M, Hq * d)
    heads = so.query_heads(rows, Hq, d)
    assert heads.shape == (M, Hq, d)
    assert heads[1].tolist() == [[12.0, 13.0, 14.0, 15.0], [16.0, 17.0, 18.0, 19.0],
                                 [20.0, 21.0, 22.0, 23.0]], heads[1]
    for m in range(M):
        for n in range(Hq * d):
            assert heads[m, n // d, n % d] == rows[m, n]
    try:
        so.query_heads(rows, Hq + 1, d)
    except ValueError:
        pass
    else:
        raise AssertionError("query_heads accepted a width that is not Hq*d")


def pin_predict_query_one_hot():
    """X = e_j picks input column j of W for every output feature."""
    rng = np.random.default_rng(3)
    W = rng.standard_normal((12, 7))
    for j in range(7):
        X = np.zeros((1, 7))
        X[0, j] = 1.0
        assert np.array_equal(so.predict_query(X, W)[0], W[:, j])


# ---------------------------------------------------------------- O2/O3: blocks and digests

def pin_blocks_hand():
    assert so.num_blocks(1024, 16) == 64
    assert so.num_blocks(33, 16) == 3
    assert so.num_blocks(16, 16) == 1
    assert so.num_blocks(1, 32) == 1
    assert list(so.block_tokens(2, 33, 16)) == [32]
    assert list(so.block_tokens(1, 33, 16)) == list(range(16, 32))


def pin_digest_mean_closed_form():
    """Keys that grow by one per token: the mean over [t0, t1) is (t0 + t1 - 1) / 2, also
    for the partial last block (divided by its own token count, reading R9)."""
    T, bs, d = 37, 8, 3
    K = np.repeat(np.arange(T, dtype=np.float64)[:, None], d, axis=1)
    K[:, 1] *= -2.0
    K[:, 2] += 0.25
    dig = so.digest_mean(K, T, bs, "f32")
    for b in range(so.num_blocks(T, bs)):
        t0, t1 = b * bs, min((b + 1) * bs, T)
        mid = (t0 + t1 - 1) / 2.0
        assert np.array_equal(dig[b], [mid, -2.0 * mid, mid + 0.25]), (b, dig[b])


def pin_digest_mean_linearity():
    """q . mean_b equals the mean over the block's tokens of q . K_t (before rounding);
    dyadic values and a last block of 8 tokens keep every step exact."""
    rng = np.random.default_rng(5)
    T, bs, d = 40, 16, 8
    K = rng.integers(-64, 64, size=(T, d)).astype(np.float64) / 16.0
    q = rng.integers(-8, 8, size=d).astype(np.float64) / 4.0
    dig = so.digest_mean(K, T, bs, "f32")
    for b in range(so.num_blocks(T, bs)):
        t = so.block_tokens(b, T, bs)
        per_token = np.array([K[i] @ q for i in t])
        assert abs(dig[b] @ q - per_token.mean()) < 1e-12


def pin_digest_mean_single_rounding():
    """A block whose float64 mean is exactly halfway between two bf16 values stores the
    even one; one just above the tie stores the upper one."""
    K = np.zeros((4, 2))
    K[:, 0] = [1.0, 1.0, 1.0, 1.0 + 4 * 2.0 ** -8]          # mean 1 + 2^-8: tie -> 1.0
    K[:, 1] = [1.0, 1.0, 1.0 + 2.0 ** -38, 1.0 + 4 * 2.0 ** -8]  # mean just above the tie
    dig = so.digest_mean(K, 4, 4, "bf16")
    assert dig[0, 0] == 1.0 and dig[0, 1] == 1.0 + 2.0 ** -7, dig


def pin_digest_mean_f32_single_rounding():
    """Float32 KV: the float64 mean of a block is rounded once to float32 -- not left
    unrounded, and not rounded onto a coarser grid (bf16, fp16).  One block of four tokens,
    one channel per case (float32 spacing 2^-23 on [1, 2)):
      mean 1 + 2^-22            on the float32 grid, not on bf16's or fp16's: kept;
      mean 1 + 2^-24 + 2^-30    just above a float32 tie: rounds up to 1 + 2^-23;
      mean 1 + 2^-24            a float32 tie: rounds to the even value 1;
    and a partial last block of two tokens whose mean 1 + 3 * 2^-24 is a tie rounding up to
    1 + 2^-22 (it divides by its own count, reading R9)."""
    K = np.ones((6, 3))
    K[3, 0] = 1.0 + 2.0 ** -20
    K[3, 1] = 1.0 + 2.0 ** -22 + 2.0 ** -28
    K[3, 2] = 1.0 + 2.0 ** -22
    K[5, :] = 1.0 + 3 * 2.0 ** -23
    dig = so.digest_mean(K, 6, 4, "f32")
    assert dig[0].tolist() == [1.0 + 2.0 ** -22, 1.0 + 2.0 ** -23, 1.0], dig[0]
    assert dig[1].tolist() == [1.0 + 2.0 ** -22] * 3, dig[1]


def pin_digest_minmax_closed_form():
    """K[t][c] = (t - c)^2 over block [t0, t1): max at an end, min 0 if c is inside."""
    T, bs, d = 20, 8, 24
    t = np.arange(T, dtype=np.float64)[:, None]
    c = np.arange(d, dtype=np.float64)[None, :]
    K = (t - c) ** 2
    dig = so.digest_minmax(K, T, bs)
    for b in range(so.num_blocks(T, bs)):
        t0, t1 = b * bs, min((b + 1) * bs, T) - 1
        for ch in range(d):
            lo = 0.0 if t0 <= ch <= t1 else min((t0 - ch) ** 2, (t1 - ch) ** 2)
            hi = max((t0 - ch) ** 2, (t1 - ch) ** 2)
            assert dig[b, 0, ch] == lo and dig[b, 1, ch] == hi, (b, ch)


# ---------------------------------------------------------------- O4: scores

def pin_minmax_score_bounds_every_token():
    """Quest's bound: for every block b, token t in b and query q,
    q . K_t <= sum_c max(q_c min_bc, q_c max_bc); summed over a GQA group too."""
    rng = np.random.default_rng(7)
    T, bs, d, G = 203, 16, 32, 3
    K = rng.standard_normal((T, d)) + rng.standard_normal((1, d))
    qs = rng.standard_normal((G, d))
    dig = so.digest_minmax(K, T, bs)
    for g in range(G):
        sig = so.score_minmax(qs[g:g + 1], dig)
        for b in range(so.num_blocks(T, bs)):
            for i in so.block_tokens(b, T, bs):
                assert K[i] @ qs[g] <= sig[b] + 1e-12
    sig_group = so.score_minmax(qs, dig)
    for b in range(so.num_blocks(T, bs)):
        for i in so.block_tokens(b, T, bs):
            assert sum(K[i] @ qs[g] for g in range(G)) <= sig_group[b] + 1e-12


def pin_scores_single_token_blocks():
    """With one token per block both digests collapse onto the key, and both scores are
    exactly the group's summed dot product with that key."""
    rng = np.random.default_rng(8)
    T, d, G = 9, 16, 4
    K = rng.integers(-20, 20, size=(T, d)).astype(np.float64) / 4.0
    qs = rng.integers(-20, 20, size=(G, d)).astype(np.float64) / 8.0
    want = np.array([sum(K[t] @ qs[g] for g in range(G)) for t in range(T)])
    assert np.array_equal(so.score_mean(qs, so.digest_mean(K, T, 1, "f32")), want)
    assert np.array_equal(so.score_minmax(qs, so.digest_minmax(K, T, 1)), want)


def pin_minmax_score_hand():
    """Two channels, one block {(1, -2), (3, 4)}: min (1, -2), max (3, 4).
    q = (1, -1): max(1, 3) + max(2, -4) = 5;  q = (-2, 0.5): max(-2, -6) + max(-1, 2) = 0."""
    dig = so.digest_minmax(np.array([[1.0, -2.0], [3.0, 4.0]]), 2, 2)
    assert so.score_minmax(np.array([[1.0, -1.0]]), dig)[0] == 5.0
    assert so.score_minmax(np.array([[-2.0, 0.5]]), dig)[0] == 0.0
    assert so.score_minmax(np.array([[1.0, -1.0], [-2.0, 0.5]]), dig)[0] == 5.0


# ---------------------------------------------------------------- O5/O6: selection

def _brute_topk(scores, k):
    """Enumerate every k-subset; keep the largest total score; among equal totals the
    lexicographically smallest sorted index tuple (lower index wins a tie)."""
    n = len(scores)
    best, best_key = None, None
    for sub in itertools.combinations(range(n), min(k, n)):
        key = (-sum(scores[i] for i in sub), sub)
        if best_key is None or key < best_key:
            best, best_key = sub, key
    return np.array(best, dtype=np.int64)


def pin_topk_brute_force():
    """The selection equals brute force over all k-subsets on small inputs (integer scores,
    so sums are exact and ties are frequent)."""
    rng = np.random.default_rng(13)
    for trial in range(300):
        n = int(rng.integers(1, 13))
        k = int(rng.integers(1, 6))
        scores = rng.integers(-3, 4, size=n).astype(np.float64)
        got = so.select_topk(scores, k)
        want = _brute_topk(list(scores), k)
        assert np.array_equal(got, want), (trial, scores, k, got, want)


def pin_topk_special_cases():
    s = np.array([0.5, 2.0, -1.0, 2.0, 3.0])
    assert so.select_topk(s, 2).tolist() == [1, 4]          # tie at 2.0 -> lower index 1
    assert so.select_topk(s, 10).tolist() == [0, 1, 2, 3, 4]  # k >= nb: all blocks
    assert so.select_topk(np.zeros(6), 3).tolist() == [0, 1, 2]
    assert so.select_topk(np.array([-0.0, 0.0, -0.0]), 1).tolist() == [0]


def _box_corner_score(q, K_block):
    """Largest q . c over the corners c of the channel-wise bounding box of a block's keys,
    by enumeration.  A linear function is largest over a box at one of its corners, so this
    is the smallest upper bound of q . K_t that sees only the box [HTML Sec. 2.2, Quest]."""
    d = K_block.shape[1]
    lo = [min(float(K_block[t, c]) for t in range(K_block.shape[0])) for c in range(d)]
    hi = [max(float(K_block[t, c]) for t in range(K_block.shape[0])) for c in range(d)]
    best = -math.inf
    for corner in itertools.product(*zip(lo, hi)):
        best = max(best, sum(float(q[c]) * corner[c] for c in range(d)))
    return best


def pin_minmax_selection_below_budget_brute_force():
    """Min/max digests with k below the block count: the selection of select_pair (and of
    forward_pair, with its split and attention) equals brute force -- each block scored as
    the sum over the group's heads of the largest q_g . c over its box corners, then the
    best k-subset by enumeration (lower index first on ties).  Dyadic keys and queries keep
    every score exact.  The cases are drawn so that mean digests select differently in
    some of them, which a pin that only sees k >= nb cannot tell apart."""
    rng = np.random.default_rng(47)
    differs = 0
    for trial in range(40):
        d, bs, G = int(rng.integers(2, 5)), int(rng.integers(1, 5)), int(rng.integers(1, 4))
        nb = int(rng.integers(3, 9))
        T = nb * bs - int(rng.integers(0, bs))          # a ragged last block
        k = int(rng.integers(1, nb))
        K = rng.integers(-12, 13, size=(T, d)).astype(np.float64) / 4.0
        V = rng.standard_normal((T, d))
        qs = rng.integers(-6, 7, size=(G, d)).astype(np.float64) / 2.0
        want_sig = []
        for b in range(nb):
            rows = K[b * bs:min((b + 1) * bs, T)]
            want_sig.append(sum(_box_corner_score(qs[g], rows) for g in range(G)))
        want = _brute_topk(want_sig, k)
        resident = rng.random(nb) < 0.5
        dig = so.digest_minmax(K, T, bs)
        sig, sel, g_blocks, c_blocks = so.select_pair(qs, dig, "minmax", k, resident)
        assert np.array_equal(sig, want_sig), (trial, sig, want_sig)
        assert sel.tolist() == want.tolist(), (trial, sel, want)
        assert g_blocks.tolist() == [b for b in want if resident[b]]
        assert c_blocks.tolist() == [b for b in want if not resident[b]]
        r = so.forward_pair(qs, qs, K, V, T, bs, dig, "minmax", k, resident, 0.5)
        assert r.selected.tolist() == want.tolist()
        rows = np.concatenate([np.arange(b * bs, min((b + 1) * bs, T)) for b in want])
        ref = _dense_ref_heads(qs, K[rows], V[rows], len(rows), 0.5)
        for g in range(G):
            _close(r.out[g].o, ref[g], 1e-12, f"min/max forward trial {trial}")
        mean_sel = _brute_topk([float(sum(qs[g] @ K[b * bs:min((b + 1) * bs, T)].mean(0)
                                          for g in range(G))) for b in range(nb)], k)
        differs += mean_sel.tolist() != want.tolist()
    assert differs >= 5, f"only {differs} cases tell min/max from mean selection"


def pin_step_minmax_hand():
    """Algorithm 1 with min/max digests, worked by hand: d = 2, blocks of 2 tokens, one
    head, W_Q^0 = I, W_Q^1 = the swap [[0, 1], [1, 0]], X^0 = (1, 0), X^1 = (0, 2), k = 1.
    Layer 0 selects with Q^0 = (1, 0): block 0 = {(1, 0), (-1, 0)} has box corners up to
    q.c = 1, block 1 = {(0.5, 0), (0.5, 0)} scores 0.5, so block 0 wins (its mean (0, 0)
    would lose to 0.5).  Its attention with Q^0 over block 0: logits (1, -1), so with
    V = e_0, e_1 the output is (1, e^-2) / (1 + e^-2), m = 1, l = 1 + e^-2.  Layer 1 selects
    with Q_pred^1 = W_Q^1 X^0 = (0, 1): block 0 = {(0, -2), (0, 1)} scores max(-2, 1) = 1,
    block 1 = {(0, 0.8), (0, 0.8)} scores 0.8 (block 0's mean (0, -0.5) would lose).  It
    attends with Q^1 = W_Q^1 X^1 = (2, 0): logits (0, 0), o = (V_0 + V_1) / 2, m = 0, l = 2."""
    I = np.eye(2)
    S = np.array([[0.0, 1.0], [1.0, 0.0]])
    V = np.array([[1.0, 0.0], [0.0, 1.0], [3.0, 3.0], [3.0, 3.0]])
    K0 = np.array([[1.0, 0.0], [-1.0, 0.0], [0.5, 0.0], [0.5, 0.0]])
    K1 = np.array([[0.0, -2.0], [0.0, 1.0], [0.0, 0.8], [0.0, 0.8]])
    dig0 = np.array([[[-1.0, 0.0], [1.0, 0.0]], [[0.5, 0.0], [0.5, 0.0]]])
    dig1 = np.array([[[0.0, -2.0], [0.0, 1.0]], [[0.0, 0.8], [0.0, 0.8]]])
    res = np.array([True, True])
    layers = [dict(X=np.array([[1.0, 0.0]]), W=I, digest=dig0, resident=res, K=K0, V=V,
                   seq_len=4, host=[so.empty_partial(2)]),
              dict(X=np.array([[0.0, 2.0]]), W=S, digest=dig1, resident=res, K=K1, V=V,
                   seq_len=4, host=[so.empty_partial(2)])]
    out = so.decode_step_pair(layers, 0, 0, 1, 2, 2, 1, 1.0, kind="minmax")
    assert out[0].scores.tolist() == [1.0, 0.5] and out[0].selected.tolist() == [0]
    e2 = math.exp(-2.0)
    _close(out[0].out[0].o, [1 / (1 + e2), e2 / (1 + e2)], 1e-15, "layer 0 output")
    assert out[0].out[0].m == 1.0 and abs(out[0].out[0].l - (1 + e2)) < 1e-15
    assert out[1].scores.tolist() == [1.0, 0.8] and out[1].selected.tolist() == [0]
    _close(out[1].out[0].o, [0.5, 0.5], 1e-15, "layer 1 output")
    assert out[1].out[0].m == 0.0 and out[1].out[0].l == 2.0


def pin_split_hand():
    sel = np.array([1, 4, 6, 9])
    res = np.zeros(10, dtype=bool)
    res[[0, 4, 9]] = True
    g, c = so.split_resident(sel, res)
    assert g.tolist() == [4, 9] and c.tolist() == [1, 6]


# ---------------------------------------------------------------- O7/O8: attention, merge

def pin_attention_closed_forms():
    rng = np.random.default_rng(17)
    d = 8
    q = rng.standard_normal(d)
    K1 = rng.standard_normal((1, d))
    V1 = rng.standard_normal((1, d))
    p = so.partial_attention(q, K1, V1, 0.5)        # one token: o = V, m = z, l = 1
    assert np.array_equal(p.o, V1[0]) and p.l == 1.0 and abs(p.m - 0.5 * K1[0] @ q) < 1e-15
    V = rng.standard_normal((5, d))                  # equal logits: o = mean V, l = T, m = 0
    p = so.partial_attention(q, np.zeros((5, d)), V, 0.3)
    _close(p.o, V.mean(axis=0), 1e-15, "equal logits")
    assert p.m == 0.0 and p.l == 5.0
    # two tokens with logits 0 and ln 3: weights 1/4, 3/4
    q2 = np.array([1.0, 0.0])
    K2 = np.array([[0.0, 0.0], [math.log(3.0), 0.0]])
    V2 = np.array([[4.0, 0.0], [0.0, 8.0]])
    p = so.partial_attention(q2, K2, V2, 1.0)
    _close(p.o, [1.0, 6.0], 1e-14, "two tokens")
    assert abs(p.m - math.log(3.0)) < 1e-15 and abs(p.l - 4.0 / 3.0) < 1e-14
    e = so.partial_attention(q, np.zeros((0, d)), np.zeros((0, d)), 1.0)
    assert e.m == -math.inf and e.l == 0.0 and not e.o.any()


def pin_attention_matches_library():
    """Dense attention equals torch's scaled_dot_product_attention in float64 (CPU)."""
    rng = np.random.default_rng(19)
    for T, d in ((1, 16), (37, 64), (300, 128)):
        q = rng.standard_normal(d)
        K = rng.standard_normal((T, d)) * 2.0
        V = rng.standard_normal((T, d))
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None, None, None, :], torch.from_numpy(K)[None, None],
            torch.from_numpy(V)[None, None]).numpy()[0, 0, 0]
        p = so.dense_attention(q, K, V, T, 1.0 / math.sqrt(d))
        _close(p.o, ref, 1e-12, "dense vs SDPA")
        z = K @ q / math.sqrt(d)
        assert abs(p.lse - float(np.log(np.exp(z - z.max()).sum()) + z.max())) < 1e-12


def pin_merge_union_invariant():
    """Merging partials over disjoint token sets equals attention over their union
    (online-softmax algebra the pages merge with); commutative, associative, and the
    empty partial is the identity."""
    rng = np.random.default_rng(23)
    for trial in range(60):
        T, d = int(rng.integers(2, 80)), int(rng.choice([4, 16, 64]))
        q = rng.standard_normal(d) * 2.0
        K = rng.standard_normal((T, d)) + rng.standard_normal((1, d)) * 3.0
        V = rng.standard_normal((T, d))
        cut = rng.permutation(T)
        a, b, c = np.split(cut, sorted(rng.choice(np.arange(1, T), 2, replace=True)))
        pa, pb, pc = (so.partial_attention(q, K[i], V[i], 0.7) for i in (a, b, c))
        whole = so.partial_attention(q, K, V, 0.7)
        for m in (so.merge(so.merge(pa, pb), pc), so.merge(pa, so.merge(pb, pc)),
                  so.merge(pc, so.merge(pb, pa))):
            _close(m.o, whole.o, 1e-12, "union o")
            assert abs(m.lse - whole.lse) < 1e-12
        e = so.empty_partial(d)
        for m in (so.merge(pa, e), so.merge(e, pa)):
            _close(m.o, pa.o, 0.0, "identity")
            assert m.m == pa.m and m.l == pa.l
    e = so.merge(so.empty_partial(4), so.empty_partial(4))
    assert e.m == -math.inf and e.l == 0.0 and not e.o.any()


# ---------------------------------------------------------------- O9: one layer, the step

def _dense_ref_heads(qs, K, V, n, scale):
    """Dense attention by the library routine for a group of query heads."""
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(np.asarray(qs))[None, :, None, :],
        torch.from_numpy(K[:n])[None, None].expand(1, len(qs), n, K.shape[1]),
        torch.from_numpy(V[:n])[None, None].expand(1, len(qs), n, V.shape[1]),
        scale=scale).numpy()[0, :, 0]
    return out


def pin_full_budget_is_dense_attention():
    """With k >= nb every block is selected, and GPU partial merged with the host partial
    is plain softmax attention over the whole context, whatever is resident
    (Transformer decode, [HTML Sec. 2.1]); both digest kinds, a ragged last block."""
    rng = np.random.default_rng(29)
    for kind in ("mean", "minmax"):
        for T, bs, G in ((100, 16, 4), (64, 16, 1), (77, 32, 5)):
            d = 32
            offsets = 0.5 * rng.standard_normal((so.num_blocks(T, bs), d))
            K = rng.standard_normal((T, d)) + np.repeat(offsets, bs, axis=0)[:T]
            V = rng.standard_normal((T, d))
            qs = rng.standard_normal((G, d))
            nb = so.num_blocks(T, bs)
            dig = so.digest_mean(K, T, bs, "f32") if kind == "mean" else so.digest_minmax(K, T, bs)
            ref = _dense_ref_heads(qs, K, V, T, 1 / math.sqrt(d))
            for res in (np.zeros(nb, bool), np.ones(nb, bool), rng.random(nb) < 0.5):
                r = so.forward_pair(qs, qs, K, V, T, bs, dig, kind, nb + 3, res, 1 / math.sqrt(d))
                assert r.selected.tolist() == list(range(nb))
                for g in range(G):
                    _close(r.out[g].o, ref[g], 1e-12, f"full budget {kind} T={T}")


def pin_sparse_equals_attention_over_selection():
    """With k < nb the merged output is attention over exactly the selected blocks' tokens
    (GPU part over S and R, host part over S minus R): checked against the library routine
    over the gathered tokens; unselected resident blocks must not contribute (R6)."""
    rng = np.random.default_rng(31)
    T, bs, d, G, k = 160, 16, 32, 2, 4
    K = rng.standard_normal((T, d))
    V = rng.standard_normal((T, d))
    qs = rng.standard_normal((G, d))
    dig = so.digest_mean(K, T, bs, "f32")
    res = np.ones(so.num_blocks(T, bs), bool)       # everything resident, incl. fillers
    r = so.forward_pair(qs, qs, K, V, T, bs, dig, "mean", k, res, 1 / math.sqrt(d))
    idx = np.concatenate([np.arange(b * bs, (b + 1) * bs) for b in r.selected])
    ref = _dense_ref_heads(qs, K[idx], V[idx], len(idx), 1 / math.sqrt(d))
    for g in range(G):
        _close(r.out[g].o, ref[g], 1e-12, "sparse = attention over selection")
    assert len(r.cpu_blocks) == 0 and len(r.gpu_blocks) == k


def pin_split_partials_indicator_hand():
    """The GPU partial covers exactly the resident selected blocks and the host partial the
    offloaded ones (Algorithm 1: A_gpu over B_gpu, A_cpu over B_cpu; R6).  Hand case with
    zero keys, so every attended token has logit 0 and weight 1: then m = 0, l = the number
    of attended tokens, and o = the mean of their values.  Values are one-hot per block
    (block b's rows all e_b), so o[b] = (tokens of b attended) / l, which shows which blocks
    each partial read.  Six blocks of 4 tokens, the last one 3 tokens long (T = 23); digests
    chosen so that the selecting query picks blocks 5, 1, 3, 4 (k = 4); blocks 1, 4 and 2
    resident.  Selection uses the selecting query, attention the other (Algorithm 1)."""
    bs, T, nb = 4, 23, 6
    K = np.zeros((T, nb))
    V = np.zeros((T, nb))
    for b in range(nb):
        V[b * bs:min((b + 1) * bs, T), b] = 1.0
    q = np.ones((1, nb))
    dig = np.array([[0.0] * nb, [5.0] + [0.0] * (nb - 1), [1.0] + [0.0] * (nb - 1),
                    [4.0] + [0.0] * (nb - 1), [3.0] + [0.0] * (nb - 1),
                    [9.0] + [0.0] * (nb - 1)])   # scores 0, 5, 1, 4, 3, 9
    res = np.array([False, True, True, False, True, False])
    # the attention query differs from the selecting one (it would pick the lowest scores);
    # with zero keys it does not change any partial
    r = so.forward_pair(q, -q, K, V, T, bs, dig, "mean", 4, res, 1.0)
    assert sorted(r.selected.tolist()) == [1, 3, 4, 5]
    assert r.gpu_blocks.tolist() == [1, 4] and r.cpu_blocks.tolist() == [3, 5]
    g, h, o = r.gpu[0], r.host[0], r.out[0]
    assert g.m == 0.0 and g.l == 8.0                       # blocks 1 and 4: 4 + 4 tokens
    assert np.array_equal(g.o, [0, 0.5, 0, 0, 0.5, 0])
    assert h.m == 0.0 and h.l == 7.0                       # blocks 3 and 5: 4 + 3 tokens
    _close(h.o, [0, 0, 0, 4 / 7, 0, 3 / 7], 1e-15, "host partial")
    assert o.m == 0.0 and o.l == 15.0                      # the union: 15 tokens
    _close(o.o, [0, 4 / 15, 0, 4 / 15, 4 / 15, 3 / 15], 1e-15, "merged")


def pin_dense_attention_indicator_hand():
    """FullKV over the first seq_len tokens: with zero keys and one-hot values per token
    position group, o is the token-count share of each group and l = seq_len (HTML Sec. 4,
    the FullKV baseline).  T = 10 tokens, groups of 3 (the last group 1 token)."""
    T, d = 10, 4
    K = np.zeros((12, d))
    V = np.zeros((12, d))
    for t in range(12):
        V[t, t // 3] = 1.0
    p = so.dense_attention(np.ones(d), K, V, T, 1.0)
    assert p.m == 0.0 and p.l == 10.0
    _close(p.o, [0.3, 0.3, 0.3, 0.1], 1e-15, "dense indicator")


def pin_layer_ahead_selection_hand():
    """Algorithm 1: layer 1 selects with Q_pred^1 = W_Q^1 X^0, not with its own Q^1, and
    attends with Q^1; layer 0 selects with Q^0.  Hand case: hidden = d = 2, one head,
    one token per block, W_Q^0 = W_Q^1 = I, X^0 = (1, 0), X^1 = (0, 1), k = 1."""
    I = np.eye(2)
    V = np.array([[5.0, 6.0], [7.0, 8.0]])
    layers = [
        dict(X=np.array([[1.0, 0.0]]), W=I, digest=np.array([[0.0, 1.0], [1.0, 0.0]]),
             resident=np.array([True, True]), K=np.array([[0.0, 1.0], [1.0, 0.0]]), V=V,
             seq_len=2, host=[so.empty_partial(2)]),
        dict(X=np.array([[0.0, 1.0]]), W=I, digest=np.array([[1.0, 0.0], [0.0, 1.0]]),
             resident=np.array([True, False]), K=np.array([[1.0, 0.0], [0.0, 1.0]]), V=V,
             seq_len=2, host=[so.Partial(np.array([1.0, -1.0]), 3.0, 2.0)]),
    ]
    out = so.decode_step_pair(layers, 0, 0, 1, 2, 1, 1, 1.0)
    # layer 0: Q^0 = (1, 0) scores blocks (0, 1) -> block 1 (key (1, 0)), resident
    assert out[0].selected.tolist() == [1] and out[0].gpu_blocks.tolist() == [1]
    # attention with Q^0 over the one token (1, 0): z = 1 -> o = V_1, m = 1, l = 1
    assert np.array_equal(out[0].out[0].o, V[1]) and out[0].out[0].m == 1.0
    # layer 1: Q_pred^1 = (1, 0) picks block 0 (its own Q^1 = (0, 1) would pick block 1)
    assert out[1].selected.tolist() == [0] and out[1].gpu_blocks.tolist() == [0]
    # attention with Q^1 = (0, 1) over key (1, 0): z = 0, o = V_0; nothing offloaded, so the
    # host partial is not merged
    assert np.array_equal(out[1].out[0].o, V[0]) and out[1].out[0].m == 0.0
    assert out[1].out[0].l == 1.0
    # make block 0 offloaded at layer 1: the output is the host partial alone
    layers[1]["resident"] = np.array([False, True])
    out = so.decode_step_pair(layers, 0, 0, 1, 2, 1, 1, 1.0)
    assert out[1].cpu_blocks.tolist() == [0] and out[1].gpu_blocks.tolist() == []
    assert np.array_equal(out[1].out[0].o, [1.0, -1.0]) and out[1].out[0].m == 3.0


def pin_step_full_budget_is_dense():
    """Every layer of the step with k >= nb and everything resident is dense attention
    with the TRUE query Q^i = W_Q^i X^i (library routine), for any layer-ahead choice."""
    rng = np.random.default_rng(37)
    L, hidden, Hq, Hkv, d, T, bs = 3, 24, 4, 2, 8, 40, 8
    G = Hq // Hkv
    layers = []
    for i in range(L):
        layers.append(dict(
            X=rng.standard_normal((2, hidden)), W=rng.standard_normal((Hq * d, hidden)) / 5,
            K=rng.standard_normal((T, d)), V=rng.standard_normal((T, d)), seq_len=T,
            resident=np.ones(so.num_blocks(T, bs), bool),
            host=[so.empty_partial(d)] * G))
        layers[-1]["digest"] = so.digest_mean(layers[-1]["K"], T, bs, "f32")
    for s in range(2):
        for h in range(Hkv):
            out = so.decode_step_pair(layers, s, h, G, d, bs, 99, 1 / math.sqrt(d))
            for i in range(L):
                Q = layers[i]["X"][s] @ layers[i]["W"].T
                qs = Q.reshape(Hq, d)[h * G:(h + 1) * G]
                ref = _dense_ref_heads(qs, layers[i]["K"], layers[i]["V"], T, 1 / math.sqrt(d))
                for g in range(G):
                    _close(out[i].out[g].o, ref[g], 1e-12, f"step layer {i}")


def pin_step_host_side_uses_predicted_query_hand():
    """Algorithm 1: the CPU side of layer i is spawned one layer ahead, so it attends the
    offloaded blocks with Q_pred^i (Q^0 at layer 0), read from the host's copy of the KV.
    Hand case of pin_layer_ahead_selection_hand with both layers' selections offloaded;
    the GPU-side rows of offloaded blocks are NaN, so reading them would show."""
    I = np.eye(2)
    V = np.array([[5.0, 6.0], [7.0, 8.0]])
    nan = np.full((2, 2), np.nan)
    layers = [
        dict(X=np.array([[1.0, 0.0]]), W=I, digest=np.array([[0.0, 1.0], [1.0, 0.0]]),
             resident=np.array([True, False]), K=nan, V=nan,
             K_host=np.array([[0.0, 1.0], [1.0, 0.0]]), V_host=V, seq_len=2),
        dict(X=np.array([[0.0, 1.0]]), W=I, digest=np.array([[1.0, 0.0], [0.0, 1.0]]),
             resident=np.array([False, True]), K=nan, V=nan,
             K_host=np.array([[1.0, 0.0], [0.0, 1.0]]), V_host=V, seq_len=2),
    ]
    out = so.decode_step_pair(layers, 0, 0, 1, 2, 1, 1, 1.0)
    # layer 0 selects block 1 (offloaded) with Q^0 = (1, 0); the CPU attends it with Q^0:
    # z = (1, 0).(1, 0) = 1, so (o, m, l) = (V_1, 1, 1) and the output is that partial
    assert out[0].cpu_blocks.tolist() == [1] and out[0].gpu_blocks.tolist() == []
    assert np.array_equal(out[0].host[0].o, V[1]) and out[0].host[0].m == 1.0
    assert np.array_equal(out[0].out[0].o, V[1]) and out[0].out[0].m == 1.0
    # layer 1 selects block 0 with Q_pred^1 = (1, 0); the CPU attends it with Q_pred^1, not
    # with Q^1 = (0, 1): z = 1 (Q^1 would give z = 0)
    assert out[1].cpu_blocks.tolist() == [0]
    assert out[1].host[0].m == 1.0 and out[1].host[0].l == 1.0
    assert np.array_equal(out[1].out[0].o, V[0]) and out[1].out[0].m == 1.0


def pin_step_host_side_merges_to_attention_over_selection():
    """With Q_pred^i = Q^i (every layer has the same X and W_Q), GPU partial over the
    resident selected blocks merged with the host's partial over the offloaded ones is
    plain softmax attention over the tokens of the whole selection (library routine), for
    any residency; a ragged last block.  Rows the other side holds are NaN on each side."""
    rng = np.random.default_rng(43)
    L, hidden, Hq, Hkv, d, T, bs, k = 3, 16, 4, 2, 8, 45, 8, 4
    G = Hq // Hkv
    nb = so.num_blocks(T, bs)
    X = rng.standard_normal((2, hidden))
    W = rng.standard_normal((Hq * d, hidden)) / 4
    layers = []
    for i in range(L):
        K = rng.standard_normal((T, d)) + rng.standard_normal(d)
        Vv = rng.standard_normal((T, d))
        res = rng.random(nb) < 0.5
        res[i % nb] = not res[i % nb]
        tok_res = np.repeat(res, bs)[:T]
        Kg, Vg, Kh, Vh = K.copy(), Vv.copy(), K.copy(), Vv.copy()
        Kg[~tok_res] = np.nan
        Vg[~tok_res] = np.nan
        Kh[tok_res] = np.nan
        Vh[tok_res] = np.nan
        layers.append(dict(X=X, W=W, digest=so.digest_mean(K, T, bs, "f32"), resident=res,
                           K=Kg, V=Vg, K_host=Kh, V_host=Vh, seq_len=T, Kfull=K, Vfull=Vv))
    scale = 1 / math.sqrt(d)
    for s in range(2):
        Q = (X[s] @ W.T).reshape(Hq, d)
        for h in range(Hkv):
            out = so.decode_step_pair(layers, s, h, G, d, bs, k, scale)
            for i in range(L):
                r = out[i]
                assert len(r.cpu_blocks) + len(r.gpu_blocks) == k
                rows = np.concatenate([np.arange(b * bs, min((b + 1) * bs, T))
                                       for b in r.selected])
                Ks, Vs = layers[i]["Kfull"][rows], layers[i]["Vfull"][rows]
                ref = _dense_ref_heads(Q[h * G:(h + 1) * G], Ks, Vs, len(rows), scale)
                for g in range(G):
                    _close(r.out[g].o, ref[g], 1e-12, f"host-side step layer {i}")


def pin_recall_hand():
    """Periodic recall, worked by hand: 8 blocks of 4 tokens (30 tokens: block 7 holds 2),
    resident {0: page 10, 2: 11, 5: 12, 6: 13}, selection B_gpu = {2}, B_cpu = {1, 3, 7};
    block 4 has no host page.  Evictable (resident, not selected, ascending): 0, 5, 6.
    With max_recall 2: block 1 takes block 0's page 10, block 3 takes block 5's page 12."""
    table = [10, -1, 11, -1, -1, 12, 13, -1]
    host = [50, 51, 52, 53, -1, 55, 56, 57]
    new, moves = so.recall_pair(table, 30, 4, [2], [1, 3, 7], host, 2)
    assert new.tolist() == [-1, 10, 11, 12, -1, -1, 13, -1]
    assert moves == [(1, 10, 51), (3, 12, 53)]
    # unlimited: block 7 takes block 6's page 13 as well
    new, moves = so.recall_pair(table, 30, 4, [2], [1, 3, 7], host, 99)
    assert new.tolist() == [-1, 10, 11, 12, -1, -1, -1, 13] and len(moves) == 3
    # a listed block that is already resident, past the sequence, or without a host page is
    # skipped; nothing to evict means nothing moves
    new, moves = so.recall_pair(table, 30, 4, [2], [0, 4, 9], host, 9)
    assert new.tolist() == table and moves == []
    new, moves = so.recall_pair(table, 30, 4, [0, 2, 5, 6], [1], host, 9)
    assert new.tolist() == table and moves == []


def pin_recall_invariants():
    """On random tables and selections: the set of pages in use is unchanged, the number of
    resident blocks is unchanged, no selected resident block loses its page, every moved
    block was offloaded and selected and is resident afterwards, and the moves are as many
    as the smallest of candidates, evictable blocks and the limit (brute force)."""
    rng = np.random.default_rng(61)
    for trial in range(200):
        nb_max = int(rng.integers(1, 40))
        bs = int(rng.integers(1, 9))
        seq_len = int(rng.integers(1, nb_max * bs + 1))
        nb = so.num_blocks(seq_len, bs)
        res = rng.random(nb_max) < rng.random()
        pages = rng.permutation(1000)[:nb_max]
        table = np.where(res, pages, -1)
        table[nb:] = -1
        host = np.where(rng.random(nb_max) < 0.9, rng.permutation(nb_max), -1)
        k = int(rng.integers(1, nb + 1))
        sel = np.sort(rng.permutation(nb)[:k])
        g, c = so.split_resident(sel, table[:nb] >= 0)
        lim = int(rng.integers(0, k + 2))
        new, moves = so.recall_pair(table, seq_len, bs, g, c, host, lim)
        used0 = sorted(int(p) for p in table if p >= 0)
        used1 = sorted(int(p) for p in new if p >= 0)
        assert used0 == used1, trial
        assert all(new[b] == table[b] for b in g), trial
        cands = [b for b in c if host[b] >= 0]
        evictable = [b for b in range(nb) if table[b] >= 0 and b not in set(sel.tolist())]
        assert len(moves) == min(len(cands), len(evictable), lim), trial
        for b, p, hp in moves:
            assert table[b] < 0 and b in set(c.tolist()) and new[b] == p and hp == host[b]


def pin_recall_due_hand():
    """The recall trigger by hand: 4 pairs, k = 8 (a budget of 32 blocks), beta = 0.12.
    3 offloaded blocks are 0.09375 (no), 4 are 0.125 (yes); the boundary 0.125 itself is not
    above beta = 0.125."""
    assert not so.recall_due([1, 1, 1, 0], 8, 0.12)
    assert so.recall_due([1, 1, 1, 1], 8, 0.12)
    assert not so.recall_due([1, 1, 1, 1], 8, 0.125)
    assert so.recall_due([0, 0, 0, 1], 8, 0.0)
    assert not so.recall_due([0, 0, 0, 0], 8, 0.0)


ALL_PINS = [v for k, v in dict(globals()).items() if k.startswith("pin_") and callable(v)]
