"""Pins for the oracle's layer-wise allocation (section 11): the single-layer
output error and the budget under one global parameter R.

gist.science/nl "Technische Samenvatting" §2.1 (layer sensitivity) and §2.3
(one 8-bit block per layer, 6-bit columns in proportion to the layer's
sensitivity scaled by a global R to meet the average bitwidth B). The pages
print no worked example, so the values below follow from the definition and
from identities that do not share the oracle's arithmetic.
"""
import itertools
import math

import numpy as np
import pytest

import oracle as orc


# ------------------------------------------------------------ output error
def test_output_error_brute_force_tiny():
    rng = np.random.default_rng(11)
    X = rng.standard_normal((3, 32)).astype(np.float32)
    W = rng.standard_normal((2, 32)).astype(np.float32)
    Yq = rng.standard_normal((3, 2))
    ref = 0.0
    for t in range(3):
        for n in range(2):
            y = 0.0
            for k in range(32):
                y += float(X[t, k]) * float(W[n, k])
            ref += (y - Yq[t, n]) ** 2
    assert orc.output_error(X, W, Yq) == pytest.approx(ref, rel=1e-12)


def test_output_error_gram_identity():
    # with Yq = 0: ||X W^T||_F^2 = sum_ij (X^T X)_ij (W^T W)_ij
    rng = np.random.default_rng(12)
    X = rng.standard_normal((20, 64)).astype(np.float32)
    W = rng.standard_normal((9, 64)).astype(np.float32)
    Xd, Wd = X.astype(np.float64), W.astype(np.float64)
    gram = float(np.sum((Xd.T @ Xd) * (Wd.T @ Wd)))
    assert orc.output_error(X, W, np.zeros((20, 9))) == pytest.approx(gram, rel=1e-10)


def test_output_error_zero_and_scaling():
    rng = np.random.default_rng(13)
    X = rng.integers(-8, 9, (7, 96)).astype(np.float32)
    W = rng.integers(-8, 9, (5, 96)).astype(np.float32)
    exact = [[sum(int(X[t, k]) * int(W[n, k]) for k in range(96)) for n in range(5)] for t in range(7)]
    assert orc.output_error(X, W, np.array(exact, np.float64)) == 0.0
    Yq = rng.standard_normal((7, 5))
    e = orc.output_error(X, W, Yq)
    assert orc.output_error(X * 2, W, Yq * 2) == 4 * e
    assert orc.output_error(X, W * 0.5, Yq * 0.5) == e / 4


# ------------------------------------------------------------ layer budget
def test_layer_budget_hand_example():
    # Two layers of 1 x 128 weights (4 blocks each), S = (1, 3). Extra bits
    # above 4: an 8-bit block +128, a 6-bit block +64; budget floor((B-4)*256).
    # Breakpoints (j - 1/2)/S: layer 1 at 1/6, 1/2, 5/6; layer 0 at 1/2, 3/2,
    # 5/2 (the two at 1/2 are taken together).
    S, rows, K = [1.0, 3.0], [1, 1], [128, 128]
    cases = {
        5.0: ([[1, 0, 3], [1, 0, 3]], 0.0),            # 256: the 8-bit blocks only
        5.25: ([[1, 0, 3], [1, 1, 2]], 0.5 / 3),        # 320: + layer 1 block 1
        5.5: ([[1, 0, 3], [1, 1, 2]], 0.5 / 3),         # 384: the pair at 1/2 needs 448
        5.75: ([[1, 1, 2], [1, 2, 1]], 0.5),            # 448: + the pair at 1/2
        6.5: ([[1, 3, 0], [1, 3, 0]], 2.5),             # 640: everything
        8.0: ([[1, 3, 0], [1, 3, 0]], 2.5),
    }
    for B, (blocks, R) in cases.items():
        got, gR = orc.layer_budget(S, rows, K, B)
        assert got.tolist() == blocks, B
        assert gR == R, B
    with pytest.raises(ValueError):
        orc.layer_budget(S, rows, K, 4.9)              # 230 < 256 for the 8-bit blocks


def _extra_bits(blocks, rows):
    return sum(32 * r * (4 * b[0] + 2 * b[1]) for b, r in zip(blocks, rows))


def _random_case(rng):
    L = int(rng.integers(1, 6))
    K = (32 * rng.integers(1, 40, L)).astype(np.int64)
    rows = rng.integers(1, 300, L).astype(np.int64)
    S = rng.exponential(1.0, L) * rng.choice([1.0, 0.0], L, p=[0.85, 0.15])
    total = float(np.sum(rows * K))
    lo = 4.0 + float(np.sum(128 * rows)) / total
    B = float(rng.uniform(lo, min(8.0, lo + 2.5)))
    return S, rows, K, B


def test_layer_budget_invariants_random():
    rng = np.random.default_rng(14)
    for _ in range(300):
        S, rows, K, B = _random_case(rng)
        total = float(np.sum(rows * K))
        allowed = math.floor((B - 4.0) * total)
        blocks, R = orc.layer_budget(S, rows, K, B)
        nb = K // 32
        assert (blocks[:, 0] == 1).all()
        assert (blocks.sum(1) == nb).all() and (blocks >= 0).all()
        assert _extra_bits(blocks, rows) <= allowed
        # n6 = number of breakpoints (j - 1/2)/S at or below R
        for l in range(len(S)):
            want = 0 if S[l] == 0 else sum(1 for j in range(1, nb[l]) if (j - 0.5) / S[l] <= R)
            assert blocks[l, 1] == want
        # maximal: the next group of breakpoints does not fit
        nxt = [((j - 0.5) / S[l], l) for l in range(len(S)) if S[l] > 0
               for j in range(1, nb[l]) if (j - 0.5) / S[l] > R]
        if nxt:
            key = min(k for k, _ in nxt)
            add = sum(64 * rows[l] for k, l in nxt if k == key)
            assert _extra_bits(blocks, rows) + add > allowed


def test_layer_budget_monotone_and_scale_free():
    rng = np.random.default_rng(15)
    for _ in range(100):
        S, rows, K, B = _random_case(rng)
        b1, R1 = orc.layer_budget(S, rows, K, B)
        b2, _ = orc.layer_budget(S, rows, K, min(8.0, B + 0.3))
        assert (b2[:, 1] >= b1[:, 1]).all()
        b3, R3 = orc.layer_budget(np.asarray(S) * 8.0, rows, K, B)   # powers of two: exact
        assert (b3 == b1).all() and R3 == R1 / 8.0


def test_layer_budget_brute_force():
    # every candidate R (0 and all breakpoints), the largest feasible wins
    rng = np.random.default_rng(16)
    for _ in range(60):
        L = int(rng.integers(1, 4))
        K = (32 * rng.integers(1, 6, L)).astype(np.int64)
        rows = rng.integers(1, 5, L).astype(np.int64)
        S = rng.integers(0, 5, L).astype(np.float64)
        total = float(np.sum(rows * K))
        B = float(rng.uniform(4.0 + float(np.sum(128 * rows)) / total, 8.0))
        allowed = math.floor((B - 4.0) * total)
        nb = K // 32
        cands = sorted({0.0} | {(j - 0.5) / S[l] for l in range(L) if S[l] > 0 for j in range(1, nb[l])})
        best = None
        for R in cands:
            blocks = [[1, 0 if S[l] == 0 else min(nb[l] - 1, sum(1 for j in range(1, nb[l]) if (j - 0.5) / S[l] <= R)), 0]
                      for l in range(L)]
            for l in range(L):
                blocks[l][2] = nb[l] - 1 - blocks[l][1]
            if _extra_bits(blocks, rows) <= allowed:
                best = (blocks, R)
        got, R = orc.layer_budget(S, rows, K, B)
        assert got.tolist() == best[0] and R == best[1]


# ------------------------------------------------------- allocate with counts
def test_allocate_blocks_matches_budgeted_allocate():
    rng = np.random.default_rng(17)
    for K, bp in itertools.product((256, 1024, 4096), ((500, 1500), (0, 0), (10000, 0), (300, 1000))):
        score = rng.exponential(1.0, K)
        n8, n6, _ = orc.budget_blocks(K, *bp)
        b1, p1 = orc.allocate(score, *bp)
        b2, p2 = orc.allocate_blocks(score, n8, n6)
        assert (b1 == b2).all() and (p1 == p2).all()
    with pytest.raises(ValueError):
        orc.allocate_blocks(np.zeros(64), 2, 1)
