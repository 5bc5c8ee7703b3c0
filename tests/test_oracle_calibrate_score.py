"""Pins for the oracle's calibration (Hessian diagonal) and column score.

Hdiag = diag(X^T X) (gist.science/nl technical summary §2.1). The pins are
the mathematics of that definition: numpy's fp64 X^T X, the correctly
rounded sum (math.fsum), exact integer arithmetic, and a hand-computed case
that fixes the documented summation order. The score
score_k = Hdiag_k * sum_n (W - Q4 W)[n,k]^2 is pinned by a brute-force
residual, by exactly representable columns (score 0) and by exact
power-of-two scaling laws.
"""
import math

import numpy as np
import pytest


def outlier_X(rng, M, K, n_ext=2, n_mild=8):
    g = np.ones(K, np.float32)
    idx = rng.permutation(K)
    g[idx[:n_ext]] = 50
    g[idx[n_ext:n_ext + n_mild]] = 4
    return (rng.standard_normal((M, K)).astype(np.float32) * g).astype(np.float32)


def test_hdiag_matches_numpy_and_fsum(orc):
    rng = np.random.default_rng(1)
    X = outlier_X(rng, 777, 96)
    h = orc.calibrate(X)
    X64 = X.astype(np.float64)
    ref = np.diagonal(X64.T @ X64)
    assert np.allclose(h, ref, rtol=1e-12, atol=0)
    for k in range(X.shape[1]):
        exact = math.fsum(float(x) * float(x) for x in X64[:, k])
        assert abs(h[k] - exact) <= 1e-12 * exact


def test_hdiag_exact_on_integers(orc):
    rng = np.random.default_rng(2)
    X = rng.integers(-1000, 1000, (1500, 64)).astype(np.float32)
    h = orc.calibrate(X)
    exact = [sum(int(x) * int(x) for x in X[:, k]) for k in range(64)]
    assert h.tolist() == [float(e) for e in exact]


def test_hdiag_accumulates_across_calls(orc):
    rng = np.random.default_rng(3)
    X = rng.integers(-50, 50, (900, 32)).astype(np.float32)
    h = orc.calibrate(X[:300])
    orc.calibrate(X[300:], h)
    assert np.array_equal(h, orc.calibrate(X))      # exact on integers
    Xr = outlier_X(rng, 600, 32)
    h = np.full(32, 0.25)
    orc.calibrate(Xr, h)
    ref = np.array([math.fsum([0.25] + [float(x) ** 2 for x in Xr[:, k]]) for k in range(32)])
    assert np.allclose(h, ref, rtol=1e-12, atol=0)


def test_hdiag_documented_order(orc):
    # One column, 9 rows: x0 = 2^27 (square 2^54, fp64 ulp 4), x1..x8 = 1.
    # Documented order: p0 = rows {0, 8} = 2^54 + 1 -> 2^54 (tie to even);
    # p1..p7 = 1; ((p0+p1)+(p2+p3)) = (2^54+1 -> 2^54) + 2 -> 2^54 (tie to even);
    # ((p4+p5)+(p6+p7)) = 4; total 2^54 + 4.
    # (A plain sequential sum gives 2^54; the exact value is 2^54 + 8.)
    X = np.ones((9, 1), np.float32)
    X[0, 0] = 2.0 ** 27
    h = orc.calibrate(X)
    assert h[0] == 2.0 ** 54 + 4
    # chunks are 256 rows: a second chunk's total is added after the first's
    X2 = np.ones((257, 1), np.float32)
    X2[256, 0] = 2.0 ** 27
    # chunk 0: 256 ones -> 256; chunk 1: 2^54; 256 + 2^54 is exact
    assert orc.calibrate(X2)[0] == 2.0 ** 54 + 256


def test_hdiag_documented_run_order(orc):
    # One column, 32 chunks (8192 rows). Chunk 0: rows 0 and 8 hold 2^26, so
    # p0 = 2^52 + 2^52 = 2^53 exactly and chunk total T0 = 2^53 (fp64 ulp 2);
    # chunks 8..31 hold one 1 each (T = 1), all other entries are 0.
    # Documented order, runs of 16 chunks: run 0 = 2^53 + 1 (x8, each a tie
    # to even -> 2^53) = 2^53; run 1 = 16 (exact); Hdiag = 0 + 2^53 + 16.
    # Chunk totals added one by one give 2^53; runs of 8 give 2^53 + 24,
    # runs of 32 give 2^53; the exact value is 2^53 + 24.
    X = np.zeros((32 * 256, 1), np.float32)
    X[0, 0] = X[8, 0] = 2.0 ** 26
    X[256 * np.arange(8, 32), 0] = 1.0
    h = orc.calibrate(X)
    assert h[0] == 2.0 ** 53 + 16
    # each call starts its own runs: Hdiag = 2^53 from a first call, then a
    # second call of 16 chunks holding one 1 each: its run total 16 is added
    # whole (2^53 + 16); adding its chunk totals one by one would give 2^53
    h = orc.calibrate(X[:256])
    X3 = np.zeros((16 * 256, 1), np.float32)
    X3[256 * np.arange(16), 0] = 1.0
    orc.calibrate(X3, h)
    assert h[0] == 2.0 ** 53 + 16


def test_hdiag_empty_and_zero(orc):
    h = orc.calibrate(np.zeros((0, 32), np.float32))
    assert not h.any()
    h = orc.calibrate(np.zeros((5, 32), np.float32))
    assert not h.any()


# ------------------------------------------------------------------------- score
def brute_residual_sq(W):
    """sum over rows of the squared uniform-MXINT4 residual, by brute-force code search."""
    N, K = W.shape
    E = np.zeros(K)
    cols = [[] for _ in range(K)]
    for n in range(N):
        for b in range(K // 32):
            v = W[n, 32 * b:32 * b + 32].astype(np.float64)
            amax = np.abs(v).max()
            if amax == 0:
                for j in range(32):
                    cols[32 * b + j].append(0.0)
                continue
            s = -127
            while not (amax / 2.0 ** s < 8):     # smallest s with amax/2^s < 8 ...
                s += 1
            while s > -127 and amax / 2.0 ** (s - 1) < 8:
                s -= 1
            grid = np.arange(-7, 8) * 2.0 ** s
            for j in range(32):
                d = np.abs(v[j] - grid)
                best = np.flatnonzero(d == d.min())
                c = best[0] if len(best) == 1 else [x for x in best if (x - 7) % 2 == 0][0]
                cols[32 * b + j].append((v[j] - grid[c]) ** 2)
    for k in range(K):
        E[k] = math.fsum(cols[k])
    return E


def test_score_unit_hdiag_is_mxint4_error(orc):
    rng = np.random.default_rng(4)
    W = (rng.standard_t(4, (40, 64)) * 0.02).astype(np.float32)
    s = orc.score(W, np.ones(64))
    ref = brute_residual_sq(W)
    assert np.allclose(s, ref, rtol=1e-12, atol=0)


def test_score_representable_columns_are_zero(orc):
    rng = np.random.default_rng(5)
    N, K = 300, 128
    c = rng.integers(-7, 8, (N, K))
    c[:, ::32] = 7                               # every block has a top-binade max code
    sexp = rng.integers(-20, 5, (N, K // 32))
    W = (c * 2.0 ** np.repeat(sexp, 32, axis=1)).astype(np.float32)
    h = rng.random(K) + 0.5
    assert not orc.score(W, h).any()


def test_score_power_of_two_laws(orc):
    rng = np.random.default_rng(6)
    W = (rng.standard_t(4, (520, 96)) * 0.02).astype(np.float32)
    h = orc.calibrate(outlier_X(rng, 300, 96))
    s = orc.score(W, h)
    assert np.array_equal(orc.score((W * np.float32(8.0)).astype(np.float32), h), s * 64.0)
    assert np.array_equal(orc.score(W, h * 0.5), s * 0.5)
    assert np.all(s >= 0)


def test_score_ranks_outlier_channels_first(orc):
    # Sanity (not a guarantee): with the tiny-layer shape, the two x50 channels
    # rank first and the eight x4 channels next.
    rng = np.random.default_rng(7)
    K = 256
    g = np.ones(K, np.float32)
    idx = rng.permutation(K)
    g[idx[:2]] = 50
    g[idx[2:10]] = 4
    X = (rng.standard_normal((64, K)).astype(np.float32) * g).astype(np.float32)
    W = (rng.standard_t(4, (256, K)) * 0.02).astype(np.float32)
    s = orc.score(W, orc.calibrate(X))
    order = np.argsort(-s, kind="stable")
    assert set(order[:2]) == set(idx[:2])
    assert set(order[2:10]) == set(idx[2:10])
