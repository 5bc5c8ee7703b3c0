"""Pins for the oracle's budget, allocation, quantize-and-pack, GEMM and KV.

Allocation follows gist.science/nl technical summary §2.3 (sort by score,
top 32 columns at 8 bits, budgeted 6-bit columns, rest at 4 bits) with
blocks kept at one width (§2.3, last paragraph). The GEMM is the plain
definition Y = deq(A) deq(W)^T. Pins: the pages' budget facts
(tests/golden/budget_from_pages.json), Python's own sort on the same key,
an independent numpy bit unpacker, exact integer matmuls and brute-force
fp64 sums.
"""
import json
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------- budget
def test_budget_golden_from_pages(orc):
    with open(os.path.join(GOLDEN, "budget_from_pages.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        n8, n6, n4 = orc.budget_blocks(c["K"], c["bp8"], c["bp6"])
        nb = c["K"] // 32
        assert n8 + n6 + n4 == nb
        if "expect_blocks" in c:
            assert [n8, n6, n4] == c["expect_blocks"], c["cite"]
        if "expect_n8_at_least" in c:
            assert n8 >= c["expect_n8_at_least"], c["cite"]
        if "max_avg_bits" in c:
            assert (8 * n8 + 6 * n6 + 4 * n4) / nb <= c["max_avg_bits"]


def test_budget_never_exceeds_average(orc):
    rng = np.random.default_rng(0)
    for _ in range(3000):
        K = 32 * int(rng.integers(1, 1000))
        bp8 = int(rng.integers(0, 3000))
        bp6 = int(rng.integers(0, 10001 - bp8))
        n8, n6, n4 = orc.budget_blocks(K, bp8, bp6)
        nb = K // 32
        assert min(n8, n6, n4) >= 0 and n8 + n6 + n4 == nb
        B = 4 + 4 * bp8 / 1e4 + 2 * bp6 / 1e4
        assert (8 * n8 + 6 * n6 + 4 * n4) / nb <= B + 1e-12
        # one 8-bit block is kept whenever the budget can pay for it
        if bp8 > 0 and nb * (2 * bp8 + bp6) // 10000 >= 2:
            assert n8 >= 1


def test_budget_config_table(orc):
    # the per-layer budgets of the benchmark workloads (8/6/4-bit column shares)
    assert orc.budget_blocks(256, 500, 1500) == (1, 0, 7)
    assert orc.budget_blocks(1024, 500, 1500) == (1, 6, 25)
    assert orc.budget_blocks(4096, 500, 1500) == (6, 20, 102)
    assert orc.budget_blocks(8192, 500, 1500) == (12, 40, 204)
    assert orc.budget_blocks(28672, 500, 1500) == (44, 136, 716)
    assert orc.budget_blocks(4096, 300, 1000) == (3, 14, 111)
    assert orc.budget_blocks(14336, 800, 2000) == (35, 91, 322)


def test_budget_rejects_bad(orc):
    for args in [(100, 0, 0), (0, 0, 0), (256, -1, 0), (256, 6000, 5000)]:
        with pytest.raises(ValueError):
            orc.budget_blocks(*args)


# ------------------------------------------------------------------- allocate
def py_allocate(score, n8, n6):
    K = len(score)
    key = lambda k: (-score[k], k)            # score descending, index ascending
    order = sorted(range(K), key=key)
    bits = np.full(K, 4, np.uint8)
    bits[order[:32 * n8]] = 8
    bits[order[32 * n8:32 * (n8 + n6)]] = 6
    perm = [k for c in (8, 6, 4) for k in range(K) if bits[k] == c]
    return bits, np.array(perm, np.int32)


@pytest.mark.parametrize("K,bp8,bp6", [(256, 500, 1500), (1024, 500, 1500), (4096, 300, 1000),
                                       (96, 0, 0), (160, 2000, 3000)])
def test_allocate_matches_python_sort(orc, K, bp8, bp6):
    rng = np.random.default_rng(K + bp8)
    s = rng.random(K) ** 3
    s[rng.integers(0, K, K // 8)] = s[0]         # ties
    n8, n6, _ = orc.budget_blocks(K, bp8, bp6)
    bits, perm = orc.allocate(s, bp8, bp6)
    rb, rp = py_allocate(s, n8, n6)
    assert np.array_equal(bits, rb) and np.array_equal(perm, rp)
    assert np.array_equal(np.sort(perm), np.arange(K))           # bijection
    for c, n in ((8, n8), (6, n6)):
        assert (bits == c).sum() == 32 * n
    # blocks of the permuted order hold one width each
    pb = bits[perm].reshape(-1, 32)
    assert np.all(pb == pb[:, :1])


def test_allocate_all4_is_identity(orc):
    s = np.random.default_rng(9).random(512)
    bits, perm = orc.allocate(s, 0, 0)
    assert np.all(bits == 4) and np.array_equal(perm, np.arange(512))


def test_allocate_nonfinite_order(orc):
    # NaN ranks above +Inf, which ranks above every finite score; ties by index
    K = 128
    s = np.zeros(K)
    s[40], s[50], s[60] = np.nan, np.inf, 1e300
    s[70:100] = 1.0
    bits, perm = orc.allocate(s, 2500, 0)       # nb=4, U=2 -> one 8-bit block
    assert set(np.flatnonzero(bits == 8)) == {40, 50, 60} | set(range(70, 99))
    s[98] = np.inf                               # Inf at 98 pushes the 1.0 at 99 out
    bits, _ = orc.allocate(s, 2500, 0)
    assert bits[98] == 8 and bits[97] == 8 and bits[99] == 4


# ------------------------------------------------------------ quantize + pack
def np_unpack(P):
    """Independent numpy unpacker of the documented plane layout."""
    q8, q6, q4, sc = P["q8"], P["q6"], P["q4"], P["sc"]
    R = sc.shape[0]
    parts = [q8.astype(np.int32)]
    if q6.shape[1]:
        b = q6.reshape(R, -1, 3).astype(np.uint32)
        w = b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16)
        f = np.stack([(w >> (6 * i)) & 63 for i in range(4)], -1).astype(np.int32)
        parts.append(np.where(f >= 32, f - 64, f).reshape(R, -1))
    if q4.shape[1]:
        lo = (q4 & 15).astype(np.int32)
        hi = (q4 >> 4).astype(np.int32)
        f = np.stack([lo, hi], -1)
        parts.append(np.where(f >= 8, f - 16, f).reshape(R, -1))
    return np.concatenate(parts, axis=1)


def test_quantize_planes_match_block_quantizer(orc):
    rng = np.random.default_rng(12)
    R, K = 9, 1024
    X = (rng.standard_normal((R, K)) * rng.choice([1, 4, 50], K)).astype(np.float32)
    h = orc.calibrate(X)
    W = (rng.standard_t(4, (64, K)) * 0.02).astype(np.float32)
    n8, n6, n4 = orc.budget_blocks(K, 500, 1500)
    bits, perm = orc.allocate(orc.score(W, h), 500, 1500)
    P = orc.quantize(X, perm, n8, n6, n4)
    codes = np_unpack(P)
    assert np.array_equal(codes, orc.unpack(P))
    for r in range(R):
        for b in range(K // 32):
            m = 8 if b < n8 else (6 if b < n8 + n6 else 4)
            c, s = orc.quantize_block(X[r, perm[32 * b:32 * b + 32]], m)
            assert np.array_equal(codes[r, 32 * b:32 * b + 32], c) and P["sc"][r, b] == s
    # gathering first and quantising with the identity gives the same planes
    P2 = orc.quantize(np.ascontiguousarray(X[:, perm]), None, n8, n6, n4)
    for key in ("q8", "q6", "q4", "sc"):
        assert np.array_equal(P[key], P2[key])


def test_all4_map_is_uniform_mxint4(orc):
    rng = np.random.default_rng(13)
    X = rng.standard_normal((5, 256)).astype(np.float32)
    bits, perm = orc.allocate(rng.random(256), 0, 0)
    P = orc.quantize(X, perm, 0, 0, 8)
    codes = np_unpack(P)
    for r in range(5):
        for b in range(8):
            c, s = orc.quantize_block(X[r, 32 * b:32 * b + 32], 4)
            assert np.array_equal(codes[r, 32 * b:32 * b + 32], c) and P["sc"][r, b] == s


def test_kv_is_uniform_4bit_along_head_dim(orc):
    rng = np.random.default_rng(14)
    kv = rng.standard_normal((3, 2, 64)).astype(np.float32)
    codes, scales = orc.quantize_kv(kv)
    P = orc.quantize(kv.reshape(6, 64), None, 0, 0, 2)
    assert np.array_equal(codes.reshape(6, 32), P["q4"]) and np.array_equal(scales.reshape(6, 2), P["sc"])


# ------------------------------------------------------------------------ GEMM
def deq_matrix(P):
    codes = np_unpack(P).astype(np.float64)
    return codes * np.repeat(2.0 ** (P["sc"].astype(np.int64) - 127), 32, axis=1)


def test_gemm_brute_force_fsum(orc):
    rng = np.random.default_rng(15)
    M, N, K = 7, 5, 1024
    X = (rng.standard_normal((M, K)) * rng.choice([1, 4, 50], K)).astype(np.float32)
    W = (rng.standard_t(4, (N, K)) * 0.02).astype(np.float32)
    n8, n6, n4 = orc.budget_blocks(K, 500, 1500)
    _, perm = orc.allocate(orc.score(W, orc.calibrate(X)), 500, 1500)
    A, B = orc.quantize(X, perm, n8, n6, n4), orc.quantize(W, perm, n8, n6, n4)
    Y, Yabs = orc.mixed_gemm(A, B)
    da, dw = deq_matrix(A), deq_matrix(B)
    for t in range(M):
        for n in range(N):
            exact = math.fsum(da[t] * dw[n])      # products exact in fp64
            assert abs(Y[t, n] - exact) <= 1e-14 * Yabs[t, n]
            assert Yabs[t, n] == pytest.approx(math.fsum(np.abs(da[t] * dw[n])), rel=1e-14)


def test_gemm_equal_scales_is_integer_matmul(orc):
    rng = np.random.default_rng(16)
    M, N, K = 6, 9, 256
    ca = rng.integers(-7, 8, (M, K))
    cw = rng.integers(-7, 8, (N, K))
    ca[:, ::32] = 7
    cw[:, ::32] = -7
    X = (ca * 2.0 ** -3).astype(np.float32)
    W = (cw * 2.0 ** 2).astype(np.float32)
    A, B = orc.quantize(X, None, 0, 0, 8), orc.quantize(W, None, 0, 0, 8)
    Y, _ = orc.mixed_gemm(A, B)
    assert np.array_equal(Y, (ca.astype(np.int64) @ cw.T.astype(np.int64)) * 2.0 ** -1)


def test_gemm_power_of_two_equivariance(orc):
    rng = np.random.default_rng(17)
    X = rng.standard_normal((4, 512)).astype(np.float32)
    W = (rng.standard_t(4, (6, 512)) * 0.02).astype(np.float32)
    n8, n6, n4 = orc.budget_blocks(512, 500, 1500)
    _, perm = orc.allocate(orc.score(W, orc.calibrate(X)), 500, 1500)
    B = orc.quantize(W, perm, n8, n6, n4)
    Y, _ = orc.mixed_gemm(orc.quantize(X, perm, n8, n6, n4), B)
    Y2, _ = orc.mixed_gemm(orc.quantize((X * np.float32(16)).astype(np.float32), perm, n8, n6, n4), B)
    assert np.array_equal(Y2, 16 * Y)


def test_gemm_all4_equals_uniform(orc):
    rng = np.random.default_rng(18)
    X = rng.standard_normal((3, 128)).astype(np.float32)
    W = rng.standard_normal((4, 128)).astype(np.float32)
    _, perm = orc.allocate(rng.random(128), 0, 0)
    Y, _ = orc.mixed_gemm(orc.quantize(X, perm, 0, 0, 4), orc.quantize(W, perm, 0, 0, 4))
    ref = np.zeros((3, 4))
    for t in range(3):
        for n in range(4):
            acc = []
            for b in range(4):
                ca, sa = orc.quantize_block(X[t, 32 * b:32 * b + 32], 4)
                cw, sw = orc.quantize_block(W[n, 32 * b:32 * b + 32], 4)
                acc.append(int(np.dot(ca.astype(np.int64), cw.astype(np.int64))) * 2.0 ** (sa + sw - 254))
            ref[t, n] = math.fsum(acc)
    assert np.allclose(Y, ref, rtol=1e-15, atol=0)
