"""Seeded random sweep of the whole path against the oracle, through the C ABI.

Each case draws K = 32 j (j in 1..64), M and N from {1, 7, 33, 64, 65, 1000},
a random 8/6-bit budget (including single-width and all-4-bit budgets), bf16
or fp32 inputs stored with a leading dimension larger than K, and the
outlier-channel activation and Student-t weight models. It then runs
calibrate, score, allocate, quantize of X and W, and the product through
mxs_mixed_gemm, mxs_mixed_gemm_mx and mxs_mixed_gemm_fused, and compares with
the oracle: bit for bit up to the planes, Y componentwise within 1e-5 of the
fp64 definition. The sweep stops at the first case that fails and names it.
"""
import numpy as np
import pytest
import torch

from bit_gemm_hdiag_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SIZES = (1, 7, 33, 64, 65, 1000)
N_CASES = 160


def draw_case(rng):
    K = 32 * int(rng.integers(1, 65))
    M = int(rng.choice(SIZES))
    N = int(rng.choice(SIZES))
    kind = int(rng.integers(0, 6))
    if kind == 0:
        bp8, bp6 = 0, 0
    elif kind == 1:
        bp8, bp6 = 10000, 0
    elif kind == 2:
        bp8, bp6 = 0, 10000
    else:
        bp8 = int(rng.integers(0, 3001))
        bp6 = int(rng.integers(0, 10001 - bp8))
    dtype = torch.bfloat16 if rng.integers(0, 2) else torch.float32
    padx = int(rng.integers(1, 17))
    padw = int(rng.integers(1, 17))
    return K, M, N, bp8, bp6, dtype, padx, padw


def strided(t, pad):
    """A copy of t living in a wider buffer: row stride K + pad, offset 1 element."""
    R, K = t.shape
    buf = torch.zeros((R, K + pad + 1), dtype=t.dtype, device=t.device)
    buf[:, 1:1 + K] = t
    return buf[:, 1:1 + K]


def gemm_ok(Y, Yref, Yabs):
    y = Y.cpu().numpy().astype(np.float64)
    err = np.abs(y - Yref)
    ok = err <= 1e-5 * Yabs
    return bool(ok.all()), float((err / np.maximum(Yabs, 1e-300)).max()) if err.size else 0.0


def test_random_sweep(orc):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import bit_gemm_hdiag_amd as mx
    rng = np.random.default_rng(20261203)
    for i in range(N_CASES):
        K, M, N, bp8, bp6, dtype, padx, padw = draw_case(rng)
        case = f"case {i}: M={M} N={N} K={K} budget={bp8}/{bp6} {dtype} ldx=K+{padx} ldw=K+{padw}"
        print(case, flush=True)
        seed = 7000 + 16 * i
        gains = synth.outlier_gains(K, seed + synth.ROLE_CHANNELS, max(1, K // 1000), max(2, K // 100))
        X = strided(synth.activations(M, K, seed + synth.ROLE_X, gains, dtype=dtype, device=DEV), padx)
        W = strided(synth.weights(N, K, seed + synth.ROLE_W, dtype=dtype, device=DEV), padw)
        Xh = np.ascontiguousarray(X.float().cpu().numpy())
        Wh = np.ascontiguousarray(W.float().cpu().numpy())

        h = mx.mxs_calibrate(X)
        h_ref = orc.calibrate(Xh)
        assert np.array_equal(h.cpu().numpy(), h_ref), f"{case}: calibrate"
        s = mx.mxs_score(W, h)
        s_ref = orc.score(Wh, h_ref)
        assert np.array_equal(s.cpu().numpy(), s_ref), f"{case}: score"
        bits, perm = mx.mxs_allocate(s, bp8, bp6)
        b_ref, p_ref = orc.allocate(s_ref, bp8, bp6)
        assert np.array_equal(bits.cpu().numpy(), b_ref), f"{case}: bit map"
        assert np.array_equal(perm.cpu().numpy(), p_ref), f"{case}: permutation"

        n8, n6, n4 = mx.mxs_budget_blocks(K, bp8, bp6)
        A = mx.mxs_quantize(X, perm, n8, n6, n4)
        B = mx.mxs_quantize(W, perm, n8, n6, n4)
        A_ref = orc.quantize(Xh, p_ref, n8, n6, n4)
        B_ref = orc.quantize(Wh, p_ref, n8, n6, n4)
        for Q, R_, what in ((A, A_ref, "X"), (B, B_ref, "W")):
            for key in ("q8", "q6", "q4", "sc"):
                g = getattr(Q, key).cpu().numpy().view(np.uint8)
                assert np.array_equal(g, R_[key].view(np.uint8)), f"{case}: {what} plane {key}"

        Yref, Yabs = orc.mixed_gemm(A_ref, B_ref)
        Y = mx.mxs_mixed_gemm(A, B)
        ok, worst = gemm_ok(Y, Yref, Yabs)
        assert ok, f"{case}: mxs_mixed_gemm worst rel {worst:.3e}"
        ok, worst = gemm_ok(mx.mxs_mixed_gemm_mx(A, B), Yref, Yabs)
        assert ok, f"{case}: mxs_mixed_gemm_mx worst rel {worst:.3e}"
        Yf = mx.mxs_mixed_gemm_fused(X, perm, B)
        assert torch.equal(Yf.view(torch.int32), Y.view(torch.int32)), f"{case}: fused differs from quantize + GEMM"
