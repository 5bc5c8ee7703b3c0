"""Prepared weights (mxs_prepare_weights, mxs_mixed_gemm_prepared,
mxs_mixed_gemm_fused_prepared) through the C ABI.

W's prefill operand is built once and reused; the product then prepares
only the activation operand. The kernels are the same as those of
mxs_mixed_gemm and mxs_mixed_gemm_fused, so Y must agree with those calls
bit for bit (raw fp32 bits, NaN included), for every path: prefill (64+
rows, including more tiles than CUs with a partial tile group and the
q_proj layer), 33..63 rows and the decode kernels (which read W's planes,
not the prepared buffer), ragged M and N, and one prepared buffer reused by
calls with different token counts. Each case is also checked against the
oracle's quantize + GEMM, componentwise within 1e-5 of the fp64 definition
(on sampled rows for the largest shapes).
"""
import numpy as np
import pytest
import torch

from bit_gemm_hdiag_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def mx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import bit_gemm_hdiag_amd as mx
    return mx


def same_bits(a, b):
    return torch.equal(a.contiguous().view(torch.int32), b.contiguous().view(torch.int32))


def operands(M, N, K, seed, dtype=torch.bfloat16):
    gains = synth.outlier_gains(K, seed + synth.ROLE_CHANNELS)
    X = synth.activations(M, K, seed + synth.ROLE_X, gains, dtype=dtype, device=DEV)
    W = synth.weights(N, K, seed + synth.ROLE_W, dtype=dtype, device=DEV)
    return X, W


def against_oracle(orc, X, W, perm, counts, Y, rows=None):
    """Y against the oracle's quantize + GEMM (on the given rows of X)."""
    p = None if perm is None else perm.cpu().numpy()
    Xs = X if rows is None else X[rows]
    Ys = Y if rows is None else Y[rows]
    Qa = orc.quantize(np.ascontiguousarray(Xs.float().cpu().numpy()), p, *counts)
    Qw = orc.quantize(np.ascontiguousarray(W.float().cpu().numpy()), p, *counts)
    Yref, Yabs = orc.mixed_gemm(Qa, Qw)
    y = Ys.cpu().numpy().astype(np.float64)
    err = np.abs(y - Yref)
    ok = err <= 1e-5 * Yabs
    assert ok.all(), f"{int((~ok).sum())} outputs off, worst rel {float((err / np.maximum(Yabs, 1e-300)).max()):.3e}"


@pytest.mark.parametrize("M,N,K,budget", [
    (64, 128, 256, (500, 1500)),          # one tile
    (300, 200, 4096, (500, 1500)),        # ragged M and N
    (130, 70, 96, (0, 3400)),             # K with a padding block
    (1100, 8192, 256, (500, 1500)),       # more tiles than CUs, partial tile group
    (2048, 4096, 4096, (500, 1500)),      # the q_proj layer
    (40, 96, 1024, (500, 1500)),          # 33..63 rows
    (8, 300, 1024, (500, 1500)),          # decode kernels
    (1, 1024, 8192, (500, 1500)),         # one token
])
def test_prepared_equals_unprepared(mx, orc, M, N, K, budget):
    seed = 7 * M + N + K
    X, W = operands(M, N, K, seed)
    n8, n6, n4 = mx.mxs_budget_blocks(K, *budget)
    perm = torch.randperm(K, generator=torch.Generator().manual_seed(seed)).to(torch.int32).to(DEV)
    Wq = mx.mxs_quantize(W, perm, n8, n6, n4)
    A = mx.mxs_quantize(X, perm, n8, n6, n4)
    wp = mx.mxs_prepare_weights(Wq)
    assert wp.numel() >= mx.mxs_prepare_weights_size(Wq)
    ref = mx.mxs_mixed_gemm(A, Wq)
    Y = mx.mxs_mixed_gemm_prepared(A, Wq, wp)
    assert same_bits(Y, ref), float((Y - ref).abs().max())
    Yf = mx.mxs_mixed_gemm_fused_prepared(X, perm, Wq, wp)
    assert same_bits(Yf, mx.mxs_mixed_gemm_fused(X, perm, Wq))
    assert same_bits(Yf, ref)
    rows = None if M <= 300 else torch.tensor(sorted({0, 1, M // 3, M // 2, M - 2, M - 1} |
                                                       set(range(0, M, 128))), device=DEV)
    against_oracle(orc, X, W, perm, (n8, n6, n4), Y, rows)


def test_one_prepared_buffer_many_calls(mx, orc):
    """One prepared W serves calls with different token counts, caller
    workspaces and a strided output; preparing twice gives the same bytes."""
    N, K = 384, 2048
    X, W = operands(600, N, K, 91)
    n8, n6, n4 = mx.mxs_budget_blocks(K, 800, 2000)
    perm = torch.randperm(K, generator=torch.Generator().manual_seed(91)).to(torch.int32).to(DEV)
    Wq = mx.mxs_quantize(W, perm, n8, n6, n4)
    wp = mx.mxs_prepare_weights(Wq)
    wp2 = mx.mxs_prepare_weights(Wq, out=torch.full_like(wp, 0x5A))
    n = mx.mxs_prepare_weights_size(Wq)
    assert torch.equal(wp[:n], wp2[:n])
    for M in (600, 64, 33, 5, 257):
        A = mx.mxs_quantize(X[:M], perm, n8, n6, n4)
        ws = torch.empty(max(1, mx.mxs_mixed_gemm_prepared_workspace(A, Wq)), dtype=torch.uint8, device=DEV)
        big = torch.full((M, N + 3), 7.0, device=DEV)
        mx.mxs_mixed_gemm_prepared(A, Wq, wp, Y=big[:, :N], ws=ws)
        assert same_bits(big[:, :N], mx.mxs_mixed_gemm(A, Wq)), M
        assert (big[:, N:] == 7.0).all()
    against_oracle(orc, X[:257], W, perm, (n8, n6, n4), big[:, :N])


def test_prepared_nonfinite_and_empty(mx):
    M, N, K = 128, 96, 512
    X, W = operands(M, N, K, 13)
    W[3, 40] = float("inf")
    X[9, 200] = float("nan")
    n8, n6, n4 = mx.mxs_budget_blocks(K, 500, 1500)
    Wq = mx.mxs_quantize(W, None, n8, n6, n4)
    A = mx.mxs_quantize(X, None, n8, n6, n4)
    wp = mx.mxs_prepare_weights(Wq)
    Y = mx.mxs_mixed_gemm_prepared(A, Wq, wp)
    assert same_bits(Y, mx.mxs_mixed_gemm(A, Wq))
    assert torch.isnan(Y[:, 3]).all() and torch.isnan(Y[9]).all()
    A0 = mx.mxs_quantize(X[:0], None, n8, n6, n4)
    assert mx.mxs_mixed_gemm_prepared(A0, Wq, wp).shape == (0, N)
    W0 = mx.mxs_quantize(W[:0], None, n8, n6, n4)
    assert mx.mxs_prepare_weights_size(W0) == 0
    assert mx.mxs_mixed_gemm_prepared(A, W0, mx.mxs_prepare_weights(W0)).shape == (M, 0)
