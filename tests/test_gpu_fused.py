"""The fused entry point (activation quantisation inside the product,
mxs_mixed_gemm_fused) through the C ABI, against the oracle and against the
two calls it replaces (mxs_quantize of X into planes, then mxs_mixed_gemm).

Every case is checked against the oracle's quantize + GEMM, componentwise
within 1e-5 of the fp64 definition (non-finite outputs where the definition
has them). The fused call and the two calls quantise with the same rule and
feed the same GEMM kernels, so Y must also agree bit for bit with them
(compared as raw fp32 bits, NaN included). Shapes cover the fused prefill
path (64+ rows, up to the 2048 x 4096 x 4096 q_proj layer), the planes path
(fewer rows, or rows too long for the LDS stage such as K = 28672), ragged
M and N, a K with a padding block, strided and misaligned X, fp32 and bf16,
the identity map and non-finite values.
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


def operands(M, N, K, seed, dtype):
    gains = synth.outlier_gains(K, seed + synth.ROLE_CHANNELS)
    X = synth.activations(M, K, seed + synth.ROLE_X, gains, dtype=dtype, device=DEV)
    W = synth.weights(N, K, seed + synth.ROLE_W, dtype=dtype, device=DEV)
    return X, W


def unfused(mx, X, perm, Wq):
    A = mx.mxs_quantize(X, perm, Wq.n8, Wq.n6, Wq.n4)
    return mx.mxs_mixed_gemm(A, Wq)


def same_bits(a, b):
    return torch.equal(a.contiguous().view(torch.int32), b.contiguous().view(torch.int32))


def against_oracle(orc, X, W, perm, counts, Y):
    """Y (device) against the oracle's quantize of X and W, then its GEMM."""
    p = None if perm is None else perm.cpu().numpy()
    Qa = orc.quantize(np.ascontiguousarray(X.float().cpu().numpy()), p, *counts)
    Qw = orc.quantize(np.ascontiguousarray(W.float().cpu().numpy()), p, *counts)
    Yref, Yabs = orc.mixed_gemm(Qa, Qw)
    y = Y.cpu().numpy().astype(np.float64)
    nan_ref = np.isnan(Yref)
    assert np.array_equal(np.isnan(y), nan_ref), "NaN pattern"
    y, Yref, Yabs = np.where(nan_ref, 0, y), np.where(nan_ref, 0, Yref), np.where(nan_ref, 1, Yabs)
    err = np.abs(y - Yref)
    ok = err <= 1e-5 * Yabs
    assert ok.all(), f"{int((~ok).sum())} outputs off, worst rel {float((err / np.maximum(Yabs, 1e-300)).max()):.3e}"


@pytest.mark.parametrize("M,N,K,budget,dtype,permuted", [
    (64, 128, 256, (500, 1500), torch.bfloat16, True),
    (300, 200, 4096, (500, 1500), torch.bfloat16, True),
    (130, 70, 96, (0, 3400), torch.float32, True),
    (256, 256, 1024, (0, 0), torch.bfloat16, False),
    (2048, 512, 4096, (300, 1200), torch.bfloat16, True),
    (128, 96, 14336, (500, 1500), torch.bfloat16, True),
    (96, 64, 28672, (500, 1500), torch.bfloat16, True),       # row too long for the stage: planes path
    (100, 80, 8192, (500, 1500), torch.float32, True),
    (8, 300, 1024, (500, 1500), torch.bfloat16, True),        # decode kernels
    (40, 64, 512, (500, 1500), torch.float32, True),          # 33..63 rows
    (40, 96, 28672, (500, 1500), torch.bfloat16, True),       # 33..63 rows, long rows
    (2048, 4096, 4096, (500, 1500), torch.bfloat16, True),    # the q_proj layer
])
def test_fused_equals_quantize_then_gemm(mx, orc, M, N, K, budget, dtype, permuted):
    seed = M + 3 * N + K
    X, W = operands(M, N, K, seed, dtype)
    n8, n6, n4 = mx.mxs_budget_blocks(K, *budget)
    perm = torch.randperm(K, generator=torch.Generator().manual_seed(seed)).to(torch.int32).to(DEV) if permuted else None
    Wq = mx.mxs_quantize(W, perm, n8, n6, n4)
    Y = mx.mxs_mixed_gemm_fused(X, perm, Wq)
    Y2 = mx.mxs_mixed_gemm_fused(X, perm, Wq)
    ref = unfused(mx, X, perm, Wq)
    assert same_bits(Y, Y2)
    assert same_bits(Y, ref), float((Y - ref).abs().max())
    against_oracle(orc, X, W, perm, (n8, n6, n4), Y)


def test_fused_strided_misaligned_and_nonfinite(mx, orc):
    M, N, K = 200, 130, 2048
    X, W = operands(M, N, K + 8, 77, torch.bfloat16)
    Xs = X[:, 3:3 + K]                        # row stride K + 8, rows start off 16-byte alignment
    Xs[5, 100] = float("inf")
    Xs[17, 7] = float("nan")
    Xs[40, :] = 0.0                           # an all-zero row
    n8, n6, n4 = mx.mxs_budget_blocks(K, 500, 1500)
    perm = torch.randperm(K, generator=torch.Generator().manual_seed(5)).to(torch.int32).to(DEV)
    Wq = mx.mxs_quantize(W[:, :K].contiguous(), perm, n8, n6, n4)
    Y = mx.mxs_mixed_gemm_fused(Xs, perm, Wq)
    ref = unfused(mx, Xs, perm, Wq)
    assert same_bits(Y, ref)
    assert torch.isnan(Y[5]).all() and torch.isnan(Y[17]).all() and (Y[40] == 0).all()
    against_oracle(orc, Xs, W[:, :K], perm, (n8, n6, n4), Y)
    # into a strided output, with a caller workspace reused twice
    big = torch.full((M, N + 10), 7.0, device=DEV)
    ws = torch.empty(mx.mxs_mixed_gemm_fused_workspace(M, torch.bfloat16, Wq), dtype=torch.uint8, device=DEV)
    for _ in range(2):
        mx.mxs_mixed_gemm_fused(Xs, perm, Wq, Y=big[:, :N], ws=ws)
    assert same_bits(big[:, :N], ref) and (big[:, N:] == 7.0).all()


def test_fused_against_oracle(mx, orc):
    M, N, K = 192, 160, 1024
    X, W = operands(M, N, K, 31, torch.bfloat16)
    n8, n6, n4 = mx.mxs_budget_blocks(K, 500, 1500)
    perm = torch.randperm(K, generator=torch.Generator().manual_seed(31)).to(torch.int32).to(DEV)
    Wq = mx.mxs_quantize(W, perm, n8, n6, n4)
    Y = mx.mxs_mixed_gemm_fused(X, perm, Wq).cpu().numpy().astype(np.float64)
    p = perm.cpu().numpy()
    Qa = orc.quantize(X.float().cpu().numpy(), p, n8, n6, n4)
    Qw = orc.quantize(W.float().cpu().numpy(), p, n8, n6, n4)
    Yref, Yabs = orc.mixed_gemm(Qa, Qw)
    assert np.all(np.abs(Y - Yref) <= 1e-5 * Yabs + 1e-30)


def test_fused_empty(mx):
    K = 256
    n8, n6, n4 = mx.mxs_budget_blocks(K, 500, 1500)
    Wq = mx.mxs_quantize(torch.randn(16, K, device=DEV), None, n8, n6, n4)
    Y = mx.mxs_mixed_gemm_fused(torch.empty(0, K, device=DEV), None, Wq)
    assert Y.shape == (0, 16)
