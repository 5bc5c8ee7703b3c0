"""mxs_mixed_gemm_noalloc (the product with its workspace in the library's
per-GPU scratch array) against mxs_mixed_gemm with a caller workspace,
through the C ABI: two calls in a row on one GPU, the second on a smaller
input, each bit-identical to the existing entry point (same kernels, same
workspace contents). Shapes whose workspace exceeds the scratch array are
rejected before anything is enqueued.
"""
import pytest
import torch

from bit_gemm_hdiag_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def operands(mx, M, N, K, seed):
    gains = synth.outlier_gains(K, seed + synth.ROLE_CHANNELS)
    X = synth.activations(M, K, seed + synth.ROLE_X, gains, device=DEV)
    W = synth.weights(N, K, seed + synth.ROLE_W, device=DEV)
    n8, n6, n4 = mx.mxs_budget_blocks(K, 500, 1500)
    perm = torch.randperm(K, generator=torch.Generator().manual_seed(seed)).to(torch.int32).to(DEV)
    return mx.mxs_quantize(X, perm, n8, n6, n4), mx.mxs_quantize(W, perm, n8, n6, n4)


def test_noalloc_matches_mixed_gemm_twice_then_smaller():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import bit_gemm_hdiag_amd as mx
    # prefill 2048 x 4096 x 4096 (prepared operands in the scratch array), then
    # prefill 256 x 1024 x 8192 (8 tiles, K split into 8 ranges: the ranges'
    # fp32 sums also in the scratch array), then decode 8 tokens (partial rows
    # in the scratch array)
    for M, N, K, seed in ((2048, 4096, 4096, 8100), (256, 1024, 8192, 8300), (8, 3000, 4096, 8200)):
        print(f"noalloc M={M} N={N} K={K}", flush=True)
        A, B = operands(mx, M, N, K, seed)
        need = mx.mxs_mixed_gemm_workspace(A, B)
        assert 0 < need <= mx.NOALLOC_SCRATCH_BYTES
        ref = mx.mxs_mixed_gemm(A, B)
        Y = torch.full((M, N), float("nan"), device=DEV)
        mx.mxs_mixed_gemm_noalloc(A, B, Y)
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int32), ref.view(torch.int32)), f"M={M}: differs from mxs_mixed_gemm"


def test_noalloc_rejects_workspace_above_scratch():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import bit_gemm_hdiag_amd as mx
    M, N, K = 2048, 8192, 8192
    A = mx.qmat_alloc(M, K, 12, 40, 204, DEV)
    B = mx.qmat_alloc(N, K, 12, 40, 204, DEV)
    assert mx.mxs_mixed_gemm_workspace(A, B) > mx.NOALLOC_SCRATCH_BYTES
    Y = torch.zeros((M, N), device=DEV)
    with pytest.raises(mx.MxsError) as ei:
        mx.mxs_mixed_gemm_noalloc(A, B, Y)
    assert ei.value.status == -6
    torch.cuda.synchronize()
    assert not Y.any()
