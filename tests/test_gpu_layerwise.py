"""Layer-wise allocation on the GPU against the oracle (through the C ABI):
the single-layer output error, the budget under one global R and the
allocation with given block counts.

Tolerance of the output error: the GPU forms X W^T on the fp32 matrix cores,
so each element may differ from the fp64 product by e = 2 K 2^-24 (|X||W|^T)
(product and accumulation roundings of a K-term fp32 sum); the squared
differences are summed in fp64. Hence |S_gpu - S_ref| <= sum (2 |dY| e + e^2)
plus fp64 summation rounding, with dY = X W^T - Yq in fp64.
"""
import numpy as np
import pytest
import torch

from bit_gemm_hdiag_amd import synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def mx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import bit_gemm_hdiag_amd as mx
    return mx


def host(t):
    return t.float().cpu().numpy()


def err_bound(X, W, Yq):
    Xd, Wd = X.astype(np.float64), W.astype(np.float64)
    dY = Xd @ Wd.T - Yq.astype(np.float64)
    e = 2 * X.shape[1] * 2.0 ** -24 * (np.abs(Xd) @ np.abs(Wd).T)
    return float(np.sum(2 * np.abs(dY) * e + e * e))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
# under 1024 output tiles of 64 x 64 the product is split along K (empty
# trailing splits at K = 32 and 96, an odd tile count at 130 x 3, two splits at
# 256 x 8192); 256 x 16384 has 1024 tiles and takes the unsplit kernel
@pytest.mark.parametrize("M,N,K", [(64, 64, 32), (70, 130, 96), (256, 200, 1024), (1, 65, 4096), (130, 3, 64),
                                   (256, 8192, 64), (256, 16384, 32)])
def test_output_error_matches_oracle(mx, orc, M, N, K, dtype):
    g = torch.Generator(device="cpu").manual_seed(M * 3 + N + K)
    X = torch.randn(M, K, generator=g).to(dtype).to(DEV)
    W = (0.02 * torch.randn(N, K, generator=g)).to(dtype).to(DEV)
    Yq = (X.float() @ W.float().T).cpu() + 0.01 * torch.randn(M, N, generator=g)
    Yq = Yq.to(DEV)
    e1 = mx.mxs_output_error(X, W, Yq).cpu().item()
    e2 = mx.mxs_output_error(X, W, Yq).cpu().item()
    assert e1 == e2                                     # deterministic
    Xh, Wh, Yh = host(X), host(W), Yq.cpu().numpy()
    ref = orc.output_error(Xh, Wh, Yh)
    assert abs(e1 - ref) <= err_bound(Xh, Wh, Yh) + 1e-12 * ref, (e1, ref)


def test_output_error_strided_and_empty(mx, orc):
    g = torch.Generator(device="cpu").manual_seed(5)
    big = torch.randn(80, 200, generator=g).to(DEV)
    X, W = big[:40, 8:136], big[40:77, 16:144]           # ld 200, rows 16-byte aligned
    Yq = torch.randn(40, 50, generator=g).to(DEV)[:, :37]
    e = mx.mxs_output_error(X, W, Yq).cpu().item()
    Xh, Wh, Yh = host(X), host(W), Yq.cpu().numpy()
    ref = orc.output_error(np.ascontiguousarray(Xh), np.ascontiguousarray(Wh), Yh)
    assert abs(e - ref) <= err_bound(Xh, Wh, Yh) + 1e-12 * ref
    Z = torch.empty(0, 128, device=DEV)
    assert mx.mxs_output_error(Z, W[:, :128].contiguous(), torch.empty(0, 37, device=DEV)).cpu().item() == 0.0


def layer_inputs(K, N, T, seed, extreme):
    gains = synth.outlier_gains(K, seed + synth.ROLE_CHANNELS, extreme=50.0 * extreme)
    X = synth.activations(T, K, seed + synth.ROLE_CALIB, gains, device=DEV)
    W = synth.weights(N, K, seed + synth.ROLE_W, device=DEV)
    return X, W


def test_layerwise_pipeline_matches_oracle(mx, orc):
    # four layers with different shapes and outlier strength; S_l from the
    # uniform-MXINT4 layer error on 192 calibration tokens
    specs = [(1024, 512, 1.0), (2048, 256, 3.0), (512, 1024, 0.5), (1024, 96, 1.0)]
    T = 192
    S, rows, Ks, layers = [], [], [], []
    for i, (K, N, extreme) in enumerate(specs):
        X, W = layer_inputs(K, N, T, 7000 + 16 * i, extreme)
        nb = K // 32
        A4 = mx.mxs_quantize(X, None, 0, 0, nb)
        W4 = mx.mxs_quantize(W, None, 0, 0, nb)
        Yq = mx.mxs_mixed_gemm(A4, W4)
        s = mx.mxs_output_error(X, W, Yq).cpu().item()
        Xh, Wh, Yh = host(X), host(W), Yq.cpu().numpy()
        ref = orc.output_error(Xh, Wh, Yh)
        assert abs(s - ref) <= err_bound(Xh, Wh, Yh) + 1e-12 * ref
        # against the oracle's own quantized product (GEMM error within its bound)
        Yo, Yabs = orc.mixed_gemm(orc.quantize(Xh, None, 0, 0, nb), orc.quantize(Wh, None, 0, 0, nb))
        assert np.all(np.abs(Yh - Yo) <= 1e-5 * Yabs + 1e-30)
        S.append(s); rows.append(N); Ks.append(K); layers.append((X, W))
    assert len(set(S)) == len(S) and min(S) > 0
    for B in (4.3, 4.5, 5.0, 6.0):
        got, R = mx.mxs_layer_budget(S, rows, Ks, B)
        want, R_ref = orc.layer_budget(S, rows, Ks, B)
        assert got == want.tolist() and R == R_ref
    blocks, _ = mx.mxs_layer_budget(S, rows, Ks, 4.5)
    for (X, W), (n8, n6, n4) in zip(layers, blocks):
        K = X.shape[1]
        hd = mx.mxs_calibrate(X)
        score = mx.mxs_score(W, hd)
        bits, perm = mx.mxs_allocate_blocks(score, n8, n6)
        b_ref, p_ref = orc.allocate_blocks(score.cpu().numpy(), n8, n6)
        assert np.array_equal(bits.cpu().numpy(), b_ref) and np.array_equal(perm.cpu().numpy(), p_ref)
        assert int((bits == 8).sum()) == 32 * n8 and int((bits == 6).sum()) == 32 * n6
