"""GPU parity at the full sizes of the Llama-3-8B MLP layers, through the C
ABI (the Llama-2-70B layers are in test_gpu_c5_pipeline.py).

Calibration, scores, the bit map and permutation, and the packed weight
planes are compared with the oracle in full and bit for bit; the GEMM is
compared on sampled tokens and output columns (the oracle computes those
outputs one by one from the same packed operands).
"""
import numpy as np
import pytest
import torch

from bit_gemm_hdiag_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GEMM_RTOL = 1e-5


@pytest.fixture(scope="module")
def mx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import bit_gemm_hdiag_amd as mx
    return mx


def host(t):
    return t.float().cpu().numpy()


def check_planes(Q, R, rows=None):
    for key in ("q8", "q6", "q4", "sc"):
        g = getattr(Q, key).cpu().numpy().view(np.uint8)
        r = R[key].view(np.uint8)
        if rows is not None:
            g = g[rows]
        assert np.array_equal(g[:, :r.shape[1]], r), key


def check_gemm(Y, Yref, Yabs, what):
    err = np.abs(Y - Yref)
    ok = err <= GEMM_RTOL * Yabs
    assert ok.all(), f"{what}: {int((~ok).sum())} outputs off"


GEMMS = ["mxs_mixed_gemm", "mxs_mixed_gemm_mx"]


def per_group_sample(n, group, gen):
    """One random index in every group of `group` consecutive indices, plus both ends."""
    picks = [g0 + int(torch.randint(0, min(group, n - g0), (1,), generator=gen)) for g0 in range(0, n, group)]
    return np.unique(np.array([0, n - 1] + picks))


def layer_pipeline(mx, orc, M, N, K, budget, calib_rows, seed, entry="mxs_mixed_gemm"):
    """calibrate -> score -> allocate -> quantize W and X -> mixed GEMM, each against the oracle."""
    gains = synth.outlier_gains(K, seed + synth.ROLE_CHANNELS)
    Xc = synth.activations(calib_rows, K, seed + synth.ROLE_CALIB, gains, device=DEV)
    W = synth.weights(N, K, seed + synth.ROLE_W, device=DEV)
    bp8, bp6 = budget
    n8, n6, n4 = mx.mxs_budget_blocks(K, bp8, bp6)

    h = mx.mxs_calibrate(Xc)
    h_ref = orc.calibrate(host(Xc))
    assert np.array_equal(h.cpu().numpy(), h_ref), "Hdiag"
    del Xc
    s = mx.mxs_score(W, h)
    Wh = host(W)
    s_ref = orc.score(Wh, h_ref)
    assert np.array_equal(s.cpu().numpy(), s_ref), "score"
    bits, perm = mx.mxs_allocate(s, bp8, bp6)
    b_ref, p_ref = orc.allocate(s_ref, bp8, bp6)
    assert np.array_equal(bits.cpu().numpy(), b_ref) and np.array_equal(perm.cpu().numpy(), p_ref), "allocate"

    B = mx.mxs_quantize(W, perm, n8, n6, n4)
    B_ref = orc.quantize(Wh, p_ref, n8, n6, n4)
    check_planes(B, B_ref)
    del Wh

    X = synth.activations(M, K, seed + synth.ROLE_X, gains, device=DEV)
    A = mx.mxs_quantize(X, perm, n8, n6, n4)
    Y = getattr(mx, entry)(A, B).cpu().numpy().astype(np.float64)
    g = torch.Generator(device="cpu").manual_seed(seed)
    rows = per_group_sample(M, 128, g)
    cols = per_group_sample(N, 128, g)
    A_ref = orc.quantize(host(X[torch.as_tensor(rows, device=DEV)]), p_ref, n8, n6, n4)
    check_planes(A, A_ref, rows)
    B_cols = {k: v[cols] for k, v in B_ref.items() if isinstance(v, np.ndarray)}
    B_cols.update({k: v for k, v in B_ref.items() if not isinstance(v, np.ndarray)})
    Yref, Yabs = orc.mixed_gemm(A_ref, B_cols)
    check_gemm(Y[np.ix_(rows, cols)], Yref, Yabs, f"{M}x{N}x{K}")


# Llama-3-8B MLP, 4096 tokens: gate/up 14336 x 4096 at 3/10/87 %, down
# 4096 x 14336 at 8/20/72 %, and the two budgets swapped (gate/up at
# 8/20/72 %, down at 3/10/87 %); calibration over 8 x 2048 tokens. Y is
# compared on one token per 128-row group and one column per 128-column group.
@pytest.mark.parametrize("N,K,budget", [(14336, 4096, (300, 1000)), (4096, 14336, (800, 2000)),
                                        (14336, 4096, (800, 2000)), (4096, 14336, (300, 1000))])
@pytest.mark.parametrize("entry", GEMMS)
def test_mlp_layer_full_size(mx, orc, N, K, budget, entry):
    layer_pipeline(mx, orc, 4096, N, K, budget, 8 * 2048, seed=3000 + K, entry=entry)
