"""GPU parity for the Llama-2-70B-shaped pipeline at full size, through the C ABI.

Every linear layer of three of the 80 70B blocks (layers 0, 39 and 79; q
8192x8192, k and v 1024x8192, o 8192x8192, gate and up 28672x8192, down
8192x28672) runs the whole path:
calibrate over 128 x 2048 synthetic tokens of its input (one call, 1024 row
chunks), score, allocate (5/15/80 % 8/6/4-bit), quantize W and X, then the
product at M = 2048 prefill tokens through every GEMM entry point
(mxs_mixed_gemm, mxs_mixed_gemm_mx, mxs_mixed_gemm_fused and, with W prepared
once, mxs_mixed_gemm_prepared). Seeds: input i of block l draws from
5000 + 16 (4 l + i), weight j (q, k, v, o, gate, up, down) from
5500 + 16 (7 l + j); block 0 is the benchmarked block.

Bar: Hdiag of every column, the scores, the bit map, the permutation and all
weight planes bit for bit against the oracle; activation planes on the
sampled rows bit for bit; Y componentwise within 1e-5 of the fp64 definition
on one sampled token per 64-row group and one sampled output column per
64-column group (every wave tile of every workgroup tile is hit); the fused
entry and the prepared entry bit-identical to quantize + mxs_mixed_gemm. The oracle computes Hdiag
column slice by column slice (the canonical order runs down each column, so
the slices give the full result).
"""
import numpy as np
import pytest
import torch

from bit_gemm_hdiag_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GEMM_RTOL = 1e-5
C5 = synth.CONFIGS[5]
LAYERS = {d["name"]: d for d in C5["layers"]}
INPUT_OF = {"q": 0, "k": 0, "v": 0, "o": 1, "gate": 2, "up": 2, "down": 3}
SLICE_COLS = 1024


@pytest.fixture(scope="module")
def mx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import bit_gemm_hdiag_amd as mx
    return mx


@pytest.fixture(scope="module")
def calib():
    return {}


BLOCKS = (0, 39, 79)


def input_seed(block, inp):
    return 5000 + 16 * (4 * block + inp)


def weight_seed(block, li):
    return 5500 + 16 * (7 * block + li)


def hdiag_of_input(mx, orc, cache, block, inp, K):
    """GPU and oracle Hdiag of one layer input over 128 x 2048 tokens, compared
    in full; cached per input (q/k/v and gate/up share theirs)."""
    if (block, inp) in cache:
        return cache[(block, inp)]
    seed = input_seed(block, inp)
    gains = synth.outlier_gains(K, seed + synth.ROLE_CHANNELS)
    Xc = synth.activations(C5["calib_rows"], K, seed + synth.ROLE_CALIB, gains, device=DEV)
    h = mx.mxs_calibrate(Xc)
    torch.cuda.synchronize()
    h_ref = np.zeros(K, np.float64)
    for c0 in range(0, K, SLICE_COLS):
        sl = Xc[:, c0:c0 + SLICE_COLS].float().cpu().numpy()
        h_ref[c0:c0 + SLICE_COLS] = orc.calibrate(sl)
        del sl
    del Xc
    torch.cuda.empty_cache()
    bad = np.flatnonzero(h.cpu().numpy() != h_ref)
    assert bad.size == 0, f"Hdiag block {block} input {inp}: {bad.size} columns differ, first {bad[:5].tolist()}"
    cache.clear()                          # one block's inputs at a time
    cache[(block, inp)] = (h, h_ref, gains)
    return cache[(block, inp)]


def per_group_sample(n, group, gen):
    """One random index in every group of `group` consecutive indices, plus both ends."""
    picks = [g0 + int(torch.randint(0, min(group, n - g0), (1,), generator=gen)) for g0 in range(0, n, group)]
    return np.unique(np.array([0, n - 1] + picks))


def assert_planes(Q, R, rows=None, what=""):
    for key in ("q8", "q6", "q4", "sc"):
        g = getattr(Q, key).cpu().numpy().view(np.uint8)
        if rows is not None:
            g = g[rows]
        r = R[key].view(np.uint8)
        bad = np.argwhere(g != r)
        assert bad.size == 0, f"{what} {key}: {len(bad)} bytes differ, first {bad[:3].tolist()}"


def assert_gemm(Y, Yref, Yabs, what):
    err = np.abs(Y - Yref)
    ok = err <= GEMM_RTOL * Yabs
    assert ok.all(), f"{what}: {int((~ok).sum())} outputs off, worst rel " \
                     f"{float((err / np.maximum(Yabs, 1e-300)).max()):.3e}"


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "gate", "up", "down"])
@pytest.mark.parametrize("block", BLOCKS)
def test_70b_block_layer(mx, orc, calib, block, name):
    lay = LAYERS[name]
    N, K, M = lay["N"], lay["K"], C5["M"]
    bp8, bp6 = C5["budget"]
    li = list(LAYERS).index(name)
    inp = INPUT_OF[name]
    print(f"70B block {block} {name}: N={N} K={K} M={M}", flush=True)
    h, h_ref, gains = hdiag_of_input(mx, orc, calib, block, inp, K)

    W = synth.weights(N, K, weight_seed(block, li) + synth.ROLE_W, device=DEV)
    s = mx.mxs_score(W, h)
    Wh = W.float().cpu().numpy()
    s_ref = orc.score(Wh, h_ref)
    assert np.array_equal(s.cpu().numpy(), s_ref), "score"
    bits, perm = mx.mxs_allocate(s, bp8, bp6)
    b_ref, p_ref = orc.allocate(s_ref, bp8, bp6)
    assert np.array_equal(bits.cpu().numpy(), b_ref), "bit map"
    assert np.array_equal(perm.cpu().numpy(), p_ref), "permutation"
    n8, n6, n4 = mx.mxs_budget_blocks(K, bp8, bp6)
    assert (n8, n6, n4) == orc.budget_blocks(K, bp8, bp6)

    B = mx.mxs_quantize(W, perm, n8, n6, n4)
    B_ref = orc.quantize(Wh, p_ref, n8, n6, n4)
    assert_planes(B, B_ref, what="W planes")
    del Wh

    X = synth.activations(M, K, input_seed(block, inp) + synth.ROLE_X, gains, device=DEV)
    A = mx.mxs_quantize(X, perm, n8, n6, n4)
    g = torch.Generator(device="cpu").manual_seed(weight_seed(block, li))
    rows = per_group_sample(M, 64, g)
    cols = per_group_sample(N, 64, g)
    A_ref = orc.quantize(X[torch.as_tensor(rows, device=DEV)].float().cpu().numpy(), p_ref, n8, n6, n4)
    assert_planes(A, A_ref, rows, what="X planes")
    B_cols = {k: (v[cols] if isinstance(v, np.ndarray) else v) for k, v in B_ref.items()}
    Yref, Yabs = orc.mixed_gemm(A_ref, B_cols)

    Y = mx.mxs_mixed_gemm(A, B)
    assert_gemm(Y.cpu().numpy()[np.ix_(rows, cols)].astype(np.float64), Yref, Yabs, f"{name} mixed_gemm")
    Yx = mx.mxs_mixed_gemm_mx(A, B)
    assert_gemm(Yx.cpu().numpy()[np.ix_(rows, cols)].astype(np.float64), Yref, Yabs, f"{name} mixed_gemm_mx")
    del Yx
    Yf = mx.mxs_mixed_gemm_fused(X, perm, B)
    assert torch.equal(Yf.view(torch.int32), Y.view(torch.int32)), f"{name}: fused differs from quantize + GEMM"
    wp = mx.mxs_prepare_weights(B)
    Yp = mx.mxs_mixed_gemm_prepared(A, B, wp)
    assert torch.equal(Yp.view(torch.int32), Y.view(torch.int32)), f"{name}: prepared differs from mixed_gemm"
    del Y, Yf, Yp, wp, A, B, W, X
    torch.cuda.empty_cache()


@pytest.mark.parametrize("entry", ["mxs_mixed_gemm", "mxs_mixed_gemm_mx", "fused"])
def test_more_tiles_than_cus_partial_group_full_y(mx, orc, entry):
    # 5 row-tiles x 64 column-tiles = 320 tiles (> 256 CUs): the tile order
    # takes groups of 8 row-tiles, and the one group here is partial (5);
    # every output is compared
    M, N, K = 1100, 8192, 256
    seed = 5900
    gains = synth.outlier_gains(K, seed + synth.ROLE_CHANNELS)
    X = synth.activations(M, K, seed + synth.ROLE_X, gains, device=DEV)
    W = synth.weights(N, K, seed + synth.ROLE_W, device=DEV)
    n8, n6, n4 = mx.mxs_budget_blocks(K, 500, 1500)
    perm = torch.randperm(K, generator=torch.Generator().manual_seed(seed)).to(torch.int32)
    B = mx.mxs_quantize(W, perm.to(DEV), n8, n6, n4)
    A = mx.mxs_quantize(X, perm.to(DEV), n8, n6, n4)
    if entry == "fused":
        Y = mx.mxs_mixed_gemm_fused(X, perm.to(DEV), B)
    else:
        Y = getattr(mx, entry)(A, B)
    A_ref = orc.quantize(X.float().cpu().numpy(), perm.numpy(), n8, n6, n4)
    B_ref = orc.quantize(W.float().cpu().numpy(), perm.numpy(), n8, n6, n4)
    assert_planes(A, A_ref, what="X planes")
    assert_planes(B, B_ref, what="W planes")
    Yref, Yabs = orc.mixed_gemm(A_ref, B_ref)
    assert_gemm(Y.cpu().numpy().astype(np.float64), Yref, Yabs, f"{M}x{N}x{K} {entry}")
