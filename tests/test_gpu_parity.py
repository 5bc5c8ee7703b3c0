"""GPU parity: every entry point of libmxsens against the CPU oracle on the
same seeded inputs (the oracle receives host copies of the device tensors).

Bar: bit-exact Hdiag, scores, bit map, permutation, codes and scales (both
sides follow one fp64 summation order and exact quantiser arithmetic);
GEMM componentwise |Y - Y_ref| <= 1e-5 * (|Qa| |Qw|^T)[t, n] against the
fp64 definition. Sizes span several tiles with ragged tails; the
full-size workloads check sampled GEMM rows.
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
    return t.float().cpu().numpy() if t.dtype in (torch.bfloat16, torch.float32) else t.cpu().numpy()


def assert_planes(Q, R, what=""):
    for key in ("q8", "q6", "q4", "sc"):
        g = getattr(Q, key).cpu().numpy().view(np.uint8)
        r = R[key].view(np.uint8)
        assert g.shape == r.shape, (what, key)
        bad = np.argwhere(g != r)
        assert bad.size == 0, f"{what} {key}: {len(bad)} mismatches, first at {bad[:3].tolist()}"


def assert_gemm(Y, Yref, Yabs, what=""):
    y = Y.cpu().numpy().astype(np.float64) if isinstance(Y, torch.Tensor) else Y
    err = np.abs(y - Yref)
    ok = err <= GEMM_RTOL * Yabs
    assert ok.all(), f"{what}: {int((~ok).sum())} outputs off, worst rel {float((err / np.maximum(Yabs, 1e-300)).max()):.3e}"
    nrm = np.linalg.norm(y - Yref) / max(np.linalg.norm(Yref), 1e-300)
    assert nrm < 1e-6, f"{what}: normwise {nrm:.3e}"


def layer(K, N, M, calib_rows, seed, dtype=torch.bfloat16, n_ext=None, n_mild=None):
    gains = synth.outlier_gains(K, seed + synth.ROLE_CHANNELS, n_ext, n_mild)
    Xc = synth.activations(calib_rows, K, seed + synth.ROLE_CALIB, gains, dtype=dtype, device=DEV)
    X = synth.activations(M, K, seed + synth.ROLE_X, gains, dtype=dtype, device=DEV)
    W = synth.weights(N, K, seed + synth.ROLE_W, dtype=dtype, device=DEV)
    return Xc, X, W


# ------------------------------------------------------------------ quantize
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("R,K,budget", [(64, 256, (500, 1500)), (7, 1024, (500, 1500)),
                                        (300, 4096, (300, 1000)), (33, 96, (0, 0))])
def test_quantize_identity_and_perm(mx, orc, dtype, R, K, budget):
    torch.manual_seed(R + K)
    gains = synth.outlier_gains(K, 11, max(1, K // 1000), max(2, K // 100))
    X = synth.activations(R, K, 12, gains, dtype=dtype, device=DEV)
    n8, n6, n4 = mx.mxs_budget_blocks(K, *budget)
    perm = torch.randperm(K, device=DEV).to(torch.int32)
    Xh = host(X)
    for p in (None, perm):
        Q = mx.mxs_quantize(X, p, n8, n6, n4)
        R_ = orc.quantize(Xh, None if p is None else p.cpu().numpy(), n8, n6, n4)
        assert_planes(Q, R_, f"R={R} K={K} perm={p is not None}")


@pytest.mark.parametrize("dtype,R,K", [(torch.bfloat16, 37, 28672), (torch.float32, 21, 16384),
                                       (torch.bfloat16, 300, 14336)])
def test_quantize_long_rows(mx, orc, dtype, R, K):
    # rows whose row and permutation do not fit twice in a CU's LDS read the
    # permutation from global memory (a second, unaligned view of the same
    # permutation takes the LDS-staged path); both must match the oracle
    gains = synth.outlier_gains(K, 31, max(1, K // 1000), max(2, K // 100))
    X = synth.activations(R, K, 32, gains, dtype=dtype, device=DEV)
    n8, n6, n4 = mx.mxs_budget_blocks(K, 800, 2000)
    perm = torch.randperm(K, generator=torch.Generator().manual_seed(K)).to(torch.int32).to(DEV)
    buf = torch.empty(K + 1, dtype=torch.int32, device=DEV)
    buf[1:] = perm
    Xh = host(X)
    ref = orc.quantize(Xh, perm.cpu().numpy(), n8, n6, n4)
    for p in (perm, buf[1:]):
        Q = mx.mxs_quantize(X, p, n8, n6, n4)
        assert_planes(Q, ref, f"R={R} K={K} {dtype} perm offset {p.data_ptr() % 16}")


def test_quantize_edge_values(mx, orc):
    # zeros, subnormals, exponent clamp, huge values, NaN/Inf blocks, ties
    K = 256
    X = np.zeros((6, K), np.float32)
    X[1, :32] = 2.0 ** -140
    X[1, 32:64] = np.array([2.0 ** -122, 2.0 ** -127, 2.0 ** -149] * 10 + [0, 0], np.float32)
    X[2, :] = np.float32(3.4e38) * np.sign(np.sin(np.arange(K)))
    X[3, 5] = np.nan
    X[3, 100] = np.inf
    X[3, 200] = -np.inf
    X[4, :] = (np.arange(K) % 16 - 8) * 0.5          # exact ties at every width
    X[5, :] = np.random.default_rng(0).standard_normal(K) * 2.0 ** 100
    for n8, n6, n4 in ((1, 0, 7), (2, 3, 3), (0, 0, 8), (8, 0, 0), (0, 8, 0)):
        for dt in (torch.float32, torch.bfloat16):
            Xd = torch.from_numpy(X).to(DEV).to(dt)
            Q = mx.mxs_quantize(Xd, None, n8, n6, n4)
            assert_planes(Q, orc.quantize(host(Xd), None, n8, n6, n4), f"edge {n8}/{n6}/{n4} {dt}")


def test_quantize_strided_and_unaligned(mx, orc):
    # ld > K and an fp32 leading dimension that is not a multiple of 4 (scalar loads)
    base = torch.randn(50, 1031, device=DEV)
    X = base[:, 3:3 + 1024]
    n8, n6, n4 = 1, 6, 25
    perm = torch.randperm(1024, device=DEV).to(torch.int32)
    for p in (None, perm):
        Q = mx.mxs_quantize(X, p, n8, n6, n4)
        ref = orc.quantize(np.ascontiguousarray(host(X)), None if p is None else p.cpu().numpy(), n8, n6, n4)
        assert_planes(Q, ref, "strided")
    # odd output strides: planes as slices of wider buffers
    q8 = torch.empty(50, 40, dtype=torch.int8, device=DEV)[:, 1:33]
    q6 = torch.empty(50, 151, dtype=torch.uint8, device=DEV)[:, 1:145]
    q4 = torch.empty(50, 403, dtype=torch.uint8, device=DEV)[:, 3:403]
    sc = torch.empty(50, 33, dtype=torch.uint8, device=DEV)[:, 1:33]
    out = mx.QMat(50, 1024, n8, n6, n4, q8, q6, q4, sc)
    mx.mxs_quantize(X, perm, n8, n6, n4, out=out)
    assert_planes(out, orc.quantize(np.ascontiguousarray(host(X)), perm.cpu().numpy(), n8, n6, n4), "odd ld")


def test_quantize_empty(mx):
    X = torch.empty(0, 256, device=DEV)
    Q = mx.mxs_quantize(X, None, 1, 0, 7)
    assert Q.rows == 0


@pytest.mark.parametrize("T,H,D", [(2048, 8, 128), (5, 3, 64), (1, 1, 32)])
def test_quantize_kv(mx, orc, T, H, D):
    kv = synth.kv(T, H, D, 2004, device=DEV)
    codes, scales = mx.mxs_quantize_kv(kv)
    c_ref, s_ref = orc.quantize_kv(host(kv))
    assert np.array_equal(codes.cpu().numpy(), c_ref) and np.array_equal(scales.cpu().numpy(), s_ref)


# ------------------------------------------------------------ calibrate/score
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("M,K", [(64, 256), (1000, 96), (257, 4096), (8 * 2048, 4096), (5000, 2048),
                                 (30000, 16384)])
def test_calibrate(mx, orc, dtype, M, K):
    # 5000 x 2048: 20 chunks, runs of 16 and 4 formed by the combine kernel;
    # 30000 x 16384: 118 chunks in 8 runs (the last 6 chunks, the last chunk
    # 48 rows), 8 x 64 = 512 workgroups that each add a whole run
    gains = synth.outlier_gains(K, 3, max(1, K // 1000), max(2, K // 100))
    X = synth.activations(M, K, 1, gains, dtype=dtype, device=DEV)
    h = mx.mxs_calibrate(X)
    ref = orc.calibrate(host(X))
    assert np.array_equal(h.cpu().numpy(), ref)


def test_calibrate_in_calls_and_strided(mx, orc):
    gains = synth.outlier_gains(4096, 2003)
    X = synth.activations(8 * 2048, 4096, 2001, gains, device=DEV)
    h = torch.zeros(4096, dtype=torch.float64, device=DEV)
    ref = np.zeros(4096)
    for i in range(8):
        mx.mxs_calibrate(X[2048 * i:2048 * (i + 1)], h)
        orc.calibrate(host(X[2048 * i:2048 * (i + 1)]), ref)
    assert np.array_equal(h.cpu().numpy(), ref)
    base = torch.randn(700, 200, device=DEV)
    Xs = base[:, 5:197]                                  # ldx = 200, unaligned start
    assert np.array_equal(mx.mxs_calibrate(Xs).cpu().numpy(), orc.calibrate(np.ascontiguousarray(host(Xs))))
    assert not mx.mxs_calibrate(torch.empty(0, 64, device=DEV)).any()


def test_calibrate_across_launches(mx, orc):
    # more chunks than one launch takes (65520 = 4095 whole runs): the first
    # launch adds whole runs per workgroup, the rest (4 chunks, the last
    # short) is one run formed by the combine kernel; one column block
    M = 65520 * 256 + 3 * 256 + 100
    g = torch.Generator(device=DEV).manual_seed(91)
    X = torch.randn(M, 32, generator=g, device=DEV).to(torch.bfloat16)
    h = mx.mxs_calibrate(X)
    ref = orc.calibrate(host(X))
    assert np.array_equal(h.cpu().numpy(), ref)


def test_calibrate_runs_onto_nonzero_hdiag(mx, orc):
    # whole runs per workgroup (30 runs x 32 column groups) added to an Hdiag
    # that already holds values: each run total is added whole, in run order
    gains = synth.outlier_gains(8192, 77)
    X = synth.activations(30 * 4096 - 100, 8192, 78, gains, device=DEV)
    h0 = np.random.default_rng(79).random(8192) * 1e6
    h = torch.from_numpy(h0.copy()).to(DEV)
    mx.mxs_calibrate(X, h)
    ref = h0.copy()
    orc.calibrate(host(X), ref)
    assert np.array_equal(h.cpu().numpy(), ref)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("N,K", [(256, 256), (1000, 96), (4096, 4096), (300, 14336)])
def test_score(mx, orc, dtype, N, K):
    W = synth.weights(N, K, 5, dtype=dtype, device=DEV)
    hd = torch.rand(K, dtype=torch.float64, device=DEV) * 100
    s = mx.mxs_score(W, hd)
    ref = orc.score(host(W), hd.cpu().numpy())
    assert np.array_equal(s.cpu().numpy(), ref)


def test_score_nonfinite_block(mx, orc):
    W = torch.randn(300, 128, device=DEV)
    W[17, 40] = float("nan")
    W[290, 100] = float("inf")
    hd = torch.ones(128, dtype=torch.float64, device=DEV)
    s = mx.mxs_score(W, hd).cpu().numpy()
    ref = orc.score(host(W), hd.cpu().numpy())
    assert np.array_equal(s, ref, equal_nan=True)
    assert np.isnan(s[32:64]).all() and np.isnan(s[96:128]).all() and np.isfinite(s[:32]).all()


# ------------------------------------------------------------------ allocate
@pytest.mark.parametrize("K,budget", [(256, (500, 1500)), (1024, (500, 1500)), (4096, (300, 1000)),
                                      (14336, (800, 2000)), (28672, (500, 1500)), (96, (0, 0))])
def test_allocate(mx, orc, K, budget):
    g = torch.Generator(device="cpu").manual_seed(K)
    s = torch.rand(K, generator=g, dtype=torch.float64) ** 4
    s[torch.randint(0, K, (K // 10,), generator=g)] = float(s[0])     # ties
    s[3] = float("inf")
    sd = s.to(DEV)
    bits, perm = mx.mxs_allocate(sd, *budget)
    rb, rp = orc.allocate(s.numpy(), *budget)
    assert np.array_equal(bits.cpu().numpy(), rb) and np.array_equal(perm.cpu().numpy(), rp)


# ----------------------------------------------------------------------- GEMM
# both entry points: int8 block sums with fp32 epilogues, and the variant on
# the block-scaled fp6 matrix cores (prefill kernels only)
GEMMS = ["mxs_mixed_gemm", "mxs_mixed_gemm_mx"]


def gemm_case(mx, orc, M, N, K, budget, seed, dtype=torch.bfloat16, sample_rows=None, entry="mxs_mixed_gemm"):
    Xc, X, W = layer(K, N, M, 512, seed, dtype)
    n8, n6, n4 = mx.mxs_budget_blocks(K, *budget)
    perm = torch.randperm(K, generator=torch.Generator().manual_seed(seed)).to(torch.int32).to(DEV)
    A = mx.mxs_quantize(X, perm, n8, n6, n4)
    B = mx.mxs_quantize(W, perm, n8, n6, n4)
    Y = getattr(mx, entry)(A, B)
    rows = np.arange(M) if sample_rows is None else sample_rows
    A_ref = orc.quantize(host(X[torch.as_tensor(rows, device=DEV)]), perm.cpu().numpy(), n8, n6, n4)
    B_ref = orc.quantize(host(W), perm.cpu().numpy(), n8, n6, n4)
    Yref, Yabs = orc.mixed_gemm(A_ref, B_ref)
    assert_gemm(Y.cpu().numpy()[rows].astype(np.float64), Yref, Yabs, f"M={M} N={N} K={K}")
    return Y


@pytest.mark.parametrize("M,N,K,budget", [(64, 256, 256, (500, 1500)), (77, 200, 1024, (500, 1500)),
                                          (1, 300, 8192, (500, 1500)), (8, 130, 8192, (500, 1500)),
                                          (32, 96, 8192, (500, 1500)), (130, 64, 4096, (300, 1000)),
                                          (129, 257, 14336, (800, 2000)), (40, 50, 96, (0, 0)),
                                          (33, 65, 512, (10000, 0)), (33, 65, 512, (0, 10000)),
                                          (300, 130, 480, (3100, 4000)), (100, 70, 352, (0, 0)),
                                          (70, 64, 288, (10000, 0)), (66, 129, 224, (0, 10000))])
@pytest.mark.parametrize("entry", GEMMS)
def test_mixed_gemm(mx, orc, M, N, K, budget, entry):
    gemm_case(mx, orc, M, N, K, budget, seed=M * 7 + N, entry=entry)


# Prefill products with fewer than 256 tiles of 256 x 128 split K into up to
# 8 ranges whose fp32 sums are added in range order: 8 and 32 tiles (8
# ranges; 256 x 1024 x 8192 is the 70B k/v shape at 256 tokens), 64 tiles (4
# ranges), 128 tiles (2 ranges). Rows sampled across every row tile.
@pytest.mark.parametrize("M,N,K", [(256, 1024, 8192), (300, 2048, 8192), (64, 8192, 8192), (512, 4096, 4096),
                                   (2048, 2048, 4096)])
def test_mixed_gemm_split_k(mx, orc, M, N, K):
    rows = np.unique(np.concatenate([np.arange(0, M, max(1, M // 12)), [M - 1]]))
    gemm_case(mx, orc, M, N, K, (500, 1500), seed=M + N + K, sample_rows=rows)


# The fp6 entry's three prefill paths, chosen by the count of 256 x 256
# output tiles: 256 or more (256 x 256 kernel, unsplit; W rows padded to 256),
# 64 to 255 (256 x 128 kernel), fewer than 64 (256 x 256 kernel with K split
# into up to 8 ranges added in order). Ragged M and N in each, whole-Y or
# rows sampled across every row tile.
@pytest.mark.parametrize("M,N,K,budget,sample", [
    (2000, 8000, 256, (500, 1500), False),     # 256 tiles, last row and column tiles partial
    (4000, 9000, 96, (0, 0), False),           # 576 tiles (2.25 passes), one 4-bit stage
    (2048, 8192, 1024, (500, 1500), True),     # 256 tiles, digit and 4-bit stages
    (1100, 8192, 256, (3100, 4000), False),    # 160 tiles: 256 x 128 kernel
    (300, 1000, 4096, (500, 1500), False),     # 8 tiles: 8 K ranges
    (520, 260, 1056, (800, 2000), False),      # 6 tiles: 6 K ranges, ragged both ways
])
def test_mixed_gemm_mx_tile_paths(mx, orc, M, N, K, budget, sample):
    rows = np.unique(np.concatenate([np.arange(0, M, 37), [M - 1]])) if sample else None
    gemm_case(mx, orc, M, N, K, budget, seed=M + 3 * N + K, sample_rows=rows, entry="mxs_mixed_gemm_mx")


@pytest.mark.parametrize("M,N,K,budget", [(1, 65, 32, (0, 0)), (2, 130, 512, (10000, 0)), (3, 64, 352, (0, 10000)),
                                          (4, 200, 480, (3100, 4000)), (4, 1000, 4096, (500, 1500)),
                                          (2, 77, 1056, (300, 1000)), (1, 129, 800, (800, 2000)),
                                          (6, 150, 2048, (500, 1500)), (8, 70, 544, (3100, 4000)),
                                          (5, 64, 96, (0, 0)), (9, 70, 544, (3100, 4000)), (16, 130, 96, (0, 0)),
                                          (31, 64, 2048, (10000, 0)), (24, 200, 352, (0, 10000)),
                                          (12, 65, 8192, (500, 1500))])
def test_mixed_gemm_vector_decode(mx, orc, M, N, K, budget):
    # the decode kernels (vector up to 8 tokens, matrix cores 9..32): one-slice
    # and many-slice cases, slice groups with fewer than four slices,
    # cases, single-width budgets, partial slices and ragged row tiles
    gemm_case(mx, orc, M, N, K, budget, seed=M * 11 + N)


@pytest.mark.parametrize("M,N,K,budget", [(200, 300, 1024, (500, 1500)), (64, 128, 8192, (300, 1000)),
                                          (3, 300, 1024, (500, 1500)), (20, 77, 4096, (300, 1000))])
@pytest.mark.parametrize("entry", GEMMS)
def test_mixed_gemm_exponent_spread(mx, orc, M, N, K, budget, entry):
    # per-block scales spread over +-2^12 so that many (row, group) pairs cannot
    # share one exponent: exercises the per-block path next to aligned groups
    g = torch.Generator(device="cpu").manual_seed(M + N)
    X = torch.randn(M, K, generator=g) * 2.0 ** torch.randint(-12, 13, (M, K // 32), generator=g).repeat_interleave(32, 1)
    W = torch.randn(N, K, generator=g) * 2.0 ** torch.randint(-12, 13, (N, K // 32), generator=g).repeat_interleave(32, 1)
    X[:, 40:72] = 0.0                                   # all-zero blocks inside groups
    W[5, 100] = float("nan") if M in (200, 3) else W[5, 100]  # one non-finite block
    X, W = X.to(DEV).to(torch.bfloat16), W.to(DEV).to(torch.bfloat16)
    n8, n6, n4 = mx.mxs_budget_blocks(K, *budget)
    perm = torch.randperm(K, generator=g).to(torch.int32).to(DEV)
    A = mx.mxs_quantize(X, perm, n8, n6, n4)
    B = mx.mxs_quantize(W, perm, n8, n6, n4)
    Y = getattr(mx, entry)(A, B).cpu().numpy().astype(np.float64)
    Yref, Yabs = orc.mixed_gemm(orc.quantize(host(X), perm.cpu().numpy(), n8, n6, n4),
                                orc.quantize(host(W), perm.cpu().numpy(), n8, n6, n4))
    nan_ref = np.isnan(Yref)
    assert np.array_equal(np.isnan(Y), nan_ref)
    assert_gemm(np.where(nan_ref, 0, Y), np.where(nan_ref, 0, Yref), np.where(nan_ref, 1, Yabs), "spread")


@pytest.mark.parametrize("M", [128, 4])
@pytest.mark.parametrize("entry", GEMMS)
def test_mixed_gemm_nonfinite_and_zero_by_class(mx, orc, entry, M):
    # NaN/Inf and all-zero blocks placed in each kind of block of the prefill
    # operand: 8-bit and 6-bit blocks (bf16 values), the 4-bit blocks that
    # round the bf16 run up to five blocks (3/4 wide blocks -> blocks 7..9),
    # and ordinary 4-bit blocks (exponent-aligned int8); M = 4 runs the
    # decode kernels on the same data
    N, K = 96, 1024
    n8, n6, n4 = 3, 4, 25
    g = torch.Generator(device="cpu").manual_seed(4242 + M)
    X = torch.randn(M, K, generator=g)
    W = torch.randn(N, K, generator=g)
    perm = torch.randperm(K, generator=g).to(torch.int32)
    col = lambda b, j=5: int(perm[32 * b + j])      # original column of position 32 b + j
    X[3 % M, col(1)] = float("nan")                  # 8-bit block of A
    W[10, col(5)] = float("inf")                      # 6-bit block of W
    X[(77 % M), col(8)] = -float("inf")              # 4-bit block carried as bf16
    W[50, col(20)] = float("nan")                     # narrow 4-bit block of W
    for b in (2, 6, 9, 25):                           # all-zero blocks, one per kind
        X[:, perm[32 * b:32 * b + 32].long()] = 0.0
        W[7, perm[32 * b:32 * b + 32].long()] = 0.0
    X, W, perm = X.to(DEV).to(torch.bfloat16), W.to(DEV).to(torch.bfloat16), perm.to(DEV)
    A = mx.mxs_quantize(X, perm, n8, n6, n4)
    B = mx.mxs_quantize(W, perm, n8, n6, n4)
    Y = getattr(mx, entry)(A, B).cpu().numpy().astype(np.float64)
    Yref, Yabs = orc.mixed_gemm(orc.quantize(host(X), perm.cpu().numpy(), n8, n6, n4),
                                orc.quantize(host(W), perm.cpu().numpy(), n8, n6, n4))
    nan_ref = np.isnan(Yref)
    assert nan_ref[3 % M].all() and nan_ref[:, 10].all() and nan_ref[:, 50].all()
    assert np.array_equal(np.isnan(Y), nan_ref)
    assert_gemm(np.where(nan_ref, 0, Y), np.where(nan_ref, 0, Yref), np.where(nan_ref, 1, Yabs), "nonfinite")


@pytest.mark.parametrize("N,K,bits", [(97, 2048, (0, 0, 64)), (130, 4096, (4, 12, 112)),
                                       (1001, 8192, (12, 40, 204)), (64, 16384, (0, 0, 512)),
                                       (257, 24576, (0, 0, 768)), (33, 28672, (45, 134, 717)),
                                       (70, 40960, (0, 0, 1280)), (50, 41024, (0, 0, 1282)),
                                       (40, 65536, (0, 0, 2048)), (40, 32800, (1025, 0, 0)),
                                       (65, 1024, (32, 0, 0)), (129, 1536, (0, 48, 0))])
@pytest.mark.parametrize("entry", GEMMS)
def test_mixed_gemm_one_token_rows(mx, orc, entry, N, K, bits):
    # one token: rows of 64 ... 2048 16-byte pieces on every (pieces per
    # lane, rows per wave, waves per row) instance, each at or near its upper
    # bound, then 2050 pieces (the slice kernel); ragged row counts;
    # single-width maps; non-finite and all-zero W blocks in each width class
    n8, n6, n4 = bits
    g = torch.Generator(device="cpu").manual_seed(N + K)
    X = torch.randn(1, K, generator=g)
    W = torch.randn(N, K, generator=g) * 2.0 ** torch.randint(-6, 7, (N, K // 32), generator=g).repeat_interleave(32, 1)
    perm = torch.randperm(K, generator=g).to(torch.int32)
    col = lambda b, j=3: int(perm[32 * b + j])
    firsts = [b for b, n in ((0, n8), (n8, n6), (n8 + n6, n4)) if n > 0]
    for i, b in enumerate(firsts):                     # one non-finite and one all-zero block per class
        W[(5 + 7 * i) % N, col(b)] = float("nan") if i != 1 else float("inf")
        W[(2 + 7 * i) % N, perm[32 * b:32 * b + 32].long()] = 0.0
    X[0, perm[32 * firsts[-1]:32 * firsts[-1] + 32].long()] = 0.0   # an all-zero block of the token
    X, W, perm = X.to(DEV).to(torch.bfloat16), W.to(DEV).to(torch.bfloat16), perm.to(DEV)
    A = mx.mxs_quantize(X, perm, n8, n6, n4)
    B = mx.mxs_quantize(W, perm, n8, n6, n4)
    Y = getattr(mx, entry)(A, B).cpu().numpy().astype(np.float64)
    Yref, Yabs = orc.mixed_gemm(orc.quantize(host(X), perm.cpu().numpy(), n8, n6, n4),
                                orc.quantize(host(W), perm.cpu().numpy(), n8, n6, n4))
    nan_ref = np.isnan(Yref)
    assert nan_ref[0, [(5 + 7 * i) % N for i in range(len(firsts))]].all() and not nan_ref.all()
    assert np.array_equal(np.isnan(Y), nan_ref)
    assert_gemm(np.where(nan_ref, 0, Y), np.where(nan_ref, 0, Yref), np.where(nan_ref, 1, Yabs), f"N={N} K={K}")


@pytest.mark.parametrize("entry", GEMMS)
def test_mixed_gemm_fp32_tiny_layer(mx, orc, entry):
    cfg = synth.CONFIGS[1]
    gemm_case(mx, orc, cfg["M"], cfg["N"], cfg["K"], cfg["budget"], seed=1000, dtype=torch.float32, entry=entry)


@pytest.mark.parametrize("entry", GEMMS)
def test_mixed_gemm_q_proj_full_size_sampled(mx, orc, entry):
    rows = np.array([0, 1, 2, 63, 64, 500, 1023, 1024, 1500, 2046, 2047])
    gemm_case(mx, orc, 2048, 4096, 4096, (500, 1500), seed=2000, sample_rows=rows, entry=entry)


_DECODE_MAPS = {}


def decode_map(mx, orc, N, K):
    """The method's own channel map of a 70B MLP weight: calibrate over 2048
    tokens, score, allocate (5/15/80 %), each compared with the oracle; W
    quantized once. Cached per shape (the token counts share it)."""
    if (N, K) in _DECODE_MAPS:
        return _DECODE_MAPS[(N, K)]
    seed = 3100 + 16 * (K // 1024)
    gains = synth.outlier_gains(K, seed + synth.ROLE_CHANNELS)
    Xc = synth.activations(2048, K, seed + synth.ROLE_CALIB, gains, device=DEV)
    W = synth.weights(N, K, seed + synth.ROLE_W, device=DEV)
    h = mx.mxs_calibrate(Xc)
    h_ref = orc.calibrate(host(Xc))
    assert np.array_equal(h.cpu().numpy(), h_ref), "calibrate"
    s = mx.mxs_score(W, h)
    Wh = host(W)
    s_ref = orc.score(Wh, h_ref)
    assert np.array_equal(s.cpu().numpy(), s_ref), "score"
    bits, perm = mx.mxs_allocate(s, 500, 1500)
    b_ref, p_ref = orc.allocate(s_ref, 500, 1500)
    assert np.array_equal(bits.cpu().numpy(), b_ref) and np.array_equal(perm.cpu().numpy(), p_ref), "allocate"
    n8, n6, n4 = mx.mxs_budget_blocks(K, 500, 1500)
    B = mx.mxs_quantize(W, perm, n8, n6, n4)
    _DECODE_MAPS.clear()
    _DECODE_MAPS[(N, K)] = (gains, seed, perm, (n8, n6, n4), B, Wh)
    return _DECODE_MAPS[(N, K)]


@pytest.mark.parametrize("M", [1, 8, 32])
@pytest.mark.parametrize("N,K", [(28672, 8192), (8192, 28672)])
def test_mixed_gemm_decode_full_size_sampled(mx, orc, N, K, M):
    # decode shapes of the 70B MLP (gate/up fused 28672 x 8192, down 8192 x
    # 28672) at batch 1/8/32 on the method's own map: every token, a sample
    # of output columns
    gains, seed, perm, (n8, n6, n4), B, Wh = decode_map(mx, orc, N, K)
    X = synth.activations(M, K, seed + synth.ROLE_X + 100 * M, gains, device=DEV)
    A = mx.mxs_quantize(X, perm, n8, n6, n4)
    Y = mx.mxs_mixed_gemm(A, B).cpu().numpy().astype(np.float64)
    g = torch.Generator(device="cpu").manual_seed(seed + M)
    cols = np.unique(np.concatenate([np.arange(0, 3), np.arange(N - 3, N),
                                     torch.randint(0, N, (40,), generator=g).numpy()]))
    p = perm.cpu().numpy()
    A_ref = orc.quantize(host(X), p, n8, n6, n4)
    B_ref = orc.quantize(Wh[cols], p, n8, n6, n4)
    Yref, Yabs = orc.mixed_gemm(A_ref, B_ref)
    assert_gemm(Y[:, cols], Yref, Yabs, f"decode M={M} N={N} K={K}")


@pytest.mark.parametrize("entry", GEMMS)
def test_mixed_gemm_strided_output_and_determinism(mx, orc, entry):
    Xc, X, W = layer(1024, 160, 70, 256, 77)
    perm = torch.arange(1024, dtype=torch.int32, device=DEV)
    A = mx.mxs_quantize(X, perm, 1, 6, 25)
    B = mx.mxs_quantize(W, perm, 1, 6, 25)
    Ybig = torch.full((70, 200), 7.0, device=DEV)
    gemm = getattr(mx, entry)
    gemm(A, B, Y=Ybig[:, 10:170])
    Y2 = gemm(A, B)
    assert torch.equal(Ybig[:, 10:170], Y2)
    assert (Ybig[:, :10] == 7).all() and (Ybig[:, 170:] == 7).all()
    Yref, Yabs = orc.mixed_gemm(orc.quantize(host(X), None, 1, 6, 25), orc.quantize(host(W), None, 1, 6, 25))
    assert_gemm(Y2, Yref, Yabs, "strided")


# ------------------------------------------------------------------- pipeline
@pytest.mark.parametrize("cfg_id", [1, 2])
def test_pipeline_matches_oracle(mx, orc, cfg_id):
    cfg = synth.CONFIGS[cfg_id]
    dt = torch.float32 if cfg["dtype"] == "f32" else torch.bfloat16
    K, N, M = cfg["K"], cfg["N"], cfg["M"]
    seed = 1000 * cfg_id
    gains = synth.outlier_gains(K, seed + synth.ROLE_CHANNELS, cfg.get("n_extreme"), cfg.get("n_mild"))
    if cfg_id == 1:
        X = synth.activations(M, K, seed + synth.ROLE_X, gains, dtype=dt, device=DEV)
        Xc = X
    else:
        Xc = synth.activations(cfg["calib_rows"], K, seed + synth.ROLE_CALIB, gains, dtype=dt, device=DEV)
        X = synth.activations(M, K, seed + synth.ROLE_X, gains, dtype=dt, device=DEV)
    W = synth.weights(N, K, seed + synth.ROLE_W, dtype=dt, device=DEV)
    bp8, bp6 = cfg["budget"]
    h = mx.mxs_calibrate(Xc)
    s = mx.mxs_score(W, h)
    bits, perm = mx.mxs_allocate(s, bp8, bp6)
    n8, n6, n4 = mx.mxs_budget_blocks(K, bp8, bp6)
    A = mx.mxs_quantize(X, perm, n8, n6, n4)
    B = mx.mxs_quantize(W, perm, n8, n6, n4)
    Y = mx.mxs_mixed_gemm(A, B)

    h_ref = orc.calibrate(host(Xc))
    s_ref = orc.score(host(W), h_ref)
    b_ref, p_ref = orc.allocate(s_ref, bp8, bp6)
    assert np.array_equal(h.cpu().numpy(), h_ref)
    assert np.array_equal(s.cpu().numpy(), s_ref)
    assert np.array_equal(bits.cpu().numpy(), b_ref) and np.array_equal(perm.cpu().numpy(), p_ref)
    rows = np.arange(M) if M <= 64 else np.array([0, 5, 700, M - 1])
    A_ref = orc.quantize(host(X[torch.as_tensor(rows, device=DEV)]), p_ref, n8, n6, n4)
    B_ref = orc.quantize(host(W), p_ref, n8, n6, n4)
    full_A = orc.quantize(host(X), p_ref, n8, n6, n4) if M <= 2048 else None
    if full_A is not None:
        assert_planes(A, full_A, "X planes")
    assert_planes(B, B_ref, "W planes")
    Yref, Yabs = orc.mixed_gemm(A_ref, B_ref)
    assert_gemm(Y.cpu().numpy()[rows].astype(np.float64), Yref, Yabs, f"config {cfg_id}")
