"""C-ABI contract checks that need no GPU: the library loads, exports every
function include/mxsens.h declares, and rejects bad arguments before any
device work (every call below fails validation, so nothing is enqueued).
The budget helper is host code and is compared with the oracle here."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxsens.h")


@pytest.fixture(scope="module")
def lib():
    from bit_gemm_hdiag_amd import build
    if not os.path.exists(build.LIB):
        build.build()
    return ctypes.CDLL(build.LIB)


@pytest.fixture(scope="module")
def mx(lib):
    import bit_gemm_hdiag_amd as mx
    return mx


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mxs_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_six_calls():
    names = declared_functions()
    for n in ("mxs_calibrate", "mxs_score", "mxs_allocate", "mxs_quantize", "mxs_mixed_gemm",
              "mxs_quantize_kv"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    from bit_gemm_hdiag_amd import build
    out = subprocess.run(["nm", "-D", "--defined-only", build.LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (mxs_\w+)", out))
    for n in declared_functions():
        assert n in exported, n
        getattr(lib, n)


def test_binding_exposes_same_names(mx):
    from bit_gemm_hdiag_amd import binding
    for n in declared_functions():
        assert n in binding.EXPORTED and callable(getattr(mx, n))


def test_budget_matches_oracle(mx, orc):
    rng = np.random.default_rng(0)
    for _ in range(500):
        K = 32 * int(rng.integers(1, 2000))
        bp8 = int(rng.integers(0, 4000))
        bp6 = int(rng.integers(0, 10001 - bp8))
        assert mx.mxs_budget_blocks(K, bp8, bp6) == orc.budget_blocks(K, bp8, bp6)


def test_status_strings(mx):
    assert mx.mxs_status_string(0) == "MXS_OK"
    assert mx.mxs_status_string(-4) == "MXS_ERR_WORKSPACE"
    assert mx.mxs_version() == 1


FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: every call below fails validation


def test_budget_errors(lib):
    out = (ctypes.c_int32 * 3)()
    f = lib.mxs_budget_blocks
    f.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    assert f(100, 0, 0, ctypes.cast(out, ctypes.c_void_p)) == -2
    assert f(256, -5, 0, ctypes.cast(out, ctypes.c_void_p)) == -3
    assert f(256, 6000, 4001, ctypes.cast(out, ctypes.c_void_p)) == -3
    assert f(256, 0, 0, None) == -1


def test_calibrate_score_errors(lib):
    P, I64, S = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    cal = lib.mxs_calibrate
    cal.argtypes = [P, ctypes.c_int32, I64, I64, I64, P, P, S, P]
    assert cal(FAKE, 1, 10, 33, 33, FAKE, None, 0, None) == -2        # K % 32
    assert cal(FAKE, 1, 10, 64, 32, FAKE, None, 0, None) == -2        # ldx < K
    assert cal(FAKE, 7, 10, 64, 64, FAKE, None, 0, None) == -1        # dtype
    assert cal(FAKE, 1, 10, 64, 64, None, None, 0, None) == -1        # hdiag NULL
    assert cal(FAKE, 1, 1000, 64, 64, FAKE, None, 0, None) == -4      # needs workspace
    need = lib.mxs_calibrate_workspace
    need.restype, need.argtypes = S, [I64, I64]
    assert need(256, 64) == 0 and need(257, 64) == 2 * 64 * 8
    assert cal(FAKE, 1, 1000, 64, 64, FAKE, FAKE, need(1000, 64) - 8, None) == -4
    sc = lib.mxs_score
    sc.argtypes = [P, ctypes.c_int32, I64, I64, I64, P, P, P, S, P]
    assert sc(FAKE, 0, 0, 64, 64, FAKE, FAKE, None, 0, None) == -2      # N = 0
    assert sc(FAKE, 0, 10, 64, 64, None, FAKE, None, 0, None) == -1
    assert sc(FAKE, 0, 600, 64, 64, FAKE, FAKE, None, 0, None) == -4
    lib.mxs_last_error.restype = ctypes.c_char_p
    assert b"workspace" in lib.mxs_last_error()


def test_allocate_errors(lib):
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    f = lib.mxs_allocate
    f.argtypes = [P, I64, ctypes.c_int32, ctypes.c_int32, P, P, P]
    assert f(FAKE, 100, 0, 0, FAKE, FAKE, None) == -2
    assert f(FAKE, 256, 9000, 2000, FAKE, FAKE, None) == -3
    assert f(None, 256, 0, 0, FAKE, FAKE, None) == -1
    assert f(FAKE, 32 * 8192, 0, 0, FAKE, FAKE, None) == -6


def qm(rows=4, K=64, n8=0, n6=1, n4=1, **kw):
    from bit_gemm_hdiag_amd.binding import _QMat
    d = dict(q8=None, ld8=0, q6=0x10000, ld6=24 * n6, q4=0x20000, ld4=16 * n4, sc=0x30000, lds=K // 32)
    d.update(kw)
    return _QMat(rows, K, n8, n6, n4, 0, d["q8"], d["ld8"], d["q6"], d["ld6"], d["q4"], d["ld4"],
                 d["sc"], d["lds"])


def test_quantize_and_gemm_errors(lib):
    P = ctypes.c_void_p
    q = lib.mxs_quantize
    q.argtypes = [P, ctypes.c_int32, ctypes.c_int64, P, P, P]
    assert q(FAKE, 0, 64, None, ctypes.byref(qm(n4=2)), None) == -2          # counts != K/32
    assert q(FAKE, 0, 32, None, ctypes.byref(qm()), None) == -2               # ldx < K
    assert q(FAKE, 0, 64, None, ctypes.byref(qm(ld6=10)), None) == -2         # ld6 < 24 n6
    assert q(FAKE, 0, 64, None, ctypes.byref(qm(q4=None)), None) == -1        # missing plane
    assert q(FAKE, 0, 64, None, None, None) == -1
    for g in (lib.mxs_mixed_gemm, lib.mxs_mixed_gemm_mx):
        g.argtypes = [P, P, P, ctypes.c_int64, P, ctypes.c_size_t, P]
        A, W = qm(rows=8), qm(rows=16, n6=0, n4=2)
        assert g(ctypes.byref(A), ctypes.byref(W), FAKE, 16, None, 0, None) == -2  # block counts differ
        W2 = qm(rows=16)
        assert g(ctypes.byref(A), ctypes.byref(W2), FAKE, 8, None, 0, None) == -2  # ldy < N
        A3 = qm(rows=8, q4=0x20004)                                                 # misaligned 4-bit plane
        assert g(ctypes.byref(A3), ctypes.byref(W2), FAKE, 16, None, 0, None) == -6
        A4 = qm(rows=128)                                                           # prefill needs a workspace
        assert g(ctypes.byref(A4), ctypes.byref(W2), FAKE, 16, None, 0, None) == -4
    for wsf in (lib.mxs_mixed_gemm_workspace, lib.mxs_mixed_gemm_mx_workspace):
        wsf.argtypes = [P, P]
        wsf.restype = ctypes.c_size_t
        assert wsf(ctypes.byref(qm(rows=128)), ctypes.byref(qm(rows=16))) > 0
        assert wsf(ctypes.byref(qm(rows=0)), ctypes.byref(qm(rows=16))) == 0
        # decode (scale rows 4-byte aligned): one token needs no partial rows, two do
        assert wsf(ctypes.byref(qm(rows=1, lds=4)), ctypes.byref(qm(rows=16, lds=4))) == 0
        assert wsf(ctypes.byref(qm(rows=2, lds=4)), ctypes.byref(qm(rows=16, lds=4))) > 0
    kv = lib.mxs_quantize_kv
    kv.argtypes = [P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, P, P, P]
    assert kv(FAKE, 1, 4, 8, 100, FAKE, FAKE, None) == -2
    assert kv(None, 1, 4, 8, 128, FAKE, FAKE, None) == -1


def test_layer_budget_matches_oracle(mx, orc):
    # host code: the library's solution for R must equal the oracle's exactly
    rng = np.random.default_rng(21)
    for _ in range(400):
        L = int(rng.integers(1, 9))
        K = (32 * rng.integers(1, 300, L)).astype(np.int64)
        rows = rng.integers(1, 30000, L).astype(np.int64)
        S = rng.lognormal(0.0, 2.0, L) * rng.choice([1.0, 0.0], L, p=[0.9, 0.1])
        if rng.random() < 0.2:
            S[:] = S[0]                                   # equal sensitivities: grouped breakpoints
        total = float(np.sum(rows * K))
        lo = 4.0 + float(np.sum(128 * rows)) / total
        B = float(rng.uniform(lo, 8.0))
        want, R = orc.layer_budget(S, rows, K, B)
        got, gR = mx.mxs_layer_budget(S, rows, K, B)
        assert got == want.tolist() and gR == R


def test_layer_budget_errors(mx, lib):
    P = ctypes.c_void_p
    S = (ctypes.c_double * 2)(1.0, 2.0)
    rows = (ctypes.c_int64 * 2)(10, 10)
    K = (ctypes.c_int64 * 2)(64, 96)
    out = (ctypes.c_int32 * 6)()
    f = lib.mxs_layer_budget
    f.restype = ctypes.c_int32
    f.argtypes = [ctypes.c_int32, P, P, P, ctypes.c_double, P, P]
    c = lambda x: ctypes.cast(x, P)
    assert f(2, c(S), c(rows), c(K), 6.0, c(out), None) == 0
    assert f(0, c(S), c(rows), c(K), 6.0, c(out), None) == -1
    assert f(2, None, c(rows), c(K), 6.0, c(out), None) == -1
    assert f(2, c(S), c(rows), c(K), 3.9, c(out), None) == -3
    assert f(2, c(S), c(rows), c(K), 4.1, c(out), None) == -3      # cannot pay the 8-bit blocks
    K[1] = 100
    assert f(2, c(S), c(rows), c(K), 6.0, c(out), None) == -2
    K[1] = 96
    S[0] = float("nan")
    assert f(2, c(S), c(rows), c(K), 6.0, c(out), None) == -1
    S[0] = float("inf")
    assert f(2, c(S), c(rows), c(K), 6.0, c(out), None) == -1
    with pytest.raises(mx.MxsError):
        mx.mxs_layer_budget([1.0, -1.0], [1, 1], [64, 64], 6.0)


def test_output_error_and_allocate_blocks_errors(lib):
    P = ctypes.c_void_p
    f = lib.mxs_output_error
    f.restype = ctypes.c_int32
    f.argtypes = [P, P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                  ctypes.c_int64, P, ctypes.c_int64, P, P, ctypes.c_size_t, P]
    lib.mxs_output_error_workspace.restype = ctypes.c_size_t
    lib.mxs_output_error_workspace.argtypes = [ctypes.c_int64, ctypes.c_int64]
    # tile sums (8 B per 64 x 64 tile); under 1024 tiles, also up to 4 K splits of
    # fp32 partial products per tile after a 16-byte alignment slack
    assert lib.mxs_output_error_workspace(130, 70) == 3 * 2 * 8 + 16 + 4 * 3 * 2 * 64 * 64 * 4
    assert lib.mxs_output_error_workspace(64 * 32, 64 * 32) == 1024 * 8          # 1024 tiles: no split
    assert lib.mxs_output_error_workspace(64 * 16, 64 * 32) == 512 * 8 + 16 + 2 * 512 * 64 * 64 * 4
    fake = P(4096)          # never dereferenced: every call below fails validation
    need = lib.mxs_output_error_workspace(64, 64)
    assert f(fake, fake, 7, 64, 64, 64, 64, 64, fake, 64, fake, fake, need, None) == -1     # dtype
    assert f(fake, fake, 0, 64, 64, 48, 64, 64, fake, 64, fake, fake, need, None) == -2     # K % 32
    assert f(fake, fake, 0, 64, 64, 64, 32, 64, fake, 64, fake, fake, need, None) == -2     # ldx < K
    assert f(fake, fake, 0, 64, 64, 64, 64, 64, fake, 63, fake, fake, need, None) == -2     # ldy < N
    assert f(None, fake, 0, 64, 64, 64, 64, 64, fake, 64, fake, fake, need, None) == -1     # X NULL
    assert f(fake, fake, 0, 64, 64, 64, 64, 64, fake, 64, None, fake, need, None) == -1     # err NULL
    assert f(P(4100), fake, 0, 64, 64, 64, 64, 64, fake, 64, fake, fake, need, None) == -6  # alignment
    assert f(fake, fake, 1, 64, 64, 64, 68, 64, fake, 64, fake, fake, need, None) == -6     # bf16 row pitch
    assert f(fake, fake, 0, 64, 64, 64, 64, 64, fake, 64, fake, fake, need - 1, None) == -4  # workspace
    assert f(fake, fake, 0, 64, 64, 64, 64, 64, fake, 64, fake, P(4104), need, None) == -4   # ws alignment
    big = 65535 * 64 + 1                                                                     # grid rows
    assert f(fake, fake, 0, big, 64, 64, 64, 64, fake, 64, fake, fake, 1 << 40, None) == -6
    g = lib.mxs_allocate_blocks
    g.restype = ctypes.c_int32
    g.argtypes = [P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, P, P, P]
    assert g(fake, 100, 1, 0, fake, fake, None) == -2
    assert g(fake, 128, 3, 2, fake, fake, None) == -3
    assert g(fake, 128, -1, 0, fake, fake, None) == -3
    assert g(None, 128, 1, 0, fake, fake, None) == -1
    assert g(fake, 262144, 1, 0, fake, fake, None) == -6


def test_attend_kv4_errors(lib):
    P = ctypes.c_void_p
    f = lib.mxs_attend_kv4
    f.restype = ctypes.c_int32
    f.argtypes = [P, P, P, P, P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                  P, P, ctypes.c_size_t, P]
    lib.mxs_attend_kv4_workspace.restype = ctypes.c_size_t
    lib.mxs_attend_kv4_workspace.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
    need = lib.mxs_attend_kv4_workspace(300, 8, 2, 64)
    assert need == 10 * 8 * (2 + 64) * 4              # 32 tokens per workgroup: 10 splits
    a = P(4096)            # never dereferenced: every call below fails validation
    args = lambda **kw: [kw.get(k, v) for k, v in (("q", a), ("kc", a), ("ks", a), ("vc", a), ("vs", a), ("T", 300),
                                                 ("Hq", 8), ("Hkv", 2), ("D", 64), ("s", 0.1), ("o", a), ("ws", a),
                                                 ("n", need), ("st", None))]
    assert f(*args(q=None)) == -1
    assert f(*args(T=0)) == -2
    assert f(*args(Hq=7)) == -2
    assert f(*args(D=48)) == -2
    assert f(*args(Hq=34, Hkv=2)) == -6            # group of 17 heads
    assert f(*args(D=288)) == -6
    assert f(*args(kc=P(4100))) == -6              # codes not 16-byte aligned
    assert f(*args(n=need - 1)) == -4


def test_gemm_fused_errors(lib):
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    f = lib.mxs_mixed_gemm_fused
    f.restype = ctypes.c_int32
    f.argtypes = [P, ctypes.c_int32, I64, I64, P, P, P, I64, P, ctypes.c_size_t, P]
    wsf = lib.mxs_mixed_gemm_fused_workspace
    wsf.restype = ctypes.c_size_t
    wsf.argtypes = [I64, ctypes.c_int32, P]
    W = qm(rows=16)
    w = ctypes.byref(W)
    assert f(FAKE, 7, 8, 64, None, w, FAKE, 16, None, 0, None) == -1         # unknown dtype
    assert f(FAKE, 1, 8, 32, None, w, FAKE, 16, None, 0, None) == -2         # ldx < K
    assert f(FAKE, 1, -1, 64, None, w, FAKE, 16, None, 0, None) == -2        # M < 0
    assert f(None, 1, 8, 64, None, w, FAKE, 16, None, 0, None) == -1         # X NULL
    assert f(FAKE, 1, 8, 64, None, w, FAKE, 8, None, 0, None) == -2          # ldy < N
    assert f(FAKE, 1, 8, 64, None, None, FAKE, 16, None, 0, None) == -1      # W NULL
    assert f(FAKE, 1, 8, 64, None, ctypes.byref(qm(rows=16, q4=0x20004)), FAKE, 16, None, 0, None) == -6
    assert f(FAKE, 1, 1 << 23, 64, None, w, FAKE, 16, None, 0, None) == -6   # too many rows
    for M in (8, 128):                                                       # planes path, fused path
        need = wsf(M, 1, w)
        assert need > 0
        assert f(FAKE, 1, M, 64, None, w, FAKE, 16, FAKE, need - 1, None) == -4
    assert wsf(0, 1, w) == 0
    assert wsf(128, 9, w) == 0



def test_prepared_weights_errors(lib):
    P, I64, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    size = lib.mxs_prepare_weights_size
    size.restype, size.argtypes = SZ, [P]
    prep = lib.mxs_prepare_weights
    prep.restype, prep.argtypes = ctypes.c_int32, [P, P, SZ, P]
    g = lib.mxs_mixed_gemm_prepared
    g.restype, g.argtypes = ctypes.c_int32, [P, P, P, SZ, P, I64, P, SZ, P]
    gws = lib.mxs_mixed_gemm_prepared_workspace
    gws.restype, gws.argtypes = SZ, [P, P]
    full = lib.mxs_mixed_gemm_workspace
    full.restype, full.argtypes = SZ, [P, P]
    W = qm(rows=16)
    w = ctypes.byref(W)
    n = size(w)
    assert n > 0 and size(None) == 0 and size(ctypes.byref(qm(rows=0))) == 0
    assert size(ctypes.byref(qm(rows=16, K=48))) == 0                          # K not a multiple of 32
    assert prep(None, FAKE, n, None) == -1
    assert prep(w, None, 0, None) == -4
    assert prep(w, FAKE, n - 1, None) == -4
    assert prep(w, ctypes.c_void_p(0x10010), n, None) == -4                     # not 256-byte aligned
    assert prep(ctypes.byref(qm(rows=16, q4=0x20004)), FAKE, n, None) == -6     # misaligned plane
    A = qm(rows=128)
    a = ctypes.byref(A)
    need = gws(a, w)
    assert 0 < need < full(a, w)                                                # A's operand only
    assert gws(ctypes.byref(qm(rows=8)), w) == full(ctypes.byref(qm(rows=8)), w)   # decode: same kernels
    assert g(a, w, None, 0, FAKE, 16, FAKE, need, None) == -4                  # no prepared weights
    assert g(a, w, FAKE, n - 1, FAKE, 16, FAKE, need, None) == -4
    assert g(a, w, FAKE, n, FAKE, 16, FAKE, need - 1, None) == -4              # workspace too small
    assert g(a, ctypes.byref(qm(rows=16, n6=0, n4=2)), FAKE, n, FAKE, 16, FAKE, need, None) == -2
    f = lib.mxs_mixed_gemm_fused_prepared
    f.restype = ctypes.c_int32
    f.argtypes = [P, ctypes.c_int32, I64, I64, P, P, P, SZ, P, I64, P, SZ, P]
    fws = lib.mxs_mixed_gemm_fused_prepared_workspace
    fws.restype, fws.argtypes = SZ, [I64, ctypes.c_int32, P]
    fneed = fws(128, 1, w)
    assert fneed > 0
    assert f(FAKE, 1, 128, 64, None, w, None, 0, FAKE, 16, FAKE, fneed, None) == -4
    assert f(FAKE, 1, 128, 64, None, w, FAKE, n, FAKE, 16, FAKE, fneed - 1, None) == -4
    assert f(FAKE, 1, 128, 32, None, w, FAKE, n, FAKE, 16, FAKE, fneed, None) == -2   # ldx < K
