"""CPU oracle for the MXSens hot path -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package. The HIP library never calls it and
shares no code with it.

The arithmetic lives in ``mxs_oracle.c`` (plain loops, fp64 sums); this module
builds it with gcc and wraps it for numpy arrays. Each wrapper names the
section of the C file it calls; the C file cites the pages.

Parity pins: every function here is checked in ``tests/test_oracle_*.py``
against closed forms, brute force or invariants (nothing is "parity
unpinned").
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from ctypes import POINTER, c_double, c_int, c_int8, c_int32, c_int64, c_uint8, c_void_p

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxs_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_mxs.so")

BLOCK = 32

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (strict IEEE: no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
               "-fPIC", "-shared", "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = c_void_p
        lib.or_quantize_block.argtypes = [P, c_int, c_int, P, P]
        lib.or_dequant_value.argtypes = [c_int, c_uint8]
        lib.or_dequant_value.restype = c_double
        lib.or_calibrate.argtypes = [P, c_int64, c_int64, c_int64, P]
        lib.or_score.argtypes = [P, c_int64, c_int64, c_int64, P, P]
        lib.or_budget_blocks.argtypes = [c_int64, c_int32, c_int32, P]
        lib.or_allocate.argtypes = [P, c_int64, c_int32, c_int32, P, P]
        lib.or_quantize.argtypes = [P, c_int64, c_int64, c_int64, P, c_int32, c_int32, c_int32,
                                    P, c_int64, P, c_int64, P, c_int64, P, c_int64]
        lib.or_unpack_row.argtypes = [c_int64, c_int64, c_int32, c_int32, c_int32,
                                      P, c_int64, P, c_int64, P, c_int64, P]
        lib.or_mixed_gemm.argtypes = [c_int64, c_int64, c_int64, c_int32, c_int32, c_int32,
                                      P, c_int64, P, c_int64, P, c_int64, P, c_int64,
                                      P, c_int64, P, c_int64, P, c_int64, P, c_int64,
                                      P, c_int64, P]
        lib.or_quantize_kv.argtypes = [P, c_int64, c_int64, c_int64, P, P]
        lib.or_allocate_blocks.argtypes = [P, c_int64, c_int32, c_int32, P, P]
        lib.or_output_error.argtypes = [P, c_int64, c_int64, c_int64, P, c_int64, c_int64, P, c_int64, P]
        lib.or_layer_budget.argtypes = [c_int32, P, P, P, c_double, P, P]
        lib.or_attend_kv4.argtypes = [P, P, P, P, P, c_int64, c_int64, c_int64, c_int64, c_double, P]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(c_void_p)


def _f32(a):
    a = np.asarray(a)
    if a.dtype != np.float32:
        raise TypeError("oracle inputs are float32 (widen bf16 exactly before the call)")
    return np.ascontiguousarray(a)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: bad argument")


# -- section 1: block quantizer ---------------------------------------------
def quantize_block(v, m: int):
    """Codes (int8[n]) and E8M0 scale byte of one block of n <= 32 values."""
    v = _f32(np.atleast_1d(v))
    codes = np.zeros(v.shape[0], np.int8)
    sb = np.zeros(1, np.uint8)
    _check(_load().or_quantize_block(_ptr(v), v.shape[0], m, _ptr(codes), _ptr(sb)), "quantize_block")
    return codes, int(sb[0])


def dequant(code: int, scale_byte: int) -> float:
    return _load().or_dequant_value(int(code), int(scale_byte))


# -- section 3: calibration --------------------------------------------------
def calibrate(X, hdiag=None):
    """hdiag += column sums of X**2 (fp64, fixed order). Returns hdiag."""
    X = _f32(X)
    M, K = X.shape
    if hdiag is None:
        hdiag = np.zeros(K, np.float64)
    assert hdiag.dtype == np.float64 and hdiag.flags.c_contiguous and hdiag.shape == (K,)
    _check(_load().or_calibrate(_ptr(X), M, K, K, _ptr(hdiag)), "calibrate")
    return hdiag


# -- section 4: score ----------------------------------------------------------
def score(W, hdiag):
    W = _f32(W)
    N, K = W.shape
    hdiag = np.ascontiguousarray(hdiag, np.float64)
    out = np.zeros(K, np.float64)
    _check(_load().or_score(_ptr(W), N, K, K, _ptr(hdiag), _ptr(out)), "score")
    return out


# -- section 5: budget -----------------------------------------------------------
def budget_blocks(K: int, bp8: int, bp6: int):
    nb = np.zeros(3, np.int32)
    _check(_load().or_budget_blocks(K, bp8, bp6, _ptr(nb)), "budget_blocks")
    return int(nb[0]), int(nb[1]), int(nb[2])


# -- section 6: allocation ---------------------------------------------------
def allocate(score_, bp8: int, bp6: int):
    """(bits uint8[K], perm int32[K]) -- perm[j] is the source column of position j."""
    s = np.ascontiguousarray(score_, np.float64)
    K = s.shape[0]
    bits = np.zeros(K, np.uint8)
    perm = np.zeros(K, np.int32)
    _check(_load().or_allocate(_ptr(s), K, bp8, bp6, _ptr(bits), _ptr(perm)), "allocate")
    return bits, perm


# -- section 7: quantize + pack ------------------------------------------------
def allocate_blocks(score_, n8: int, n6: int):
    """allocate() with the block counts given instead of the budget."""
    sc = np.ascontiguousarray(score_, dtype=np.float64)
    K = sc.shape[0]
    bits = np.zeros(K, np.uint8)
    perm = np.zeros(K, np.int32)
    _check(_load().or_allocate_blocks(_ptr(sc), K, n8, n6, _ptr(bits), _ptr(perm)), "allocate_blocks")
    return bits, perm


def quantize(X, perm, n8: int, n6: int, n4: int):
    """Planes dict(q8 int8[R,32 n8], q6 uint8[R,24 n6], q4 uint8[R,16 n4], sc uint8[R,nb])."""
    X = _f32(X)
    R, K = X.shape
    nb = K // BLOCK
    q8 = np.zeros((R, 32 * n8), np.int8)
    q6 = np.zeros((R, 24 * n6), np.uint8)
    q4 = np.zeros((R, 16 * n4), np.uint8)
    sc = np.zeros((R, nb), np.uint8)
    p = None if perm is None else np.ascontiguousarray(perm, np.int32)
    _check(_load().or_quantize(_ptr(X), R, K, K, _ptr(p), n8, n6, n4,
                               _ptr(q8), max(32 * n8, 1), _ptr(q6), max(24 * n6, 1),
                               _ptr(q4), max(16 * n4, 1), _ptr(sc), nb), "quantize")
    return dict(q8=q8, q6=q6, q4=q4, sc=sc, n8=n8, n6=n6, n4=n4, K=K, rows=R)


def _planes_args(P):
    n8, n6, n4 = P["n8"], P["n6"], P["n4"]
    q8 = np.ascontiguousarray(P["q8"], np.int8)
    q6 = np.ascontiguousarray(P["q6"], np.uint8)
    q4 = np.ascontiguousarray(P["q4"], np.uint8)
    sc = np.ascontiguousarray(P["sc"], np.uint8)
    return (q8, max(q8.shape[1], 1), q6, max(q6.shape[1], 1), q4, max(q4.shape[1], 1),
            sc, sc.shape[1]), (n8, n6, n4)


def unpack(P):
    """Codes int32[R, K] (permuted order) from planes (section 8)."""
    (q8, l8, q6, l6, q4, l4, sc, ls), (n8, n6, n4) = _planes_args(P)
    R, K = sc.shape[0], sc.shape[1] * BLOCK
    out = np.zeros((R, K), np.int32)
    lib = _load()
    for r in range(R):
        _check(lib.or_unpack_row(r, K, n8, n6, n4, _ptr(q8), l8, _ptr(q6), l6, _ptr(q4), l4,
                                 _ptr(out[r])), "unpack")
    return out


# -- section 9: mixed GEMM -------------------------------------------------------
def mixed_gemm(A, W):
    """(Y, Yabs) float64[M, N]: Y = deq(A) deq(W)^T, Yabs = |deq(A)| |deq(W)|^T."""
    (a8, la8, a6, la6, a4, la4, asc, las), na = _planes_args(A)
    (w8, lw8, w6, lw6, w4, lw4, wsc, lws), nw = _planes_args(W)
    if na != nw or asc.shape[1] != wsc.shape[1]:
        raise ValueError("A and W must share K and block counts")
    M, N, K = asc.shape[0], wsc.shape[0], asc.shape[1] * BLOCK
    Y = np.zeros((M, N), np.float64)
    Yabs = np.zeros((M, N), np.float64)
    _check(_load().or_mixed_gemm(M, N, K, *na, _ptr(a8), la8, _ptr(a6), la6, _ptr(a4), la4,
                                 _ptr(asc), las, _ptr(w8), lw8, _ptr(w6), lw6, _ptr(w4), lw4,
                                 _ptr(wsc), lws, _ptr(Y), N, _ptr(Yabs)), "mixed_gemm")
    return Y, Yabs


# -- section 10: KV ----------------------------------------------------------------
def quantize_kv(kv):
    """codes uint8[T, H, D/2], scales uint8[T, H, D/32] for kv float32[T, H, D]."""
    kv = _f32(kv)
    T, H, D = kv.shape
    codes = np.zeros((T, H, D // 2), np.uint8)
    scales = np.zeros((T, H, D // BLOCK), np.uint8)
    _check(_load().or_quantize_kv(_ptr(kv), T, H, D, _ptr(codes), _ptr(scales)), "quantize_kv")
    return codes, scales


# -- section 11: layer-wise allocation ----------------------------------------
def output_error(X, W, Yq):
    """sum over (t, n) of (X W^T - Yq)^2 in fp64 (X [M, K], W [N, K] float32,
    Yq [M, N] any float)."""
    X, W = _f32(X), _f32(W)
    Yq = np.ascontiguousarray(Yq, dtype=np.float64)
    M, K = X.shape
    N = W.shape[0]
    err = np.zeros(1, np.float64)
    _check(_load().or_output_error(_ptr(X), M, K, K, _ptr(W), N, K, _ptr(Yq), N, _ptr(err)), "output_error")
    return float(err[0])


def layer_budget(S, rows, K, B: float):
    """(blocks int32[L, 3] = (n8, n6, n4) per layer, R) for layer
    sensitivities S, weight rows and columns per layer and average width B."""
    S = np.ascontiguousarray(S, dtype=np.float64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    K = np.ascontiguousarray(K, dtype=np.int64)
    L = S.shape[0]
    out = np.zeros((L, 3), np.int32)
    R = np.zeros(1, np.float64)
    _check(_load().or_layer_budget(L, _ptr(S), _ptr(rows), _ptr(K), float(B), _ptr(out), _ptr(R)), "layer_budget")
    return out, float(R[0])


# -- section 12: attention over the 4-bit K/V cache ----------------------------
def attend_kv4(q, kc, ks, vc, vs, scale: float):
    """out float64[Hq, D] for one query token q float32[Hq, D] over K/V codes
    uint8[T, Hkv, D/2] and scales uint8[T, Hkv, D/32] (section 10 layout)."""
    q = _f32(q)
    kc, ks, vc, vs = (np.ascontiguousarray(a, np.uint8) for a in (kc, ks, vc, vs))
    Hq, D = q.shape
    T, Hkv = kc.shape[0], kc.shape[1]
    out = np.zeros((Hq, D), np.float64)
    _check(_load().or_attend_kv4(_ptr(q), _ptr(kc), _ptr(ks), _ptr(vc), _ptr(vs), T, Hq, Hkv, D, float(scale),
                                 _ptr(out)), "attend_kv4")
    return out
