"""ctypes binding of libmxsens (include/mxsens.h), same names as the C ABI.

Argument marshalling only: tensors must already live in GPU memory; the
binding checks dtypes and layouts, allocates outputs and workspaces with
torch when the caller passes none, and enqueues the C call on the current
HIP stream. Every step of the method runs in the library's kernels. There
is no CPU fallback: a missing library raises at import.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_char_p, c_double, c_int32, c_int64, c_size_t, c_void_p
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "_lib", "libmxsens.so")

MXS_F32, MXS_BF16 = 0, 1
STATUS = {0: "MXS_OK", -1: "MXS_ERR_ARG", -2: "MXS_ERR_SHAPE", -3: "MXS_ERR_BUDGET",
          -4: "MXS_ERR_WORKSPACE", -5: "MXS_ERR_DEVICE", -6: "MXS_ERR_UNSUPPORTED"}


class MxsError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: {STATUS.get(status, status)}: {msg}")
        self.status = status


class _QMat(Structure):
    _fields_ = [("rows", c_int64), ("K", c_int64), ("n8", c_int32), ("n6", c_int32),
                ("n4", c_int32), ("reserved", c_int32),
                ("q8", c_void_p), ("ld8", c_int64), ("q6", c_void_p), ("ld6", c_int64),
                ("q4", c_void_p), ("ld4", c_int64), ("sc", c_void_p), ("lds", c_int64)]


def library_path() -> str:
    return _LIB_PATH


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"libmxsens.so is not built ({_LIB_PATH}); run __graft_entry__.build() "
                          "or python -m bit_gemm_hdiag_amd.build")
    lib = ctypes.CDLL(_LIB_PATH)
    P, S = c_void_p, c_int32
    sig = {
        "mxs_status_string": (c_char_p, [S]),
        "mxs_last_error": (c_char_p, []),
        "mxs_version": (c_int32, []),
        "mxs_budget_blocks": (S, [c_int64, c_int32, c_int32, P]),
        "mxs_calibrate_workspace": (c_size_t, [c_int64, c_int64]),
        "mxs_score_workspace": (c_size_t, [c_int64, c_int64]),
        "mxs_calibrate": (S, [P, c_int32, c_int64, c_int64, c_int64, P, P, c_size_t, P]),
        "mxs_score": (S, [P, c_int32, c_int64, c_int64, c_int64, P, P, P, c_size_t, P]),
        "mxs_allocate": (S, [P, c_int64, c_int32, c_int32, P, P, P]),
        "mxs_quantize": (S, [P, c_int32, c_int64, P, POINTER(_QMat), P]),
        "mxs_mixed_gemm_workspace": (c_size_t, [POINTER(_QMat), POINTER(_QMat)]),
        "mxs_mixed_gemm": (S, [POINTER(_QMat), POINTER(_QMat), P, c_int64, P, c_size_t, P]),
        "mxs_mixed_gemm_noalloc": (S, [POINTER(_QMat), POINTER(_QMat), P, c_int64, P]),
        "mxs_mixed_gemm_mx_workspace": (c_size_t, [POINTER(_QMat), POINTER(_QMat)]),
        "mxs_mixed_gemm_mx": (S, [POINTER(_QMat), POINTER(_QMat), P, c_int64, P, c_size_t, P]),
        "mxs_quantize_kv": (S, [P, c_int32, c_int64, c_int64, c_int64, P, P, P]),
        "mxs_allocate_blocks": (S, [P, c_int64, c_int32, c_int32, P, P, P]),
        "mxs_output_error_workspace": (c_size_t, [c_int64, c_int64]),
        "mxs_output_error": (S, [P, P, c_int32, c_int64, c_int64, c_int64, c_int64, c_int64, P, c_int64, P, P,
                                 c_size_t, P]),
        "mxs_layer_budget": (S, [c_int32, P, P, P, c_double, P, P]),
        "mxs_attend_kv4_workspace": (c_size_t, [c_int64, c_int64, c_int64, c_int64]),
        "mxs_attend_kv4": (S, [P, P, P, P, P, c_int64, c_int64, c_int64, c_int64, ctypes.c_float, P, P, c_size_t, P]),
        "mxs_mixed_gemm_fused_workspace": (c_size_t, [c_int64, c_int32, POINTER(_QMat)]),
        "mxs_mixed_gemm_fused": (S, [P, c_int32, c_int64, c_int64, P, POINTER(_QMat), P, c_int64, P, c_size_t, P]),
        "mxs_prepare_weights_size": (c_size_t, [POINTER(_QMat)]),
        "mxs_prepare_weights": (S, [POINTER(_QMat), P, c_size_t, P]),
        "mxs_mixed_gemm_prepared_workspace": (c_size_t, [POINTER(_QMat), POINTER(_QMat)]),
        "mxs_mixed_gemm_prepared": (S, [POINTER(_QMat), POINTER(_QMat), P, c_size_t, P, c_int64, P, c_size_t, P]),
        "mxs_mixed_gemm_fused_prepared_workspace": (c_size_t, [c_int64, c_int32, POINTER(_QMat)]),
        "mxs_mixed_gemm_fused_prepared": (S, [P, c_int32, c_int64, c_int64, P, POINTER(_QMat), P, c_size_t, P,
                                              c_int64, P, c_size_t, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    return lib


_lib = _load()
EXPORTED = ("mxs_status_string", "mxs_last_error", "mxs_version", "mxs_budget_blocks",
            "mxs_calibrate_workspace", "mxs_score_workspace", "mxs_calibrate", "mxs_score",
            "mxs_allocate", "mxs_quantize", "mxs_mixed_gemm_workspace", "mxs_mixed_gemm", "mxs_mixed_gemm_noalloc",
            "mxs_mixed_gemm_mx_workspace", "mxs_mixed_gemm_mx", "mxs_quantize_kv", "mxs_allocate_blocks",
            "mxs_output_error_workspace", "mxs_output_error", "mxs_layer_budget", "mxs_attend_kv4_workspace",
            "mxs_attend_kv4", "mxs_mixed_gemm_fused_workspace", "mxs_mixed_gemm_fused",
            "mxs_prepare_weights_size", "mxs_prepare_weights", "mxs_mixed_gemm_prepared_workspace",
            "mxs_mixed_gemm_prepared", "mxs_mixed_gemm_fused_prepared_workspace", "mxs_mixed_gemm_fused_prepared")


def _check(status: int, where: str):
    if status != 0:
        raise MxsError(status, where, _lib.mxs_last_error().decode())


def _stream(dev) -> c_void_p:
    return c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MXS_BF16
    if t.dtype == torch.float32:
        return MXS_F32
    raise TypeError(f"unsupported element type {t.dtype} (bf16 or fp32)")


def _dev2d(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with unit column stride")
    return t.data_ptr(), t.stride(0)


def _ptr(t):
    return None if t is None or t.numel() == 0 else t.data_ptr()


def _workspace(nbytes: int, dev, ws):
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    return ws.data_ptr(), ws.numel() * ws.element_size()


# --------------------------------------------------------------------- plain calls
def mxs_version() -> int:
    return _lib.mxs_version()


def mxs_status_string(status: int) -> str:
    return _lib.mxs_status_string(status).decode()


def mxs_last_error() -> str:
    return _lib.mxs_last_error().decode()


def mxs_budget_blocks(K: int, bp8: int, bp6: int):
    out = (c_int32 * 3)()
    _check(_lib.mxs_budget_blocks(K, bp8, bp6, ctypes.cast(out, c_void_p)), "mxs_budget_blocks")
    return int(out[0]), int(out[1]), int(out[2])


def mxs_calibrate_workspace(M: int, K: int) -> int:
    return int(_lib.mxs_calibrate_workspace(M, K))


def mxs_score_workspace(N: int, K: int) -> int:
    return int(_lib.mxs_score_workspace(N, K))


def mxs_calibrate(X: torch.Tensor, hdiag: torch.Tensor | None = None, ws=None) -> torch.Tensor:
    """hdiag[k] += sum_t X[t, k]^2 (fp64, fixed order). X [M, K] bf16/fp32 on the GPU."""
    px, ldx = _dev2d(X, "X")
    M, K = X.shape
    if hdiag is None:
        hdiag = torch.zeros(K, dtype=torch.float64, device=X.device)
    if hdiag.dtype != torch.float64 or not hdiag.is_contiguous() or hdiag.numel() != K:
        raise ValueError("hdiag must be a contiguous fp64 [K] tensor")
    pw, nw = _workspace(mxs_calibrate_workspace(M, K), X.device, ws)
    _check(_lib.mxs_calibrate(px, _dtype(X), M, K, ldx, hdiag.data_ptr(), pw, nw, _stream(X.device)),
           "mxs_calibrate")
    return hdiag


def mxs_score(W: torch.Tensor, hdiag: torch.Tensor, score: torch.Tensor | None = None, ws=None):
    """score[k] = hdiag[k] * sum_n (W - Q4(W))[n, k]^2, fp64 [K]."""
    pw_, ldw = _dev2d(W, "W")
    N, K = W.shape
    if score is None:
        score = torch.empty(K, dtype=torch.float64, device=W.device)
    if hdiag.dtype != torch.float64 or not hdiag.is_contiguous() or hdiag.numel() != K:
        raise ValueError("hdiag must be a contiguous fp64 [K] tensor")
    p, n = _workspace(mxs_score_workspace(N, K), W.device, ws)
    _check(_lib.mxs_score(pw_, _dtype(W), N, K, ldw, hdiag.data_ptr(), score.data_ptr(), p, n,
                          _stream(W.device)), "mxs_score")
    return score


def mxs_allocate(score: torch.Tensor, bp8: int, bp6: int, bits=None, perm=None):
    """(bits uint8 [K] in {8, 6, 4}, perm int32 [K] gather form)."""
    if not score.is_cuda or score.dtype != torch.float64 or not score.is_contiguous():
        raise ValueError("score must be a contiguous fp64 GPU tensor")
    K = score.numel()
    if bits is None:
        bits = torch.empty(K, dtype=torch.uint8, device=score.device)
    if perm is None:
        perm = torch.empty(K, dtype=torch.int32, device=score.device)
    _check(_lib.mxs_allocate(score.data_ptr(), K, bp8, bp6, bits.data_ptr(), perm.data_ptr(),
                             _stream(score.device)), "mxs_allocate")
    return bits, perm


@dataclass(frozen=True)
class QMat:
    """Planes of a matrix quantised with one bit map (see mxs_qmat). Frozen:
    the C struct is built once, on first use, and reused by every call."""
    rows: int
    K: int
    n8: int
    n6: int
    n4: int
    q8: torch.Tensor
    q6: torch.Tensor
    q4: torch.Tensor
    sc: torch.Tensor

    def c_struct(self) -> _QMat:
        q = self.__dict__.get("_c")
        if q is not None:
            return q

        def ld(t, width):
            return t.stride(0) if t.numel() else max(width, 1)
        for t in (self.q8, self.q6, self.q4, self.sc):
            if t.numel() and t.stride(1) != 1:
                raise ValueError("planes need unit column stride")
        q = _QMat(self.rows, self.K, self.n8, self.n6, self.n4, 0,
                  _ptr(self.q8), ld(self.q8, 32 * self.n8), _ptr(self.q6), ld(self.q6, 24 * self.n6),
                  _ptr(self.q4), ld(self.q4, 16 * self.n4), _ptr(self.sc), ld(self.sc, self.K // 32))
        object.__setattr__(self, "_c", q)
        return q

    def rows_slice(self, r0: int, r1: int) -> "QMat":
        return QMat(r1 - r0, self.K, self.n8, self.n6, self.n4, self.q8[r0:r1], self.q6[r0:r1],
                    self.q4[r0:r1], self.sc[r0:r1])


def qmat_alloc(rows: int, K: int, n8: int, n6: int, n4: int, device) -> QMat:
    kw = dict(device=device)
    return QMat(rows, K, n8, n6, n4,
                torch.empty((rows, 32 * n8), dtype=torch.int8, **kw),
                torch.empty((rows, 24 * n6), dtype=torch.uint8, **kw),
                torch.empty((rows, 16 * n4), dtype=torch.uint8, **kw),
                torch.empty((rows, K // 32), dtype=torch.uint8, **kw))


def mxs_quantize(X: torch.Tensor, perm: torch.Tensor | None, n8: int, n6: int, n4: int,
                 out: QMat | None = None) -> QMat:
    """MXINT 8/6/4 planes of X[:, perm] (perm None = identity)."""
    px, ldx = _dev2d(X, "X")
    R, K = X.shape
    if perm is not None and (perm.dtype != torch.int32 or not perm.is_contiguous() or perm.numel() != K
                             or not perm.is_cuda):
        raise ValueError("perm must be a contiguous int32 [K] GPU tensor")
    if out is None:
        out = qmat_alloc(R, K, n8, n6, n4, X.device)
    if out.rows != R or out.K != K:
        raise ValueError("output planes do not match X")
    q = out.c_struct()
    _check(_lib.mxs_quantize(px, _dtype(X), ldx, _ptr(perm), ctypes.byref(q), _stream(X.device)),
           "mxs_quantize")
    return out


def mxs_mixed_gemm_workspace(A: QMat, W: QMat) -> int:
    a, w = A.c_struct(), W.c_struct()
    return int(_lib.mxs_mixed_gemm_workspace(ctypes.byref(a), ctypes.byref(w)))


def _gemm(fn, wsfn, name, A: QMat, W: QMat, Y, ws) -> torch.Tensor:
    dev = A.sc.device
    if Y is None:
        Y = torch.empty((A.rows, W.rows), dtype=torch.float32, device=dev)
    if Y.dtype != torch.float32:
        raise TypeError("Y must be fp32")
    py, ldy = _dev2d(Y, "Y")
    a, w = ctypes.byref(A.c_struct()), ctypes.byref(W.c_struct())
    if ws is None:
        p, n = _workspace(int(wsfn(a, w)), dev, None)
    else:
        p, n = ws.data_ptr(), ws.numel() * ws.element_size()
    _check(fn(a, w, py, ldy, p, n, _stream(dev)), name)
    return Y


def mxs_mixed_gemm(A: QMat, W: QMat, Y: torch.Tensor | None = None, ws=None) -> torch.Tensor:
    """Y [M, N] fp32 = Qa(X) Qw(W)^T with per-block MX scales."""
    return _gemm(_lib.mxs_mixed_gemm, _lib.mxs_mixed_gemm_workspace, "mxs_mixed_gemm", A, W, Y, ws)


# bytes of the device scratch array behind mxs_mixed_gemm_noalloc (per GPU)
NOALLOC_SCRATCH_BYTES = 48 << 20


def mxs_mixed_gemm_noalloc(A: QMat, W: QMat, Y: torch.Tensor) -> torch.Tensor:
    """mxs_mixed_gemm with its workspace in the library's per-GPU scratch
    array: the C call allocates nothing (Y is the caller's fp32 [M, N])."""
    if Y.dtype != torch.float32:
        raise TypeError("Y must be fp32")
    py, ldy = _dev2d(Y, "Y")
    a, w = ctypes.byref(A.c_struct()), ctypes.byref(W.c_struct())
    _check(_lib.mxs_mixed_gemm_noalloc(a, w, py, ldy, _stream(Y.device)), "mxs_mixed_gemm_noalloc")
    return Y


def mxs_mixed_gemm_fused_workspace(M: int, dtype: torch.dtype, W: QMat) -> int:
    dt = MXS_BF16 if dtype == torch.bfloat16 else MXS_F32
    return int(_lib.mxs_mixed_gemm_fused_workspace(M, dt, ctypes.byref(W.c_struct())))


def _fused_args(X: torch.Tensor, perm, W: QMat, Y):
    px, ldx = _dev2d(X, "X")
    M, K = X.shape
    if K != W.K:
        raise ValueError("X and W differ in K")
    if perm is not None and (perm.dtype != torch.int32 or not perm.is_contiguous() or perm.numel() != K
                             or not perm.is_cuda):
        raise ValueError("perm must be a contiguous int32 [K] GPU tensor")
    if Y is None:
        Y = torch.empty((M, W.rows), dtype=torch.float32, device=X.device)
    if Y.dtype != torch.float32:
        raise TypeError("Y must be fp32")
    py, ldy = _dev2d(Y, "Y")
    return px, ldx, M, Y, py, ldy


def mxs_mixed_gemm_fused(X: torch.Tensor, perm: torch.Tensor | None, W: QMat, Y: torch.Tensor | None = None,
                         ws=None) -> torch.Tensor:
    """Y [M, N] fp32 = mixed_gemm(quantize(X[:, perm] at W's block counts), W), X quantized inside the call."""
    px, ldx, M, Y, py, ldy = _fused_args(X, perm, W, Y)
    w = W.c_struct()
    dt = _dtype(X)
    if ws is None:
        p, n = _workspace(int(_lib.mxs_mixed_gemm_fused_workspace(M, dt, ctypes.byref(w))), X.device, None)
    else:
        p, n = ws.data_ptr(), ws.numel() * ws.element_size()
    _check(_lib.mxs_mixed_gemm_fused(px, dt, M, ldx, _ptr(perm), ctypes.byref(w), py, ldy, p, n,
                                     _stream(X.device)), "mxs_mixed_gemm_fused")
    return Y


# ------------------------------------------------------------ prepared weights
def mxs_prepare_weights_size(W: QMat) -> int:
    return int(_lib.mxs_prepare_weights_size(ctypes.byref(W.c_struct())))


def mxs_prepare_weights(W: QMat, out: torch.Tensor | None = None) -> torch.Tensor:
    """W's prefill operand built once (uint8 device buffer, contents private
    to the library), for mxs_mixed_gemm_prepared / mxs_mixed_gemm_fused_prepared."""
    n = mxs_prepare_weights_size(W)
    if out is None:
        out = torch.empty(max(n, 1), dtype=torch.uint8, device=W.sc.device)
    if out.dtype != torch.uint8 or not out.is_cuda or not out.is_contiguous():
        raise ValueError("out must be a contiguous uint8 GPU tensor")
    _check(_lib.mxs_prepare_weights(ctypes.byref(W.c_struct()), out.data_ptr(), out.numel(),
                                    _stream(out.device)), "mxs_prepare_weights")
    return out


def mxs_mixed_gemm_prepared_workspace(A: QMat, W: QMat) -> int:
    return int(_lib.mxs_mixed_gemm_prepared_workspace(ctypes.byref(A.c_struct()), ctypes.byref(W.c_struct())))


def mxs_mixed_gemm_prepared(A: QMat, W: QMat, wprep: torch.Tensor, Y: torch.Tensor | None = None,
                            ws=None) -> torch.Tensor:
    """mxs_mixed_gemm with W's operand taken from mxs_prepare_weights(W)."""
    dev = A.sc.device
    if Y is None:
        Y = torch.empty((A.rows, W.rows), dtype=torch.float32, device=dev)
    if Y.dtype != torch.float32:
        raise TypeError("Y must be fp32")
    py, ldy = _dev2d(Y, "Y")
    a, w = ctypes.byref(A.c_struct()), ctypes.byref(W.c_struct())
    if ws is None:
        p, n = _workspace(int(_lib.mxs_mixed_gemm_prepared_workspace(a, w)), dev, None)
    else:
        p, n = ws.data_ptr(), ws.numel() * ws.element_size()
    _check(_lib.mxs_mixed_gemm_prepared(a, w, wprep.data_ptr(), wprep.numel() * wprep.element_size(), py, ldy,
                                        p, n, _stream(dev)), "mxs_mixed_gemm_prepared")
    return Y


def mxs_mixed_gemm_fused_prepared_workspace(M: int, dtype: torch.dtype, W: QMat) -> int:
    dt = MXS_BF16 if dtype == torch.bfloat16 else MXS_F32
    return int(_lib.mxs_mixed_gemm_fused_prepared_workspace(M, dt, ctypes.byref(W.c_struct())))


def mxs_mixed_gemm_fused_prepared(X: torch.Tensor, perm: torch.Tensor | None, W: QMat, wprep: torch.Tensor,
                                  Y: torch.Tensor | None = None, ws=None) -> torch.Tensor:
    """mxs_mixed_gemm_fused with W's operand taken from mxs_prepare_weights(W)."""
    px, ldx, M, Y, py, ldy = _fused_args(X, perm, W, Y)
    w = W.c_struct()
    dt = _dtype(X)
    if ws is None:
        p, n = _workspace(int(_lib.mxs_mixed_gemm_fused_prepared_workspace(M, dt, ctypes.byref(w))), X.device,
                          None)
    else:
        p, n = ws.data_ptr(), ws.numel() * ws.element_size()
    _check(_lib.mxs_mixed_gemm_fused_prepared(px, dt, M, ldx, _ptr(perm), ctypes.byref(w), wprep.data_ptr(),
                                              wprep.numel() * wprep.element_size(), py, ldy, p, n,
                                              _stream(X.device)), "mxs_mixed_gemm_fused_prepared")
    return Y


def mxs_mixed_gemm_mx_workspace(A: QMat, W: QMat) -> int:
    a, w = A.c_struct(), W.c_struct()
    return int(_lib.mxs_mixed_gemm_mx_workspace(ctypes.byref(a), ctypes.byref(w)))


def mxs_mixed_gemm_mx(A: QMat, W: QMat, Y: torch.Tensor | None = None, ws=None) -> torch.Tensor:
    """The same product, prefill on the block-scaled fp6 matrix cores."""
    return _gemm(_lib.mxs_mixed_gemm_mx, _lib.mxs_mixed_gemm_mx_workspace, "mxs_mixed_gemm_mx", A, W, Y, ws)


def mxs_quantize_kv(kv: torch.Tensor, codes=None, scales=None):
    """codes uint8 [T, H, D/2], scales uint8 [T, H, D/32] for kv [T, H, D]."""
    if not kv.is_cuda or kv.dim() != 3 or not kv.is_contiguous():
        raise ValueError("kv must be a contiguous [T, H, D] GPU tensor")
    T, H, D = kv.shape
    if codes is None:
        codes = torch.empty((T, H, D // 2), dtype=torch.uint8, device=kv.device)
    if scales is None:
        scales = torch.empty((T, H, D // 32), dtype=torch.uint8, device=kv.device)
    _check(_lib.mxs_quantize_kv(kv.data_ptr(), _dtype(kv), T, H, D, _ptr(codes), _ptr(scales),
                                _stream(kv.device)), "mxs_quantize_kv")
    return codes, scales


# ------------------------------------------------------------ layer-wise budget
def mxs_allocate_blocks(score: torch.Tensor, n8: int, n6: int, bits=None, perm=None):
    """mxs_allocate with the block counts given: (bits, perm)."""
    if not score.is_cuda or score.dtype != torch.float64 or not score.is_contiguous():
        raise ValueError("score must be a contiguous fp64 GPU tensor")
    K = score.numel()
    if bits is None:
        bits = torch.empty(K, dtype=torch.uint8, device=score.device)
    if perm is None:
        perm = torch.empty(K, dtype=torch.int32, device=score.device)
    _check(_lib.mxs_allocate_blocks(score.data_ptr(), K, n8, n6, bits.data_ptr(), perm.data_ptr(),
                                    _stream(score.device)), "mxs_allocate_blocks")
    return bits, perm


def mxs_output_error_workspace(M: int, N: int) -> int:
    return int(_lib.mxs_output_error_workspace(M, N))


def mxs_output_error(X: torch.Tensor, W: torch.Tensor, Yq: torch.Tensor, err=None, ws=None) -> torch.Tensor:
    """err (fp64 [1] on the GPU) = sum over (t, n) of (X W^T - Yq)^2."""
    px, ldx = _dev2d(X, "X")
    pw, ldw = _dev2d(W, "W")
    py, ldy = _dev2d(Yq, "Yq")
    if X.dtype != W.dtype:
        raise TypeError("X and W must have the same element type")
    if Yq.dtype != torch.float32:
        raise TypeError("Yq must be fp32")
    M, K = X.shape
    N = W.shape[0]
    if W.shape[1] != K or tuple(Yq.shape) != (M, N):
        raise ValueError("shapes do not match: X [M, K], W [N, K], Yq [M, N]")
    if err is None:
        err = torch.empty(1, dtype=torch.float64, device=X.device)
    p, n = _workspace(mxs_output_error_workspace(M, N), X.device, ws)
    _check(_lib.mxs_output_error(px, pw, _dtype(X), M, N, K, ldx, ldw, py, ldy, err.data_ptr(), p, n,
                                 _stream(X.device)), "mxs_output_error")
    return err


def mxs_layer_budget(S, rows, K, B: float):
    """(blocks [L][3] as (n8, n6, n4) lists, R) for layer sensitivities S."""
    L = len(S)
    s_arr = (ctypes.c_double * L)(*[float(x) for x in S])
    r_arr = (c_int64 * L)(*[int(x) for x in rows])
    k_arr = (c_int64 * L)(*[int(x) for x in K])
    out = (c_int32 * (3 * L))()
    R = c_double(0.0)
    _check(_lib.mxs_layer_budget(L, ctypes.cast(s_arr, c_void_p), ctypes.cast(r_arr, c_void_p),
                                 ctypes.cast(k_arr, c_void_p), float(B), ctypes.cast(out, c_void_p),
                                 ctypes.byref(R)), "mxs_layer_budget")
    return [[out[3 * i], out[3 * i + 1], out[3 * i + 2]] for i in range(L)], R.value


# ------------------------------------------------------- attention over KV4
def mxs_attend_kv4_workspace(T: int, Hq: int, Hkv: int, D: int) -> int:
    return int(_lib.mxs_attend_kv4_workspace(T, Hq, Hkv, D))


def mxs_attend_kv4(q: torch.Tensor, k_cache, v_cache, scale: float, out=None, ws=None) -> torch.Tensor:
    """out [Hq, D] fp32: attention of one query token q [Hq, D] (fp32) over K/V
    caches given as (codes [T, Hkv, D/2], scales [T, Hkv, D/32]) from
    mxs_quantize_kv."""
    kc, ks = k_cache
    vc, vs = v_cache
    if not q.is_cuda or q.dtype != torch.float32 or q.dim() != 2 or not q.is_contiguous():
        raise ValueError("q must be a contiguous fp32 [Hq, D] GPU tensor")
    for t in (kc, ks, vc, vs):
        if not t.is_cuda or t.dtype != torch.uint8 or t.dim() != 3 or not t.is_contiguous():
            raise ValueError("caches must be contiguous uint8 [T, Hkv, ...] GPU tensors")
    Hq, D = q.shape
    T, Hkv = kc.shape[0], kc.shape[1]
    if tuple(kc.shape) != (T, Hkv, D // 2) or tuple(vc.shape) != (T, Hkv, D // 2) \
            or tuple(ks.shape) != (T, Hkv, D // 32) or tuple(vs.shape) != (T, Hkv, D // 32):
        raise ValueError("cache shapes do not match q")
    if out is None:
        out = torch.empty((Hq, D), dtype=torch.float32, device=q.device)
    p, n = _workspace(mxs_attend_kv4_workspace(T, Hq, Hkv, D), q.device, ws)
    _check(_lib.mxs_attend_kv4(q.data_ptr(), kc.data_ptr(), ks.data_ptr(), vc.data_ptr(), vs.data_ptr(), T, Hq,
                               Hkv, D, float(scale), out.data_ptr(), p, n, _stream(q.device)), "mxs_attend_kv4")
    return out
