"""MXSens hot path on MI355X: Python binding of the C-ABI library ``libmxsens.so``.

The binding only marshals arguments (torch tensors in device memory and the
current HIP stream) onto the ``mxs_*`` entry points declared in
``include/mxsens.h``; every step runs in the library's HIP kernels. The
library is loaded on first use of an ``mxs_*`` name and the import fails
loudly if it has not been built.
"""
from __future__ import annotations

_BINDING_NAMES = None


def __getattr__(name):
    if name.startswith("mxs_") or name in ("MxsError", "QMat", "qmat_alloc", "library_path",
                                          "STATUS", "NOALLOC_SCRATCH_BYTES"):
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
