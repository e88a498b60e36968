"""ctypes loader for ``libkdn.so`` (the HIP library).  Argument marshalling
only: every step of the computation runs in the library's kernels.

The library must have been built (``python -m kalman_delta_rule_amd.build``);
there is no fallback: a missing library raises ``KdnLibraryMissing``.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkdn.so")

KDN_F32, KDN_BF16 = 0, 1
KDN_DIAG, KDN_ISO = 0, 1
KDN_MATH_BF16 = 0x100  # OR-ed into io_dtype: single bf16 products in the Diagonal bf16 forward
KDN_OUT_F32 = 0x200    # OR-ed into io_dtype: fp32 o from bf16 q, k, v (Diagonal, split products)

_lib = None


class KdnLibraryMissing(RuntimeError):
    pass


class KdnError(RuntimeError):
    def __init__(self, status: int, name: str, message: str):
        super().__init__("%s (%d): %s" % (name, status, message))
        self.status = status
        self.name = name
        self.message = message


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise KdnLibraryMissing(
            "libkdn.so is not built (expected at %s); run "
            "`python -m kalman_delta_rule_amd.build`" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    vp, fp, i, f, sz = (ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_float,
                        ctypes.c_size_t)
    L.kdn_fwd_workspace_size.restype = sz
    L.kdn_fwd_workspace_size.argtypes = [i] * 7
    fwd_args = [i] * 6 + [f] + [vp] * 3 + [fp] * 5 + [vp, fp, fp, vp, sz, vp]
    for name in ("kdn_diag_fwd", "kdn_iso_fwd"):
        fn = getattr(L, name)
        fn.restype = i
        fn.argtypes = fwd_args
    L.kdn_step.restype = i
    L.kdn_step.argtypes = [i] * 6 + [f] + [vp] * 3 + [fp] * 3 + [fp, fp, vp, vp]
    L.kdn_fwd_ex.restype = i
    L.kdn_fwd_ex.argtypes = ([i] * 7 + [f] + [fp] + [vp] * 3 + [fp] * 6 + [vp] + [fp] * 3
                             + [vp, sz, vp])
    L.kdn_dense_fwd.restype = i
    L.kdn_dense_fwd.argtypes = [i] * 6 + [vp] * 3 + [fp] * 5 + [vp] + [fp] * 3 + [vp]
    L.kdn_fwd_preact_workspace_size.restype = sz
    L.kdn_fwd_preact_workspace_size.argtypes = [i] * 5
    L.kdn_fwd_preact.restype = i
    L.kdn_fwd_preact.argtypes = ([i] * 7 + [f] + [fp] + [vp] * 6 + [f] + [fp] * 3 + [vp]
                                 + [fp] * 3 + [vp, sz, vp])
    L.kdn_gates_from_preact.restype = i
    L.kdn_gates_from_preact.argtypes = [i] * 6 + [vp] * 3 + [f] + [fp] * 3 + [vp]
    L.kdn_bwd_preact_workspace_size.restype = sz
    L.kdn_bwd_preact_workspace_size.argtypes = [i] * 6
    L.kdn_bwd_preact.restype = i
    L.kdn_bwd_preact.argtypes = ([i] * 7 + [f] + [fp] + [vp] * 6 + [f] + [fp] * 3 + [vp]
                                 + [fp] * 2 + [vp] * 3 + [fp] * 6 + [vp, sz, vp])
    L.kdn_bwd_workspace_size.restype = sz
    L.kdn_bwd_workspace_size.argtypes = [i] * 6
    L.kdn_bwd.restype = i
    L.kdn_bwd.argtypes = ([i] * 7 + [f] + [fp] + [vp] * 3 + [fp] * 6 + [vp] + [fp] * 2
                          + [vp] * 3 + [fp] * 6 + [vp, sz, vp])
    L.kdn_step_ex.restype = i
    L.kdn_step_ex.argtypes = [i] * 6 + [f] + [fp] + [vp] * 3 + [fp] * 5 + [vp, fp, vp]
    L.kdn_gain_workspace_size.restype = sz
    L.kdn_gain_workspace_size.argtypes = [i] * 5
    L.kdn_gain_scan.restype = i
    L.kdn_gain_scan.argtypes = [i] * 6 + [f] + [vp] + [fp] * 4 + [fp, fp, vp, sz, vp]
    L.kdn_gain_scan_static_max_bytes.restype = sz
    L.kdn_gain_scan_static_max_bytes.argtypes = []
    L.kdn_gain_scan_static.restype = i
    L.kdn_gain_scan_static.argtypes = [i] * 6 + [f] + [vp] + [fp] * 4 + [fp, fp, vp]
    L.kdn_status_string.restype = ctypes.c_char_p
    L.kdn_status_string.argtypes = [i]
    L.kdn_last_error_message.restype = ctypes.c_char_p
    L.kdn_last_error_message.argtypes = []
    L.kdn_version.restype = ctypes.c_char_p
    L.kdn_version.argtypes = []
    _lib = L
    return L


EXPORTED = ("kdn_fwd_workspace_size", "kdn_diag_fwd", "kdn_iso_fwd", "kdn_step",
            "kdn_fwd_ex", "kdn_step_ex", "kdn_dense_fwd", "kdn_bwd_workspace_size", "kdn_bwd",
            "kdn_fwd_preact_workspace_size", "kdn_fwd_preact", "kdn_gates_from_preact",
            "kdn_bwd_preact_workspace_size", "kdn_bwd_preact",
            "kdn_gain_workspace_size", "kdn_gain_scan", "kdn_gain_scan_static_max_bytes",
            "kdn_gain_scan_static", "kdn_status_string",
            "kdn_last_error_message", "kdn_version")


def check(status: int) -> None:
    if status != 0:
        L = lib()
        raise KdnError(status, L.kdn_status_string(status).decode(),
                       L.kdn_last_error_message().decode())
