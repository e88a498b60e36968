"""kalman_delta_rule_amd -- Kalman Delta Network (KDN) mixer on MI355X (gfx950).

The compute lives in the HIP library ``libkdn.so`` (C ABI in
``include/kdn.h``); ``api`` is a thin torch binding with the same entry-point
names.  Importing the package does not load the library; the first call
does, and fails loudly if it has not been built.
"""
from .api import (  # noqa: F401
    KDN_BF16,
    KDN_DIAG,
    KDN_F32,
    KDN_ISO,
    KDN_MATH_BF16,
    KDN_OUT_F32,
    KdnError,
    fwd_launcher,
    kdn_diag_fwd,
    kdn_bwd,
    kdn_bwd_preact,
    kdn_dense_fwd,
    kdn_fwd_ex,
    kdn_fwd_preact,
    kdn_gates_from_preact,
    kdn_fwd_workspace_size,
    kdn_gain_scan,
    kdn_iso_fwd,
    kdn_step,
    kdn_version,
)

__all__ = [
    "kdn_diag_fwd",
    "kdn_iso_fwd",
    "kdn_step",
    "kdn_fwd_ex",
    "kdn_fwd_preact",
    "kdn_gates_from_preact",
    "kdn_dense_fwd",
    "kdn_bwd",
    "kdn_bwd_preact",
    "kdn_gain_scan",
    "kdn_fwd_workspace_size",
    "kdn_version",
    "fwd_launcher",
    "KdnError",
]
