"""Python binding of the KDN C ABI (``include/kdn.h``) over torch tensors.

Same entry-point names as the C library.  This layer only checks tensor
metadata, allocates outputs / workspace with torch (device memory) and passes
raw pointers plus torch's current HIP stream; every step of the method runs
in the library's kernels.  Layouts: activations [B,T,H,D], state [B,H,dk,dv],
variances [B,H,dk] (Diagonal) or [B,H] (Isotropic).
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import (KDN_BF16, KDN_DIAG, KDN_F32, KDN_ISO, KDN_MATH_BF16, KDN_OUT_F32,  # noqa: F401
                   KdnError)


def _io_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KDN_BF16
    if t.dtype == torch.float32:
        return KDN_F32
    raise TypeError("q, k, v must be bfloat16 or float32, got %s" % t.dtype)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, shape, dtype, device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _math_flag(math: Optional[str]) -> int:
    """Contraction precision of the bf16 forward: None (the library's
    default: split-operand products for Diagonal, single bf16 products for
    Isotropic) or "bf16" (single bf16 products)."""
    if math is None:
        return 0
    if math == "bf16":
        return KDN_MATH_BF16
    raise ValueError("math must be None or 'bf16', got %r" % (math,))


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _head_vec(t, name, H, dev):
    if t is not None:
        _need(t, name, (H,), torch.float32, dev)
    return t


def _fwd(variant: int, q, k, v, alpha, omega, r, S0, var0, mu, o, S_T, var_T,
         ext: bool = False, mu_h=None, c0_h=None, beta_eff=None, sequence_parallel=True,
         math=None, o_dtype=None, prepare=False):
    """Checks the tensors, allocates what is missing, and launches the
    forward (or, with ``prepare``, returns (outputs, launch) where launch()
    repeats the call on the same tensors and stream without re-checking)."""
    L = _lib.lib()
    if q.dim() != 4:
        raise ValueError("q must be [B,T,H,dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    io = _io_code(q)
    _need(q, "q", (B, T, H, dk), q.dtype, dev)
    _need(k, "k", (B, T, H, dk), q.dtype, dev)
    _need(v, "v", (B, T, H, dv), q.dtype, dev)
    _need(alpha, "alpha", (B, T, H, dk), torch.float32, dev)
    wshape = (B, T, H, dk) if variant == KDN_DIAG else (B, T, H)
    _need(omega, "omega", wshape, torch.float32, dev)
    _need(r, "r", (B, T, H), torch.float32, dev)
    vshape = (B, H, dk) if variant == KDN_DIAG else (B, H)
    if S0 is not None:
        _need(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    if var0 is not None:
        _need(var0, "p0" if variant == KDN_DIAG else "b0", vshape, torch.float32, dev)
    o_dtype = q.dtype if o_dtype is None else o_dtype
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=o_dtype, device=dev)
    _need(o, "o", (B, T, H, dv), o_dtype, dev)
    if S_T is None:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    _need(S_T, "S_T", (B, H, dk, dv), torch.float32, dev)
    if var_T is None:
        var_T = torch.empty(vshape, dtype=torch.float32, device=dev)
    _need(var_T, "var_T", vshape, torch.float32, dev)
    mu = float(dk if mu is None else mu)
    io |= _math_flag(math)
    if o_dtype != q.dtype:
        if not (q.dtype == torch.bfloat16 and o_dtype == torch.float32):
            raise TypeError("o may differ from q's dtype only as fp32 with bf16 inputs")
        io |= KDN_OUT_F32
    # with the workspace, shapes with few heads and long sequences run sequence-parallel
    ws_bytes = L.kdn_fwd_workspace_size(variant, B, T, H, dk, dv, io) if sequence_parallel else 0
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    if ext:
        _head_vec(mu_h, "mu_h", H, dev)
        _head_vec(c0_h, "c0_h", H, dev)
        if beta_eff is not None:
            _need(beta_eff, "beta_eff", (B, T, H), torch.float32, dev)
        fn = L.kdn_fwd_ex
        args = (variant, B, T, H, dk, dv, io, mu, _ptr(mu_h), _ptr(q), _ptr(k), _ptr(v),
                _ptr(alpha), _ptr(omega), _ptr(r), _ptr(S0), _ptr(var0), _ptr(c0_h), _ptr(o),
                _ptr(S_T), _ptr(var_T), _ptr(beta_eff), _ptr(ws), ws_bytes)
    else:
        fn = L.kdn_diag_fwd if variant == KDN_DIAG else L.kdn_iso_fwd
        args = (B, T, H, dk, dv, io, mu, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(omega),
                _ptr(r), _ptr(S0), _ptr(var0), _ptr(o), _ptr(S_T), _ptr(var_T), _ptr(ws),
                ws_bytes)
    stream = _stream(dev)
    keep = (q, k, v, alpha, omega, r, S0, var0, o, S_T, var_T, mu_h, c0_h, beta_eff, ws)

    def launch():
        _lib.check(fn(*args, stream))
        return keep  # the tensors stay alive as long as the launcher does

    if prepare:
        return (o, S_T, var_T), launch
    with torch.cuda.device(dev):
        launch()
    return o, S_T, var_T


def kdn_diag_fwd(q, k, v, alpha, omega, r, S0=None, p0=None, mu=None, o=None, S_T=None,
                 p_T=None, math=None, o_dtype=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Diagonal KDN forward.  Returns (o [B,T,H,dv], S_T [B,H,dk,dv], p_T [B,H,dk]).
    With bf16 q/k/v the contractions run split-operand products (near fp32)
    unless math="bf16" asks for single bf16 products; o_dtype=torch.float32
    then writes o in fp32."""
    return _fwd(KDN_DIAG, q, k, v, alpha, omega, r, S0, p0, mu, o, S_T, p_T, math=math,
                o_dtype=o_dtype)


def fwd_launcher(variant: str, q, k, v, alpha, omega, r, S0=None, var0=None, mu=None,
                 o=None, S_T=None, var_T=None, math=None, o_dtype=None):
    """Check the arguments once and return ((o, S_T, var_T), launch): each
    launch() runs the same forward (kdn_diag_fwd / kdn_iso_fwd) on the same
    tensors and on the stream that was current here, without re-checking or
    allocating (a workspace the shape needs is allocated once, now)."""
    var = {"diag": KDN_DIAG, "iso": KDN_ISO}[variant]
    return _fwd(var, q, k, v, alpha, omega, r, S0, var0, mu, o, S_T, var_T, math=math,
                o_dtype=o_dtype, prepare=True)


def kdn_iso_fwd(q, k, v, alpha, omega, r, S0=None, b0=None, mu=None, o=None, S_T=None,
                b_T=None, math=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Isotropic KDN forward.  Returns (o [B,T,H,dv], S_T [B,H,dk,dv], b_T [B,H])."""
    return _fwd(KDN_ISO, q, k, v, alpha, omega, r, S0, b0, mu, o, S_T, b_T, math=math)


def kdn_fwd_ex(variant: str, q, k, v, alpha, omega, r, S0=None, var0=None, mu=None,
               mu_h=None, c0_h=None, want_beta_eff: bool = False, o=None, S_T=None,
               var_T=None, sequence_parallel: bool = True, math=None, o_dtype=None):
    """Forward with per-head mu_h [H] and c0_h [H] (both optional) and the
    effective write strength.  Returns (o, S_T, var_T, beta_eff [B,T,H] or
    None).  sequence_parallel=False withholds the workspace, so that shapes the
    library would split over the sequence run the serial walk instead."""
    var = {"diag": KDN_DIAG, "iso": KDN_ISO}[variant]
    beta = None
    if want_beta_eff:
        B, T, H, _ = q.shape
        beta = torch.empty((B, T, H), dtype=torch.float32, device=q.device)
    o, S_T, var_T = _fwd(var, q, k, v, alpha, omega, r, S0, var0, mu, o, S_T, var_T,
                         ext=True, mu_h=mu_h, c0_h=c0_h, beta_eff=beta,
                         sequence_parallel=sequence_parallel, math=math, o_dtype=o_dtype)
    return o, S_T, var_T, beta


def kdn_dense_fwd(q, k, v, alpha, omega, r, S0=None, P0=None, want_beta_eff: bool = False,
                  o=None, S_T=None, P_T=None):
    """Exact dense-covariance Kalman memory with diag(alpha) / diag(omega)
    gates, for small d_k.  Returns (o [B,T,H,dv], S_T [B,H,dk,dv],
    P_T [B,H,dk,dk], beta_eff [B,T,H] or None)."""
    L = _lib.lib()
    if q.dim() != 4:
        raise ValueError("q must be [B,T,H,dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    io = _io_code(q)
    _need(q, "q", (B, T, H, dk), q.dtype, dev)
    _need(k, "k", (B, T, H, dk), q.dtype, dev)
    _need(v, "v", (B, T, H, dv), q.dtype, dev)
    _need(alpha, "alpha", (B, T, H, dk), torch.float32, dev)
    _need(omega, "omega", (B, T, H, dk), torch.float32, dev)
    _need(r, "r", (B, T, H), torch.float32, dev)
    if S0 is not None:
        _need(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    if P0 is not None:
        _need(P0, "P0", (B, H, dk, dk), torch.float32, dev)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    _need(o, "o", (B, T, H, dv), q.dtype, dev)
    if S_T is None:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if P_T is None:
        P_T = torch.empty((B, H, dk, dk), dtype=torch.float32, device=dev)
    _need(S_T, "S_T", (B, H, dk, dv), torch.float32, dev)
    _need(P_T, "P_T", (B, H, dk, dk), torch.float32, dev)
    beta = torch.empty((B, T, H), dtype=torch.float32, device=dev) if want_beta_eff else None
    with torch.cuda.device(dev):
        st = L.kdn_dense_fwd(B, T, H, dk, dv, io, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                             _ptr(omega), _ptr(r), _ptr(S0), _ptr(P0), _ptr(o), _ptr(S_T),
                             _ptr(P_T), _ptr(beta), _stream(dev))
    _lib.check(st)
    return o, S_T, P_T, beta


def kdn_fwd_preact(variant: str, q, k, v, a_pre, w_pre, r_pre, r_min: float = 0.01, S0=None,
                   var0=None, mu=None, mu_h=None, c0_h=None, want_beta_eff: bool = False,
                   o=None, S_T=None, var_T=None, workspace=None, math=None):
    """Forward from the gates' pre-activations (alpha = sigmoid(a_pre),
    omega = softplus(w_pre), r = r_min + softplus(r_pre)); pre-activations in
    the io dtype of q.  Returns (o, S_T, var_T, beta_eff or None)."""
    L = _lib.lib()
    var = {"diag": KDN_DIAG, "iso": KDN_ISO}[variant]
    if q.dim() != 4:
        raise ValueError("q must be [B,T,H,dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    io = _io_code(q)
    iso = var == KDN_ISO
    f32 = torch.float32
    _need(q, "q", (B, T, H, dk), q.dtype, dev)
    _need(k, "k", (B, T, H, dk), q.dtype, dev)
    _need(v, "v", (B, T, H, dv), q.dtype, dev)
    _need(a_pre, "a_pre", (B, T, H, dk), q.dtype, dev)
    _need(w_pre, "w_pre", (B, T, H) if iso else (B, T, H, dk), q.dtype, dev)
    _need(r_pre, "r_pre", (B, T, H), q.dtype, dev)
    var_shape = (B, H) if iso else (B, H, dk)
    for t, n, shp in ((S0, "S0", (B, H, dk, dv)), (var0, "var0", var_shape),
                      (mu_h, "mu_h", (H,)), (c0_h, "c0_h", (H,))):
        if t is not None:
            _need(t, n, shp, f32, dev)
    mu = float(dk if mu is None else mu)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    if S_T is None:
        S_T = torch.empty((B, H, dk, dv), dtype=f32, device=dev)
    if var_T is None:
        var_T = torch.empty(var_shape, dtype=f32, device=dev)
    beta = torch.empty((B, T, H), dtype=f32, device=dev) if want_beta_eff else None
    need = int(L.kdn_fwd_preact_workspace_size(var, B, T, H, dk))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        st = L.kdn_fwd_preact(var, B, T, H, dk, dv, io | _math_flag(math), mu, _ptr(mu_h),
                              _ptr(q), _ptr(k), _ptr(v),
                              _ptr(a_pre), _ptr(w_pre), _ptr(r_pre), float(r_min), _ptr(S0),
                              _ptr(var0), _ptr(c0_h), _ptr(o), _ptr(S_T), _ptr(var_T),
                              _ptr(beta), _ptr(workspace), workspace.numel(), _stream(dev))
    _lib.check(st)
    return o, S_T, var_T, beta


def kdn_gates_from_preact(variant: str, a_pre, w_pre, r_pre, r_min: float = 0.01):
    """The gates (alpha, omega, r), fp32, from their pre-activations, with the
    arithmetic the forward from pre-activations uses (kdn_fwd_ex on these
    gates equals kdn_fwd_preact bit for bit)."""
    L = _lib.lib()
    var = {"diag": KDN_DIAG, "iso": KDN_ISO}[variant]
    if a_pre.dim() != 4:
        raise ValueError("a_pre must be [B,T,H,dk]")
    B, T, H, dk = a_pre.shape
    dev = a_pre.device
    io = _io_code(a_pre)
    iso = var == KDN_ISO
    _need(w_pre, "w_pre", (B, T, H) if iso else (B, T, H, dk), a_pre.dtype, dev)
    _need(r_pre, "r_pre", (B, T, H), a_pre.dtype, dev)
    f32 = torch.float32
    alpha = torch.empty((B, T, H, dk), dtype=f32, device=dev)
    omega = torch.empty(tuple(w_pre.shape), dtype=f32, device=dev)
    r = torch.empty((B, T, H), dtype=f32, device=dev)
    with torch.cuda.device(dev):
        st = L.kdn_gates_from_preact(var, B, T, H, dk, io, _ptr(a_pre), _ptr(w_pre), _ptr(r_pre),
                                     float(r_min), _ptr(alpha), _ptr(omega), _ptr(r), _stream(dev))
    _lib.check(st)
    return alpha, omega, r


def kdn_bwd(variant: str, q, k, v, alpha, omega, r, d_o, S0=None, var0=None, mu=None,
            mu_h=None, c0_h=None, dS_T=None, dvar_T=None, want_state_grads: bool = True,
            workspace=None) -> dict:
    """Backward pass of the forward given by the same arguments (see kdn_fwd_ex)
    for dL/do = d_o, dL/dS_T = dS_T and dL/dvar_T = dvar_T (both optional).
    Returns a dict with dq, dk, dv (io dtype), dalpha, domega, dr (fp32) and,
    with ``want_state_grads``, dS0, dvar0 and dmu [B,H] (fp32).  A given
    ``workspace`` (uint8) is passed as it is: the library requires its base
    size and splits the sequence (bf16 io, few heads) only when it holds all
    of kdn_bwd_workspace_size; without one, that size is allocated."""
    L = _lib.lib()
    var = {"diag": KDN_DIAG, "iso": KDN_ISO}[variant]
    if q.dim() != 4:
        raise ValueError("q must be [B,T,H,dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    io = _io_code(q)
    iso = var == KDN_ISO
    var_shape = (B, H) if iso else (B, H, dk)
    f32 = torch.float32
    _need(q, "q", (B, T, H, dk), q.dtype, dev)
    _need(k, "k", (B, T, H, dk), q.dtype, dev)
    _need(v, "v", (B, T, H, dv), q.dtype, dev)
    _need(d_o, "d_o", (B, T, H, dv), q.dtype, dev)
    _need(alpha, "alpha", (B, T, H, dk), f32, dev)
    _need(omega, "omega", (B, T, H) if iso else (B, T, H, dk), f32, dev)
    _need(r, "r", (B, T, H), f32, dev)
    for t, n, shp in ((S0, "S0", (B, H, dk, dv)), (dS_T, "dS_T", (B, H, dk, dv)),
                      (var0, "var0", var_shape), (dvar_T, "dvar_T", var_shape),
                      (mu_h, "mu_h", (H,)), (c0_h, "c0_h", (H,))):
        if t is not None:
            _need(t, n, shp, f32, dev)
    mu = float(dk if mu is None else mu)
    g = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
         "dalpha": torch.empty_like(alpha), "domega": torch.empty_like(omega),
         "dr": torch.empty_like(r)}
    if want_state_grads:
        g["dS0"] = torch.empty((B, H, dk, dv), dtype=f32, device=dev)
        g["dvar0"] = torch.empty(var_shape, dtype=f32, device=dev)
        g["dmu"] = torch.empty((B, H), dtype=f32, device=dev)
    if workspace is None:
        need = int(L.kdn_bwd_workspace_size(var, B, T, H, dk, dv))
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        st = L.kdn_bwd(var, B, T, H, dk, dv, io, mu, _ptr(mu_h), _ptr(q), _ptr(k), _ptr(v),
                       _ptr(alpha), _ptr(omega), _ptr(r), _ptr(S0), _ptr(var0), _ptr(c0_h),
                       _ptr(d_o), _ptr(dS_T), _ptr(dvar_T), _ptr(g["dq"]), _ptr(g["dk"]),
                       _ptr(g["dv"]), _ptr(g["dalpha"]), _ptr(g["domega"]), _ptr(g["dr"]),
                       _ptr(g.get("dS0")), _ptr(g.get("dvar0")), _ptr(g.get("dmu")),
                       _ptr(workspace), workspace.numel(), _stream(dev))
    _lib.check(st)
    return g


def kdn_bwd_preact(variant: str, q, k, v, a_pre, w_pre, r_pre, d_o, r_min: float = 0.01,
                   S0=None, var0=None, mu=None, mu_h=None, c0_h=None, dS_T=None, dvar_T=None,
                   workspace=None) -> dict:
    """Backward of kdn_fwd_preact: dq, dk, dv (io dtype), da_pre, dw_pre,
    dr_pre (fp32), dS0, dvar0, dmu."""
    L = _lib.lib()
    var = {"diag": KDN_DIAG, "iso": KDN_ISO}[variant]
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    io = _io_code(q)
    iso = var == KDN_ISO
    f32 = torch.float32
    _need(q, "q", (B, T, H, dk), q.dtype, dev)
    _need(k, "k", (B, T, H, dk), q.dtype, dev)
    _need(v, "v", (B, T, H, dv), q.dtype, dev)
    _need(d_o, "d_o", (B, T, H, dv), q.dtype, dev)
    _need(a_pre, "a_pre", (B, T, H, dk), q.dtype, dev)
    _need(w_pre, "w_pre", (B, T, H) if iso else (B, T, H, dk), q.dtype, dev)
    _need(r_pre, "r_pre", (B, T, H), q.dtype, dev)
    var_shape = (B, H) if iso else (B, H, dk)
    for t, n, shp in ((S0, "S0", (B, H, dk, dv)), (dS_T, "dS_T", (B, H, dk, dv)),
                      (var0, "var0", var_shape), (dvar_T, "dvar_T", var_shape),
                      (mu_h, "mu_h", (H,)), (c0_h, "c0_h", (H,))):
        if t is not None:
            _need(t, n, shp, f32, dev)
    mu = float(dk if mu is None else mu)
    g = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
         "da_pre": torch.empty(a_pre.shape, dtype=f32, device=dev),
         "dw_pre": torch.empty(w_pre.shape, dtype=f32, device=dev),
         "dr_pre": torch.empty(r_pre.shape, dtype=f32, device=dev),
         "dS0": torch.empty((B, H, dk, dv), dtype=f32, device=dev),
         "dvar0": torch.empty(var_shape, dtype=f32, device=dev),
         "dmu": torch.empty((B, H), dtype=f32, device=dev)}
    need = int(L.kdn_bwd_preact_workspace_size(var, B, T, H, dk, dv))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        st = L.kdn_bwd_preact(var, B, T, H, dk, dv, io, mu, _ptr(mu_h), _ptr(q), _ptr(k), _ptr(v),
                              _ptr(a_pre), _ptr(w_pre), _ptr(r_pre), float(r_min), _ptr(S0),
                              _ptr(var0), _ptr(c0_h), _ptr(d_o), _ptr(dS_T), _ptr(dvar_T),
                              *[_ptr(g[n]) for n in ("dq", "dk", "dv", "da_pre", "dw_pre",
                                                     "dr_pre", "dS0", "dvar0", "dmu")],
                              _ptr(workspace), workspace.numel(), _stream(dev))
    _lib.check(st)
    return g


def kdn_step(variant: str, q, k, v, alpha, omega, r, S, var_state, mu=None,
             o=None, mu_h=None, beta_eff=None) -> torch.Tensor:
    """One decode step; S [B,H,dk,dv] and var_state are updated in place.
    ``variant`` is "diag" or "iso".  Returns o [B,H,dv]."""
    L = _lib.lib()
    var = {"diag": KDN_DIAG, "iso": KDN_ISO}[variant]
    B, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    io = _io_code(q)
    _need(q, "q", (B, H, dk), q.dtype, dev)
    _need(k, "k", (B, H, dk), q.dtype, dev)
    _need(v, "v", (B, H, dv), q.dtype, dev)
    _need(alpha, "alpha", (B, H, dk), torch.float32, dev)
    _need(omega, "omega", (B, H, dk) if var == KDN_DIAG else (B, H), torch.float32, dev)
    _need(r, "r", (B, H), torch.float32, dev)
    _need(S, "S", (B, H, dk, dv), torch.float32, dev)
    _need(var_state, "var_state", (B, H, dk) if var == KDN_DIAG else (B, H), torch.float32, dev)
    if o is None:
        o = torch.empty((B, H, dv), dtype=q.dtype, device=dev)
    _need(o, "o", (B, H, dv), q.dtype, dev)
    mu = float(dk if mu is None else mu)
    if mu_h is not None or beta_eff is not None:
        # extended step: per-head information scale and / or the effective
        # write strength [B,H]
        _head_vec(mu_h, "mu_h", H, dev)
        if beta_eff is not None:
            _need(beta_eff, "beta_eff", (B, H), torch.float32, dev)
        with torch.cuda.device(dev):
            st = L.kdn_step_ex(var, B, H, dk, dv, io, mu, _ptr(mu_h), _ptr(q), _ptr(k), _ptr(v),
                               _ptr(alpha), _ptr(omega), _ptr(r), _ptr(S), _ptr(var_state),
                               _ptr(o), _ptr(beta_eff), _stream(dev))
        _lib.check(st)
        return o
    with torch.cuda.device(dev):
        st = L.kdn_step(var, B, H, dk, dv, io, mu, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                        _ptr(omega), _ptr(r), _ptr(S), _ptr(var_state), _ptr(o), _stream(dev))
    _lib.check(st)
    return o


def kdn_gain_scan(variant: str, k, alpha, omega, r, var0=None, mu=None,
                  want_kappa: bool = True):
    """Gain scan alone.  Returns (kappa [B,T,H,dk] fp32 or None, var_T)."""
    L = _lib.lib()
    var = {"diag": KDN_DIAG, "iso": KDN_ISO}[variant]
    B, T, H, dk = k.shape
    dev = k.device
    io = _io_code(k)
    _need(alpha, "alpha", (B, T, H, dk), torch.float32, dev)
    _need(omega, "omega", (B, T, H, dk) if var == KDN_DIAG else (B, T, H), torch.float32, dev)
    _need(r, "r", (B, T, H), torch.float32, dev)
    vshape = (B, H, dk) if var == KDN_DIAG else (B, H)
    if var0 is not None:
        _need(var0, "var0", vshape, torch.float32, dev)
    if not k.is_contiguous():
        raise ValueError("k must be contiguous")
    kappa = torch.empty((B, T, H, dk), dtype=torch.float32, device=dev) if want_kappa else None
    var_T = torch.empty(vshape, dtype=torch.float32, device=dev)
    mu = float(dk if mu is None else mu)
    ws_bytes = L.kdn_gain_workspace_size(var, B, T, H, dk)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        st = L.kdn_gain_scan(var, B, T, H, dk, io, mu, _ptr(k), _ptr(alpha), _ptr(omega),
                             _ptr(r), _ptr(var0), _ptr(kappa), _ptr(var_T), _ptr(ws),
                             ws.numel(), _stream(dev))
    _lib.check(st)
    return kappa, var_T


def kdn_gain_scan_static(variant: str, k, alpha, omega, r, var0=None, mu=None, kappa=None,
                         var_T=None):
    """Gain scan through the allocation-free entry point: its scratch is the
    library's static device array, so the call itself allocates nothing (give
    kappa and var_T to allocate nothing here either; kappa may be None to skip
    the gain).  Returns (kappa, var_T)."""
    L = _lib.lib()
    var = {"diag": KDN_DIAG, "iso": KDN_ISO}[variant]
    B, T, H, dk = k.shape
    dev = k.device
    io = _io_code(k)
    _need(k, "k", (B, T, H, dk), k.dtype, dev)
    _need(alpha, "alpha", (B, T, H, dk), torch.float32, dev)
    _need(omega, "omega", (B, T, H, dk) if var == KDN_DIAG else (B, T, H), torch.float32, dev)
    _need(r, "r", (B, T, H), torch.float32, dev)
    vshape = (B, H, dk) if var == KDN_DIAG else (B, H)
    if var0 is not None:
        _need(var0, "var0", vshape, torch.float32, dev)
    if kappa is not None:
        _need(kappa, "kappa", (B, T, H, dk), torch.float32, dev)
    if var_T is None:
        var_T = torch.empty(vshape, dtype=torch.float32, device=dev)
    _need(var_T, "var_T", vshape, torch.float32, dev)
    mu = float(dk if mu is None else mu)
    with torch.cuda.device(dev):
        st = L.kdn_gain_scan_static(var, B, T, H, dk, io, mu, _ptr(k), _ptr(alpha), _ptr(omega),
                                    _ptr(r), _ptr(var0), _ptr(kappa), _ptr(var_T), _stream(dev))
    _lib.check(st)
    return kappa, var_T


def kdn_fwd_workspace_size(variant: str, B, T, H, dk, dv, io_dtype: torch.dtype) -> int:
    var = {"diag": KDN_DIAG, "iso": KDN_ISO}[variant]
    io = KDN_BF16 if io_dtype == torch.bfloat16 else KDN_F32
    return int(_lib.lib().kdn_fwd_workspace_size(var, B, T, H, dk, dv, io))


def kdn_version() -> str:
    return _lib.lib().kdn_version().decode()
