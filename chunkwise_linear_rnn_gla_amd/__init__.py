"""MI355X-native Gated Linear Attention (chunkwise forward and backward).

The computation runs in ``libgla.so`` (HIP kernels for gfx950, C ABI in
``include/gla.h``).  This package only marshals arguments: PyTorch supplies
device memory and the current HIP stream.

``fwd`` / ``bwd`` allocate outputs and workspace with torch and call the
library; ``_abi`` exposes the raw C entry points under their C names.
"""
from __future__ import annotations

from . import _abi
from ._abi import (BWD_ALGOS, FWD_ALGOS, GLA_BF16, GLA_FP32, GlaBwdConfig,  # noqa: F401
                   GlaDims, GlaError, GlaFwdConfig, ggla_bwd, ggla_bwd_workspace_size, ggla_fwd,
                   ggla_fwd_workspace_size, gla_abi_version, gla_bwd, gla_bwd_ex,
                   gla_bwd_ex_workspace_size, gla_bwd_workspace_size, gla_decode, gla_fwd,
                   gla_fwd_ex, gla_fwd_ex_workspace_size, gla_fwd_workspace_size,
                   gla_status_string)

__all__ = ["fwd", "bwd", "decode", "fwd_general", "bwd_general", "dims_for", "fwd_config",
           "bwd_config", "gla_fwd", "gla_fwd_ex", "gla_bwd", "gla_bwd_ex", "gla_decode", "ggla_fwd", "ggla_bwd",
           "ggla_fwd_workspace_size", "ggla_bwd_workspace_size", "gla_fwd_workspace_size",
           "gla_fwd_ex_workspace_size", "gla_bwd_workspace_size", "gla_abi_version",
           "gla_status_string", "GlaDims", "GlaFwdConfig", "GlaError", "GLA_FP32", "GLA_BF16"]


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return GLA_BF16
    if t.dtype == torch.float32:
        return GLA_FP32
    raise TypeError(f"unsupported I/O dtype {t.dtype}")


def dims_for(q, v, chunk=64, subchunk=16) -> GlaDims:
    B, H, L, dk = q.shape
    return GlaDims(B, H, L, dk, v.shape[-1], chunk, subchunk)


def _check(t, name, dtype=None, shape=None, device=None, require_device=True):
    """Reject a tensor the library could not use as described: wrong dtype,
    shape, layout or device.  Runs before any call into the library, so a
    wrong buffer never reaches a kernel (the C side sees only a pointer)."""
    if t is None:
        return
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if require_device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def fwd_config(algo="auto", recur_waves=0, recur_segments=0):
    """A GlaFwdConfig for gla_fwd_ex: algo in "auto", "two_pass", "fused",
    "materialized"; recur_waves / recur_segments 0 for automatic."""
    if algo not in FWD_ALGOS:
        raise ValueError(f"unknown forward algo {algo!r}; one of {sorted(FWD_ALGOS)}")
    return GlaFwdConfig(FWD_ALGOS[algo], int(recur_waves), int(recur_segments))


def _stream(device):
    return _torch().cuda.current_stream(device).cuda_stream


def bwd_config(algo="auto"):
    """A GlaBwdConfig for gla_bwd_ex: algo in "auto", "materialized", "recurrent"."""
    if algo not in BWD_ALGOS:
        raise ValueError(f"unknown backward algo {algo!r}; one of {sorted(BWD_ALGOS)}")
    return GlaBwdConfig(BWD_ALGOS[algo])


def fwd(q, k, v, log_alpha, h0=None, chunk=64, subchunk=16, final_state=True, workspace=None,
        out=None, algo="auto", recur_waves=0, recur_segments=0):
    """GLA forward.  q, k [B,H,L,dk], v [B,H,L,dv] (fp32 or bf16), log_alpha
    [B,H,L,dk] fp32, h0 [B,H,dk,dv] fp32 or None.  algo / recur_waves /
    recur_segments select the forward path (see fwd_config; the defaults are
    gla_fwd's automatic choice).  Returns (o, hT or None)."""
    torch = _torch()
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    io = q.dtype
    dev = q.device
    _check(q, "q", io)
    _check(k, "k", io, q.shape, dev)
    _check(v, "v", io, (B, H, L, dv), dev)
    _check(log_alpha, "log_alpha", torch.float32, q.shape, dev)
    _check(h0, "h0", torch.float32, (B, H, dk, dv), dev)
    _check(out, "out", io, (B, H, L, dv), dev)
    _check(workspace, "workspace", torch.uint8, None, dev)
    dims = GlaDims(B, H, L, dk, dv, chunk, subchunk)
    code = _dtype_code(q)
    cfg = fwd_config(algo, recur_waves, recur_segments)
    o = out if out is not None else torch.empty(B, H, L, dv, dtype=io, device=dev)
    hT = torch.empty(B, H, dk, dv, dtype=torch.float32, device=dev) if final_state else None
    n = gla_fwd_ex_workspace_size(dims, code, cfg)
    if workspace is None or workspace.numel() < n:
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    st = gla_fwd_ex(dims, code, cfg, q, k, v, log_alpha, h0, o, hT, workspace,
                    workspace.numel(), _stream(dev))
    if st != 0:
        raise GlaError(st, "gla_fwd_ex")
    return o, hT


def bwd(q, k, v, log_alpha, h0, dout, dhT=None, chunk=64, subchunk=16, want_dh0=True,
        workspace=None, algo="auto"):
    """GLA backward.  algo selects the path (see bwd_config; the default is
    gla_bwd's automatic choice).  Returns (dq, dk, dv, dlog_alpha, dh0 or None)."""
    torch = _torch()
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    io = q.dtype
    _check(q, "q", io)
    _check(k, "k", io, q.shape, q.device)
    _check(v, "v", io, (B, H, L, dv), q.device)
    _check(log_alpha, "log_alpha", torch.float32, q.shape, q.device)
    _check(h0, "h0", torch.float32, (B, H, dk, dv), q.device)
    _check(dout, "dout", io, (B, H, L, dv), q.device)
    _check(dhT, "dhT", torch.float32, (B, H, dk, dv), q.device)
    _check(workspace, "workspace", torch.uint8, None, q.device)
    dims = GlaDims(B, H, L, dk, dv, chunk, subchunk)
    code = _dtype_code(q)
    dq = torch.empty_like(q)
    dkk = torch.empty_like(k)
    dvv = torch.empty_like(v)
    dla = torch.empty_like(log_alpha)
    dh0 = torch.empty(B, H, dk, dv, dtype=torch.float32, device=q.device) if want_dh0 else None
    cfg = bwd_config(algo)
    n = gla_bwd_ex_workspace_size(dims, code, cfg)
    if workspace is None or workspace.numel() < n:
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    st = gla_bwd_ex(dims, code, cfg, q, k, v, log_alpha, h0, dout, dhT, dq, dkk, dvv, dla, dh0,
                    workspace, workspace.numel(), _stream(q.device))
    if st != 0:
        raise GlaError(st, "gla_bwd_ex")
    return dq, dkk, dvv, dla, dh0


def decode(q, k, v, log_alpha, state, out=None):
    """One token of the recurrent form, in place on `state`.  q, k [B,H,dk],
    v [B,H,dv] (fp32 or bf16), log_alpha [B,H,dk] fp32, state [B,H,dk,dv]
    fp32 (updated).  Returns o [B,H,dv]."""
    torch = _torch()
    B, H, dk = q.shape
    dv = v.shape[-1]
    io = q.dtype
    _check(q, "q", io)
    _check(k, "k", io, q.shape, q.device)
    _check(v, "v", io, (B, H, dv), q.device)
    _check(log_alpha, "log_alpha", torch.float32, q.shape, q.device)
    _check(state, "state", torch.float32, (B, H, dk, dv), q.device)
    o = out if out is not None else torch.empty(B, H, dv, dtype=io, device=q.device)
    _check(o, "out", io, (B, H, dv), q.device)
    st = gla_decode(GlaDims(B, H, 1, dk, dv, 64, 16), _dtype_code(q), q, k, v, log_alpha, state,
                    o, _stream(q.device))
    if st != 0:
        raise GlaError(st, "gla_decode")
    return o


def fwd_general(q, k, v, log_alpha, log_beta, h0=None, final_state=True, workspace=None,
                out=None):
    """Forward with the general gate G_t = alpha_t^T beta_t.  As ``fwd``, plus
    log_beta [B,H,L,dv] fp32 (the column gate).  Returns (o, hT or None)."""
    torch = _torch()
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    io = q.dtype
    _check(q, "q", io)
    _check(k, "k", io, q.shape, q.device)
    _check(v, "v", io, (B, H, L, dv), q.device)
    _check(log_alpha, "log_alpha", torch.float32, q.shape, q.device)
    _check(log_beta, "log_beta", torch.float32, (B, H, L, dv), q.device)
    _check(h0, "h0", torch.float32, (B, H, dk, dv), q.device)
    _check(out, "out", io, (B, H, L, dv), q.device)
    _check(workspace, "workspace", torch.uint8, None, q.device)
    dims = GlaDims(B, H, L, dk, dv, 16, 16)
    code = _dtype_code(q)
    o = out if out is not None else torch.empty(B, H, L, dv, dtype=io, device=q.device)
    hT = torch.empty(B, H, dk, dv, dtype=torch.float32, device=q.device) if final_state else None
    n = ggla_fwd_workspace_size(dims, code)
    if workspace is None or workspace.numel() < n:
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    st = ggla_fwd(dims, code, q, k, v, log_alpha, log_beta, h0, o, hT, workspace,
                  workspace.numel(), _stream(q.device))
    if st != 0:
        raise GlaError(st, "ggla_fwd")
    return o, hT


def bwd_general(q, k, v, log_alpha, log_beta, h0, dout, dhT=None, want_dh0=True,
                workspace=None):
    """Backward of ``fwd_general``.  Returns (dq, dk, dv, dlog_alpha, dlog_beta,
    dh0 or None)."""
    torch = _torch()
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    io = q.dtype
    _check(q, "q", io)
    _check(k, "k", io, q.shape, q.device)
    _check(v, "v", io, (B, H, L, dv), q.device)
    _check(log_alpha, "log_alpha", torch.float32, q.shape, q.device)
    _check(log_beta, "log_beta", torch.float32, (B, H, L, dv), q.device)
    _check(h0, "h0", torch.float32, (B, H, dk, dv), q.device)
    _check(dout, "dout", io, (B, H, L, dv), q.device)
    _check(dhT, "dhT", torch.float32, (B, H, dk, dv), q.device)
    dims = GlaDims(B, H, L, dk, dv, 16, 16)
    code = _dtype_code(q)
    dq, dkk, dvv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dla, dlb = torch.empty_like(log_alpha), torch.empty_like(log_beta)
    dh0 = torch.empty(B, H, dk, dv, dtype=torch.float32, device=q.device) if want_dh0 else None
    n = ggla_bwd_workspace_size(dims, code)
    if workspace is None or workspace.numel() < n:
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    st = ggla_bwd(dims, code, q, k, v, log_alpha, log_beta, h0, dout, dhT, dq, dkk, dvv, dla,
                  dlb, dh0, workspace, workspace.numel(), _stream(q.device))
    if st != 0:
        raise GlaError(st, "ggla_bwd")
    return dq, dkk, dvv, dla, dlb, dh0
