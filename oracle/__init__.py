"""The oracle: plain, slow, fp64 CPU implementations of GLA.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package.  The HIP library never
links, loads or calls anything here, and nothing here imports the HIP
package: the two share no code.

Contents
--------
* ``fwd`` / ``bwd``: the token-by-token recurrence and its back-propagation
  through time, in C (``gla_oracle.c``), threaded over (batch, head).
* ``chunkwise_fwd``: the chunkwise form with secondary chunking in NumPy
  (``chunkwise.py``), an independent formulation used to pin ``fwd``.
* ``closed_form_dlog_alpha``: the pages' closed-form gate gradient, used to pin
  ``bwd`` (and, through it, the GPU path's use of that closed form).
* ``ggla_fwd`` / ``ggla_bwd``: the general gate G_t = alpha_t^T beta_t (notes,
  App. C) as the same token recurrence and BPTT in C;
  ``closed_form_general``: its closed-form dlog alpha and dlog beta.

All functions take and return NumPy float64 arrays laid out [B, H, L, d]
(states [B, H, dk, dv]).

Pins: every function here is checked in ``tests/test_oracle_pins.py``
against results fixed by the pages and by mathematics (parallel form at
alpha == 1, brute-force per-pair decay products, chunk-size invariance,
constant-gate closed form, segment splitting, finite differences, autograd of
an independent formulation).  No function is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .chunkwise import chunkwise_fwd  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gla_oracle.c")
_LIB = os.path.join(_HERE, "libgla_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile gla_oracle.c into libgla_oracle.so with the host C compiler."""
    global _lib
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", tmp, _SRC,
               "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
        _lib = None
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        i = ctypes.c_int
        lib.gla_oracle_fwd.argtypes = [i, i, i, i, i, dp, dp, dp, dp, dp, dp, dp, i]
        lib.gla_oracle_fwd.restype = i
        lib.gla_oracle_bwd.argtypes = [i, i, i, i, i] + [dp] * 12 + [i]
        lib.gla_oracle_bwd.restype = i
        lib.ggla_oracle_fwd.argtypes = [i, i, i, i, i] + [dp] * 8 + [i]
        lib.ggla_oracle_fwd.restype = i
        lib.ggla_oracle_bwd.argtypes = [i, i, i, i, i] + [dp] * 14 + [i]
        lib.ggla_oracle_bwd.restype = i
        _lib = lib
    return _lib


def default_threads() -> int:
    """Threads for the oracle: the CPUs this process may use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _p(x):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _c64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def fwd(q, k, v, log_alpha, h0=None, nthreads=None):
    """Token-by-token GLA forward in fp64. Returns (o, hT)."""
    q, k, v, a, h0 = (_c64(x) for x in (q, k, v, log_alpha, h0))
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and a.shape == q.shape and v.shape == (B, H, L, dv)
    if h0 is not None:
        assert h0.shape == (B, H, dk, dv)
    o = np.empty((B, H, L, dv))
    hT = np.empty((B, H, dk, dv))
    rc = _load().gla_oracle_fwd(B, H, L, dk, dv, _p(q), _p(k), _p(v), _p(a), _p(h0),
                                _p(o), _p(hT), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"gla_oracle_fwd failed ({rc})")
    return o, hT


def bwd(q, k, v, log_alpha, h0, dout, dhT=None, nthreads=None):
    """BPTT of the recurrence in fp64. Returns (dq, dk, dv, dlog_alpha, dh0)."""
    q, k, v, a, h0, do, dhT = (_c64(x) for x in (q, k, v, log_alpha, h0, dout, dhT))
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    assert do.shape == v.shape
    dq = np.empty_like(q)
    dkk = np.empty_like(k)
    dvv = np.empty_like(v)
    da = np.empty_like(a)
    dh0 = np.empty((B, H, dk, dv))
    rc = _load().gla_oracle_bwd(B, H, L, dk, dv, _p(q), _p(k), _p(v), _p(a), _p(h0),
                                _p(do), _p(dhT), _p(dq), _p(dkk), _p(dvv), _p(da),
                                _p(dh0), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"gla_oracle_bwd failed ({rc})")
    return dq, dkk, dvv, da, dh0


def closed_form_dlog_alpha(q, k, dq, dk, hT=None, dhT=None):
    """The pages' closed-form gate gradient, in fp64.

    zako-mio deep-reading report, ch. 3.4 technique B; papercache.org notes
    §4.3 and App. B (derivation of dlog alpha): with b_t the cumulative gate
    product, dlog b_t = q_t ⊙ dq_t - k_t ⊙ dk_t and dlog alpha_t is the sum of
    dlog b_i over i >= t.  When the final state hT also receives a gradient dhT,
    log b_L enters hT = diag(b_L) (...) directly, which adds rowsum(hT ⊙ dhT)
    to dlog b_L and hence to every dlog alpha_t (derived; the pages take
    dhT = 0).
    """
    dlogb = np.asarray(q, np.float64) * dq - np.asarray(k, np.float64) * dk
    out = np.flip(np.cumsum(np.flip(dlogb, axis=-2), axis=-2), axis=-2)
    if dhT is not None:
        out = out + np.sum(np.asarray(hT) * np.asarray(dhT), axis=-1)[..., None, :]
    return out


def ggla_fwd(q, k, v, log_alpha, log_beta, h0=None, nthreads=None):
    """Token-by-token forward with the general gate G_t = alpha_t^T beta_t
    (log_beta [B, H, L, dv]) in fp64.  Returns (o, hT)."""
    q, k, v, a, b, h0 = (_c64(x) for x in (q, k, v, log_alpha, log_beta, h0))
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and a.shape == q.shape and v.shape == (B, H, L, dv)
    assert b.shape == v.shape
    if h0 is not None:
        assert h0.shape == (B, H, dk, dv)
    o = np.empty((B, H, L, dv))
    hT = np.empty((B, H, dk, dv))
    rc = _load().ggla_oracle_fwd(B, H, L, dk, dv, _p(q), _p(k), _p(v), _p(a), _p(b), _p(h0),
                                 _p(o), _p(hT), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"ggla_oracle_fwd failed ({rc})")
    return o, hT


def ggla_bwd(q, k, v, log_alpha, log_beta, h0, dout, dhT=None, nthreads=None):
    """BPTT of the general-gate recurrence in fp64.
    Returns (dq, dk, dv, dlog_alpha, dlog_beta, dh0)."""
    q, k, v, a, b, h0, do, dhT = (_c64(x) for x in (q, k, v, log_alpha, log_beta, h0, dout,
                                                    dhT))
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    assert do.shape == v.shape and b.shape == v.shape
    dq = np.empty_like(q)
    dkk = np.empty_like(k)
    dvv = np.empty_like(v)
    da = np.empty_like(a)
    db = np.empty_like(b)
    dh0 = np.empty((B, H, dk, dv))
    rc = _load().ggla_oracle_bwd(B, H, L, dk, dv, _p(q), _p(k), _p(v), _p(a), _p(b), _p(h0),
                                 _p(do), _p(dhT), _p(dq), _p(dkk), _p(dvv), _p(da), _p(db),
                                 _p(dh0), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"ggla_oracle_bwd failed ({rc})")
    return dq, dkk, dvv, da, db, dh0


def closed_form_general(q, k, v, o, dq, dk, dv, dout, hT=None, dhT=None):
    """Closed-form gate gradients of the general gate, in fp64.

    Notes, App. C (memory-efficient gradients of the general form): with the
    cumulative products b_t of alpha and d_t of beta, the parallel form puts
    b_t on q_t, 1/b_s on k_s, 1/d_s on v_s and d_t on o_t, so
        dlog b_t = q_t ⊙ dq_t - k_t ⊙ dk_t,   dlog d_t = o_t ⊙ do_t - v_t ⊙ dv_t
    and each dlog gate is the sum of its dlog cumulative product over later
    tokens.  hT carries b_L and d_L as well, which adds the row sums
    (alpha) and column sums (beta) of hT ⊙ dhT to the last token's terms.
    Returns (dlog_alpha, dlog_beta)."""
    f = lambda x: np.asarray(x, np.float64)
    rev = lambda x: np.flip(np.cumsum(np.flip(x, axis=-2), axis=-2), axis=-2)
    da = rev(f(q) * f(dq) - f(k) * f(dk))
    db = rev(f(o) * f(dout) - f(v) * f(dv))
    if dhT is not None:
        P = f(hT) * f(dhT)
        da = da + np.sum(P, axis=-1)[..., None, :]
        db = db + np.sum(P, axis=-2)[..., None, :]
    return da, db
