"""ctypes binding of libgla.so (include/gla.h).  Argument marshalling only.

The functions here carry the C names.  Tensors are passed as device pointers;
every step of the computation runs in the library's HIP kernels.  If the
library is missing the first call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgla.so")

GLA_FP32 = 0
GLA_BF16 = 1
STATUS = {0: "GLA_OK", 1: "GLA_ERR_NULL", 2: "GLA_ERR_SHAPE", 3: "GLA_ERR_DTYPE",
          4: "GLA_ERR_ALIGN", 5: "GLA_ERR_WORKSPACE", 6: "GLA_ERR_HIP"}

# Every symbol include/gla.h declares.
EXPORTS = ("gla_abi_version", "gla_status_string", "gla_fwd_workspace_size",
           "gla_bwd_workspace_size", "gla_fwd", "gla_bwd", "gla_fwd_ex_workspace_size",
           "gla_fwd_ex", "gla_fwd_noalloc", "gla_bwd_ex_workspace_size", "gla_bwd_ex",
           "gla_decode", "ggla_fwd_workspace_size",
           "ggla_bwd_workspace_size", "ggla_fwd", "ggla_bwd", "gla_profile_begin",
           "gla_profile_end", "gla_profile_count", "gla_profile_get")


class GlaDims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("L", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("subchunk", ctypes.c_int32)]


# gla_fwd_algo
GLA_FWD_AUTO, GLA_FWD_TWO_PASS, GLA_FWD_FUSED, GLA_FWD_MATERIALIZED = 0, 1, 2, 3
FWD_ALGOS = {"auto": GLA_FWD_AUTO, "two_pass": GLA_FWD_TWO_PASS, "fused": GLA_FWD_FUSED,
             "materialized": GLA_FWD_MATERIALIZED}


class GlaFwdConfig(ctypes.Structure):
    _fields_ = [("algo", ctypes.c_int32), ("recur_waves", ctypes.c_int32),
                ("recur_segments", ctypes.c_int32)]


# gla_bwd_algo
GLA_BWD_AUTO, GLA_BWD_MATERIALIZED, GLA_BWD_RECURRENT = 0, 1, 2
BWD_ALGOS = {"auto": GLA_BWD_AUTO, "materialized": GLA_BWD_MATERIALIZED,
             "recurrent": GLA_BWD_RECURRENT}


class GlaBwdConfig(ctypes.Structure):
    _fields_ = [("algo", ctypes.c_int32)]


class GlaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({status_string(status)})")


_lib = None


def load():
    """Load libgla.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m chunkwise_linear_rnn_gla_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    dims_p = ctypes.POINTER(GlaDims)
    lib.gla_abi_version.argtypes = []
    lib.gla_abi_version.restype = i32
    lib.gla_status_string.argtypes = [i32]
    lib.gla_status_string.restype = ctypes.c_char_p
    for f in (lib.gla_fwd_workspace_size, lib.gla_bwd_workspace_size):
        f.argtypes = [dims_p, i32, ctypes.POINTER(sz)]
        f.restype = i32
    lib.gla_fwd.argtypes = [dims_p, i32] + [vp] * 7 + [vp, sz, vp]
    lib.gla_fwd.restype = i32
    lib.gla_bwd.argtypes = [dims_p, i32] + [vp] * 12 + [vp, sz, vp]
    lib.gla_bwd.restype = i32
    cfg_p = ctypes.POINTER(GlaFwdConfig)
    lib.gla_fwd_ex_workspace_size.argtypes = [dims_p, i32, cfg_p, ctypes.POINTER(sz)]
    lib.gla_fwd_ex_workspace_size.restype = i32
    lib.gla_fwd_ex.argtypes = [dims_p, i32, cfg_p] + [vp] * 7 + [vp, sz, vp]
    lib.gla_fwd_ex.restype = i32
    bcfg_p = ctypes.POINTER(GlaBwdConfig)
    lib.gla_bwd_ex_workspace_size.argtypes = [dims_p, i32, bcfg_p, ctypes.POINTER(sz)]
    lib.gla_bwd_ex_workspace_size.restype = i32
    lib.gla_bwd_ex.argtypes = [dims_p, i32, bcfg_p] + [vp] * 12 + [vp, sz, vp]
    lib.gla_bwd_ex.restype = i32
    lib.gla_fwd_noalloc.argtypes = [dims_p, i32] + [vp] * 7 + [vp]
    lib.gla_fwd_noalloc.restype = i32
    lib.gla_decode.argtypes = [dims_p, i32] + [vp] * 6 + [vp]
    lib.gla_decode.restype = i32
    for f in (lib.ggla_fwd_workspace_size, lib.ggla_bwd_workspace_size):
        f.argtypes = [dims_p, i32, ctypes.POINTER(sz)]
        f.restype = i32
    lib.ggla_fwd.argtypes = [dims_p, i32] + [vp] * 8 + [vp, sz, vp]
    lib.ggla_fwd.restype = i32
    lib.ggla_bwd.argtypes = [dims_p, i32] + [vp] * 14 + [vp, sz, vp]
    lib.ggla_bwd.restype = i32
    lib.gla_profile_begin.argtypes = [i32]
    lib.gla_profile_begin.restype = i32
    lib.gla_profile_end.argtypes = []
    lib.gla_profile_end.restype = None
    lib.gla_profile_count.argtypes = []
    lib.gla_profile_count.restype = i32
    lib.gla_profile_get.argtypes = [i32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_float)]
    lib.gla_profile_get.restype = i32
    _lib = lib
    return lib


def gla_abi_version() -> int:
    return load().gla_abi_version()


def status_string(status: int) -> str:
    return load().gla_status_string(int(status)).decode()


gla_status_string = status_string


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def gla_fwd_workspace_size(dims: GlaDims, dtype: int) -> int:
    n = ctypes.c_size_t(0)
    st = load().gla_fwd_workspace_size(ctypes.byref(dims), dtype, ctypes.byref(n))
    if st != 0:
        raise GlaError(st, "gla_fwd_workspace_size")
    return n.value


def gla_bwd_workspace_size(dims: GlaDims, dtype: int) -> int:
    n = ctypes.c_size_t(0)
    st = load().gla_bwd_workspace_size(ctypes.byref(dims), dtype, ctypes.byref(n))
    if st != 0:
        raise GlaError(st, "gla_bwd_workspace_size")
    return n.value


def gla_fwd(dims, dtype, q, k, v, log_alpha, h0, o, hT, workspace, workspace_bytes, stream):
    """Raw call; pointer arguments are tensors, ints or None.  Returns the status."""
    return load().gla_fwd(ctypes.byref(dims), dtype, _ptr(q), _ptr(k), _ptr(v),
                          _ptr(log_alpha), _ptr(h0), _ptr(o), _ptr(hT), _ptr(workspace),
                          workspace_bytes, stream)


def _cfg(cfg):
    return None if cfg is None else ctypes.byref(cfg)


def gla_fwd_ex_workspace_size(dims: GlaDims, dtype: int, cfg) -> int:
    n = ctypes.c_size_t(0)
    st = load().gla_fwd_ex_workspace_size(ctypes.byref(dims), dtype, _cfg(cfg), ctypes.byref(n))
    if st != 0:
        raise GlaError(st, "gla_fwd_ex_workspace_size")
    return n.value


def gla_fwd_ex(dims, dtype, cfg, q, k, v, log_alpha, h0, o, hT, workspace, workspace_bytes,
               stream):
    """Raw call with a GlaFwdConfig (or None); returns the status."""
    return load().gla_fwd_ex(ctypes.byref(dims), dtype, _cfg(cfg), _ptr(q), _ptr(k), _ptr(v),
                             _ptr(log_alpha), _ptr(h0), _ptr(o), _ptr(hT), _ptr(workspace),
                             workspace_bytes, stream)


def gla_bwd_ex_workspace_size(dims: GlaDims, dtype: int, cfg) -> int:
    n = ctypes.c_size_t(0)
    st = load().gla_bwd_ex_workspace_size(ctypes.byref(dims), dtype, _cfg(cfg), ctypes.byref(n))
    if st != 0:
        raise GlaError(st, "gla_bwd_ex_workspace_size")
    return n.value


def gla_bwd_ex(dims, dtype, cfg, q, k, v, log_alpha, h0, dout, dhT, dq, dk, dv, dlog_alpha, dh0,
               workspace, workspace_bytes, stream):
    """Raw call with a GlaBwdConfig (or None); returns the status."""
    return load().gla_bwd_ex(ctypes.byref(dims), dtype, _cfg(cfg), _ptr(q), _ptr(k), _ptr(v),
                             _ptr(log_alpha), _ptr(h0), _ptr(dout), _ptr(dhT), _ptr(dq), _ptr(dk),
                             _ptr(dv), _ptr(dlog_alpha), _ptr(dh0), _ptr(workspace),
                             workspace_bytes, stream)


def gla_fwd_noalloc(dims, dtype, q, k, v, log_alpha, h0, o, hT, stream):
    """Raw call of the allocation-free forward (scratch in the library's
    static device array); returns the status."""
    return load().gla_fwd_noalloc(ctypes.byref(dims), dtype, _ptr(q), _ptr(k), _ptr(v),
                                  _ptr(log_alpha), _ptr(h0), _ptr(o), _ptr(hT), stream)


def gla_bwd(dims, dtype, q, k, v, log_alpha, h0, dout, dhT, dq, dk, dv, dlog_alpha, dh0,
            workspace, workspace_bytes, stream):
    """Raw call; pointer arguments are tensors, ints or None.  Returns the status."""
    return load().gla_bwd(ctypes.byref(dims), dtype, _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                          _ptr(h0), _ptr(dout), _ptr(dhT), _ptr(dq), _ptr(dk), _ptr(dv),
                          _ptr(dlog_alpha), _ptr(dh0), _ptr(workspace), workspace_bytes, stream)


def ggla_fwd_workspace_size(dims: GlaDims, dtype: int) -> int:
    n = ctypes.c_size_t(0)
    st = load().ggla_fwd_workspace_size(ctypes.byref(dims), dtype, ctypes.byref(n))
    if st != 0:
        raise GlaError(st, "ggla_fwd_workspace_size")
    return n.value


def ggla_bwd_workspace_size(dims: GlaDims, dtype: int) -> int:
    n = ctypes.c_size_t(0)
    st = load().ggla_bwd_workspace_size(ctypes.byref(dims), dtype, ctypes.byref(n))
    if st != 0:
        raise GlaError(st, "ggla_bwd_workspace_size")
    return n.value


def ggla_fwd(dims, dtype, q, k, v, log_alpha, log_beta, h0, o, hT, workspace, workspace_bytes,
             stream):
    """Raw call; pointer arguments are tensors, ints or None.  Returns the status."""
    return load().ggla_fwd(ctypes.byref(dims), dtype, _ptr(q), _ptr(k), _ptr(v),
                           _ptr(log_alpha), _ptr(log_beta), _ptr(h0), _ptr(o), _ptr(hT),
                           _ptr(workspace), workspace_bytes, stream)


def ggla_bwd(dims, dtype, q, k, v, log_alpha, log_beta, h0, dout, dhT, dq, dk, dv, dlog_alpha,
             dlog_beta, dh0, workspace, workspace_bytes, stream):
    """Raw call; pointer arguments are tensors, ints or None.  Returns the status."""
    return load().ggla_bwd(ctypes.byref(dims), dtype, _ptr(q), _ptr(k), _ptr(v),
                           _ptr(log_alpha), _ptr(log_beta), _ptr(h0), _ptr(dout), _ptr(dhT),
                           _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dlog_alpha), _ptr(dlog_beta),
                           _ptr(dh0), _ptr(workspace), workspace_bytes, stream)


def gla_decode(dims, dtype, q, k, v, log_alpha, state, o, stream):
    """Raw call; pointer arguments are tensors, ints or None.  Returns the status."""
    return load().gla_decode(ctypes.byref(dims), dtype, _ptr(q), _ptr(k), _ptr(v),
                             _ptr(log_alpha), _ptr(state), _ptr(o), stream)


def gla_profile_begin(capacity: int) -> None:
    st = load().gla_profile_begin(int(capacity))
    if st != 0:
        raise GlaError(st, "gla_profile_begin")


def gla_profile_end() -> None:
    load().gla_profile_end()


def gla_profile_count() -> int:
    return load().gla_profile_count()


def gla_profile_get(index: int):
    """(kernel name, duration in ms) of the index-th launch record."""
    name = ctypes.c_char_p()
    ms = ctypes.c_float(0.0)
    st = load().gla_profile_get(int(index), ctypes.byref(name), ctypes.byref(ms))
    if st != 0:
        raise GlaError(st, "gla_profile_get")
    return name.value.decode(), ms.value
