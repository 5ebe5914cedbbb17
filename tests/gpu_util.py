"""Helpers for the GPU parity tests: move seeded inputs to the device, call the
HIP path through the C ABI binding, compare with the oracle in fp64."""
import numpy as np
import torch

import oracle
from chunkwise_linear_rnn_gla_amd import GLA_BF16, GLA_FP32, GlaDims, GlaError, _abi
from chunkwise_linear_rnn_gla_amd import bwd as gla_bwd_t
from chunkwise_linear_rnn_gla_amd import fwd as gla_fwd_t
from chunkwise_linear_rnn_gla_amd import (bwd_config, fwd_config, gla_bwd_ex_workspace_size,
                                          gla_fwd_ex_workspace_size)
from chunkwise_linear_rnn_gla_amd.inputs import as_f64

# Tolerances (relative L2 per output tensor): the required bar for fp32 I/O and
# for bf16 I/O with fp32 accumulation.
TOL = {"fp32": 1e-5, "bf16": 5e-3}


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (n if n > 0 else 1.0))


def dtype_name(x):
    return "bf16" if x.q.dtype == torch.bfloat16 else "fp32"


# The kernel that marks each forward path in the launch records.
PATH_KERNEL = {"two_pass": "chunk_prep", "fused": "seg_output", "materialized": "chunk_output"}


def fwd_path_supported(x, chunk, algo, **cfg):
    """Whether the library accepts `algo` (and cfg) for this shape: the
    workspace query validates exactly as the call does."""
    if algo == "auto" and not cfg:
        return True
    B, H, L, dk = x.q.shape
    dims = GlaDims(B, H, L, dk, x.v.shape[-1], chunk, 16)
    code = GLA_BF16 if x.q.dtype == torch.bfloat16 else GLA_FP32
    try:
        gla_fwd_ex_workspace_size(dims, code, fwd_config(algo, **cfg))
    except GlaError as e:
        if e.status == 2:
            return False
        raise
    return True


def run_fwd(x, chunk=64, subchunk=16, dev="cuda", algo="auto", **cfg):
    """The forward through the C ABI; returns (o, hT, names of the launched
    kernels)."""
    d = x.to(dev)
    _abi.gla_profile_begin(64)
    o, hT = gla_fwd_t(d.q, d.k, d.v, d.log_alpha, d.h0, chunk=chunk, subchunk=subchunk,
                      algo=algo, **cfg)
    torch.cuda.synchronize()
    _abi.gla_profile_end()
    names = [_abi.gla_profile_get(i)[0] for i in range(_abi.gla_profile_count())]
    return as_f64(o), as_f64(hT), names


def oracle_fwd(x):
    return oracle.fwd(as_f64(x.q), as_f64(x.k), as_f64(x.v), as_f64(x.log_alpha), as_f64(x.h0))


def bwd_path_supported(x, chunk, algo):
    """Whether the library accepts the backward path `algo` for this shape."""
    if algo == "auto":
        return True
    B, H, L, dk = x.q.shape
    dims = GlaDims(B, H, L, dk, x.v.shape[-1], chunk, 16)
    code = GLA_BF16 if x.q.dtype == torch.bfloat16 else GLA_FP32
    try:
        gla_bwd_ex_workspace_size(dims, code, bwd_config(algo))
    except GlaError as e:
        if e.status == 2:
            return False
        raise
    return True


def run_bwd(x, chunk=64, subchunk=16, dev="cuda", algo="auto", names=None):
    """The backward through the C ABI; the launched kernels' names are
    appended to `names` when a list is given."""
    d = x.to(dev)
    _abi.gla_profile_begin(64)
    g = gla_bwd_t(d.q, d.k, d.v, d.log_alpha, d.h0, d.do, d.dhT, chunk=chunk, subchunk=subchunk,
                  algo=algo)
    torch.cuda.synchronize()
    _abi.gla_profile_end()
    if names is not None:
        names.extend(_abi.gla_profile_get(i)[0] for i in range(_abi.gla_profile_count()))
    return tuple(as_f64(t) for t in g)


def oracle_bwd(x):
    return oracle.bwd(as_f64(x.q), as_f64(x.k), as_f64(x.v), as_f64(x.log_alpha), as_f64(x.h0),
                      as_f64(x.do), as_f64(x.dhT))


def say(*a):
    print(*a, flush=True)
