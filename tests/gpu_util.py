"""Helpers for the GPU parity tests: move seeded inputs to the device, call the
HIP path through the C ABI binding, compare with the oracle in fp64."""
import numpy as np
import torch

import oracle
from chunkwise_linear_rnn_gla_amd import bwd as gla_bwd_t
from chunkwise_linear_rnn_gla_amd import fwd as gla_fwd_t
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


def run_fwd(x, chunk=64, subchunk=16, dev="cuda"):
    d = x.to(dev)
    o, hT = gla_fwd_t(d.q, d.k, d.v, d.log_alpha, d.h0, chunk=chunk, subchunk=subchunk)
    torch.cuda.synchronize()
    return as_f64(o), as_f64(hT)


def oracle_fwd(x):
    return oracle.fwd(as_f64(x.q), as_f64(x.k), as_f64(x.v), as_f64(x.log_alpha), as_f64(x.h0))


def run_bwd(x, chunk=64, subchunk=16, dev="cuda"):
    d = x.to(dev)
    g = gla_bwd_t(d.q, d.k, d.v, d.log_alpha, d.h0, d.do, d.dhT, chunk=chunk, subchunk=subchunk)
    torch.cuda.synchronize()
    return tuple(as_f64(t) for t in g)


def oracle_bwd(x):
    return oracle.bwd(as_f64(x.q), as_f64(x.k), as_f64(x.v), as_f64(x.log_alpha), as_f64(x.h0),
                      as_f64(x.do), as_f64(x.dhT))


def say(*a):
    print(*a, flush=True)
