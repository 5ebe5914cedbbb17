"""GPU test of gla_fwd_noalloc, the forward whose scratch is the library's
static device array: through the C ABI, against gla_fwd (the same two-pass
kernels on a caller-supplied workspace) on the same inputs.  The two must
agree bit for bit, which is within the parity bar; the second call uses a
smaller input than the first (the array keeps the first call's contents,
which the kernels must not depend on).  Both also meet the oracle's bar."""
import numpy as np
import pytest
import torch

from chunkwise_linear_rnn_gla_amd import GLA_BF16, GLA_FP32, GlaDims, _abi
from chunkwise_linear_rnn_gla_amd.inputs import WORKLOADS, make_inputs, workload_inputs
from gpu_util import TOL, dtype_name, oracle_fwd, rel_l2, say

pytestmark = pytest.mark.gpu


def _both(x, chunk):
    d = x.to("cuda")
    B, H, L, dk = x.q.shape
    dv = x.v.shape[-1]
    dims = GlaDims(B, H, L, dk, dv, chunk, 16)
    code = GLA_BF16 if x.q.dtype == torch.bfloat16 else GLA_FP32
    stream = torch.cuda.current_stream().cuda_stream
    o1 = torch.empty(B, H, L, dv, dtype=x.q.dtype, device="cuda")
    h1 = torch.empty(B, H, dk, dv, dtype=torch.float32, device="cuda")
    o2 = torch.full_like(o1, float("nan"))
    h2 = torch.full_like(h1, float("nan"))
    ws = torch.empty(max(1, _abi.gla_fwd_workspace_size(dims, code)), dtype=torch.uint8,
                     device="cuda")
    assert _abi.gla_fwd(dims, code, d.q, d.k, d.v, d.log_alpha, d.h0, o1, h1, ws, ws.numel(),
                        stream) == 0
    assert _abi.gla_fwd_noalloc(dims, code, d.q, d.k, d.v, d.log_alpha, d.h0, o2, h2,
                                stream) == 0
    torch.cuda.synchronize()
    return o1, h1, o2, h2


def _check(x, chunk, tag):
    say(f"[noalloc] {tag} dtype={dtype_name(x)} shape={tuple(x.q.shape)} dv={x.v.shape[-1]}")
    o1, h1, o2, h2 = _both(x, chunk)
    assert torch.equal(o1, o2), "o differs from gla_fwd's"
    assert torch.equal(h1, h2), "hT differs from gla_fwd's"
    ro, rh = oracle_fwd(x)
    to64 = lambda t: t.double().cpu().numpy()
    eo, eh = rel_l2(to64(o2), ro), rel_l2(to64(h2), rh)
    say(f"      rel_l2 vs oracle o={eo:.3e} hT={eh:.3e}")
    assert eo <= TOL[dtype_name(x)] and eh <= TOL[dtype_name(x)]


def test_noalloc_matches_gla_fwd_on_two_calls():
    w = WORKLOADS["gla340m_fwd"]            # 41 MiB of records
    _check(workload_inputs(w), w.chunk, "first call, GLA-340M layer shape")
    x = make_inputs(1, 2, 200, 64, 128, "fp32", seed=901, h0_std=0.5)
    _check(x, 64, "second call, smaller, ragged")


def test_noalloc_rejects_oversized_and_unsupported():
    q = torch.empty(16, dtype=torch.uint8, device="cuda")
    big = GlaDims(16, 4, 2048, 128, 256, 64, 16)      # 82 MiB of records
    assert _abi.gla_fwd_noalloc(big, GLA_BF16, q, q, q, q, None, q, None, None) == 5
    odd = GlaDims(1, 1, 64, 256, 64, 64, 16)          # fp32 dk 256: no two-pass kernels
    assert _abi.gla_fwd_noalloc(odd, GLA_FP32, q, q, q, q, None, q, None, None) == 2
