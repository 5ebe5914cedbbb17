"""GPU parity of the one-token decode step (gla_decode): T calls in a row, each
updating the state in place, against the fp64 token recurrence of the oracle
over the same T tokens (relative L2 of every step's output and of the final
state: <= 1e-5 for fp32 I/O, <= 5e-3 for bf16 I/O)."""
import numpy as np
import pytest
import torch

from chunkwise_linear_rnn_gla_amd import decode as gla_decode_t
from chunkwise_linear_rnn_gla_amd.inputs import as_f64, make_inputs
from gpu_util import TOL, oracle_fwd, rel_l2, say

pytestmark = pytest.mark.gpu


def run_decode_steps(x, dev="cuda"):
    """Feed the tokens of x one by one; returns (o [B,H,T,dv], final state)."""
    d = x.to(dev)
    B, H, T, dk = d.q.shape
    dv = d.v.shape[-1]
    state = (d.h0.clone() if d.h0 is not None
             else torch.zeros(B, H, dk, dv, dtype=torch.float32, device=dev))
    outs = []
    for t in range(T):
        tok = lambda z: z[:, :, t, :].contiguous()
        outs.append(gla_decode_t(tok(d.q), tok(d.k), tok(d.v), tok(d.log_alpha), state))
    torch.cuda.synchronize()
    return as_f64(torch.stack(outs, dim=2)), as_f64(state)


@pytest.mark.parametrize("dtype,B,H,dk,dv,gate", [
    ("fp32", 1, 1, 16, 32, "sigmoid16"),
    ("fp32", 2, 3, 64, 48, "sigmoid16"),     # d_v not a multiple of 64
    ("fp32", 1, 2, 128, 256, "extreme"),
    ("bf16", 2, 2, 128, 256, "sigmoid16"),
    ("bf16", 1, 3, 64, 96, "zero"),          # alpha = 1; d_v not a multiple of 64
    ("bf16", 1, 2, 256, 512, "sigmoid16"),   # largest head dims
    ("bf16", 32, 4, 64, 256, "sigmoid16"),   # 64-column workgroups (large grid)
    ("fp32", 16, 8, 32, 240, "extreme"),     # 64-column workgroups, ragged d_v
])
def test_decode_steps_match_oracle(dtype, B, H, dk, dv, gate):
    x = make_inputs(B, H, 6, dk, dv, dtype, seed=31 + dk + dv, gate=gate, h0_std=0.5)
    say(f"[decode] dtype={dtype} B={B} H={H} dk={dk} dv={dv} gate={gate} T=6")
    o, st = run_decode_steps(x)
    ro, rst = oracle_fwd(x)
    eo, es = rel_l2(o, ro), rel_l2(st, rst)
    say(f"      rel_l2 o={eo:.3e} state={es:.3e}")
    assert np.isfinite(o).all() and np.isfinite(st).all()
    assert eo <= TOL[dtype], f"o rel_l2 {eo}"
    assert es <= TOL[dtype], f"state rel_l2 {es}"


def test_decode_from_zero_state_bench_shape():
    # the bench's decode shape (B8 H4 dk128 dv256, bf16), one step from zero
    x = make_inputs(8, 4, 1, 128, 256, "bf16", seed=77)
    say("[decode] bench shape, one step from a zero state")
    o, st = run_decode_steps(x)
    ro, rst = oracle_fwd(x)
    assert rel_l2(o, ro) <= TOL["bf16"] and rel_l2(st, rst) <= TOL["bf16"]


def test_decode_zero_batch_is_a_no_op():
    e = torch.empty(0, 4, 64, device="cuda", dtype=torch.bfloat16)
    s = torch.empty(0, 4, 64, 64, device="cuda", dtype=torch.float32)
    a = torch.empty(0, 4, 64, device="cuda", dtype=torch.float32)
    o = gla_decode_t(e, e, e, a, s)
    torch.cuda.synchronize()
    assert o.shape == (0, 4, 64)
