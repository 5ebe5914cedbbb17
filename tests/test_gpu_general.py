"""GPU parity of the general gate G_t = alpha_t^T beta_t (ggla_fwd / ggla_bwd
through the C ABI) against the fp64 oracle's token recurrence and its BPTT,
element by element (relative L2 per tensor: <= 1e-5 for fp32 I/O, <= 5e-3 for
bf16 I/O).  Shapes span several 16-token chunks with ragged tails, both
gates sharp enough to take the log-space intra-chunk path, a unit column gate
(where the row-gated path must agree), d_k up to 256 and d_v up to 512, and empty
sequences and batches."""
import numpy as np
import pytest
import torch

import oracle
from chunkwise_linear_rnn_gla_amd import bwd_general, fwd, fwd_general
from chunkwise_linear_rnn_gla_amd.inputs import as_f64, make_inputs, make_log_beta
from gpu_util import TOL, rel_l2, say

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, B, H, L, dk, dv, alpha gate, beta gate, h0 std
    ("fp32", 1, 1, 37, 16, 32, "sigmoid16", "sigmoid16", 0.0),
    ("fp32", 2, 2, 100, 64, 48, "sigmoid16", "sigmoid16", 0.5),
    ("fp32", 1, 2, 70, 128, 64, "extreme", "extreme", 0.5),
    ("fp32", 1, 1, 33, 256, 256, "sigmoid16", "sigmoid16", 0.5),
    ("bf16", 2, 2, 130, 64, 96, "sigmoid16", "sigmoid16", 0.5),
    ("bf16", 1, 2, 256, 128, 256, "sigmoid16", "sigmoid16", 0.0),
    ("bf16", 1, 1, 64, 256, 256, "sigmoid16", "sigmoid16", 0.5),
    ("bf16", 2, 1, 90, 32, 224, "extreme", "extreme", 0.5),
    ("bf16", 1, 2, 50, 96, 64, "zero", "const", 0.5),
    # fp32 I/O on a grid that fills the chip (512 workgroups of 128-row tiles):
    # two waves per tile, the next chunk's column work formed a step early
    ("fp32", 8, 4, 80, 128, 256, "sigmoid16", "sigmoid16", 0.5),
    # d_v = 512: the backward's transposed passes hold 512 state rows over four waves
    ("fp32", 1, 1, 45, 32, 512, "sigmoid16", "sigmoid16", 0.5),
    ("bf16", 1, 2, 70, 256, 512, "sigmoid16", "sigmoid16", 0.5),
]


def _rev_cumsum(x):
    return np.flip(np.cumsum(np.flip(x, axis=-2), axis=-2), axis=-2)


def gate_grad_bounds(q, k, v, do, o, dq, dk, dv, dla, dlb):
    """Relative-L2 bounds for the fp32 gate gradients under sharp gates.

    The closed form forms each dlog gate as a reverse sum of differences
    (q ⊙ dq - k ⊙ dk, o ⊙ do - v ⊙ dv) whose terms, the same-token parts taken
    out (they cancel exactly and the kernels leave them out), are kappa times
    larger than the result; kappa comes from the oracle's fp64 values.  Each
    term carries the fp32 error of a dot product over d channels, about
    2^-24 sqrt(d) relative, so the result is held to 2^-24 sqrt(d) kappa (and
    never below the 1e-5 bar)."""
    vd = np.sum(v * do, axis=-1, keepdims=True)
    qk = np.sum(q * k, axis=-1, keepdims=True)
    ta = np.abs(q * (dq - vd * k)) + np.abs(k * (dk - vd * q))
    tb = np.abs((o - qk * v) * do) + np.abs(v * (dv - qk * do))
    d = max(q.shape[-1], v.shape[-1])
    bound = lambda t, g: 2.0 ** -24 * np.sqrt(d) * np.linalg.norm(_rev_cumsum(t)) / np.linalg.norm(g)
    return max(TOL["fp32"], bound(ta, dla)), max(TOL["fp32"], bound(tb, dlb))


def _inputs(dtype, B, H, L, dk, dv, ga, gb, h0, seed):
    x = make_inputs(B, H, L, dk, dv, dtype, seed=seed, gate=ga, h0_std=h0, with_do=True,
                    dhT_std=0.5)
    lb = make_log_beta(B, H, L, dv, seed=seed, gate=gb)
    return x, lb


def _dev(x, lb):
    d = x.to("cuda")
    return d, lb.to("cuda")


@pytest.mark.parametrize("dtype,B,H,L,dk,dv,ga,gb,h0", CASES)
def test_general_forward_matches_oracle(dtype, B, H, L, dk, dv, ga, gb, h0):
    x, lb = _inputs(dtype, B, H, L, dk, dv, ga, gb, h0, seed=L + dk + dv)
    say(f"[ggla fwd] {dtype} B={B} H={H} L={L} dk={dk} dv={dv} gates={ga}/{gb} h0={h0}")
    d, lbd = _dev(x, lb)
    o, hT = fwd_general(d.q, d.k, d.v, d.log_alpha, lbd, d.h0)
    torch.cuda.synchronize()
    ro, rhT = oracle.ggla_fwd(as_f64(x.q), as_f64(x.k), as_f64(x.v), as_f64(x.log_alpha),
                              as_f64(lb), as_f64(x.h0))
    eo, eh = rel_l2(as_f64(o), ro), rel_l2(as_f64(hT), rhT)
    say(f"      rel_l2 o={eo:.3e} hT={eh:.3e}")
    assert np.isfinite(as_f64(o)).all()
    assert eo <= TOL[dtype] and eh <= TOL[dtype]


@pytest.mark.parametrize("dtype,B,H,L,dk,dv,ga,gb,h0", CASES)
def test_general_backward_matches_oracle(dtype, B, H, L, dk, dv, ga, gb, h0):
    x, lb = _inputs(dtype, B, H, L, dk, dv, ga, gb, h0, seed=3 * L + dk)
    say(f"[ggla bwd] {dtype} B={B} H={H} L={L} dk={dk} dv={dv} gates={ga}/{gb} h0={h0}")
    d, lbd = _dev(x, lb)
    g = bwd_general(d.q, d.k, d.v, d.log_alpha, lbd, d.h0, d.do, d.dhT)
    torch.cuda.synchronize()
    f = [as_f64(t) for t in (x.q, x.k, x.v, x.log_alpha)]
    ref = oracle.ggla_bwd(*f, as_f64(lb), as_f64(x.h0), as_f64(x.do), as_f64(x.dhT))
    tol = {n: TOL[dtype] for n in ("dq", "dk", "dv", "dlog_alpha", "dlog_beta", "dh0")}
    if dtype == "fp32" and "extreme" in (ga, gb):
        o, _ = oracle.ggla_fwd(*f, as_f64(lb), as_f64(x.h0))
        tol["dlog_alpha"], tol["dlog_beta"] = gate_grad_bounds(
            f[0], f[1], f[2], as_f64(x.do), o, ref[0], ref[1], ref[2], ref[3], ref[4])
    for name, got, want in zip(("dq", "dk", "dv", "dlog_alpha", "dlog_beta", "dh0"), g, ref):
        e = rel_l2(as_f64(got), want)
        say(f"      {name}: rel_l2 {e:.3e} (bar {tol[name]:.2e})")
        assert np.isfinite(as_f64(got)).all(), name
        assert e <= tol[name], f"{name} rel_l2 {e}"


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_general_backward_without_dhT(dtype):
    # dhT absent: the dv pass starts from a zero state; dh0 is still its
    # final state times token 0's gate, and hT enters no gate gradient
    x, lb = _inputs(dtype, 2, 2, 77, 64, 96, "sigmoid16", "sigmoid16", 0.5, seed=91)
    say(f"[ggla bwd] {dtype} without dhT, B2 H2 L77 dk64 dv96")
    d, lbd = _dev(x, lb)
    g = bwd_general(d.q, d.k, d.v, d.log_alpha, lbd, d.h0, d.do, None)
    torch.cuda.synchronize()
    ref = oracle.ggla_bwd(as_f64(x.q), as_f64(x.k), as_f64(x.v), as_f64(x.log_alpha),
                          as_f64(lb), as_f64(x.h0), as_f64(x.do), None)
    for name, got, want in zip(("dq", "dk", "dv", "dlog_alpha", "dlog_beta", "dh0"), g, ref):
        e = rel_l2(as_f64(got), want)
        say(f"      {name}: rel_l2 {e:.3e}")
        assert e <= TOL[dtype], f"{name} rel_l2 {e}"


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("L", [1, 16, 17])
def test_general_chunk_edges(dtype, L):
    # one token, exactly one 16-token chunk, one token past it; h0 and dhT set
    x, lb = _inputs(dtype, 1, 2, L, 32, 64, "sigmoid16", "sigmoid16", 0.5, seed=200 + L)
    say(f"[ggla] chunk edges {dtype} L={L}")
    d, lbd = _dev(x, lb)
    o, hT = fwd_general(d.q, d.k, d.v, d.log_alpha, lbd, d.h0)
    g = bwd_general(d.q, d.k, d.v, d.log_alpha, lbd, d.h0, d.do, d.dhT)
    torch.cuda.synchronize()
    f = [as_f64(t) for t in (x.q, x.k, x.v, x.log_alpha)]
    ro, rhT = oracle.ggla_fwd(*f, as_f64(lb), as_f64(x.h0))
    ref = oracle.ggla_bwd(*f, as_f64(lb), as_f64(x.h0), as_f64(x.do), as_f64(x.dhT))
    pairs = [("o", o, ro), ("hT", hT, rhT)]
    pairs += list(zip(("dq", "dk", "dv", "dlog_alpha", "dlog_beta", "dh0"), g, ref))
    for name, got, want in pairs:
        e = rel_l2(as_f64(got), want)
        say(f"      {name}: rel_l2 {e:.3e}")
        assert e <= TOL[dtype], f"{name} rel_l2 {e}"


def test_unit_column_gate_matches_row_gated_path():
    # log beta = 0: the general path and gla_fwd compute the same o and hT
    x = make_inputs(2, 2, 200, 128, 256, "bf16", seed=21, h0_std=0.5)
    lb = torch.zeros(2, 2, 200, 256)
    d, lbd = _dev(x, lb)
    say("[ggla] unit column gate vs gla_fwd, bf16 B2 H2 L200 dk128 dv256")
    o1, h1 = fwd_general(d.q, d.k, d.v, d.log_alpha, lbd, d.h0)
    o2, h2 = fwd(d.q, d.k, d.v, d.log_alpha, d.h0)
    torch.cuda.synchronize()
    ro, rh = oracle.fwd(as_f64(x.q), as_f64(x.k), as_f64(x.v), as_f64(x.log_alpha), as_f64(x.h0))
    for got in (o1, o2):
        assert rel_l2(as_f64(got), ro) <= TOL["bf16"]
    assert rel_l2(as_f64(h1), rh) <= TOL["bf16"] and rel_l2(as_f64(h2), rh) <= TOL["bf16"]


@pytest.mark.parametrize("B,dk,dv", [(8, 128, 256), (4, 256, 512)], ids=["gla340m", "gla1p3b"])
def test_general_layer_shapes_forward_and_backward(B, dk, dv):
    # the GLA-340M and GLA-1.3B head shapes at full length (H4 L2048 bf16)
    x, lb = _inputs("bf16", B, 4, 2048, dk, dv, "sigmoid16", "sigmoid16", 0.0, seed=1001 + dv)
    say(f"[ggla] layer shape B{B} H4 L2048 dk{dk} dv{dv} bf16, forward and backward")
    d, lbd = _dev(x, lb)
    o, hT = fwd_general(d.q, d.k, d.v, d.log_alpha, lbd)
    g = bwd_general(d.q, d.k, d.v, d.log_alpha, lbd, None, d.do, None, want_dh0=False)
    torch.cuda.synchronize()
    f = [as_f64(t) for t in (x.q, x.k, x.v, x.log_alpha)]
    ro, rhT = oracle.ggla_fwd(*f, as_f64(lb))
    assert rel_l2(as_f64(o), ro) <= TOL["bf16"] and rel_l2(as_f64(hT), rhT) <= TOL["bf16"]
    ref = oracle.ggla_bwd(*f, as_f64(lb), None, as_f64(x.do), None)
    for name, got, want in zip(("dq", "dk", "dv", "dlog_alpha", "dlog_beta"), g[:5], ref[:5]):
        e = rel_l2(as_f64(got), want)
        say(f"      {name}: rel_l2 {e:.3e}")
        assert e <= TOL["bf16"], name


def test_general_long_sequence():
    # 1,024 chunks in sequence with an initial state: no drift over a long run
    x, lb = _inputs("bf16", 1, 4, 16384, 128, 256, "sigmoid16", "sigmoid16", 0.1, seed=1004)
    say("[ggla] long sequence B1 H4 L16384 dk128 dv256 bf16, h0 std 0.1")
    d, lbd = _dev(x, lb)
    o, hT = fwd_general(d.q, d.k, d.v, d.log_alpha, lbd, d.h0)
    torch.cuda.synchronize()
    ro, rhT = oracle.ggla_fwd(as_f64(x.q), as_f64(x.k), as_f64(x.v), as_f64(x.log_alpha),
                              as_f64(lb), as_f64(x.h0))
    eo, eh = rel_l2(as_f64(o), ro), rel_l2(as_f64(hT), rhT)
    # the last 512 tokens on their own as well: a late drift would show there
    el = rel_l2(as_f64(o)[:, :, -512:], ro[:, :, -512:])
    say(f"      rel_l2 o={eo:.3e} (last 512: {el:.3e}) hT={eh:.3e}")
    assert eo <= TOL["bf16"] and el <= TOL["bf16"] and eh <= TOL["bf16"]


def test_general_empty_sequence_and_batch():
    q = torch.empty(1, 2, 0, 64, device="cuda", dtype=torch.bfloat16)
    v = torch.empty(1, 2, 0, 96, device="cuda", dtype=torch.bfloat16)
    la = torch.empty(1, 2, 0, 64, device="cuda")
    lb = torch.empty(1, 2, 0, 96, device="cuda")
    h0 = torch.randn(1, 2, 64, 96, device="cuda")
    o, hT = fwd_general(q, q, v, la, lb, h0)
    dhT = torch.randn(1, 2, 64, 96, device="cuda")
    g = bwd_general(q, q, v, la, lb, h0, v, dhT)
    torch.cuda.synchronize()
    assert o.shape == (1, 2, 0, 96) and torch.equal(hT, h0) and torch.equal(g[5], dhT)
    e = torch.empty(0, 2, 16, 64, device="cuda")
    ev = torch.empty(0, 2, 16, 32, device="cuda")
    o, _ = fwd_general(e, e, ev, e, ev)
    torch.cuda.synchronize()
    assert o.shape == (0, 2, 16, 32)
