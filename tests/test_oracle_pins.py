"""Pins for the fp64 oracle, checked against what the pages and mathematics fix.

None of these use the HIP library.  Each pin is chosen so that a plausible
mistake in the oracle (a dropped term, a wrong sign or index, a transposed
operand, a decay applied at the wrong step) fails at least one of them:

* alpha == 1 reduces GLA to unnormalised causal linear attention, whose
  parallel form is O = (Q K^T ⊙ M) V with M lower-triangular including the
  diagonal (papercache.org notes §2.1, "Eq. 1" and the parallel form).
* Brute force with explicit per-pair gate products b_t / b_i (notes §4.1,
  parallel form via b_t = prod alpha_j), no logs and no cumsum, tiny inputs.
* The chunkwise form with secondary chunking (notes §4.2 equations, §4.3 /
  Figure 3 block split), independent code, equal for C in {1, 16, 64, L}
  (notes §2.2).
* A data-independent decay gamma (RetNet-style, notes §4 intro; Table 1) gives
  ((Q K^T) ⊙ D) V with D_ti = gamma^(t-i); a channel-shared scalar gate
  (Mamba-2 style, notes §4.1) gives D_ti = prod_{s=i+1..t} gamma_s.
* Segment splitting with S_0 := previous segment's state (notes §2.2).
* Gradients: central finite differences, torch fp64 autograd of the log-space
  parallel form (a different formulation), and the pages' closed-form gate
  gradient (zako-mio report ch. 3.4; notes §4.3 and App. B).
"""
import math

import numpy as np
import pytest
import torch

from chunkwise_linear_rnn_gla_amd.inputs import as_f64, make_inputs


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    n = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (n if n > 0 else 1.0)


def f64_inputs(B, H, L, dk, dv, seed, gate="sigmoid16", h0_std=0.0, with_do=False, dhT_std=0.0,
               **kw):
    x = make_inputs(B, H, L, dk, dv, "fp32", seed, gate=gate, h0_std=h0_std, with_do=with_do,
                    dhT_std=dhT_std, **kw)
    return {n: as_f64(getattr(x, n)) for n in ("q", "k", "v", "log_alpha", "h0", "do", "dhT")}


# --------------------------------------------------------------------------- forward pins

def test_alpha_one_is_causal_linear_attention(oracle_mod):
    x = f64_inputs(2, 3, 37, 5, 7, seed=1, gate="zero")
    o, hT = oracle_mod.fwd(x["q"], x["k"], x["v"], x["log_alpha"])
    mask = np.tril(np.ones((37, 37)))
    ref = np.matmul(np.matmul(x["q"], np.swapaxes(x["k"], -1, -2)) * mask, x["v"])
    assert rel(o, ref) < 1e-13
    assert rel(hT, np.matmul(np.swapaxes(x["k"], -1, -2), x["v"])) < 1e-13


def _brute_head(q, k, v, a, h0):
    """Explicit per-pair gate products, pure Python loops, no logs or cumsums."""
    L, dk = q.shape
    dv = v.shape[1]
    alpha = [[math.exp(a[t][i]) for i in range(dk)] for t in range(L)]

    def prod(lo, hi, i):  # product of alpha_s[i] for s in [lo, hi]
        p = 1.0
        for s in range(lo, hi + 1):
            p *= alpha[s][i]
        return p

    o = np.zeros((L, dv))
    for t in range(L):
        for j in range(dv):
            acc = 0.0
            for i in range(dk):
                acc += q[t][i] * prod(0, t, i) * h0[i][j]
                for s in range(t + 1):
                    acc += q[t][i] * k[s][i] * prod(s + 1, t, i) * v[s][j]
            o[t][j] = acc
    hT = np.zeros((dk, dv))
    for i in range(dk):
        for j in range(dv):
            acc = prod(0, L - 1, i) * h0[i][j]
            for s in range(L):
                acc += prod(s + 1, L - 1, i) * k[s][i] * v[s][j]
            hT[i][j] = acc
    return o, hT


@pytest.mark.parametrize("gate", ["sigmoid16", "extreme"])
def test_bruteforce_pair_products(oracle_mod, gate):
    x = f64_inputs(1, 2, 11, 3, 4, seed=2, gate=gate, h0_std=0.7)
    o, hT = oracle_mod.fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"])
    for h in range(2):
        ob, hb = _brute_head(x["q"][0, h], x["k"][0, h], x["v"][0, h], x["log_alpha"][0, h],
                             x["h0"][0, h])
        assert rel(o[0, h], ob) < 1e-13
        assert rel(hT[0, h], hb) < 1e-13


@pytest.mark.parametrize("C", [1, 16, 64, 128])
def test_chunk_size_invariance(oracle_mod, C):
    x = f64_inputs(1, 2, 128, 8, 12, seed=3, h0_std=0.5)
    o, hT = oracle_mod.fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"])
    oc, hc = oracle_mod.chunkwise_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"], C=C,
                                      c=min(16, C))
    assert rel(oc, o) < 1e-12
    assert rel(hc, hT) < 1e-12


def test_chunkwise_with_strong_decay(oracle_mod):
    # Gates whose cumulative products underflow fp64 over the sequence: the
    # log-space / reference-row chunkwise form must still equal the recurrence.
    x = f64_inputs(1, 1, 64, 4, 6, seed=4, gate="extreme")
    o, hT = oracle_mod.fwd(x["q"], x["k"], x["v"], x["log_alpha"])
    oc, hc = oracle_mod.chunkwise_fwd(x["q"], x["k"], x["v"], x["log_alpha"], None, C=32, c=16)
    assert rel(oc, o) < 1e-12
    assert rel(hc, hT) < 1e-12


def test_constant_gate_closed_form(oracle_mod):
    gamma = 0.93
    x = f64_inputs(2, 2, 40, 6, 5, seed=5, gate="const", gate_value=math.log(gamma))
    x["log_alpha"][:] = math.log(gamma)
    o, _ = oracle_mod.fwd(x["q"], x["k"], x["v"], x["log_alpha"])
    t = np.arange(40)
    D = np.where(t[:, None] >= t[None, :], gamma ** (t[:, None] - t[None, :]).clip(min=0), 0.0)
    ref = np.matmul(np.matmul(x["q"], np.swapaxes(x["k"], -1, -2)) * D, x["v"])
    assert rel(o, ref) < 1e-13


def test_scalar_gate_closed_form(oracle_mod):
    # One gate value per token shared by every key channel.
    x = f64_inputs(1, 1, 30, 5, 4, seed=6)
    g = x["log_alpha"][0, 0, :, 0].copy()
    x["log_alpha"][0, 0] = g[:, None]
    o, _ = oracle_mod.fwd(x["q"], x["k"], x["v"], x["log_alpha"])
    gam = np.exp(g)
    D = np.zeros((30, 30))
    for t in range(30):
        for i in range(t + 1):
            D[t, i] = np.prod(gam[i + 1:t + 1])
    ref = ((x["q"][0, 0] @ x["k"][0, 0].T) * D) @ x["v"][0, 0]
    assert rel(o[0, 0], ref) < 1e-13


def test_segment_split(oracle_mod):
    x = f64_inputs(2, 2, 90, 6, 10, seed=7, h0_std=0.3)
    q, k, v, a, h0 = x["q"], x["k"], x["v"], x["log_alpha"], x["h0"]
    o, hT = oracle_mod.fwd(q, k, v, a, h0)
    s = 37
    o1, h1 = oracle_mod.fwd(q[:, :, :s], k[:, :, :s], v[:, :, :s], a[:, :, :s], h0)
    o2, h2 = oracle_mod.fwd(q[:, :, s:], k[:, :, s:], v[:, :, s:], a[:, :, s:], h1)
    assert rel(np.concatenate([o1, o2], axis=2), o) < 1e-13
    assert rel(h2, hT) < 1e-13


def test_empty_sequence(oracle_mod):
    x = f64_inputs(1, 2, 0, 4, 6, seed=8, h0_std=1.0)
    o, hT = oracle_mod.fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"])
    assert o.shape == (1, 2, 0, 6)
    assert np.array_equal(hT, x["h0"])


def test_threads_do_not_change_bits(oracle_mod):
    x = f64_inputs(3, 3, 50, 8, 8, seed=9, h0_std=0.2, with_do=True)
    o1, h1 = oracle_mod.fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"], nthreads=1)
    o4, h4 = oracle_mod.fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"], nthreads=4)
    assert np.array_equal(o1, o4) and np.array_equal(h1, h4)
    g1 = oracle_mod.bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"], x["do"], nthreads=1)
    g4 = oracle_mod.bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"], x["do"], nthreads=4)
    for a, b in zip(g1, g4):
        assert np.array_equal(a, b)


# --------------------------------------------------------------------------- backward pins

def _loss(oracle_mod, q, k, v, a, h0, do, dhT):
    o, hT = oracle_mod.fwd(q, k, v, a, h0, nthreads=1)
    return float(np.sum(o * do) + np.sum(hT * dhT))


def test_bptt_matches_finite_differences(oracle_mod):
    x = f64_inputs(1, 1, 7, 3, 4, seed=10, h0_std=0.8, with_do=True, dhT_std=0.6)
    args = [x["q"], x["k"], x["v"], x["log_alpha"], x["h0"]]
    grads = oracle_mod.bwd(*args, x["do"], x["dhT"], nthreads=1)
    names = ["q", "k", "v", "log_alpha", "h0"]
    order = [0, 1, 2, 3, 4]  # bwd returns dq, dk, dv, dlog_alpha, dh0
    eps = 1e-6
    for ai, gi in zip(range(5), order):
        base = args[ai]
        fd = np.zeros_like(base)
        it = np.nditer(base, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[ai][idx] += eps
            minus[ai][idx] -= eps
            fd[idx] = (_loss(oracle_mod, *plus, x["do"], x["dhT"]) -
                       _loss(oracle_mod, *minus, x["do"], x["dhT"])) / (2 * eps)
        assert rel(grads[gi], fd) < 1e-7, names[ai]


def _parallel_form_torch(q, k, v, a, h0):
    """Log-space parallel form (notes §4.1 Eq. 4 with the h0 term), fp64 torch."""
    Bc = torch.cumsum(a, dim=-2)                        # log b_t
    L = q.shape[-2]
    mask = torch.tril(torch.ones(L, L, dtype=torch.float64))
    diff = Bc[..., :, None, :] - Bc[..., None, :, :]    # [.., t, i, k] = log b_t - log b_i
    diff = torch.where(mask[..., None] > 0, diff, torch.full_like(diff, -1e300))
    P = torch.einsum("...tk,...ik,...tik->...ti", q, k, torch.exp(diff))
    o = P @ v + (q * torch.exp(Bc)) @ h0
    bl = Bc[..., -1:, :]                                # log b_L
    hT = torch.exp(bl).transpose(-1, -2) * h0 + (k * torch.exp(bl - Bc)).transpose(-1, -2) @ v
    return o, hT


def test_bptt_matches_autograd_of_parallel_form(oracle_mod):
    x = f64_inputs(2, 2, 20, 4, 6, seed=11, h0_std=0.5, with_do=True, dhT_std=0.4)
    t = {n: torch.tensor(x[n], requires_grad=True) for n in ("q", "k", "v", "log_alpha", "h0")}
    o, hT = _parallel_form_torch(t["q"], t["k"], t["v"], t["log_alpha"], t["h0"])
    ref_o, ref_h = oracle_mod.fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"])
    assert rel(o.detach().numpy(), ref_o) < 1e-12
    assert rel(hT.detach().numpy(), ref_h) < 1e-12
    loss = (o * torch.tensor(x["do"])).sum() + (hT * torch.tensor(x["dhT"])).sum()
    loss.backward()
    g = oracle_mod.bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"], x["do"], x["dhT"])
    for got, n in zip(g, ("q", "k", "v", "log_alpha", "h0")):
        assert rel(got, t[n].grad.numpy()) < 1e-11, n


@pytest.mark.parametrize("with_dhT", [False, True])
def test_closed_form_gate_gradient(oracle_mod, with_dhT):
    x = f64_inputs(2, 2, 100, 8, 16, seed=12, h0_std=0.5, with_do=True,
                   dhT_std=0.7 if with_dhT else 0.0)
    dq, dk, dv, da, dh0 = oracle_mod.bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"],
                                         x["do"], x["dhT"])
    _, hT = oracle_mod.fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"])
    cf = oracle_mod.closed_form_dlog_alpha(x["q"], x["k"], dq, dk, hT, x["dhT"])
    assert rel(cf, da) < 1e-11
    if with_dhT:  # the extra final-state term is needed, not optional
        cf0 = oracle_mod.closed_form_dlog_alpha(x["q"], x["k"], dq, dk)
        assert rel(cf0, da) > 1e-3


# --------------------------------------------------------------------------- inputs

def test_inputs_are_deterministic_and_exactly_upcast():
    a = make_inputs(2, 2, 33, 32, 64, "bf16", seed=5, h0_std=0.1, with_do=True)
    b = make_inputs(2, 2, 33, 32, 64, "bf16", seed=5, h0_std=0.1, with_do=True)
    for n in ("q", "k", "v", "log_alpha", "h0", "do"):
        assert torch.equal(getattr(a, n), getattr(b, n))
    q64 = as_f64(a.q)
    assert np.array_equal(torch.tensor(q64).to(torch.bfloat16).to(torch.float64).numpy(), q64)
    assert a.log_alpha.dtype == torch.float32 and float(a.log_alpha.max()) < 0.0
