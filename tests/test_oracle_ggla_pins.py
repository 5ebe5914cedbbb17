"""Pins of the general-gate oracle (G_t = alpha_t^T beta_t; papercache.org
notes on GLA, App. C) against results fixed by the mathematics:

* beta = 1 reduces it to the row-gated recurrence (pinned on its own);
* App. C.1's parallel form with cumulative products, written out as a
  brute-force sum over token pairs on a short sequence;
* finite differences of the forward for every input's gradient;
* the closed-form gate gradients (App. C, memory-efficient gradients);
* the role-swap identities the GPU backward is built on: dq is a forward of
  the same recurrence with (q, k, v, alpha, beta) -> (do, v, k, beta, alpha);
  dv and dk are forwards on the time-reversed sequence with the gates shifted
  by one token.
"""
import numpy as np
import pytest

import oracle


def _inputs(B, H, L, dk, dv, seed, h0=True, dhT=True, gate_scale=1.0):
    r = np.random.default_rng(seed)
    q = r.normal(size=(B, H, L, dk)) * dk ** -0.5
    k = r.normal(size=(B, H, L, dk))
    v = r.normal(size=(B, H, L, dv))
    a = -r.uniform(0.0, gate_scale, size=(B, H, L, dk))
    b = -r.uniform(0.0, gate_scale, size=(B, H, L, dv))
    s0 = r.normal(size=(B, H, dk, dv)) * 0.5 if h0 else None
    do = r.normal(size=(B, H, L, dv))
    dh = r.normal(size=(B, H, dk, dv)) if dhT else None
    return q, k, v, a, b, s0, do, dh


def _rel(x, y):
    return np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-300)


def test_unit_beta_is_the_row_gated_recurrence(oracle_mod):
    q, k, v, a, _, h0, do, dhT = _inputs(2, 2, 37, 5, 7, seed=1)
    b = np.zeros_like(v)
    o, hT = oracle.fwd(q, k, v, a, h0)
    og, hTg = oracle.ggla_fwd(q, k, v, a, b, h0)
    assert np.array_equal(o, og) and np.array_equal(hT, hTg)
    g1 = oracle.bwd(q, k, v, a, h0, do, dhT)
    g2 = oracle.ggla_bwd(q, k, v, a, b, h0, do, dhT)
    for x, y in zip(g1, (g2[0], g2[1], g2[2], g2[3], g2[5])):
        assert _rel(y, x) < 1e-13


def test_parallel_form_brute_force(oracle_mod):
    # App. C.1: O = ((Q ⊙ B)(K / B)^T ⊙ M)(V / D) ⊙ D, with B, D the cumulative
    # products of alpha, beta from the first token and M the causal mask
    # (output scaled by D, the plain reading that reproduces the recurrence),
    # plus the initial state's term (Q ⊙ B) S_0 ⊙ D
    q, k, v, a, b, h0, _, _ = _inputs(1, 2, 11, 3, 4, seed=2, gate_scale=0.5)
    o, hT = oracle.ggla_fwd(q, k, v, a, b, h0)
    Bc, Dc = np.exp(np.cumsum(a, axis=-2)), np.exp(np.cumsum(b, axis=-2))
    L = q.shape[-2]
    want = np.zeros_like(o)
    for h in range(q.shape[1]):
        for t in range(L):
            for s in range(t + 1):
                w = np.sum(q[0, h, t] * Bc[0, h, t] * k[0, h, s] / Bc[0, h, s])
                want[0, h, t] += w * v[0, h, s] / Dc[0, h, s] * Dc[0, h, t]
            want[0, h, t] += (q[0, h, t] * Bc[0, h, t]) @ h0[0, h] * Dc[0, h, t]
    assert _rel(o, want) < 1e-12
    # final state: sum_s (b_L / b_s)(d_L / d_s) k_s^T v_s + (b_L d_L) ⊙ S_0
    S = np.einsum("hs,hsi,hsj,hsj->hij", np.ones((2, L)), k[0] / Bc[0], v[0], 1 / Dc[0])
    S = (S + h0[0]) * Bc[0, :, -1][:, :, None] * Dc[0, :, -1][:, None, :]
    assert _rel(hT[0], S) < 1e-12


def test_gradients_match_finite_differences(oracle_mod):
    q, k, v, a, b, h0, do, dhT = _inputs(1, 1, 6, 3, 4, seed=3, gate_scale=0.8)
    g = oracle.ggla_bwd(q, k, v, a, b, h0, do, dhT)
    args = [q, k, v, a, b, h0]

    def loss(xs):
        o, hT = oracle.ggla_fwd(*xs)
        return np.sum(o * do) + np.sum(hT * dhT)

    for which, grad in zip(range(6), (g[0], g[1], g[2], g[3], g[4], g[5])):
        x = args[which]
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = [y.copy() for y in args]
            xm = [y.copy() for y in args]
            xp[which][idx] += 1e-6
            xm[which][idx] -= 1e-6
            num[idx] = (loss(xp) - loss(xm)) / 2e-6
        assert _rel(grad, num) < 1e-7, which


def test_closed_form_gate_gradients(oracle_mod):
    q, k, v, a, b, h0, do, dhT = _inputs(2, 2, 45, 6, 5, seed=4)
    o, hT = oracle.ggla_fwd(q, k, v, a, b, h0)
    dq, dk, dv, da, db, _ = oracle.ggla_bwd(q, k, v, a, b, h0, do, dhT)
    ca, cb = oracle.closed_form_general(q, k, v, o, dq, dk, dv, do, hT, dhT)
    assert _rel(ca, da) < 1e-12 and _rel(cb, db) < 1e-12


def _rev(x):
    return np.ascontiguousarray(np.flip(x, axis=-2))


def _shift_rev(g):
    """Gates of the time-reversed pass: position u takes the gate of original
    token L - u (u >= 1) and 1 at u = 0."""
    out = np.zeros_like(g)
    out[..., 1:, :] = _rev(g)[..., :-1, :]
    return out


def _t(s):
    return np.ascontiguousarray(np.swapaxes(s, -1, -2))


@pytest.mark.parametrize("L", [1, 23])
def test_role_swap_identities(oracle_mod, L):
    q, k, v, a, b, h0, do, dhT = _inputs(1, 2, L, 4, 6, seed=5 + L)
    dq, dk, dv, da, db, dh0 = oracle.ggla_bwd(q, k, v, a, b, h0, do, dhT)
    # dq_t = S_t do_t: the transposed state runs the same recurrence
    xq, _ = oracle.ggla_fwd(do, v, k, b, a, _t(h0))
    assert _rel(xq, dq) < 1e-12
    # dv_s = k_s dS_s and dk_s = dS_s v_s with dS_s = G_{s+1} ⊙ dS_{s+1} + q_s^T do_s,
    # dS_{L-1} including dhT: a forward on the reversed sequence
    xv, fin = oracle.ggla_fwd(_rev(k), _rev(q), _rev(do), _shift_rev(a), _shift_rev(b), dhT)
    assert _rel(_rev(xv), dv) < 1e-12
    xk, _ = oracle.ggla_fwd(_rev(v), _rev(do), _rev(q), _shift_rev(b), _shift_rev(a), _t(dhT))
    assert _rel(_rev(xk), dk) < 1e-12
    # dh0 = G_0 ⊙ dS_0, the reversed pass's final state decayed by token 0's gate
    G0 = np.exp(a[..., 0, :])[..., :, None] * np.exp(b[..., 0, :])[..., None, :]
    assert _rel(G0 * fin, dh0) < 1e-12
