"""CPU pins of the fp64 layer reference used by the layer's GPU parity tests:
its gradients against finite differences, and its forward, with every gate
at 1, against causal linear attention written as one masked product."""
import torch

from chunkwise_linear_rnn_gla_amd.layer import GlaLayer
from layer_ref import causal_linear_attention, layer_fwd, layer_params


def _layer(d, heads, seed):
    return GlaLayer(d, heads, seed=seed, dtype=torch.float64, device="cpu")


def test_layer_reference_gradients_match_finite_differences(oracle_mod):
    lay = _layer(8, 2, seed=3)                        # d_k = 2, d_v = 4 per head
    P = layer_params(lay)
    x = torch.randn(1, 5, 8, dtype=torch.float64, generator=torch.Generator().manual_seed(4))
    names = ["w_q", "w_k", "w_v", "w_a1", "w_a2", "b_a"]

    def f(x_, *ws):
        Q = dict(P, **dict(zip(names, ws)))
        return layer_fwd(Q, x_, lay.h, lay.temp)

    args = [x.requires_grad_(True)] + [P[n] for n in names]
    assert torch.autograd.gradcheck(f, args, eps=1e-6, atol=1e-7, rtol=1e-5)


def test_layer_reference_with_unit_gates_is_causal_linear_attention(oracle_mod):
    lay = _layer(32, 2, seed=5)
    P = layer_params(lay)
    with torch.no_grad():
        P["w_a2"].zero_()
        P["b_a"].fill_(60.0)                          # logsigmoid(60) / 16 ~ -5e-28
    x = torch.randn(2, 37, 32, dtype=torch.float64, generator=torch.Generator().manual_seed(6))
    got = layer_fwd(P, x, lay.h, lay.temp)
    want = layer_fwd(P, x, lay.h, lay.temp, core=causal_linear_attention)
    assert torch.allclose(got, want, rtol=1e-10, atol=1e-12)


# ---- the layer's non-core operations (zako-mio report ch. 3.5: per-head
# states, each head's output normalised by LayerNorm before the heads are
# concatenated, a Swish output gate r_t, then W_O).  Each pin checks a
# property the pages fix without retyping the reference's formula.

def _gate_free(P, c):
    """Output gate made a constant swish(c) (W_r = 0, b_r = c) and W_O = I, so
    that y is swish(c) times the concatenated normalised head outputs."""
    with torch.no_grad():
        P["w_r"].zero_()
        P["b_r"].fill_(c)
        P["w_o"].copy_(torch.eye(P["w_o"].shape[0], dtype=P["w_o"].dtype))
    return P


def test_layer_reference_normalises_each_head_separately(oracle_mod):
    d, heads = 24, 3
    lay = _layer(d, heads, seed=11)
    P = _gate_free(layer_params(lay), 2.0)
    x = torch.randn(2, 19, d, dtype=torch.float64, generator=torch.Generator().manual_seed(12))
    y = layer_fwd(P, x, lay.h, lay.temp).detach() / torch.nn.functional.silu(torch.tensor(2.0))
    per_head = y.view(2, 19, heads, d // heads)      # heads concatenated in order
    # every head of every token: zero mean and unit (population) variance over
    # its d_v values, up to LayerNorm's epsilon: the variance is
    # s2 / (s2 + 1e-5) for a raw variance s2, never above 1, and above 0.99
    # for these inputs (raw variances above 1e-3; a norm over the wrong axis
    # gives per-head variances far from 1)
    mean = per_head.mean(-1)
    var = per_head.var(-1, unbiased=False)
    assert mean.abs().max() < 1e-12
    assert var.max() <= 1 + 1e-12 and var.min() > 0.99
    # while the concatenation as a whole is not normalised per token across
    # heads in general: each head carries its own statistics, so a norm over
    # all of d would differ
    whole = torch.nn.functional.layer_norm(y, (d,))
    assert not torch.allclose(whole, y, atol=1e-6)


def test_layer_reference_is_equivariant_to_a_permutation_of_heads(oracle_mod):
    # Heads are independent (their own state and norm), so reordering the
    # heads' column blocks of W_Q, W_K, W_V, W_a2, b_a and the matching blocks
    # of W_r's columns and W_O's rows leaves the output unchanged.  A head
    # split along the wrong axis would mix channels of different heads.
    d, heads = 24, 3
    dk, dv = d // (2 * heads), d // heads
    lay = _layer(d, heads, seed=13)
    P = layer_params(lay)
    x = torch.randn(1, 23, d, dtype=torch.float64, generator=torch.Generator().manual_seed(14))
    with torch.no_grad():
        P["b_a"].copy_(torch.randn(P["b_a"].shape, dtype=torch.float64,
                                   generator=torch.Generator().manual_seed(15)))
        P["b_r"].copy_(torch.randn(P["b_r"].shape, dtype=torch.float64,
                                   generator=torch.Generator().manual_seed(16)))
    perm = [2, 0, 1]
    ck = torch.cat([torch.arange(h * dk, (h + 1) * dk) for h in perm])
    cv = torch.cat([torch.arange(h * dv, (h + 1) * dv) for h in perm])
    Q = {n: t.detach().clone() for n, t in P.items()}
    Q["w_q"], Q["w_k"] = P["w_q"][:, ck], P["w_k"][:, ck]
    Q["w_a2"], Q["b_a"] = P["w_a2"][:, ck], P["b_a"][ck]
    Q["w_v"], Q["w_r"], Q["b_r"] = P["w_v"][:, cv], P["w_r"][:, cv], P["b_r"][cv]
    Q["w_o"] = P["w_o"][cv, :]
    a = layer_fwd(P, x, lay.h, lay.temp)
    b = layer_fwd(Q, x, lay.h, lay.temp)
    assert torch.allclose(a, b, rtol=1e-12, atol=1e-13)
    # and a permutation of channels that crosses heads does change it
    Q2 = {n: t.detach().clone() for n, t in P.items()}
    cross = torch.roll(torch.arange(d), 1)
    Q2["w_v"], Q2["w_r"], Q2["b_r"] = P["w_v"][:, cross], P["w_r"][:, cross], P["b_r"][cross]
    Q2["w_o"] = P["w_o"][cross, :]
    assert not torch.allclose(a, layer_fwd(Q2, x, lay.h, lay.temp), atol=1e-6)


def test_layer_reference_output_gate_is_swish(oracle_mod):
    # r = swish(x W_r + b_r) = t sigma(t): zero at t = 0, and with a constant
    # pre-activation c the output scales by swish(c) (so c = 1 and c = -1
    # give outputs in the ratio swish(1) / swish(-1) = -e).
    d, heads = 16, 2
    lay = _layer(d, heads, seed=17)
    x = torch.randn(1, 9, d, dtype=torch.float64, generator=torch.Generator().manual_seed(18))
    P0 = layer_params(lay)
    with torch.no_grad():
        P0["w_r"].zero_()
        P0["b_r"].zero_()
    assert torch.count_nonzero(layer_fwd(P0, x, lay.h, lay.temp)) == 0
    ys = {}
    for c in (1.0, -1.0):
        P = layer_params(lay)
        with torch.no_grad():
            P["w_r"].zero_()
            P["b_r"].fill_(c)
        ys[c] = layer_fwd(P, x, lay.h, lay.temp).detach()
    import math
    assert torch.allclose(ys[1.0], -math.e * ys[-1.0], rtol=1e-12, atol=1e-14)
