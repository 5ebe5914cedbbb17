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
