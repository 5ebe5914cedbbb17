"""GPU parity of the op-level GLA layer (projections and gates in torch, the
recurrence in the HIP kernels) against its fp64 CPU reference with the oracle's
recurrence: the output and the gradients of the input and of every weight.

Tolerances (relative L2 per tensor).  fp32: 1e-4, ten fp32 stages (GEMMs over
d <= 512, the norm, the gates), each well inside the kernels' 1e-5 bar.  bf16:
2e-2, about ten roundings of intermediates to bf16 (unit roundoff 2^-9, rms
about 1.1e-3 each, so about 3.5e-3 summed) with a margin for the norm's and
the gradient chain's amplification."""
import numpy as np
import pytest
import torch

from chunkwise_linear_rnn_gla_amd.layer import GlaLayer
from gpu_util import rel_l2, say
from layer_ref import layer_fwd, layer_params

pytestmark = pytest.mark.gpu

TOL_LAYER = {"fp32": 1e-4, "bf16": 2e-2}


@pytest.mark.parametrize("dtype,B,L,d,heads", [
    ("fp32", 2, 200, 256, 2),      # d_k 64, d_v 128; ragged last chunk
    ("bf16", 2, 200, 256, 2),
    ("bf16", 1, 130, 512, 4),      # d_k 64, d_v 128, four heads
    ("fp32", 1, 64, 512, 2),       # d_k 128, d_v 256 (the 340M head shape)
])
def test_layer_matches_reference(dtype, B, L, d, heads):
    tdt = torch.float32 if dtype == "fp32" else torch.bfloat16
    say(f"[layer] dtype={dtype} B={B} L={L} d={d} heads={heads}")
    lay = GlaLayer(d, heads, seed=11 + d, dtype=tdt, device="cuda")
    g = torch.Generator().manual_seed(12 + L)
    x = torch.randn(B, L, d, generator=g).to(tdt)
    dy = torch.randn(B, L, d, generator=g).to(tdt)

    xg = x.cuda().requires_grad_(True)
    y = lay(xg)
    y.backward(dy.cuda())
    torch.cuda.synchronize()

    P = layer_params(lay)
    x64 = x.double().requires_grad_(True)
    y64 = layer_fwd(P, x64, heads, lay.temp)
    y64.backward(dy.double())

    tol = TOL_LAYER[dtype]
    pairs = [("y", y, y64), ("dx", xg.grad, x64.grad)]
    pairs += [("d" + n, p.grad, P[n].grad) for n, p in lay.named_parameters()]
    for name, got, want in pairs:
        got = got.detach().double().cpu().numpy()
        want = want.detach().numpy()
        e = rel_l2(got, want)
        say(f"      {name}: rel_l2 {e:.3e}")
        assert np.isfinite(got).all(), name
        assert e <= tol, f"{name} rel_l2 {e}"
