"""Op-level GLA layer around the library's kernels, on synthetic weights.

The layer of the pages' GLA Transformer (zako-mio deep-reading report ch. 3.5
on §4.4; gate parametrisation ch. 2.3): for input x [B, L, d] and H heads,

    q = x W_q,  k = x W_k  (d -> d/2),   v = x W_v  (d -> d),
    log alpha = logsigmoid(x W_a1 W_a2 + b_a) / 16      (rank-16 gate, d -> d/2)
    o^h = GLA(q^h d_k^{-1/2}, k^h, v^h, alpha^h)        (per head, the kernels)
    o = concat_h LayerNorm(o^h),   r = swish(x W_r + b_r),   y = (o ⊙ r) W_o

with d_k = d / (2 H) and d_v = d / H per head.  The projections, the gate
producer, the norms and the output gate are torch operations (plain 2-D
matrix products on the library GEMMs); the recurrence, forward and backward,
runs in the HIP kernels through `GlaFunction`.  Weights are seeded random
draws: the layer is a workload for the kernels, not a trained model.
"""
from __future__ import annotations

import torch
import torch.nn.functional as F

from . import bwd as _gla_bwd
from . import fwd as _gla_fwd


class GlaFunction(torch.autograd.Function):
    """o = GLA(q, k, v, log_alpha) per (batch, head) with h0 = 0, through
    gla_fwd / gla_bwd.  q, k, v [B, H, L, d] in the I/O dtype, log_alpha
    [B, H, L, dk] fp32."""

    @staticmethod
    def forward(ctx, q, k, v, log_alpha, chunk):
        q, k, v, log_alpha = (t.contiguous() for t in (q, k, v, log_alpha))
        o, _ = _gla_fwd(q, k, v, log_alpha, None, chunk=chunk, final_state=False)
        ctx.save_for_backward(q, k, v, log_alpha)
        ctx.chunk = chunk
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, log_alpha = ctx.saved_tensors
        dq, dk, dv, dla, _ = _gla_bwd(q, k, v, log_alpha, None, do.contiguous(),
                                      chunk=ctx.chunk, want_dh0=False)
        return dq, dk, dv, dla, None


def _mm(x2d, w):
    """x2d [N, i] @ w [i, o], both contiguous (2-D products only)."""
    return torch.matmul(x2d, w)


class GlaLayer(torch.nn.Module):
    """The GLA attention layer above; weights stored [in, out], contiguous."""

    def __init__(self, d: int, heads: int, gate_rank: int = 16, gate_temp: float = 16.0,
                 chunk: int = 64, seed: int = 0, dtype=torch.bfloat16, device="cuda"):
        super().__init__()
        if d % (2 * heads):
            raise ValueError("d must be a multiple of 2 * heads")
        self.d, self.h, self.chunk, self.temp = d, heads, chunk, gate_temp
        self.dk, self.dv = d // (2 * heads), d // heads
        g = torch.Generator().manual_seed(int(seed))

        def w(i, o, scale=None):
            t = torch.randn(i, o, generator=g) * (scale if scale is not None else i ** -0.5)
            return torch.nn.Parameter(t.to(dtype).to(device))

        self.w_q, self.w_k, self.w_v = w(d, d // 2), w(d, d // 2), w(d, d)
        self.w_a1, self.w_a2 = w(d, gate_rank), w(gate_rank, d // 2)
        self.b_a = torch.nn.Parameter(torch.zeros(d // 2, dtype=torch.float32, device=device))
        self.w_r, self.w_o = w(d, d), w(d, d)
        self.b_r = torch.nn.Parameter(torch.zeros(d, dtype=dtype, device=device))

    def heads(self, t, dh):
        B, L, _ = t.shape
        return t.view(B, L, self.h, dh).transpose(1, 2).contiguous()

    def forward(self, x):
        B, L, d = x.shape
        x2 = x.reshape(B * L, d)
        q = _mm(x2, self.w_q).view(B, L, -1) * self.dk ** -0.5
        k = _mm(x2, self.w_k).view(B, L, -1)
        v = _mm(x2, self.w_v).view(B, L, -1)
        gl = _mm(_mm(x2, self.w_a1), self.w_a2).float() + self.b_a
        la = (F.logsigmoid(gl) / self.temp).view(B, L, -1)
        o = GlaFunction.apply(self.heads(q.to(x.dtype), self.dk), self.heads(k, self.dk),
                              self.heads(v, self.dv), self.heads(la, self.dk), self.chunk)
        o = F.layer_norm(o.float(), (self.dv,)).to(x.dtype)          # per head
        o = o.transpose(1, 2).reshape(B * L, d)
        r = F.silu(_mm(x2, self.w_r) + self.b_r)
        return _mm((o * r).contiguous(), self.w_o).view(B, L, d)

    def flops_fwd(self, B: int, L: int) -> float:
        """Matrix-product FLOPs of one forward: the projections plus the stated
        count of the GLA core (2 L C (dk + dv) + 4 L dk dv per head)."""
        d, r = self.d, self.w_a1.shape[1]
        proj = 2.0 * B * L * (d * d / 2 * 2 + d * d * 3 + d * r + r * d / 2)
        core = B * self.h * (2.0 * L * self.chunk * (self.dk + self.dv)
                             + 4.0 * L * self.dk * self.dv)
        return proj + core


__all__ = ["GlaFunction", "GlaLayer"]
