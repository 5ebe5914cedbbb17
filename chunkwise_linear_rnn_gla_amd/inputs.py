"""Seeded synthetic inputs for the GLA layer, shared by the HIP path's tests,
the benchmark and the oracle's callers.

This module holds no arithmetic of the method itself: it only draws random
tensors with the shapes and distributions of the layer shapes on the pages
(4 heads, d_k = d_v / 2, training length 2048; the GLA-340M and GLA-1.3B
layers) and casts them to the I/O dtype.

Recipe (the same for every workload):
* a CPU ``torch.Generator`` seeded with ``seed``; tensors drawn in the order
  q, k, v, z, then h0 (only if the workload has a nonzero initial state), then
  the upstream gradient do (only if it has a backward), then dhT (only if
  requested);
* q ~ N(0,1) * d_k^-1/2, k, v ~ N(0,1), drawn in fp32, then rounded once to the
  I/O dtype (round-to-nearest-even for bf16);
* gate: log alpha = logsigmoid(z) / 16 with z ~ N(0,1) per (b, h, t, key
  channel), kept in fp32.  This mirrors the pages' gate parametrisation
  alpha = sigmoid(x W1 W2 + b)^(1/tau) with tau = 16 (zako-mio report, ch. 3.3;
  papercache.org notes §4.1), with the low-rank projection output replaced by
  N(0,1) draws since no trained weights are involved;
* h0 ~ N(0,1) * h0_std in fp32; do ~ N(0,1) in the I/O dtype.

Optional gate modes for edge cases: "zero" (alpha == 1), "const" (one
log-decay value everywhere), "channel_const" (one value per key channel,
shared over time), "extreme" (log alpha ~ -U(0, 20): gates that underflow
fp32 products within a few steps), "spiky" (the sigmoid gate with one entry in
2,048 replaced by -U(10, 40): rare abrupt forgets, so that some 16-token spans
of a channel decay far more than the rest).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch
import torch.nn.functional as F

DTYPES = {"fp32": torch.float32, "bf16": torch.bfloat16}


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str          # "fp32" or "bf16": dtype of q, k, v, o (and do, dq, dk, dv)
    B: int
    H: int
    L: int
    dk: int
    dv: int
    chunk: int = 64
    subchunk: int = 16
    h0_std: float = 0.0
    backward: bool = False
    seed: int = 0

    @property
    def tokens(self) -> int:
        return self.B * self.L

    def stated_flops_fwd(self) -> int:
        """FLOPs by the stated count: per head 2*L*C*(dk+dv) + 4*L*dk*dv."""
        per_head = 2 * self.L * self.chunk * (self.dk + self.dv) + 4 * self.L * self.dk * self.dv
        return self.B * self.H * per_head


# The five workloads of the benchmark contract (seed = 1000 + number).
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", "fp32", 1, 1, 64, 16, 32, chunk=16, seed=1001),
    "gla340m_fwd": Workload("gla340m_fwd", "bf16", 8, 4, 2048, 128, 256, seed=1002),
    "gla1p3b_fwd": Workload("gla1p3b_fwd", "bf16", 4, 4, 2048, 256, 512, seed=1003),
    "long16k_fwd": Workload("long16k_fwd", "bf16", 1, 4, 16384, 128, 256, h0_std=0.1, seed=1004),
    "gla340m_fwdbwd": Workload("gla340m_fwdbwd", "bf16", 8, 4, 2048, 128, 256, backward=True,
                               seed=1005),
}


@dataclasses.dataclass
class Inputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    log_alpha: torch.Tensor
    h0: Optional[torch.Tensor]
    do: Optional[torch.Tensor]
    dhT: Optional[torch.Tensor]

    def to(self, device) -> "Inputs":
        f = lambda t: None if t is None else t.to(device).contiguous()
        return Inputs(*(f(getattr(self, x.name)) for x in dataclasses.fields(self)))


def make_inputs(B, H, L, dk, dv, dtype="bf16", seed=0, gate="sigmoid16", h0_std=0.0,
                with_do=False, dhT_std=0.0, gate_value=-0.05) -> Inputs:
    """Draw one seeded set of CPU tensors laid out [B, H, L, d] (h0 [B, H, dk, dv])."""
    g = torch.Generator().manual_seed(int(seed))
    io = DTYPES[dtype]
    q = (torch.randn(B, H, L, dk, generator=g) * dk ** -0.5).to(io)
    k = torch.randn(B, H, L, dk, generator=g).to(io)
    v = torch.randn(B, H, L, dv, generator=g).to(io)
    z = torch.randn(B, H, L, dk, generator=g)
    if gate == "sigmoid16":
        a = F.logsigmoid(z) / 16.0
    elif gate == "zero":
        a = torch.zeros_like(z)
    elif gate == "const":
        a = torch.full_like(z, float(gate_value))
    elif gate == "channel_const":
        a = (F.logsigmoid(z[:, :, :1, :]) / 16.0).expand_as(z).contiguous()
    elif gate == "extreme":
        a = -20.0 * torch.rand(B, H, L, dk, generator=g)
    elif gate == "spiky":
        spike = torch.rand(B, H, L, dk, generator=g) < 1.0 / 2048
        depth = 10.0 + 30.0 * torch.rand(B, H, L, dk, generator=g)
        a = torch.where(spike, -depth, F.logsigmoid(z) / 16.0)
    else:
        raise ValueError(f"unknown gate mode {gate!r}")
    a = a.to(torch.float32).contiguous()
    h0 = torch.randn(B, H, dk, dv, generator=g) * h0_std if h0_std else None
    do = torch.randn(B, H, L, dv, generator=g).to(io) if with_do else None
    dhT = torch.randn(B, H, dk, dv, generator=g) * dhT_std if dhT_std else None
    return Inputs(q, k, v, a, h0, do, dhT)


def make_log_beta(B, H, L, dv, seed=0, gate="sigmoid16", gate_value=-0.05):
    """Seeded column gate log beta [B, H, L, dv] (fp32) for the general gate
    G = alpha^T beta, drawn from its own generator (seed + 7919) so that the
    draws of make_inputs with the same seed are unchanged.  Same modes as the
    row gate: logsigmoid(z) / 16, zero, constant, per-channel constant and
    "extreme" (-U(0, 20))."""
    g = torch.Generator().manual_seed(int(seed) + 7919)
    z = torch.randn(B, H, L, dv, generator=g)
    if gate == "sigmoid16":
        b = F.logsigmoid(z) / 16.0
    elif gate == "zero":
        b = torch.zeros_like(z)
    elif gate == "const":
        b = torch.full_like(z, float(gate_value))
    elif gate == "channel_const":
        b = (F.logsigmoid(z[:, :, :1, :]) / 16.0).expand_as(z).contiguous()
    elif gate == "extreme":
        b = -20.0 * torch.rand(B, H, L, dv, generator=g)
    else:
        raise ValueError(f"unknown gate mode {gate!r}")
    return b.to(torch.float32).contiguous()


def workload_inputs(w: Workload) -> Inputs:
    return make_inputs(w.B, w.H, w.L, w.dk, w.dv, w.dtype, w.seed, h0_std=w.h0_std,
                       with_do=w.backward)


def as_f64(t):
    """Exact upcast of a CPU tensor (any float dtype) to a float64 NumPy array."""
    if t is None:
        return None
    return t.detach().to("cpu", torch.float64).numpy()
