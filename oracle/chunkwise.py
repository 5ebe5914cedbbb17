"""fp64 NumPy chunkwise form of GLA with secondary chunking.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

A second, independent statement of what the layer computes, used only to pin
the token-by-token recurrence in ``gla_oracle.c``: the two must agree for
every chunk size C (papercache.org notes on "Gated Linear Attention
Transformers with Hardware-Efficient Training", §2.2: C = L is the parallel
form, C = 1 the recurrent form).  It is written from the matrix equations of
the chunkwise form (notes §4.2) and the block split of secondary chunking
(notes §4.3, Figure 3), one whole-chunk or whole-block array operation per
equation:

* Per chunk, B is the cumulative sum of a = log alpha from the chunk's first
  row (inclusive), so Lambda = e^B is the decay from the chunk start, b = B
  at the last row is the chunk's total log decay, gamma = e^b and
  Gamma = e^{b - B} the decay from a row to the chunk end.
* Output:  O = (Q ⊙ Lambda) S_prev + P V, with the chunk's causal gated
  score matrix P[m, r] = sum_k q_mk k_rk exp(B_mk - B_rk) for r <= m.
* State:   S = diag(gamma) S_prev + (K ⊙ Gamma)^T V.
* P by sub-chunks of c rows (Figure 3): blocks on the diagonal in log space
  (the pairwise differences B_m - B_r masked to r <= m before the
  exponential); blocks below the diagonal as one matrix product per query
  sub-chunk j through the reference row z = B at its first row,
  (Q_j ⊙ e^{B_j - z}) (K_{<j} ⊙ e^{z - B_{<j}})^T, where both factors are <= 1.
* S_0 = h0 (a previous segment's state, notes §2.2, or zeros); hT = the state
  after the last chunk.
"""
from __future__ import annotations

import numpy as np


def chunk_scores(q, k, B, c):
    """The causal gated score matrix P (C x C) of one chunk, by sub-chunks of
    c rows: log space on the diagonal blocks, reference-row products below."""
    C = q.shape[0]
    t = np.arange(C)
    on_diag_block = (t[:, None] // c == t[None, :] // c) & (t[:, None] >= t[None, :])
    diff = np.where(on_diag_block[:, :, None], B[:, None, :] - B[None, :, :], -np.inf)
    P = np.einsum("mk,rk,mrk->mr", q, k, np.exp(diff))
    for j in range(1, C // c):
        rows, z = slice(j * c, (j + 1) * c), B[j * c]
        P[rows, : j * c] = (q[rows] * np.exp(B[rows] - z)) @ (k[: j * c] * np.exp(z - B[: j * c])).T
    return P


def _head(q, k, v, a, h0, C, c):
    L, dk = q.shape
    S = np.zeros((dk, v.shape[1])) if h0 is None else np.array(h0, dtype=np.float64)
    o = np.empty((L, v.shape[1]))
    for n0 in range(0, L, C):
        rows = slice(n0, n0 + C)
        Q, K, V = q[rows], k[rows], v[rows]
        B = np.cumsum(a[rows], axis=0)
        b = B[-1]
        o[rows] = (Q * np.exp(B)) @ S + chunk_scores(Q, K, B, c) @ V
        S = np.exp(b)[:, None] * S + (K * np.exp(b - B)).T @ V
    return o, S


def chunkwise_fwd(q, k, v, log_alpha, h0=None, C=64, c=16):
    """Chunkwise GLA forward in fp64. Arrays are [B, H, L, d] (h0 [B, H, dk, dv]).

    Returns (o, hT).  Requires L % C == 0 and C % c == 0.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    a = np.asarray(log_alpha, dtype=np.float64)
    Bn, H, L, dk = q.shape
    dv = v.shape[-1]
    if L % C or C % c:
        raise ValueError("chunkwise_fwd needs L % C == 0 and C % c == 0")
    o = np.zeros((Bn, H, L, dv))
    hT = np.zeros((Bn, H, dk, dv))
    for b in range(Bn):
        for h in range(H):
            hh = None if h0 is None else np.asarray(h0, dtype=np.float64)[b, h]
            o[b, h], hT[b, h] = _head(q[b, h], k[b, h], v[b, h], a[b, h], hh, C, c)
    return o, hT
