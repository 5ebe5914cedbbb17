"""fp64 NumPy chunkwise form of GLA with secondary chunking.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

This is a second, independent statement of what the layer computes: the
chunkwise-parallel form of "Gated Linear Attention Transformers with
Hardware-Efficient Training" (papercache.org notes, §4.2 chunkwise form and
§4.3 / Figure 3 secondary chunking; App. B, the PyTorch-style listing of the
secondary-chunking forward).  It is used only to pin the token-by-token
recurrence in ``gla_oracle.c``: the two must agree for every chunk size C
(notes §2.2: C = L is the parallel form, C = 1 the recurrent form).

Per head, with a = log alpha and chunk size C, sub-chunk size c:

* B = inclusive cumsum of a *within each chunk* (the listing's cumsum; its
  printed loop body indexes a[i] / B[i] where the chunk-local position
  i*C + j is meant -- taken that way here, which is the only reading under
  which the listing reproduces the recurrence).
* Inter-chunk: O_n += (Q ⊙ e^B) S_{n-1};  S_n = diag(e^{b}) S_{n-1} +
  (K ⊙ e^{b - B})^T V, with b = B at the chunk's last row.
* Intra-chunk, per sub-chunk j:
    - diagonal block in full precision log space:
      P[m, r] = sum_k q_mk k_rk exp(B_mk - B_rk) for r <= m;
    - earlier sub-chunks u < j via the reference row z = B at sub-chunk j's
      first row: (Q_j ⊙ e^{B_j - z}) (K_u ⊙ e^{z - B_u})^T, both factors <= 1.
* h0 / hT: S_0 = h0 (the chunk state may come from a previous segment,
  notes §2.2); hT = S_{L/C}.  The listing itself starts from zeros and does
  not return the final state; adding both is the plain extension.

Nothing here is blocked, fused or reordered beyond those steps.
"""
from __future__ import annotations

import numpy as np


def _head(q, k, v, a, h0, C, c):
    L, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if h0 is None else np.array(h0, dtype=np.float64)
    o = np.zeros((L, dv))
    for n in range(L // C):
        rows = slice(n * C, (n + 1) * C)
        bq, bk, bv, ba = q[rows], k[rows], v[rows], a[rows]
        Bc = np.cumsum(ba, axis=0)            # chunk-local inclusive cumsum
        b_last = Bc[-1]
        oc = (bq * np.exp(Bc)) @ S            # inter-chunk contribution
        S = np.exp(b_last)[:, None] * S + (bk * np.exp(b_last - Bc)).T @ bv
        for j in range(C // c):
            t = slice(j * c, (j + 1) * c)
            qj, kj, vj, Bj = bq[t], bk[t], bv[t], Bc[t]
            P = np.zeros((c, c))
            for m in range(c):
                for r in range(m + 1):
                    P[m, r] = np.sum(qj[m] * kj[r] * np.exp(Bj[m] - Bj[r]))
            oc[t] += P @ vj
            z = Bj[0]
            qs = qj * np.exp(Bj - z)
            for u in range(j):
                y = slice(u * c, (u + 1) * c)
                ks = bk[y] * np.exp(z - Bc[y])
                oc[t] += (qs @ ks.T) @ bv[y]
        o[rows] = oc
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
