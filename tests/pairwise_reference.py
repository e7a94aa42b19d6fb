"""Independent whole-sequence (pairwise-decay attention) form of the gated delta
rule, for tiny inputs only.  Used to pin the token-serial oracle.

It shares nothing with the oracle's recurrence: decays are explicit products
of per-token factors (no cumulative sums, no state loop), the delta system is
solved by textbook forward substitution, and the output and final state are
assembled from the solved deltas.  For one (batch, head), with a_t = exp(g_t)
(per key channel), E_ij = prod_{s=j+1..i} a_s and Gam_i = prod_{s=0..i} a_s:

    d_i + sum_{j<i} beta_i <k_i, k_j * E_ij> d_j = beta_i (v_i - h0^T (k_i * Gam_i))
    o_i  = scale * (h0^T (q_i * Gam_i) + sum_{j<=i} <q_i, k_j * E_ij> d_j)
    hT   = Gam_{T-1} * h0 + sum_j (k_j * E_{T-1,j}) d_j^T

which is the chunked view of the recurrence with the whole sequence as one
chunk (the Marin note's "Background": later queries scored against earlier
keys, decayed by the per-channel factor between the two tokens).
"""
from __future__ import annotations

import math

import numpy as np


def _prod(a, lo, hi):
    """prod_{s=lo..hi} a_s (rows), explicit left-to-right multiplication."""
    out = np.ones(a.shape[1])
    for s in range(lo, hi + 1):
        out = out * a[s]
    return out


def head_forward(q, k, v, g, beta, scale, h0=None):
    """One head.  q,k [T,Dk]; v [T,Dv]; g [T,Dk] or [T]; beta [T]; h0 [Dk,Dv]."""
    T, Dk = q.shape
    Dv = v.shape[1]
    g = np.asarray(g, dtype=np.float64)
    if g.ndim == 1:
        g = np.repeat(g[:, None], Dk, axis=1)
    a = np.array([[math.exp(x) for x in row] for row in g])
    h0 = np.zeros((Dk, Dv)) if h0 is None else np.asarray(h0, dtype=np.float64)
    E = np.zeros((T, T, Dk))
    for i in range(T):
        for j in range(i + 1):
            E[i, j] = _prod(a, j + 1, i)
    Gam = np.array([_prod(a, 0, i) for i in range(T)])
    P = np.zeros((T, T))
    A = np.zeros((T, T))
    for i in range(T):
        for j in range(i + 1):
            P[i, j] = sum(q[i, c] * k[j, c] * E[i, j, c] for c in range(Dk))
            if j < i:
                A[i, j] = beta[i] * sum(k[i, c] * k[j, c] * E[i, j, c] for c in range(Dk))
    rhs = np.zeros((T, Dv))
    for i in range(T):
        kg = k[i] * Gam[i]
        rhs[i] = beta[i] * (v[i] - np.array([sum(kg[c] * h0[c, n] for c in range(Dk))
                                             for n in range(Dv)]))
    D = np.zeros((T, Dv))
    for i in range(T):  # forward substitution, unit lower triangular (I + A)
        acc = rhs[i].copy()
        for j in range(i):
            acc = acc - A[i, j] * D[j]
        D[i] = acc
    O = np.zeros((T, Dv))
    for i in range(T):
        qg = q[i] * Gam[i]
        val = np.array([sum(qg[c] * h0[c, n] for c in range(Dk)) for n in range(Dv)])
        for j in range(i + 1):
            val = val + P[i, j] * D[j]
        O[i] = scale * val
    hT = Gam[T - 1][:, None] * h0
    for j in range(T):
        hT = hT + np.outer(k[j] * E[T - 1, j], D[j])
    return O, hT, P, A


def forward(q, k, v, g, beta, scale, h0=None):
    """All heads; arrays in the library layout, float64."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    O = np.zeros((B, T, H, Dv))
    HT = np.zeros((B, H, Dk, Dv))
    for b in range(B):
        for h in range(H):
            o, hT, _, _ = head_forward(q[b, :, h], k[b, :, h], v[b, :, h],
                                       g[b, :, h], beta[b, :, h], scale,
                                       None if h0 is None else h0[b, h])
            O[b, :, h] = o
            HT[b, h] = hT
    return O, HT
