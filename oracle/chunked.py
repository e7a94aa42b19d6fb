"""Chunked form of the gated delta rule with the numerical-safety options
(float64, plain torch CPU ops, dense matrices).

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this module.  It shares nothing with
the HIP library.

The chunked algorithm (Marin note, "Background": the sequence in chunks of C
tokens, later queries scored against earlier keys inside a chunk, a state
carried between chunks; atomic_ops card, "Features": chunk scores, WY block
solve, recompute, inter-chunk scan).  For one chunk with start state S
(rows t of the chunk, g the per-key-channel log-decays, G their inclusive
cumulative sum inside the chunk, Gamma = exp(G)):

    P[i, j] = sum_c q[i, c] k[j, c] exp(G[i, c] - G[j, c])            j <= i
    A[i, j] = beta[i] sum_c k[i, c] k[j, c] exp(G[i, c] - G[j, c])     j <  i
    T = ((1 + wy_eps) I + A)^-1
    U = T diag(beta) V,   W = T diag(beta) (K o Gamma),   D = U - W S
    O = scale ((Q o Gamma) S + P D)
    S <- diag(exp(G[C-1])) S + (K o exp(G[C-1] - G))^T D

With wy_eps = 0 this is the token recurrence exactly (D holds the tokens'
deltas); the token-serial oracle pins it there.  The options (atomic_ops card,
"Features": clipping + nan_to_num at every kernel boundary, optional wy_eps
Tikhonov-style damping of the WY solve; "Debugging": per-stage reports of
non-finite or > 1e6 values that never change values):

  wy_eps  damping of the WY solve: (1 + wy_eps) on the diagonal of I + A
  clip    at each boundary between the pages' four forward stages (scores P
          and A, the solve's T, the recompute's U and W, the outputs O and the
          final state) NaN -> 0, +-inf -> +-clip, then clamp to [-clip, clip]
  diag    counts per boundary, before clipping: non-finite values, and finite
          values with |x| > 1e6 (DIAG_STAGES order)

Gradients come from torch autograd through this forward with the clipping
taken as the identity (it is the identity wherever values are finite and
inside the bound); with clip set, the returned gradients are clipped too.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _f64, l2norm, l2norm_backward

DIAG_STAGES = ("P", "A", "T", "U", "W", "o", "hT")
DIAG_LARGE = 1e6


class _Clip(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, c):
        return torch.clamp(torch.nan_to_num(x, nan=0.0, posinf=c, neginf=-c), -c, c)

    @staticmethod
    def backward(ctx, gr):
        return gr, None


def _boundary(x, stage, clip, counts, valid=None):
    """A stage boundary: count (before clipping) and clip."""
    if counts is not None:
        xv = x.detach() if valid is None else x.detach()[valid]
        fin = torch.isfinite(xv)
        counts[stage][0] += int((~fin).sum())
        counts[stage][1] += int((fin & (xv.abs() > DIAG_LARGE)).sum())
    return _Clip.apply(x, clip) if clip else x


def _forward_t(q, k, v, g, beta, scale, h0, chunk, wy_eps, clip, counts):
    """Torch float64 tensors [B,T,H,*] -> (o [B,T,H,Dv], hT [B,H,Dk,Dv])."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    C = chunk
    NC = (T + C - 1) // C
    pad = NC * C - T
    if g.dim() == 3:  # one log-decay per head: the same value in every key channel
        g = g[..., None].expand(B, T, H, Dk)

    def padt(x):  # padding tokens: q = k = v = 0, g = 0, beta = 0 (they change nothing)
        if not pad:
            return x
        shp = list(x.shape)
        shp[1] = pad
        return torch.cat([x, x.new_zeros(shp)], dim=1)

    # [B, H, NC, C, *]
    def chunks(x):
        x = padt(x)
        return x.reshape(B, NC, C, H, *x.shape[3:]).movedim(3, 1)

    Q, K, V, Gl, Bt = chunks(q), chunks(k), chunks(v), chunks(g), chunks(beta)
    S = h0.clone() if h0 is not None else q.new_zeros(B, H, Dk, Dv)
    low_incl = torch.tril(torch.ones(C, C, dtype=torch.bool))
    low_strict = torch.tril(torch.ones(C, C, dtype=torch.bool), -1)
    eye = torch.eye(C, dtype=q.dtype)
    outs = []
    for n in range(NC):
        q_, k_, v_, b_ = Q[:, :, n], K[:, :, n], V[:, :, n], Bt[:, :, n]
        G = torch.cumsum(Gl[:, :, n], dim=2)                       # [B,H,C,Dk]
        diff = G[:, :, :, None, :] - G[:, :, None, :, :]           # G_i - G_j  [B,H,C,C,Dk]
        E = torch.exp(torch.where(low_incl[:, :, None], diff, torch.zeros_like(diff)))
        qk = (q_[:, :, :, None, :] * k_[:, :, None, :, :] * E).sum(-1)
        kk = (k_[:, :, :, None, :] * k_[:, :, None, :, :] * E).sum(-1)
        P = torch.where(low_incl, qk, torch.zeros_like(qk))
        A = torch.where(low_strict, b_[..., None] * kk, torch.zeros_like(kk))
        P = _boundary(P, "P", clip, counts)
        A = _boundary(A, "A", clip, counts)
        M = (1.0 + wy_eps) * eye + A
        Tm = torch.linalg.solve_triangular(M, eye.expand_as(M), upper=False)
        Tm = _boundary(Tm, "T", clip, counts)
        Gam = torch.exp(G)
        U = Tm @ (b_[..., None] * v_)
        W = Tm @ (b_[..., None] * k_ * Gam)
        U = _boundary(U, "U", clip, counts)
        W = _boundary(W, "W", clip, counts)
        D = U - W @ S
        O = scale * ((q_ * Gam) @ S + P @ D)
        outs.append(O)
        Gl_last = G[:, :, -1:, :]                                  # [B,H,1,Dk]
        S = torch.exp(Gl_last[:, :, 0, :, None]) * S + (k_ * torch.exp(Gl_last - G)).transpose(-1, -2) @ D
    o = torch.stack(outs, dim=2).reshape(B, H, NC * C, Dv)[:, :, :T].movedim(1, 2)
    o = _boundary(o, "o", clip, counts)
    hT = _boundary(S, "hT", clip, counts)
    return o, hT


def _tensors(*xs):
    return [None if x is None else torch.from_numpy(_f64(x)) for x in xs]


def forward(q, k, v, g, beta, scale, h0=None, *, chunk=64, wy_eps=0.0, clip=0.0,
            qk_l2norm=False, diag=False):
    """Returns (o, hT) as float64 arrays, and with diag also the counts
    {stage: (non-finite, large)}."""
    if qk_l2norm:
        q, k = l2norm(q), l2norm(k)
    counts = {s: [0, 0] for s in DIAG_STAGES} if diag else None
    tq, tk, tv, tg, tb, th = _tensors(q, k, v, g, beta, h0)
    with torch.no_grad():
        o, hT = _forward_t(tq, tk, tv, tg, tb, float(scale), th, chunk, float(wy_eps),
                           float(clip), counts)
    res = (o.numpy(), hT.numpy())
    if diag:
        return res + ({s: tuple(c) for s, c in counts.items()},)
    return res


def backward(q, k, v, g, beta, scale, dO, h0=None, dhT=None, *, chunk=64, wy_eps=0.0, clip=0.0,
             qk_l2norm=False):
    """Gradients of sum(o * dO) + sum(hT * dhT) (dq, dk with respect to the raw
    rows when qk_l2norm), float64 arrays."""
    q_raw, k_raw = q, k
    if qk_l2norm:
        q, k = l2norm(q), l2norm(k)
    if h0 is None:  # the gradient at a zero start state is still wanted (dh0)
        h0 = np.zeros((q.shape[0], q.shape[2], q.shape[3], v.shape[3]))
    ts = _tensors(q, k, v, g, beta, h0)
    for t in ts:
        if t is not None:
            t.requires_grad_(True)
    tq, tk, tv, tg, tb, th = ts
    o, hT = _forward_t(tq, tk, tv, tg, tb, float(scale), th, chunk, float(wy_eps), float(clip),
                       None)
    loss = (o * torch.from_numpy(_f64(dO))).sum()
    if dhT is not None:
        loss = loss + (hT * torch.from_numpy(_f64(dhT))).sum()
    want = [t for t in ts if t is not None]
    grads = torch.autograd.grad(loss, want, allow_unused=True)
    gmap = dict(zip([id(t) for t in want], grads))
    names = ("dq", "dk", "dv", "dg", "dbeta", "dh0")
    out = {}
    for name, t in zip(names, ts):
        gr = gmap.get(id(t))
        out[name] = (torch.zeros_like(t) if gr is None else gr).numpy()
    if qk_l2norm:
        out["dq"] = l2norm_backward(q_raw, out["dq"])
        out["dk"] = l2norm_backward(k_raw, out["dk"])
    if clip:
        for name in names:
            x = out[name]
            out[name] = np.clip(np.nan_to_num(x, nan=0.0, posinf=clip, neginf=-clip), -clip, clip)
    return out


def forward_inputs(inp: dict, **kw):
    kw.setdefault("qk_l2norm", bool(inp["meta"].get("qk_l2norm", False)))
    kw.setdefault("chunk", inp["meta"].get("chunk", 64))
    return forward(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["meta"]["scale"],
                   h0=inp.get("h0"), **kw)


def backward_inputs(inp: dict, **kw):
    kw.setdefault("qk_l2norm", bool(inp["meta"].get("qk_l2norm", False)))
    kw.setdefault("chunk", inp["meta"].get("chunk", 64))
    return backward(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["meta"]["scale"],
                    inp["dO"], h0=inp.get("h0"), dhT=inp.get("dhT"), **kw)
