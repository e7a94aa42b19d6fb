"""Pins of the CPU oracle: checks against what the pages and the mathematics fix,
independent of the oracle's own code.  Each pin takes the loaded oracle library
(``oracle.load()`` or a planted-mistake variant of it) and raises
AssertionError on failure.

Pages cited:
* "Factoring GDN-2 decay on TPU" (Marin research note), sections Background
  and Approach;
* "gated-deltanet" (Hugging Face kernels card), sections Method and Correctness;
* "atomic_ops" (PyPI card), section Correctness & testing.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import gdn_inputs as gi
import oracle
from pairwise_reference import forward as pairwise_forward

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rel_err(x, y) -> float:
    """max|x - y| / max|y| (y the expected value)."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    den = float(np.max(np.abs(y))) if y.size else 0.0
    num = float(np.max(np.abs(x - y))) if y.size else 0.0
    return num / den if den > 0 else num


def _rand(seed, B, T, H, Dk, Dv, decay="channel", h0_std=None, grads=False):
    return gi.f64_inputs(gi.make_inputs(B, T, H, Dk, Dv, decay=decay, seed=seed,
                                        h0_std=h0_std, grads=grads))


def _fwd(lib, d, **kw):
    args = dict(h0=d.get("h0"))
    args.update(kw)
    return oracle.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["meta"]["scale"],
                          lib=lib, **args)


# --------------------------------------------------------------------------
# P1  worked decay example (Marin note, Approach)
# --------------------------------------------------------------------------
def pin_worked_example(lib):
    ex = golden("worked_decay_example.json")
    cum = ex["cumulative_log_decay"]
    kf = ex["key_to_boundary_exponent"]
    qf = ex["boundary_to_query_exponents"]
    pf = ex["pair_factor_exponents"]
    # the page's own arithmetic: pair factor = key factor * query factor
    assert cum["boundary"] - cum["key"] == kf
    for i in range(2):
        assert cum["queries"][i] - cum["boundary"] == qf[i]
        assert kf + qf[i] == pf[i]
    # one 64-token chunk split 32|32: key at token 30, boundary at token 31
    # (last token of the earlier block), queries at 32 and 33, one live channel.
    T, Dk, Dv = 64, 4, 4
    g = np.zeros((1, T, 1, Dk))
    g[0, 30, 0, 0] = cum["key"]
    g[0, 31, 0, 0] = cum["boundary"] - cum["key"]
    g[0, 32, 0, 0] = cum["queries"][0] - cum["boundary"]
    g[0, 33, 0, 0] = cum["queries"][1] - cum["queries"][0]
    q = np.zeros((1, T, 1, Dk)); k = np.zeros((1, T, 1, Dk)); v = np.zeros((1, T, 1, Dv))
    beta = np.zeros((1, T, 1))
    k[0, 30, 0, 0] = 1.0; v[0, 30, 0, 0] = 1.0; beta[0, 30, 0] = 1.0
    q[0, 32, 0, 0] = 1.0; q[0, 33, 0, 0] = 1.0
    o, hT = oracle.forward(q, k, v, g, beta, 1.0, lib=lib)
    for i, t in enumerate((32, 33)):
        want = math.exp(pf[i])
        assert abs(o[0, t, 0, 0] - want) <= 1e-15 * want, (t, o[0, t, 0, 0], want)
    assert np.all(o[0, :32] == 0.0)
    # the decayed write of token 30 reaches the end of the chunk as exp(G_63 - G_30)
    assert abs(hT[0, 0, 0, 0] - math.exp(cum["queries"][1] - cum["key"])) <= 1e-15


# --------------------------------------------------------------------------
# P2  beta = 0 leaves the state untouched except for the decay (card, Correctness)
# --------------------------------------------------------------------------
def pin_beta_zero(lib):
    gs = golden("gate_semantics.json")
    assert gs["beta_zero_leaves_state_untouched"]
    for decay in ("channel", "head"):
        d = _rand(11, 1, 12, 2, 5, 3, decay=decay, h0_std=1.0)
        d["beta"][:] = 0.0
        o, hT = _fwd(lib, d)
        for h in range(2):
            S = d["h0"][0, h].copy()
            for t in range(12):
                gt = d["g"][0, t, h]
                a = np.array([math.exp(x) for x in np.broadcast_to(gt, (5,))])
                S = S * a[:, None]
                want_o = d["meta"]["scale"] * (d["q"][0, t, h] @ S)
                assert rel_err(o[0, t, h], want_o) <= 1e-14
            assert np.array_equal(hT[0, h], S), "beta=0 must leave the state untouched"


# --------------------------------------------------------------------------
# P3  g = 0 and beta = 0 is the exact identity (card, Correctness)
# --------------------------------------------------------------------------
def pin_identity(lib):
    gs = golden("gate_semantics.json")
    assert gs["g_zero_and_beta_zero_is_identity"]
    for decay in ("channel", "head"):
        d = _rand(12, 2, 9, 2, 6, 4, decay=decay, h0_std=1.0)
        d["g"][:] = 0.0
        d["beta"][:] = 0.0
        o, hT = _fwd(lib, d)
        assert np.array_equal(hT, d["h0"])
        want = d["meta"]["scale"] * np.einsum("bthi,bhij->bthj", d["q"], d["h0"])
        assert rel_err(o, want) <= 1e-14


# --------------------------------------------------------------------------
# P4  rewriting the same unit key does not double it (card, Method)
# --------------------------------------------------------------------------
def pin_rewrite(lib):
    fx = golden("delta_rewrite.json")
    rng = np.random.default_rng(5)
    Dk, Dv = 7, 5
    kvec = rng.standard_normal(Dk); kvec *= fx["key_norm"] / np.linalg.norm(kvec)
    vvec = rng.standard_normal(Dv)
    h0 = rng.standard_normal((1, 1, Dk, Dv))
    T = fx["writes"]
    k = np.tile(kvec, (1, T, 1, 1)); q = k.copy(); v = np.tile(vvec, (1, T, 1, 1))
    g = np.full((1, T, 1, Dk), fx["g"]); beta = np.full((1, T, 1), fx["beta"])
    o, hT = oracle.forward(q, k, v, g, beta, 1.0, h0=h0, lib=lib)
    for t in range(T):  # o_t = S_t^T k = v after every write
        assert rel_err(o[0, t, 0], vvec) <= 1e-13
    assert rel_err(hT[0, 0].T @ kvec, vvec) <= 1e-13
    once = h0[0, 0] + np.outer(kvec, vvec - h0[0, 0].T @ kvec)
    assert rel_err(hT[0, 0], once) <= 1e-13


# --------------------------------------------------------------------------
# P5  chunked equals whole; token by token equals batched (card, Correctness)
# --------------------------------------------------------------------------
def pin_chunk_split(lib):
    fx = golden("chunk_split.json")
    T, n, L = fx["total_tokens"], fx["calls"], fx["tokens_per_call"]
    assert n * L == T
    for decay in ("channel", "head"):
        d = _rand(13, 2, T, 2, 8, 6, decay=decay, h0_std=0.5)
        o_all, h_all = _fwd(lib, d)
        for step in (L, 1):
            S = d["h0"]
            outs = []
            for t0 in range(0, T, step):
                sl = slice(t0, t0 + step)
                o, S = oracle.forward(d["q"][:, sl], d["k"][:, sl], d["v"][:, sl], d["g"][:, sl],
                                      d["beta"][:, sl], d["meta"]["scale"], h0=S, lib=lib)
                outs.append(o)
            assert np.array_equal(np.concatenate(outs, axis=1), o_all)
            assert np.array_equal(S, h_all)


# --------------------------------------------------------------------------
# P6  independent pairwise-decay attention form, tiny inputs
# --------------------------------------------------------------------------
def pin_pairwise(lib):
    for seed in range(3):
        for decay in ("channel", "head"):
            for h0_std in (None, 0.7):
                d = _rand(20 + seed, 1, 10, 2, 5, 3, decay=decay, h0_std=h0_std)
                o, hT = _fwd(lib, d)
                o2, hT2 = pairwise_forward(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                           d["meta"]["scale"], d.get("h0"))
                assert rel_err(o, o2) <= 1e-12, rel_err(o, o2)
                assert rel_err(hT, hT2) <= 1e-12, rel_err(hT, hT2)


# --------------------------------------------------------------------------
# P7  Dk = Dv = 1: a first-order linear recurrence in closed form
#     s_t = a_t (1 - beta_t k_t^2) s_{t-1} + beta_t k_t v_t,  o_t = scale q_t s_t
# --------------------------------------------------------------------------
def pin_scalar(lib):
    rng = np.random.default_rng(7)
    T = 40
    q = rng.standard_normal((1, T, 1, 1)); k = rng.standard_normal((1, T, 1, 1)) * 0.8
    v = rng.standard_normal((1, T, 1, 1)); beta = rng.uniform(0.0, 1.0, (1, T, 1))
    g = -rng.uniform(0.0, 2.0, (1, T, 1, 1)); h0 = rng.standard_normal((1, 1, 1, 1))
    o, hT = oracle.forward(q, k, v, g, beta, 0.37, h0=h0, lib=lib)
    s = h0[0, 0, 0, 0]
    for t in range(T):
        a = math.exp(g[0, t, 0, 0]); kt = k[0, t, 0, 0]; bt = beta[0, t, 0]
        s = a * (1.0 - bt * kt * kt) * s + bt * kt * v[0, t, 0, 0]
        assert abs(o[0, t, 0, 0] - 0.37 * q[0, t, 0, 0] * s) <= 1e-13 * (1 + abs(s))
    assert abs(hT[0, 0, 0, 0] - s) <= 1e-13 * (1 + abs(s))


# --------------------------------------------------------------------------
# P8  distinct one-hot keys, zero state: the delta terms vanish and the layer
#     reduces to per-channel gated linear attention
#     o_t = scale * sum_{j<=t} beta_j q_t[c_j] prod_{s=j+1..t} exp(g_s[c_j]) v_j
# --------------------------------------------------------------------------
def pin_onehot(lib):
    rng = np.random.default_rng(8)
    Dk, Dv, T = 8, 3, 8
    perm = rng.permutation(Dk)
    k = np.zeros((1, T, 1, Dk))
    for t in range(T):
        k[0, t, 0, perm[t]] = 1.0
    q = rng.standard_normal((1, T, 1, Dk)); v = rng.standard_normal((1, T, 1, Dv))
    beta = rng.uniform(0.1, 0.9, (1, T, 1)); g = -rng.uniform(0.0, 1.5, (1, T, 1, Dk))
    scale = 0.5
    o, hT = oracle.forward(q, k, v, g, beta, scale, lib=lib)
    for t in range(T):
        want = np.zeros(Dv)
        for j in range(t + 1):
            c = perm[j]
            dec = 1.0
            for s in range(j + 1, t + 1):
                dec *= math.exp(g[0, s, 0, c])
            want += beta[0, j, 0] * q[0, t, 0, c] * dec * v[0, j, 0]
        assert rel_err(o[0, t, 0], scale * want) <= 1e-13


# --------------------------------------------------------------------------
# P9  a large negative g wipes the state by nine orders of magnitude
# --------------------------------------------------------------------------
def pin_wipe(lib):
    gs = golden("gate_semantics.json")
    d = _rand(14, 1, 1, 3, 8, 8, decay="head", h0_std=1.0)
    d["g"][:] = gs["large_negative_g_used"]
    d["beta"][:] = 0.0
    _, hT = _fwd(lib, d)
    for h in range(3):
        ratio = np.max(np.abs(hT[0, h])) / np.max(np.abs(d["h0"][0, h]))
        assert round(-math.log10(ratio)) == gs["large_negative_g_shrink_orders_of_magnitude"]
        assert abs(ratio - math.exp(gs["large_negative_g_used"])) <= 1e-12 * ratio


# --------------------------------------------------------------------------
# P10 the reverse pass equals central finite differences of the forward
#     (atomic_ops card, Correctness & testing: derivation-independent checks)
# --------------------------------------------------------------------------
def _loss(lib, d, dO, dhT):
    o, hT = _fwd(lib, d)
    return float(np.sum(o * dO) + np.sum(hT * dhT))


def pin_fd_gradients(lib, seeds=(0, 1, 2, 3, 4), h=1e-6, tol=1e-6):
    names = ("q", "k", "v", "g", "beta", "h0")
    gmap = dict(q="dq", k="dk", v="dv", g="dg", beta="dbeta", h0="dh0")
    for seed in seeds:
        for decay in ("channel", "head"):
            d = _rand(100 + seed, 1, 9, 1, 4, 3, decay=decay, h0_std=0.5, grads=True)
            dO, dhT = d["dO"], d["dhT"]
            gr = oracle.backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["meta"]["scale"],
                                 dO, h0=d["h0"], dhT=dhT, lib=lib)
            for nm in names:
                x = d[nm]
                num = np.zeros_like(x)
                for idx in np.ndindex(*x.shape):
                    x0 = x[idx]
                    x[idx] = x0 + h; lp = _loss(lib, d, dO, dhT)
                    x[idx] = x0 - h; lm = _loss(lib, d, dO, dhT)
                    x[idx] = x0
                    num[idx] = (lp - lm) / (2 * h)
                err = rel_err(gr[gmap[nm]], num)
                assert err <= tol, (seed, decay, nm, err)


# --------------------------------------------------------------------------
# P11 determinism (card, Correctness)
# --------------------------------------------------------------------------
def pin_determinism(lib):
    d = _rand(15, 2, 33, 2, 6, 5, decay="channel", h0_std=0.3, grads=True)
    a = _fwd(lib, d)
    b = _fwd(lib, d)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


# --------------------------------------------------------------------------
# P12 the use_qk_l2norm prologue (card, Usage): rows scaled to unit length
# --------------------------------------------------------------------------
def pin_l2norm_rows(lib):
    """Closed form: every normalised row has squared length s / (s + eps)
    (exactly 1 with eps = 0) and points along the raw row."""
    x = np.random.default_rng(7).standard_normal((6, 3, 11)) * np.array([1e-2, 1.0, 30.0])[:, None]
    for eps in (0.0, 1e-6):
        y = oracle.l2norm(x, eps=eps, lib=lib)
        s = np.sum(x * x, axis=-1)
        assert np.allclose(np.sum(y * y, axis=-1), s / (s + eps), rtol=1e-14, atol=0)
        cos = np.sum(x * y, axis=-1) / np.sqrt(s * np.sum(y * y, axis=-1))
        assert np.allclose(cos, 1.0, rtol=0, atol=1e-14)


def pin_l2norm_scale_invariance(lib):
    """With normalisation the layer sees only the directions of q and k:
    rescaling every row by a positive factor changes nothing but the eps
    guard's share, at most ~eps / |x|^2."""
    d = _rand(21, 2, 40, 2, 8, 5, decay="channel", h0_std=0.2)
    rng = np.random.default_rng(3)
    cq = rng.uniform(0.5, 4.0, d["q"].shape[:3])[..., None]
    ck = rng.uniform(0.5, 4.0, d["k"].shape[:3])[..., None]
    o1, h1 = _fwd(lib, d, qk_l2norm=True)
    d2 = dict(d, q=d["q"] * cq, k=d["k"] * ck)
    o2, h2 = _fwd(lib, d2, qk_l2norm=True)
    assert rel_err(o2, o1) < 1e-5 and rel_err(h2, h1) < 1e-5


def pin_l2norm_gradient_orthogonal(lib):
    """The loss depends on q only through q/|q|, so its gradient has no
    component along q (up to eps / |q|^2): dq . q ~ 0 for every row."""
    d = _rand(23, 1, 30, 2, 8, 6, decay="head", grads=True)
    gr = oracle.backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["meta"]["scale"], d["dO"],
                         dhT=d["dhT"], lib=lib, qk_l2norm=True)
    for x, dx in ((d["q"], gr["dq"]), (d["k"], gr["dk"])):
        along = np.abs(np.sum(x * dx, axis=-1)) / (np.linalg.norm(x, axis=-1) * np.linalg.norm(dx, axis=-1) + 1e-300)
        assert float(np.max(along)) < 1e-5


def _loss_l2(lib, d, dO, dhT):
    o, hT = _fwd(lib, d, qk_l2norm=True)
    return float(np.sum(o * dO) + np.sum(hT * dhT))


def pin_l2norm_fd(lib, seeds=(0, 1), h=1e-6, tol=1e-6):
    """Central finite differences of the loss with respect to the raw q and k
    against the backward's dq, dk through the normalisation."""
    for seed in seeds:
        d = _rand(140 + seed, 1, 7, 1, 4, 3, decay="channel", h0_std=0.5, grads=True)
        dO, dhT = d["dO"], d["dhT"]
        gr = oracle.backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["meta"]["scale"], dO,
                             h0=d["h0"], dhT=dhT, lib=lib, qk_l2norm=True)
        for nm, gn in (("q", "dq"), ("k", "dk")):
            x = d[nm]
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                x0 = x[idx]
                x[idx] = x0 + h; lp = _loss_l2(lib, d, dO, dhT)
                x[idx] = x0 - h; lm = _loss_l2(lib, d, dO, dhT)
                x[idx] = x0
                num[idx] = (lp - lm) / (2 * h)
            err = rel_err(gr[gn], num)
            assert err <= tol, (seed, nm, err)


FORWARD_PINS = [pin_worked_example, pin_beta_zero, pin_identity, pin_rewrite, pin_chunk_split,
                pin_pairwise, pin_scalar, pin_onehot, pin_wipe, pin_determinism,
                pin_l2norm_rows, pin_l2norm_scale_invariance, pin_l2norm_gradient_orthogonal]
ALL_PINS = FORWARD_PINS + [pin_fd_gradients, pin_l2norm_fd]
