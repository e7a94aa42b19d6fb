"""Pins of the chunked oracle and its numerical-safety options (wy_eps damping,
clip, stage diagnostics; atomic_ops card, "Features" and "Debugging").  Each
pin takes the module under test, so planted mistakes in a copy of it can be
shown to fail at least one of them.

What fixes the expected values:
  * wy_eps = 0, no clip: the token recurrence, i.e. the token-serial oracle
    (itself pinned by tests/pins.py);
  * chunks of one token, or keys orthogonal inside each chunk with one decay
    per head: the block matrix A vanishes, the damped solve is 1 / (1 + wy_eps)
    and the layer equals the token recurrence with beta / (1 + wy_eps);
  * one token from a zero state: every stage has a closed form
    (P = q.k, T = 1 / (1 + eps), U = beta v / (1 + eps), o = scale P U,
    hT = k U^T), so clipping and the counts can be written down;
  * a query only reaches its own output row: a NaN in q_t leaves every other
    output as it was and o_t, cleaned, is 0;
  * gradients: central differences of the forward.
"""
from __future__ import annotations

import numpy as np

import gdn_inputs as gi
import oracle


def rel_err(x, y):
    den = float(np.max(np.abs(y)))
    return float(np.max(np.abs(np.asarray(x) - np.asarray(y)))) / (den if den else 1.0)


def _inp(B, T, H, Dk, Dv, decay, seed, h0_std=0.3, grads=True, chunk=16):
    d = gi.make_inputs(B, T, H, Dk, Dv, decay=decay, seed=seed, h0_std=h0_std, grads=grads)
    d["meta"]["chunk"] = chunk
    return gi.f64_inputs(d)


def pin_equals_token_serial(ch):
    """wy_eps = 0 and no clip: the chunked form is the token recurrence, for any
    chunk size, ragged tails, both decay modes, with and without h0 and L2 norm."""
    for decay, C, T, h0, l2 in (("channel", 1, 9, 0.3, False), ("channel", 4, 37, 0.3, False),
                                ("channel", 16, 40, None, False), ("head", 8, 37, 0.3, False),
                                ("head", 16, 16, 0.3, True)):
        d = _inp(2, T, 2, 8, 6, decay, seed=C + T, h0_std=h0)
        kw = dict(qk_l2norm=l2)
        o1, h1 = ch.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["meta"]["scale"],
                            d.get("h0"), chunk=C, **kw)
        o2, h2 = oracle.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["meta"]["scale"],
                                d.get("h0"), **kw)
        assert rel_err(o1, o2) < 1e-12 and rel_err(h1, h2) < 1e-12, (decay, C, T)
        g1 = ch.backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["meta"]["scale"], d["dO"],
                         d.get("h0"), d["dhT"], chunk=C, **kw)
        g2 = oracle.backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["meta"]["scale"],
                             d["dO"], h0=d.get("h0"), dhT=d["dhT"], **kw)
        for name in g2:
            assert rel_err(g1[name], g2[name]) < 1e-11, (decay, C, T, name)


def _check_scaled_beta(ch, d, C, eps, grads_to_check):
    sc = d["meta"]["scale"]
    o1, h1 = ch.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], sc, d["h0"], chunk=C,
                        wy_eps=eps)
    b2 = d["beta"] / (1.0 + eps)
    o2, h2 = oracle.forward(d["q"], d["k"], d["v"], d["g"], b2, sc, d["h0"])
    assert rel_err(o1, o2) < 1e-12 and rel_err(h1, h2) < 1e-12
    g1 = ch.backward(d["q"], d["k"], d["v"], d["g"], d["beta"], sc, d["dO"], d["h0"], d["dhT"],
                     chunk=C, wy_eps=eps)
    g2 = oracle.backward(d["q"], d["k"], d["v"], d["g"], b2, sc, d["dO"], h0=d["h0"],
                         dhT=d["dhT"])
    g2["dbeta"] = g2["dbeta"] / (1.0 + eps)  # chain rule through beta / (1 + eps)
    for name in grads_to_check:
        assert rel_err(g1[name], g2[name]) < 1e-11, name


def pin_damping_single_token_chunks(ch):
    """Chunks of one token: A = 0, so the damped layer is the recurrence with
    beta / (1 + eps), whatever the keys and decays."""
    d = _inp(1, 11, 2, 8, 5, "channel", seed=5)
    _check_scaled_beta(ch, d, 1, 0.37, ("dq", "dk", "dv", "dg", "dbeta", "dh0"))


def pin_damping_orthogonal_keys(ch):
    """Keys orthogonal inside each chunk and one decay per head: A = 0 inside
    every chunk, so again the recurrence with beta / (1 + eps).  (Perturbing k
    breaks the orthogonality, so dk is not compared.)"""
    C, Dk = 8, 8
    d = _inp(1, 3 * C, 2, Dk, 5, "head", seed=6)
    rng = np.random.default_rng(11)
    for n in range(3):
        for h in range(2):
            Qm, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
            d["k"][0, n * C:(n + 1) * C, h] = Qm[:C]
    _check_scaled_beta(ch, d, C, 0.25, ("dq", "dv", "dg", "dbeta", "dh0"))


def pin_damping_changes_values(ch):
    """Damping is not the identity when keys interact (guards a dropped eps)."""
    d = _inp(1, 16, 1, 8, 4, "channel", seed=7)
    sc = d["meta"]["scale"]
    o0, _ = ch.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], sc, d["h0"], chunk=16)
    o1, _ = ch.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], sc, d["h0"], chunk=16, wy_eps=0.5)
    assert rel_err(o1, o0) > 1e-3


def _one_token(seed, vscale=1.0):
    rng = np.random.default_rng(seed)
    Dk, Dv = 6, 5
    q = rng.standard_normal((1, 1, 1, Dk))
    k = rng.standard_normal((1, 1, 1, Dk)) / np.sqrt(Dk)
    v = rng.standard_normal((1, 1, 1, Dv)) * vscale
    g = -np.abs(rng.standard_normal((1, 1, 1, Dk)))
    beta = np.array([[[0.7]]])
    return q, k, v, g, beta


def pin_clip_single_token_closed_form(ch):
    """One token from a zero state, with v large enough that clipping engages at
    U and at the outputs: o = clip(scale * clip(q.k) * clip(beta v / (1 + eps))),
    hT = clip(k clip(beta v / (1 + eps))^T).  The decay of a lone token does not
    reach its own write."""
    q, k, v, g, beta = _one_token(1, vscale=50.0)
    eps, c, sc = 0.2, 3.0, 0.4
    cl = lambda x: np.clip(x, -c, c)
    U = cl(beta[0, 0, 0] * v[0, 0, 0] / (1 + eps))
    P = cl(float(q[0, 0, 0] @ k[0, 0, 0]))
    o_ref = cl(sc * P * U)
    h_ref = cl(np.outer(k[0, 0, 0], U))
    for C in (1, 4):
        o, hT = ch.forward(q, k, v, g, beta, sc, None, chunk=C, wy_eps=eps, clip=c)
        assert np.allclose(o[0, 0, 0], o_ref, rtol=0, atol=1e-14)
        assert np.allclose(hT[0, 0], h_ref, rtol=0, atol=1e-14)


def pin_clip_passthrough(ch):
    """A bound no value reaches changes nothing, bit for bit."""
    d = _inp(1, 20, 2, 8, 4, "channel", seed=8)
    sc = d["meta"]["scale"]
    a = ch.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], sc, d["h0"], chunk=8)
    b = ch.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], sc, d["h0"], chunk=8, clip=1e30)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def pin_clip_nan_query(ch):
    """A NaN in q_t reaches only o_t: cleaned to 0; every other output and the
    state are those of the run with a finite q_t."""
    d = _inp(1, 20, 2, 8, 4, "channel", seed=9)
    sc = d["meta"]["scale"]
    t, h = 13, 1
    qn = d["q"].copy()
    qn[0, t, h, 3] = np.nan
    o1, h1 = ch.forward(qn, d["k"], d["v"], d["g"], d["beta"], sc, d["h0"], chunk=8, clip=100.0)
    o0, h0 = ch.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], sc, d["h0"], chunk=8)
    assert np.all(o1[0, t, h] == 0.0)
    mask = np.ones(o0.shape, dtype=bool)
    mask[0, t, h] = False
    assert np.array_equal(o1[mask], o0[mask]) and np.array_equal(h1, h0)


def pin_diag_counts(ch):
    """Counts per stage: a NaN in q_t makes row t of P non-finite at the keys
    j <= t of its chunk and o_t non-finite in every value column; one token with
    a huge v makes U = beta v / (1 + eps) large where it exceeds 1e6, and the
    counts never change values."""
    d = _inp(1, 20, 2, 8, 4, "channel", seed=10)
    sc = d["meta"]["scale"]
    t, h, C = 13, 0, 8
    qn = d["q"].copy()
    qn[0, t, h, 0] = np.nan
    o, hT, cnt = ch.forward(qn, d["k"], d["v"], d["g"], d["beta"], sc, d["h0"], chunk=C,
                            diag=True)
    o2, h2 = ch.forward(qn, d["k"], d["v"], d["g"], d["beta"], sc, d["h0"], chunk=C)
    assert np.array_equal(np.nan_to_num(o), np.nan_to_num(o2)) and np.array_equal(hT, h2)
    exp = {s: (0, 0) for s in cnt}
    exp["P"] = (t % C + 1, 0)
    exp["o"] = (4, 0)
    assert cnt == exp, cnt
    # the counts are taken before clipping: the same with clip on
    *_, cnt_c = ch.forward(qn, d["k"], d["v"], d["g"], d["beta"], sc, d["h0"], chunk=C,
                           clip=100.0, diag=True)
    assert cnt_c == exp, cnt_c
    q, k, v, g, beta = _one_token(2, vscale=1e7)
    eps = 0.1
    U = beta[0, 0, 0] * v[0, 0, 0] / (1 + eps)
    *_, cnt = ch.forward(q, k, v, g, beta, 0.5, None, chunk=4, wy_eps=eps, diag=True)
    assert cnt["U"] == (0, int(np.sum(np.abs(U) > 1e6))), cnt
    assert cnt["T"] == (0, 0) and cnt["P"] == (0, 0)


def pin_damped_fd(ch, h=1e-6, tol=1e-6):
    """Central differences of the damped forward against its gradients."""
    d = _inp(1, 6, 1, 4, 3, "channel", seed=12, grads=True)
    sc, eps, C = d["meta"]["scale"], 0.4, 4
    gr = ch.backward(d["q"], d["k"], d["v"], d["g"], d["beta"], sc, d["dO"], d["h0"], d["dhT"],
                     chunk=C, wy_eps=eps)

    def loss():
        o, hT = ch.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], sc, d["h0"], chunk=C,
                           wy_eps=eps)
        return float(np.sum(o * d["dO"]) + np.sum(hT * d["dhT"]))

    for nm, gn in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"),
                   ("h0", "dh0")):
        x = d[nm]
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            x0 = x[idx]
            x[idx] = x0 + h; lp = loss()
            x[idx] = x0 - h; lm = loss()
            x[idx] = x0
            num[idx] = (lp - lm) / (2 * h)
        assert rel_err(gr[gn], num) <= tol, (nm, rel_err(gr[gn], num))


ALL_PINS = [pin_equals_token_serial, pin_damping_single_token_chunks, pin_damping_orthogonal_keys,
            pin_damping_changes_values, pin_clip_single_token_closed_form, pin_clip_passthrough,
            pin_clip_nan_query, pin_diag_counts, pin_damped_fd]
