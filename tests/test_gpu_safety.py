"""The numerical-safety options of the chunked calls on the GPU (wy_eps damping
of the WY solve, clip + nan_to_num at the stage boundaries, per-stage counts of
non-finite and large values) against the chunked float64 oracle with the same
options (oracle/chunked.py, pinned to the token-serial oracle and to closed
forms)."""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
from oracle import chunked
from gpu_util import TOL, host, log, rel_err, to_dev_inputs

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def run(inp, *, grads=True, **opts):
    import gated_delta_rule_52_amd as gdn
    d = to_dev_inputs(inp)
    m = inp["meta"]
    kw = dict(scale=m["scale"], chunk=m["chunk"], **opts)
    sh = gdn.make_shape(d["q"], d["v"], d["g"], m["scale"], m["chunk"],
                        wy_eps=opts.get("wy_eps", 0.0), clip=opts.get("clip", 0.0),
                        diag=opts.get("diag", False))
    ws = gdn.workspace(sh, True, d["q"].device)
    o, hT, ws = gdn.gdn_forward_train(d["q"], d["k"], d["v"], d["g"], d["beta"], d.get("h0"),
                                      ws=ws, **kw)
    out = {"o": o, "hT": hT}
    if opts.get("diag"):
        out["counts"] = gdn.gdn_diag_read(sh, ws)
    if grads:
        g = gdn.gdn_backward_train(d["q"], d["k"], d["v"], d["g"], d["beta"], d["dO"], ws,
                                   d.get("dhT"), **kw)
        out.update(zip(NAMES, g))
    torch.cuda.synchronize()
    return out


def compare(got, inp, tol, label, grads=True, **opts):
    o_ref, h_ref = chunked.forward_inputs(inp, **opts)
    errs = {"o": rel_err(host(got["o"]), o_ref), "hT": rel_err(host(got["hT"]), h_ref)}
    if grads:
        ref = chunked.backward_inputs(inp, **opts)
        errs.update({k: rel_err(host(got[k]), ref[k]) for k in NAMES})
    log(f"  {label}: " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, bad


def make(B, T, H, D, *, decay="channel", dtype="f32", seed=0, chunk=64):
    inp = gi.make_inputs(B, T, H, D, D, decay=decay, dtype=dtype, seed=seed, h0_std=0.2,
                         grads=True)
    inp["meta"]["chunk"] = chunk
    return inp


@pytest.mark.parametrize("seed", range(2))
def test_damped_chunk16(seed):
    inp = make(1, 70, 2, 16, seed=seed, chunk=16)
    compare(run(inp, wy_eps=0.3), inp, TOL["f32"], f"damped chunk16 seed={seed}", wy_eps=0.3)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("decay", ["channel", "head"])
@pytest.mark.parametrize("D", [64, 128])
def test_damped(dtype, decay, D):
    inp = make(2, 150, 2, D, decay=decay, dtype=dtype, seed=3)
    compare(run(inp, wy_eps=0.25), inp, TOL[dtype], f"damped {dtype} {decay} D={D}", wy_eps=0.25)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_eps_and_unreached_clip_change_nothing(dtype):
    """wy_eps = 0 multiplies by exactly 1, and a bound no value reaches is the
    identity: bitwise the plain results."""
    inp = make(2, 100, 2, 128, dtype=dtype, seed=4)
    a = run(inp)
    b = run(inp, wy_eps=0.0, clip=1e30)
    for k in ("o", "hT") + NAMES:
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("dtype,D,chunk", [("f32", 16, 16), ("f32", 64, 64), ("bf16", 128, 64)])
def test_clip_engaged(dtype, D, chunk):
    """Values beyond the bound: a few tokens' v scaled by 1e3, clip 64 (exact
    in bf16); outputs and gradients against the oracle with the same clipping."""
    inp = make(1, 90, 2, D, dtype=dtype, seed=6, chunk=chunk)
    v = inp["v"]
    if dtype == "bf16":
        f = gi.bf16_bits_to_f32(v)
        f[0, [5, 40, 77]] *= 1e3
        inp["v"] = gi.f32_to_bf16_bits(f.astype(np.float32))
    else:
        v[0, [5, 40, 77]] *= 1e3
    opts = dict(wy_eps=0.1, clip=64.0)
    got = run(inp, **opts)
    assert float(got["o"].abs().max()) <= 64.0 and float(got["hT"].abs().max()) <= 64.0
    compare(got, inp, TOL[dtype], f"clip {dtype} D={D}", **opts)


@pytest.mark.parametrize("dtype,D,chunk", [("f32", 16, 16), ("f32", 128, 64), ("bf16", 128, 64)])
def test_nan_query_cleaned(dtype, D, chunk):
    """A NaN in one query reaches only its own output row, which the clip
    cleans to 0; every other output and the state are bitwise the clean run's."""
    inp = make(1, 100, 2, D, dtype=dtype, seed=7, chunk=chunk)
    t, h = 70, 1
    bad = {k: (v.copy() if isinstance(v, np.ndarray) else dict(v)) for k, v in inp.items()}
    if dtype == "bf16":
        bad["q"][0, t, h, 3] = 0x7FC0  # bf16 NaN
    else:
        bad["q"][0, t, h, 3] = np.nan
    a = run(bad, grads=False, clip=100.0)
    b = run(inp, grads=False, clip=100.0)
    assert torch.all(a["o"][0, t, h] == 0)
    mask = torch.ones_like(a["o"], dtype=torch.bool)
    mask[0, t, h] = False
    assert torch.equal(a["o"][mask], b["o"][mask]) and torch.equal(a["hT"], b["hT"])


def _poison(inp, dtype, nan_at=None, huge_at=None):
    if dtype == "bf16":
        if nan_at:
            inp["q"][nan_at] = 0x7FC0  # bf16 NaN
        if huge_at:
            f = gi.bf16_bits_to_f32(inp["v"])
            f[huge_at] *= 1e8
            inp["v"] = gi.f32_to_bf16_bits(f.astype(np.float32))
    else:
        if nan_at:
            inp["q"][nan_at] = np.nan
        if huge_at:
            inp["v"][huge_at] *= 1e8


def _check_counts(inp, dtype, D, label, exact):
    for clip in (0.0, 50.0):
        got = run(inp, grads=False, diag=True, clip=clip)
        *_, ref = chunked.forward_inputs(inp, diag=True, clip=clip)
        log(f"  counts {label} {dtype} D={D} clip={clip}: {got['counts']}")
        if exact:
            assert got["counts"] == ref, (got["counts"], ref)
        else:
            # bf16 operands move values by ~1%: an entry within that of the
            # 1e6 threshold may land on either side
            for st, (nf, big) in ref.items():
                gnf, gbig = got["counts"][st]
                assert gnf == nf and abs(gbig - big) <= max(2, 0.01 * big), (st, got["counts"], ref)
        plain = run(inp, grads=False, clip=clip)
        assert torch.equal(torch.nan_to_num(got["o"]), torch.nan_to_num(plain["o"]))
        assert torch.equal(torch.nan_to_num(got["hT"]), torch.nan_to_num(plain["hT"]))


@pytest.mark.parametrize("dtype,D,chunk", [("f32", 16, 16), ("f32", 128, 64), ("bf16", 128, 64)])
def test_diag_counts_nan_query(dtype, D, chunk):
    """A NaN query: row t of P at the keys j <= t of its chunk and o_t are
    non-finite, nothing else; with and without clipping (counted before it),
    the counts equal the oracle's and change no value."""
    inp = make(1, 100, 2, D, dtype=dtype, seed=8, chunk=chunk)
    _poison(inp, dtype, nan_at=(0, 70, 0, 0))
    _check_counts(inp, dtype, D, "nan", exact=True)


@pytest.mark.parametrize("dtype,D,chunk", [("f32", 16, 16), ("f32", 128, 64), ("bf16", 128, 64)])
def test_diag_counts_large(dtype, D, chunk):
    """One token's v times 1e8: U, o and hT hold values above 1e6."""
    inp = make(1, 100, 2, D, dtype=dtype, seed=8, chunk=chunk)
    _poison(inp, dtype, huge_at=(0, 20, 1))
    _check_counts(inp, dtype, D, "large", exact=dtype == "f32")


@pytest.mark.parametrize("decay", ["channel", "head"])
def test_training_pair_equals_separate_calls(decay):
    import gated_delta_rule_52_amd as gdn
    inp = make(2, 130, 2, 128, decay=decay, dtype="bf16", seed=9)
    d = to_dev_inputs(inp)
    kw = dict(scale=inp["meta"]["scale"], wy_eps=0.2, clip=32.0)
    o1, h1 = gdn.gdn_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], **kw)
    g1 = gdn.gdn_backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["dO"], d["h0"], d["dhT"], **kw)
    o2, h2, ws = gdn.gdn_forward_train(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], **kw)
    g2 = gdn.gdn_backward_train(d["q"], d["k"], d["v"], d["g"], d["beta"], d["dO"], ws, d["dhT"],
                                **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
