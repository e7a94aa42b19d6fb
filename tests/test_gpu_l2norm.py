"""use_qk_l2norm on the GPU (the q/k L2-normalisation prologue and its
adjoint, fused into the chunked kernels and the decode step) against the
oracle, which normalises in float64 before its token-serial loop and maps the
gradients back through the normalisation.  Inputs are raw q, k rows with
log-normal lengths (gdn_inputs qk_scale)."""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from gpu_util import TOL, dev, host, log, rel_err, to_dev_inputs
from test_gpu_forward import sub_heads

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def raw(B, T, H, D, *, decay="channel", dtype="f32", seed=0, chunk=64, h0_std=0.1, grads=False,
        qk_scale=1.0):
    inp = gi.make_inputs(B, T, H, D, D, decay=decay, dtype=dtype, seed=seed, h0_std=h0_std,
                         grads=grads, qk_scale=qk_scale)
    inp["meta"]["chunk"] = chunk
    return inp


def gpu_forward(inp):
    import gated_delta_rule_52_amd as gdn
    d = to_dev_inputs(inp)
    m = inp["meta"]
    o, hT = gdn.gdn_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d.get("h0"),
                            scale=m["scale"], chunk=m["chunk"], use_qk_l2norm=True)
    torch.cuda.synchronize()
    return o, hT


def gpu_backward(inp):
    import gated_delta_rule_52_amd as gdn
    d = to_dev_inputs(inp)
    m = inp["meta"]
    out = gdn.gdn_backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["dO"], d.get("h0"),
                           d.get("dhT"), scale=m["scale"], chunk=m["chunk"], use_qk_l2norm=True)
    torch.cuda.synchronize()
    return dict(zip(NAMES, out))


def check_forward(inp, tol, label):
    o, hT = gpu_forward(inp)
    o_ref, h_ref = oracle.forward_inputs(inp)
    eo, eh = rel_err(host(o), o_ref), rel_err(host(hT), h_ref)
    log(f"  {label}: o {eo:.2e}  hT {eh:.2e}")
    assert eo <= tol and eh <= tol, (eo, eh)


def check_backward(inp, tol, label):
    got = gpu_backward(inp)
    ref = oracle.backward_inputs(inp)
    errs = {k: rel_err(host(got[k]), ref[k]) for k in NAMES if got[k] is not None}
    log(f"  {label}: " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, bad


@pytest.mark.parametrize("seed", range(3))
def test_tiny_chunk16(seed):
    """B=1 T=64 H=2 16x16, chunk 16, fp32: forward and gradients."""
    inp = raw(1, 64, 2, 16, seed=seed, chunk=16, grads=True)
    check_forward(inp, TOL["f32"], f"tiny seed={seed} fwd")
    check_backward(inp, TOL["f32"], f"tiny seed={seed} bwd")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("decay", ["channel", "head"])
@pytest.mark.parametrize("D", [64, 128])
def test_medium(dtype, decay, D):
    """B=2 T=200 H=3 (several chunks and a ragged tail), chunk 64."""
    inp = raw(2, 200, 3, D, decay=decay, dtype=dtype, seed=31, grads=True)
    check_forward(inp, TOL[dtype], f"medium {dtype} {decay} D={D} fwd")
    check_backward(inp, TOL[dtype], f"medium {dtype} {decay} D={D} bwd")


@pytest.mark.parametrize("T", [1, 63, 65])
def test_ragged_bf16(T):
    inp = raw(2, T, 2, 128, dtype="bf16", seed=50 + T, grads=True)
    check_forward(inp, TOL["bf16"], f"ragged T={T} fwd")
    check_backward(inp, TOL["bf16"], f"ragged T={T} bwd")


def test_zero_rows():
    """All-zero q and k rows: x_hat = 0 there, and the gradient is r dx_hat
    with r = 1/sqrt(eps) (the degenerate case the guard exists for)."""
    inp = raw(1, 70, 2, 64, seed=4, grads=True)
    for name in ("q", "k"):
        inp[name][0, 5] = 0.0
        inp[name][0, 66, 1] = 0.0
    check_forward(inp, TOL["f32"], "zero rows fwd")
    check_backward(inp, TOL["f32"], "zero rows bwd")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_normalised_inputs_match_plain_path(dtype):
    """On rows that already have unit length the option changes each row by
    the factor 1/sqrt(1 + eps) only: outputs agree with the plain path."""
    import gated_delta_rule_52_amd as gdn
    inp = gi.make_inputs(2, 130, 2, 128, 128, dtype=dtype, seed=12, h0_std=0.1)
    d = to_dev_inputs(inp)
    sc = inp["meta"]["scale"]
    o1, h1 = gdn.gdn_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], scale=sc)
    o2, h2 = gdn.gdn_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], scale=sc,
                             use_qk_l2norm=True)
    torch.cuda.synchronize()
    tol = 1e-5 if dtype == "f32" else 2e-2
    assert rel_err(host(o2), host(o1)) <= tol and rel_err(host(h2), host(h1)) <= tol


@pytest.mark.parametrize("decay", ["channel", "head"])
def test_training_pair_equals_separate_calls(decay):
    """gdn_forward_train + gdn_backward_train with the option give bitwise the
    same results as gdn_forward + gdn_backward with it."""
    import gated_delta_rule_52_amd as gdn
    inp = raw(2, 200, 3, 128, decay=decay, dtype="bf16", seed=22, grads=True)
    d = to_dev_inputs(inp)
    sc = inp["meta"]["scale"]
    kw = dict(scale=sc, use_qk_l2norm=True)
    o1, h1 = gdn.gdn_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], **kw)
    g1 = gdn.gdn_backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["dO"], d["h0"], d["dhT"],
                          **kw)
    o2, h2, ws = gdn.gdn_forward_train(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], **kw)
    g2 = gdn.gdn_backward_train(d["q"], d["k"], d["v"], d["g"], d["beta"], d["dO"], ws, d["dhT"],
                                **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_deterministic():
    inp = raw(2, 200, 3, 128, dtype="bf16", seed=9, grads=True)
    a = gpu_backward(inp)
    b = gpu_backward(inp)
    for k in NAMES:
        assert torch.equal(a[k], b[k]), k


def test_training_shape_sampled():
    """B=8 T=4096 H=6 128x128 bf16, per-channel decay, raw q, k: forward and
    gradients of three sampled heads against the oracle."""
    import gated_delta_rule_52_amd as gdn
    log("training-shape use_qk_l2norm bf16")
    inp = gi.train(dtype="bf16", grads=True, qk_scale=1.0)
    d = to_dev_inputs(inp)
    sc = inp["meta"]["scale"]
    o, hT, ws = gdn.gdn_forward_train(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=sc,
                                      use_qk_l2norm=True)
    grads = gdn.gdn_backward_train(d["q"], d["k"], d["v"], d["g"], d["beta"], d["dO"], ws,
                                   d["dhT"], scale=sc, use_qk_l2norm=True)
    torch.cuda.synchronize()
    pairs = [(0, 0), (7, 5), (3, 2)]
    s = sub_heads(inp, pairs)
    o_ref, h_ref = oracle.forward(s["q"], s["k"], s["v"], s["g"], s["beta"], sc, qk_l2norm=True)
    ref = oracle.backward(s["q"], s["k"], s["v"], s["g"], s["beta"], sc, s["dO"], dhT=s["dhT"],
                          qk_l2norm=True)
    o_gpu = np.stack([host(o[b, :, h]) for b, h in pairs], axis=1)[None]
    h_gpu = np.stack([host(hT[b, h]) for b, h in pairs])[None]
    errs = {"o": rel_err(o_gpu, o_ref), "hT": rel_err(h_gpu, h_ref)}
    for name, x in zip(NAMES, grads):
        if name == "dh0":
            sel = np.stack([host(x[b, h]) for b, h in pairs])[None]
        else:
            sel = np.stack([host(x[b, :, h]) for b, h in pairs], axis=1)[None]
        errs[name] = rel_err(sel, ref[name])
    log("  " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= TOL["bf16"]}
    assert not bad, bad


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("decay", ["channel", "head"])
@pytest.mark.parametrize("D", [16, 128])
def test_decode_steps(dtype, decay, D):
    """Token-by-token decode with the option equals the oracle's normalised
    forward over the same tokens, state included."""
    import gated_delta_rule_52_amd as gdn
    inp = gi.make_inputs(3, 12, 4, D, D, decay=decay, dtype=dtype, seed=5, h0_std=0.1,
                         qk_scale=1.0)
    d = to_dev_inputs(inp)
    sc = inp["meta"]["scale"]
    state = d["h0"].clone()
    outs = []
    for t in range(inp["meta"]["T"]):
        sl = lambda x: x[:, t:t + 1].contiguous()
        outs.append(gdn.gdn_decode_step(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["g"]),
                                        sl(d["beta"]), state, scale=sc, use_qk_l2norm=True))
    o = torch.cat(outs, dim=1)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle.forward_inputs(inp)
    eo, eh = rel_err(host(o), o_ref), rel_err(host(state), h_ref)
    log(f"  decode {dtype} {decay} D={D}: o {eo:.2e}  state {eh:.2e}")
    assert eo <= TOL[dtype] and eh <= TOL[dtype], (eo, eh)
