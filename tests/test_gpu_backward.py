"""Chunked backward on the GPU against the oracle's token-serial reverse pass
(which is itself pinned to central finite differences)."""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from gpu_util import TOL, host, log, rel_err, to_dev_inputs
from test_gpu_forward import gpu_forward, sub_heads

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def gpu_backward(inp, chunk=None, h0=True, dhT=True):
    import gated_delta_rule_52_amd as gdn
    d = to_dev_inputs(inp)
    m = inp["meta"]
    out = gdn.gdn_backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["dO"],
                           h0=d.get("h0") if h0 else None, dhT=d.get("dhT") if dhT else None,
                           scale=m["scale"], chunk=chunk or m.get("chunk"))
    torch.cuda.synchronize()
    return dict(zip(NAMES, out))


def compare(got, ref, tol, label):
    errs = {k: rel_err(host(got[k]), ref[k]) for k in NAMES if got[k] is not None}
    log(f"  {label}: " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, bad


@pytest.mark.parametrize("seed", range(5))
def test_tiny_gradients(seed):
    """B=1 T=64 H=2 16x16, chunk 16, fp32, with h0 and dhT."""
    inp = gi.make_inputs(1, 64, 2, 16, 16, decay="channel", seed=seed, h0_std=0.3, grads=True)
    inp["meta"]["chunk"] = 16
    got = gpu_backward(inp)
    ref = oracle.backward_inputs(inp)
    compare(got, ref, TOL["f32"], f"tiny seed={seed}")


@pytest.mark.parametrize("chunk", [16, 64])
@pytest.mark.parametrize("T", [1, 37, 64, 100])
def test_ragged_gradients(chunk, T):
    D = 16 if chunk == 16 else 64
    inp = gi.make_inputs(2, T, 2, D, D, decay="channel", seed=40 + T, h0_std=0.2, grads=True)
    got = gpu_backward(inp, chunk=chunk)
    ref = oracle.backward_inputs(inp)
    compare(got, ref, TOL["f32"], f"ragged T={T} chunk={chunk}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("decay", ["channel", "head"])
@pytest.mark.parametrize("D", [64, 128])
def test_medium_gradients(dtype, decay, D):
    inp = gi.make_inputs(2, 320, 3, D, D, decay=decay, dtype=dtype, seed=17, h0_std=0.1,
                         grads=True)
    inp["meta"]["chunk"] = 64
    got = gpu_backward(inp)
    ref = oracle.backward_inputs(inp)
    compare(got, ref, TOL[dtype], f"medium {dtype} {decay} D={D}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("decay", ["channel", "head"])
def test_weak_decay_gradients(dtype, decay):
    """Decay a hundred times weaker than the default draw (a chunk keeps about
    e^-0.5 of its start state instead of e^-50), so the state carried across
    chunks, the saved chunk-start states and the whole-chunk decay gradient
    weigh in every output and gradient."""
    log(f"weak decay {dtype} {decay}")
    inp = gi.make_inputs(2, 512, 3, 128, 128, decay=decay, dtype=dtype, seed=23, h0_std=0.1,
                         grads=True, g_scale=0.01)
    inp["meta"]["chunk"] = 64
    o, hT = gpu_forward(inp)
    o_ref, h_ref = oracle.forward_inputs(inp)
    eo, eh = rel_err(host(o), o_ref), rel_err(host(hT), h_ref)
    log(f"  forward: o {eo:.2e}  hT {eh:.2e}")
    assert eo <= TOL[dtype] and eh <= TOL[dtype]
    got = gpu_backward(inp)
    ref = oracle.backward_inputs(inp)
    compare(got, ref, TOL[dtype], f"weak decay {dtype} {decay}")


@pytest.mark.parametrize("decay,D", [("channel", 128), ("head", 128), ("channel", 64)])
def test_more_chunk_heads_than_workgroups(decay, D):
    """B=3 T=1000 H=6: 288 chunk-heads (more than the chip has CUs) with a
    ragged last chunk, so the persistent backward kernel takes several
    chunk-heads per workgroup, loading each next one during the tail of the
    one before; weak decay lets the chunk-start states weigh in.  At 64x64
    the Dv loop is one prefetching tile and the last."""
    log(f"more chunk-heads than workgroups, bf16 {decay} D={D}")
    inp = gi.make_inputs(3, 1000, 6, D, D, decay=decay, dtype="bf16", seed=37, h0_std=0.1,
                         grads=True, g_scale=0.01)
    inp["meta"]["chunk"] = 64
    got = gpu_backward(inp)
    ref = oracle.backward_inputs(inp)
    compare(got, ref, TOL["bf16"], f"many chunk-heads {decay} D={D}")


def test_no_h0_no_dhT():
    inp = gi.make_inputs(2, 130, 2, 64, 64, decay="channel", seed=3, grads=True)
    inp.pop("dhT")
    got = gpu_backward(inp, h0=False, dhT=False)
    ref = oracle.backward_inputs(inp)
    compare(got, ref, TOL["f32"], "no h0 / dhT")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_training_shape_gradients_sampled(dtype):
    """B=8 T=4096 H=6 128x128 per-channel; dO ~ N(0,1) in the input dtype,
    dhT ~ N(0, 0.01); oracle reverse pass on sampled heads."""
    log(f"training-shape backward {dtype}")
    inp = gi.train(dtype=dtype, grads=True)
    got = gpu_backward(inp, h0=False)
    pairs = [(0, 0), (7, 5), (3, 2)]
    s = sub_heads(inp, pairs)
    ref = oracle.backward(s["q"], s["k"], s["v"], s["g"], s["beta"], inp["meta"]["scale"], s["dO"],
                          dhT=s["dhT"])
    sel = {}
    for name in NAMES:
        x = got[name]
        if name == "dh0":
            sel[name] = torch.stack([x[b, h] for b, h in pairs])[None]
        else:
            sel[name] = torch.stack([x[b, :, h] for b, h in pairs], dim=1)[None]
    compare(sel, ref, TOL[dtype], f"train {dtype} sampled")


def test_backward_deterministic():
    inp = gi.make_inputs(2, 200, 3, 128, 128, decay="channel", dtype="bf16", seed=8, grads=True)
    a = gpu_backward(inp, h0=False)
    b = gpu_backward(inp, h0=False)
    for k in NAMES:
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("decay", ["channel", "head"])
def test_training_pair_equals_separate_calls(dtype, decay):
    """gdn_forward_train + gdn_backward_train (residuals kept) give bitwise the
    same outputs and gradients as gdn_forward + gdn_backward (recompute)."""
    import gated_delta_rule_52_amd as gdn
    inp = gi.make_inputs(2, 200, 3, 128, 128, decay=decay, dtype=dtype, seed=21, h0_std=0.1,
                         grads=True)
    d = to_dev_inputs(inp)
    sc = inp["meta"]["scale"]
    o1, h1 = gdn.gdn_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], scale=sc)
    g1 = gdn.gdn_backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["dO"], d["h0"], d["dhT"],
                          scale=sc)
    o2, h2, ws = gdn.gdn_forward_train(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], scale=sc)
    g2 = gdn.gdn_backward_train(d["q"], d["k"], d["v"], d["g"], d["beta"], d["dO"], ws, d["dhT"],
                                scale=sc)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("decay", ["channel", "head"])
def test_long_state_carry_training_shape(dtype, decay):
    """B=8 T=4096 H=6 128x128 (the training shape) with a decay a hundred times
    weaker than the default draw: each 64-token chunk keeps about e^-0.5 of its
    start state, so the state is carried through all 64 chunks (the gated-deltanet
    card, Requirements: the state is a long chain of products) and the saved
    chunk-start states, chunk deltas and state gradients weigh in every result.
    h0 ~ N(0, 0.1).
    gdn_forward, and the training pair gdn_forward_train + gdn_backward_train,
    against the oracle on sampled heads: o, hT and all six gradients."""
    import gated_delta_rule_52_amd as gdn
    log(f"long state carry, training shape, {dtype} {decay}")
    inp = gi.make_inputs(8, 4096, 6, 128, 128, decay=decay, dtype=dtype, seed=29, h0_std=0.1,
                         grads=True, g_scale=0.01)
    d = to_dev_inputs(inp)
    sc = inp["meta"]["scale"]
    o1, h1 = gdn.gdn_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], scale=sc)
    o2, h2, ws = gdn.gdn_forward_train(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], scale=sc)
    grads = gdn.gdn_backward_train(d["q"], d["k"], d["v"], d["g"], d["beta"], d["dO"], ws, d["dhT"],
                                   scale=sc)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    pairs = [(0, 0), (7, 5), (3, 2), (5, 1)]
    s = sub_heads(inp, pairs)
    o_ref, h_ref = oracle.forward(s["q"], s["k"], s["v"], s["g"], s["beta"], sc, h0=s["h0"])
    ref = oracle.backward(s["q"], s["k"], s["v"], s["g"], s["beta"], sc, s["dO"], h0=s["h0"],
                          dhT=s["dhT"])
    eo = rel_err(np.stack([host(o1[b, :, h]) for b, h in pairs], axis=1)[None], o_ref)
    eh = rel_err(np.stack([host(h1[b, h]) for b, h in pairs])[None], h_ref)
    log(f"  forward: o {eo:.2e}  hT {eh:.2e}")
    assert eo <= TOL[dtype] and eh <= TOL[dtype]
    sel = {}
    for name, x in zip(NAMES, grads):
        if name == "dh0":
            sel[name] = torch.stack([x[b, h] for b, h in pairs])[None]
        else:
            sel[name] = torch.stack([x[b, :, h] for b, h in pairs], dim=1)[None]
    compare(sel, ref, TOL[dtype], f"long carry {dtype} {decay}")
