"""Chunked forward on the GPU against the token-serial oracle."""
import math

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from gpu_util import TOL, dev, host, log, rel_err, to_dev_inputs

pytestmark = pytest.mark.gpu


def gpu_forward(inp, h0=True, chunk=None, **kw):
    import gated_delta_rule_52_amd as gdn
    d = to_dev_inputs(inp)
    m = inp["meta"]
    o, hT = gdn.gdn_forward(d["q"], d["k"], d["v"], d["g"], d["beta"],
                            d.get("h0") if h0 else None, scale=m["scale"],
                            chunk=chunk or m.get("chunk"), **kw)
    torch.cuda.synchronize()
    return o, hT


def sub_heads(inp, pairs):
    """The workload restricted to the given (b, h) pairs (oracle on a sample)."""
    out = {}
    for name, x in inp.items():
        if not isinstance(x, np.ndarray):
            continue
        if name in ("h0", "dhT"):
            out[name] = np.stack([x[b, h] for b, h in pairs])[None]
        else:
            out[name] = np.stack([x[b, :, h] for b, h in pairs], axis=1)[None]
    return out


def check_sampled(inp, o, hT, pairs, tol):
    s = sub_heads(inp, pairs)
    o_ref, h_ref = oracle.forward(s["q"], s["k"], s["v"], s["g"], s["beta"], inp["meta"]["scale"],
                                  h0=s.get("h0"))
    o_gpu = np.stack([host(o[b, :, h]) for b, h in pairs], axis=1)[None]
    h_gpu = np.stack([host(hT[b, h]) for b, h in pairs])[None]
    eo, eh = rel_err(o_gpu, o_ref), rel_err(h_gpu, h_ref)
    log(f"  sampled {len(pairs)} heads: o {eo:.3e}  hT {eh:.3e}")
    assert eo <= tol and eh <= tol, (eo, eh)


@pytest.mark.parametrize("seed", range(5))
def test_tiny_per_channel(seed):
    """B=1 T=64 H=2 16x16, chunk 16, fp32, zero state."""
    log(f"tiny seed={seed}")
    inp = gi.tiny(seed)
    o, hT = gpu_forward(inp)
    o_ref, h_ref = oracle.forward_inputs(inp)
    assert rel_err(host(o), o_ref) <= TOL["f32"], rel_err(host(o), o_ref)
    assert rel_err(host(hT), h_ref) <= TOL["f32"]


@pytest.mark.parametrize("chunk", [16, 64])
@pytest.mark.parametrize("T", [1, 15, 16, 37, 64, 100, 130])
def test_ragged_lengths(chunk, T):
    """Any T, with a ragged last chunk (identity padding)."""
    D = 16 if chunk == 16 else 64
    log(f"ragged T={T} chunk={chunk} D={D}")
    inp = gi.make_inputs(2, T, 3, D, D, decay="channel", seed=T, h0_std=0.3)
    o, hT = gpu_forward(inp, chunk=chunk)
    o_ref, h_ref = oracle.forward_inputs(inp)
    assert rel_err(host(o), o_ref) <= TOL["f32"]
    assert rel_err(host(hT), h_ref) <= TOL["f32"]


@pytest.mark.parametrize("T", [1, 63, 64, 65, 130, 200, 256])
def test_ragged_lengths_bf16(T):
    """bf16 tables at chunk 64: one, two, three and four chunks (odd and even
    counts), ragged and whole last chunks, from a random start state."""
    D = 128
    log(f"ragged bf16 T={T} D={D}")
    inp = gi.make_inputs(2, T, 3, D, D, decay="channel", dtype="bf16", seed=100 + T, h0_std=0.1)
    o, hT = gpu_forward(inp)
    o_ref, h_ref = oracle.forward_inputs(inp)
    eo, eh = rel_err(host(o), o_ref), rel_err(host(hT), h_ref)
    log(f"  o {eo:.3e} hT {eh:.3e}")
    assert eo <= TOL["bf16"] and eh <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("decay", ["channel", "head"])
@pytest.mark.parametrize("D", [64, 128])
def test_medium(dtype, decay, D):
    log(f"medium dtype={dtype} decay={decay} D={D}")
    inp = gi.make_inputs(2, 320, 3, D, D, decay=decay, dtype=dtype, seed=7, h0_std=0.1)
    o, hT = gpu_forward(inp)
    o_ref, h_ref = oracle.forward_inputs(inp)
    eo, eh = rel_err(host(o), o_ref), rel_err(host(hT), h_ref)
    log(f"  o {eo:.3e} hT {eh:.3e}")
    assert eo <= TOL[dtype] and eh <= TOL[dtype]


def test_worked_example_on_gpu():
    """The Marin note's worked example through the device path: key at
    cumulative log-decay -1 (token 30), boundary -2 (token 31, last token of
    the earlier 32-token block), queries at -3 and -4 (tokens 32, 33)."""
    import json, os
    ex = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                     "worked_decay_example.json")))
    T, D = 64, 64
    g = np.zeros((1, T, 1, D), np.float32)
    cum = ex["cumulative_log_decay"]
    g[0, 30, 0, 0] = cum["key"]
    g[0, 31, 0, 0] = cum["boundary"] - cum["key"]
    g[0, 32, 0, 0] = cum["queries"][0] - cum["boundary"]
    g[0, 33, 0, 0] = cum["queries"][1] - cum["queries"][0]
    q = np.zeros((1, T, 1, D), np.float32); k = q.copy(); v = q.copy()
    beta = np.zeros((1, T, 1), np.float32)
    k[0, 30, 0, 0] = v[0, 30, 0, 0] = beta[0, 30, 0] = 1.0
    q[0, 32, 0, 0] = q[0, 33, 0, 0] = 1.0
    import gated_delta_rule_52_amd as gdn
    o, hT = gdn.gdn_forward(dev(q), dev(k), dev(v), dev(g), dev(beta), scale=1.0, chunk=64)
    torch.cuda.synchronize()
    o = host(o)
    for i, t in enumerate((32, 33)):
        want = math.exp(ex["pair_factor_exponents"][i])
        assert abs(o[0, t, 0, 0] - want) <= 1e-6 * want, (t, o[0, t, 0, 0], want)


def test_head_wipe_and_split_calls():
    """Per-head decay, B=2 T=2048 H=8 128x128 fp32, wipes g=-20 at every 256th
    token, h0 ~ N(0, 0.1); also as 16 calls of 128 tokens carrying the state."""
    import gated_delta_rule_52_amd as gdn
    log("head-wipe B=2 T=2048 H=8")
    inp = gi.head_wipe()
    o, hT = gpu_forward(inp)
    o_ref, h_ref = oracle.forward_inputs(inp)
    eo, eh = rel_err(host(o), o_ref), rel_err(host(hT), h_ref)
    log(f"  one call: o {eo:.3e}  hT {eh:.3e}")
    assert eo <= TOL["f32"] and eh <= TOL["f32"]
    d = to_dev_inputs(inp)
    S = d["h0"].clone()
    outs = []
    for t0 in range(0, 2048, 128):
        sl = slice(t0, t0 + 128)
        o_c, _ = gdn.gdn_forward(d["q"][:, sl].contiguous(), d["k"][:, sl].contiguous(),
                                 d["v"][:, sl].contiguous(), d["g"][:, sl].contiguous(),
                                 d["beta"][:, sl].contiguous(), S, scale=inp["meta"]["scale"],
                                 hT=S)
        outs.append(o_c)
    torch.cuda.synchronize()
    o_split = torch.cat(outs, dim=1)
    same = torch.equal(o_split, o) and torch.equal(S, hT)
    log(f"  16x128 calls bitwise equal to one call: {same}")
    assert same


@pytest.mark.parametrize("dtype,B", [("bf16", 8), ("f32", 8), ("bf16", 4)])
def test_training_shape_sampled(dtype, B):
    """B=8 (and 4) T=4096 H=6 128x128 per-channel, zero state; sampled heads."""
    log(f"training shape dtype={dtype} B={B}")
    inp = gi.train(dtype=dtype, B=B)
    o, hT = gpu_forward(inp, h0=False)
    assert torch.isfinite(o.float()).all() and torch.isfinite(hT).all()
    pairs = [(0, 0), (B - 1, 5), (B // 2, 2)]
    check_sampled(inp, o, hT, pairs, TOL[dtype])


def test_gates_identity_bitwise():
    """g = 0 and beta = 0: the state passes through exactly (gated-deltanet card,
    Correctness), and beta = 0 alone leaves it decayed only."""
    inp = gi.make_inputs(2, 200, 3, 128, 128, decay="channel", seed=4, h0_std=1.0)
    inp["g"][:] = 0.0
    inp["beta"][:] = 0.0
    o, hT = gpu_forward(inp)
    assert np.array_equal(host(hT), inp["h0"].astype(np.float64))
    # short enough that the decayed state stays far above the fp32 range limit
    inp2 = gi.make_inputs(2, 20, 3, 128, 128, decay="channel", seed=4, h0_std=1.0)
    inp2["beta"][:] = 0.0
    o2, h2 = gpu_forward(inp2)
    o_ref, h_ref = oracle.forward_inputs(inp2)
    assert rel_err(host(h2), h_ref) <= TOL["f32"] and rel_err(host(o2), o_ref) <= TOL["f32"]


def test_forward_deterministic():
    inp = gi.make_inputs(2, 300, 6, 128, 128, decay="channel", dtype="bf16", seed=5)
    a = gpu_forward(inp, h0=False)
    b = gpu_forward(inp, h0=False)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_decode_equals_chunked():
    """Token-by-token decoding equals the batched pass, state included
    (gated-deltanet card, Correctness), within the fp32 tolerance."""
    import gated_delta_rule_52_amd as gdn
    inp = gi.make_inputs(4, 64, 4, 128, 128, decay="channel", seed=6, h0_std=0.1)
    o, hT = gpu_forward(inp)
    d = to_dev_inputs(inp)
    S = d["h0"].clone()
    outs = []
    for t in range(64):
        outs.append(gdn.gdn_decode_step(d["q"][:, t].contiguous(), d["k"][:, t].contiguous(),
                                        d["v"][:, t].contiguous(), d["g"][:, t].contiguous(),
                                        d["beta"][:, t].contiguous(), S,
                                        scale=inp["meta"]["scale"]))
    torch.cuda.synchronize()
    o_dec = torch.cat(outs, dim=1)
    assert rel_err(host(o_dec), host(o)) <= TOL["f32"]
    assert rel_err(host(S), host(hT)) <= TOL["f32"]


@pytest.mark.parametrize("decay", ["channel", "head"])
def test_bf16_split_calls_in_place(decay):
    """bf16 inputs, B=2 T=1024 H=4 128x128 with h0 ~ N(0, 0.1) and weak decay (the
    state carries across chunks): 8 calls of 128 tokens, each writing its final
    state over its initial state (hT aliasing h0, the in-place carry the
    gated-deltanet card's Usage describes), equal one call bitwise."""
    import gated_delta_rule_52_amd as gdn
    log(f"bf16 split calls in place, {decay}")
    inp = gi.make_inputs(2, 1024, 4, 128, 128, decay=decay, dtype="bf16", seed=19, h0_std=0.1,
                         g_scale=0.01)
    d = to_dev_inputs(inp)
    sc = inp["meta"]["scale"]
    o, hT = gdn.gdn_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], scale=sc)
    S = d["h0"].clone()
    outs = []
    for t0 in range(0, 1024, 128):
        sl = slice(t0, t0 + 128)
        o_c, _ = gdn.gdn_forward(d["q"][:, sl].contiguous(), d["k"][:, sl].contiguous(),
                                 d["v"][:, sl].contiguous(), d["g"][:, sl].contiguous(),
                                 d["beta"][:, sl].contiguous(), S, scale=sc, hT=S)
        outs.append(o_c)
    torch.cuda.synchronize()
    o_split = torch.cat(outs, dim=1)
    assert torch.equal(o_split, o) and torch.equal(S, hT)
    o_ref, h_ref = oracle.forward_inputs(inp)
    assert rel_err(host(o), o_ref) <= TOL["bf16"] and rel_err(host(hT), h_ref) <= TOL["bf16"]
