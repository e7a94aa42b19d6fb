"""Decode from a checkpoint plus a buffer of recent tokens (gdn_replay_*) on
the GPU: every step's output and, after folding the buffer in, the state equal
the token-serial oracle's; and they agree with the plain decode step."""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from gpu_util import TOL, host, log, rel_err, to_dev_inputs

pytestmark = pytest.mark.gpu


def replay_run(inp, depth, fold_at=()):
    """Run every token through gdn_replay_step; fold at the given steps (and at
    the end).  Returns (o [B,T,H,Dv], final state)."""
    import gated_delta_rule_52_amd as gdn
    d = to_dev_inputs(inp)
    m = inp["meta"]
    B, T, H, Dk, Dv = m["B"], m["T"], m["H"], m["Dk"], m["Dv"]
    pch = m["decay"] == "channel"
    ckpt = d["h0"].clone() if "h0" in d else gdn.gdn_new_state(B, H, Dk, Dv)
    buf = gdn.gdn_replay_buffer(B, H, Dk, Dv, depth, per_channel=pch)
    outs = []
    for t in range(T):
        sl = lambda x: x[:, t:t + 1].contiguous()
        outs.append(gdn.gdn_replay_step(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["g"]),
                                        sl(d["beta"]), ckpt, buf, depth, scale=m["scale"]))
        if t in fold_at:
            gdn.gdn_replay_fold(ckpt, buf, depth, per_channel=pch)
    gdn.gdn_replay_fold(ckpt, buf, depth, per_channel=pch)
    torch.cuda.synchronize()
    return torch.cat(outs, dim=1), ckpt


def check(inp, depth, label, fold_at=()):
    o, S = replay_run(inp, depth, fold_at)
    o_ref, h_ref = oracle.forward_inputs(inp)
    eo, eh = rel_err(host(o), o_ref), rel_err(host(S), h_ref)
    log(f"  {label}: o {eo:.2e}  state {eh:.2e}")
    tol = TOL[inp["meta"]["dtype"]]
    assert eo <= tol and eh <= tol, (eo, eh)
    return o, S


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("decay", ["channel", "head"])
@pytest.mark.parametrize("D", [16, 64, 128])
@pytest.mark.parametrize("depth", [1, 5, 16])
def test_replay_matches_oracle(dtype, decay, D, depth):
    T = 2 * depth + 3  # the buffer fills and folds, and ends part-full
    inp = gi.make_inputs(3, T, 4, D, D, decay=decay, dtype=dtype, seed=depth + D, h0_std=0.1)
    check(inp, depth, f"replay {dtype} {decay} D={D} depth={depth}")


def test_fold_mid_sequence():
    """Folding early (a part-full buffer) then continuing changes nothing but rounding."""
    inp = gi.make_inputs(2, 30, 3, 128, 128, decay="channel", seed=3, h0_std=0.1)
    check(inp, 8, "fold at steps 2, 3, 13", fold_at=(2, 3, 13))


def test_wipes():
    """Retention-gate wipes (g = -20 every 7th token) inside and across buffers."""
    inp = gi.make_inputs(2, 40, 2, 64, 64, decay="head", seed=5, h0_std=0.1, wipe_period=7)
    check(inp, 16, "wipes")


@pytest.mark.parametrize("decay", ["channel", "head"])
def test_agrees_with_decode_step(decay):
    import gated_delta_rule_52_amd as gdn
    inp = gi.make_inputs(4, 20, 4, 128, 128, decay=decay, seed=7, h0_std=0.1)
    o_r, S_r = replay_run(inp, 8)
    d = to_dev_inputs(inp)
    state = d["h0"].clone()
    outs = []
    for t in range(20):
        sl = lambda x: x[:, t:t + 1].contiguous()
        outs.append(gdn.gdn_decode_step(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["g"]),
                                        sl(d["beta"]), state, scale=inp["meta"]["scale"]))
    o_d = torch.cat(outs, dim=1)
    torch.cuda.synchronize()
    assert rel_err(host(o_r), host(o_d)) < 1e-5 and rel_err(host(S_r), host(state)) < 1e-5


def test_deterministic():
    inp = gi.make_inputs(2, 25, 3, 128, 128, decay="channel", dtype="bf16", seed=9, h0_std=0.1)
    a = replay_run(inp, 8)
    b = replay_run(inp, 8)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
