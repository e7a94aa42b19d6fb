"""Decode step on the GPU against the token-serial oracle."""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from gpu_util import TOL, dev, host, log, rel_err, to_dev_inputs

pytestmark = pytest.mark.gpu


def run_decode(inp, steps):
    import gated_delta_rule_52_amd as gdn
    d = to_dev_inputs(inp)
    m = inp["meta"]
    if "h0" in d:
        state = d["h0"].clone()
    else:
        state = gdn.new_state(m["B"], m["H"], m["Dk"], m["Dv"])
    outs = []
    for t in range(steps):
        o = gdn.gdn_decode_step(d["q"][:, t].contiguous(), d["k"][:, t].contiguous(),
                                d["v"][:, t].contiguous(), d["g"][:, t].contiguous(),
                                d["beta"][:, t].contiguous(), state, scale=m["scale"])
        outs.append(o)
    torch.cuda.synchronize()
    return np.concatenate([host(o) for o in outs], axis=1), host(state)


@pytest.mark.parametrize("decay", ["channel", "head"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [16, 64, 128])
def test_decode_small(decay, dtype, D):
    log(f"decode small decay={decay} dtype={dtype} D={D}")
    inp = gi.make_inputs(3, 20, 5, D, D, decay=decay, dtype=dtype, seed=3, h0_std=0.1)
    o, S = run_decode(inp, 20)
    o_ref, S_ref = oracle.forward_inputs(inp)
    assert rel_err(o, o_ref) <= TOL[dtype], rel_err(o, o_ref)
    assert rel_err(S, S_ref) <= TOL[dtype], rel_err(S, S_ref)


def test_decode_serving_shape_64_steps():
    """B=256, H=16, 128x128 fp32 state (268 MB), 64 steps from h0 ~ N(0, 0.1)."""
    log("decode B=256 H=16 D=128 x64 steps")
    inp = gi.decode()
    o, S = run_decode(inp, 64)
    o_ref, S_ref = oracle.forward_inputs(inp)
    eo, es = rel_err(o, o_ref), rel_err(S, S_ref)
    log(f"  o rel err {eo:.3e}  state rel err {es:.3e}")
    assert eo <= TOL["f32"] and es <= TOL["f32"]
    # per step too
    for t in (0, 31, 63):
        assert rel_err(o[:, t], o_ref[:, t]) <= TOL["f32"]


def test_decode_identity_gates_bitwise():
    """g = 0 and beta = 0 leave the state exactly unchanged (gated-deltanet
    card, Correctness)."""
    import gated_delta_rule_52_amd as gdn
    inp = gi.make_inputs(4, 1, 3, 128, 128, decay="channel", seed=9, h0_std=1.0)
    d = to_dev_inputs(inp)
    d["g"].zero_()
    d["beta"].zero_()
    state = d["h0"].clone()
    gdn.gdn_decode_step(d["q"][:, 0].contiguous(), d["k"][:, 0].contiguous(),
                        d["v"][:, 0].contiguous(), d["g"][:, 0].contiguous(),
                        d["beta"][:, 0].contiguous(), state)
    torch.cuda.synchronize()
    assert torch.equal(state, d["h0"])


def test_decode_deterministic():
    import gated_delta_rule_52_amd as gdn
    inp = gi.make_inputs(8, 1, 4, 128, 128, decay="channel", seed=10, h0_std=0.1)
    d = to_dev_inputs(inp)
    outs = []
    for _ in range(2):
        s = d["h0"].clone()
        o = gdn.gdn_decode_step(d["q"][:, 0].contiguous(), d["k"][:, 0].contiguous(),
                                d["v"][:, 0].contiguous(), d["g"][:, 0].contiguous(),
                                d["beta"][:, 0].contiguous(), s)
        outs.append((o, s))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
