"""The float32 instantiation of the oracle (same C source compiled with
-DORACLE_REAL=float; timed as a second CPU baseline) agrees with the float64
oracle to float32 rounding, forward and reverse pass, both decay kinds."""
import numpy as np
import pytest

import gdn_inputs as gi
import oracle


@pytest.mark.parametrize("decay", ["channel", "head"])
def test_f32_instantiation_matches_f64(decay):
    inp = gi.make_inputs(2, 150, 3, 32, 32, decay=decay, seed=11, h0_std=0.1, grads=True)
    m = inp["meta"]
    o, h = oracle.forward_inputs(inp)
    o32, h32 = oracle.forward_f32(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], m["scale"],
                                  h0=inp["h0"])
    assert o32.dtype == np.float32 and h32.dtype == np.float32

    def rel(x, y):
        return float(np.max(np.abs(x.astype(np.float64) - y)) / np.max(np.abs(y)))

    assert rel(o32, o) < 1e-5 and rel(h32, h) < 1e-5
    g = oracle.backward_inputs(inp)
    g32 = oracle.backward_f32(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], m["scale"],
                              inp["dO"], h0=inp["h0"], dhT=inp["dhT"])
    for name in g:
        assert rel(g32[name], g[name]) < 1e-5, name
