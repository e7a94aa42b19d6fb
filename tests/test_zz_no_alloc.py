"""gdn_forward_noalloc (the forward for callers that cannot allocate: its
workspace is the library's static per-device array) called through the C ABI
gives what gdn_forward gives, on two calls in a row, the second smaller; a
shape whose workspace does not fit is refused before any launch."""
import ctypes

import pytest
import torch

import gdn_inputs as gi
from gpu_util import TOL, host, log, rel_err, to_dev_inputs

pytestmark = pytest.mark.gpu


def _noalloc(inp, o, hT, h0=None):
    import gated_delta_rule_52_amd as gdn
    d = to_dev_inputs(inp)
    sh = gdn.make_shape(d["q"], d["v"], d["g"], inp["meta"]["scale"], inp["meta"].get("chunk"))
    need = gdn.gdn_workspace_bytes(sh, False)
    rc = gdn.lib().gdn_forward_noalloc(
        ctypes.byref(sh), ctypes.c_void_p(d["q"].data_ptr()), ctypes.c_void_p(d["k"].data_ptr()),
        ctypes.c_void_p(d["v"].data_ptr()), ctypes.c_void_p(d["g"].data_ptr()),
        ctypes.c_void_p(d["beta"].data_ptr()),
        ctypes.c_void_p(h0.data_ptr()) if h0 is not None else None,
        ctypes.c_void_p(o.data_ptr()), ctypes.c_void_p(hT.data_ptr()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return rc, need, d


def test_noalloc_matches_gdn_forward_twice():
    import gated_delta_rule_52_amd as gdn
    cases = [
        # bf16, per channel, ragged T, h0: 96 chunk-heads (about 14 MB of workspace)
        dict(B=1, T=1000, H=6, D=128, decay="channel", dtype="bf16", h0=True),
        # then a smaller one: fp32, per head, 64 x 64, zero state
        dict(B=2, T=100, H=2, D=64, decay="head", dtype="f32", h0=False),
    ]
    for i, c in enumerate(cases):
        log(f"noalloc call {i}: {c}")
        inp = gi.make_inputs(c["B"], c["T"], c["H"], c["D"], c["D"], decay=c["decay"],
                             dtype=c["dtype"], seed=50 + i, h0_std=0.1 if c["h0"] else None)
        inp["meta"]["chunk"] = 64
        d0 = to_dev_inputs(inp)
        o = torch.full_like(d0["v"], float("nan"))
        hT = torch.full((c["B"], c["H"], c["D"], c["D"]), float("nan"), device="cuda")
        rc, need, d = _noalloc(inp, o, hT, d0.get("h0"))
        assert rc == 0, gdn.lib().gdn_status_string(rc)
        assert 0 < need <= gdn.GDN_NOALLOC_SCRATCH_BYTES
        o_ref, h_ref = gdn.gdn_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d0.get("h0"),
                                       scale=inp["meta"]["scale"], chunk=64)
        torch.cuda.synchronize()
        eo, eh = rel_err(host(o), host(o_ref)), rel_err(host(hT), host(h_ref))
        log(f"  vs gdn_forward: o {eo:.1e}  hT {eh:.1e}  bitwise {torch.equal(o, o_ref) and torch.equal(hT, h_ref)}")
        assert eo <= TOL[c["dtype"]] and eh <= TOL[c["dtype"]]
        assert torch.equal(o, o_ref) and torch.equal(hT, h_ref)


def test_noalloc_refuses_what_does_not_fit():
    import gated_delta_rule_52_amd as gdn
    # B=8 T=4096 H=6 128x128 needs far more than the static array holds
    inp = gi.make_inputs(1, 64, 1, 128, 128, dtype="bf16", seed=3)
    d = to_dev_inputs(inp)
    sh = gdn.GdnShape(8, 4096, 6, 128, 128, gdn.GDN_BF16, gdn.GDN_DECAY_PER_CHANNEL, 0.0, 64,
                      0, 0.0, 0.0, 0)
    assert gdn.gdn_workspace_bytes(sh, False) > gdn.GDN_NOALLOC_SCRATCH_BYTES
    p = ctypes.c_void_p(d["q"].data_ptr())  # never dereferenced: refused before any launch
    rc = gdn.lib().gdn_forward_noalloc(ctypes.byref(sh), p, p, p, p, p, None, p, p, None)
    assert rc == 4  # GDN_ERR_WORKSPACE
    sh.B, sh.T, sh.diag = 1, 64, 1
    rc = gdn.lib().gdn_forward_noalloc(ctypes.byref(sh), p, p, p, p, p, None, p, p, None)
    assert rc == 2  # GDN_ERR_UNSUPPORTED: diag counters would sit in the shared array
