"""HIP-graph capture of the training pair and of the forward: the library
allocates nothing and issues no memset when the caller passes every output
and the workspace, so one call can be captured and replayed.  Every replay
must reproduce the eager call bitwise (the kernels are deterministic), with
the outputs overwritten before each replay and eager calls and
synchronizations between replays."""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from gpu_util import TOL, host, log, rel_err, to_dev_inputs

pytestmark = pytest.mark.gpu


def _replay_checks(fn, outs, n=4):
    fn()
    torch.cuda.synchronize()
    want = [x.clone() for x in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    for i in range(n):
        for x in outs:
            x.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for x, y in zip(outs, want):
            assert torch.equal(x, y), f"replay {i} differs from the eager call"
        fn()  # eager work between replays
        torch.cuda.synchronize()
    del graph
    return want


@pytest.mark.parametrize("decay", ["channel", "head"])
def test_training_pair_graph_replays(decay):
    import gated_delta_rule_52_amd as gdn
    log(f"graph replay of the training pair, bf16 {decay}")
    inp = gi.make_inputs(2, 200, 3, 128, 128, decay=decay, dtype="bf16", seed=29, h0_std=0.1,
                         grads=True)
    d = to_dev_inputs(inp)
    sc = inp["meta"]["scale"]
    q, k, v, g, beta, h0, dO, dhT = (d[n] for n in ("q", "k", "v", "g", "beta", "h0", "dO", "dhT"))
    sh = gdn.make_shape(q, v, g, sc, 64)
    ws = gdn.workspace(sh, True, q.device)
    o = torch.empty_like(v)
    hT = torch.empty((2, 3, 128, 128), dtype=torch.float32, device="cuda")
    gout = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(g),
            torch.empty_like(beta), torch.empty_like(hT))

    def step():
        gdn.gdn_forward_train(q, k, v, g, beta, h0, scale=sc, chunk=64, o=o, hT=hT, ws=ws)
        gdn.gdn_backward_train(q, k, v, g, beta, dO, ws, dhT, scale=sc, chunk=64, out=gout)

    want = _replay_checks(step, (o, hT) + gout)
    # and the replayed results are the layer's: against the oracle
    ref = oracle.backward_inputs(inp)
    o_ref, h_ref = oracle.forward_inputs(inp)
    assert rel_err(host(want[0]), o_ref) <= TOL["bf16"] and rel_err(host(want[1]), h_ref) <= TOL["bf16"]
    for name, x in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), want[2:]):
        assert rel_err(host(x), ref[name]) <= TOL["bf16"], name


def test_forward_graph_replays():
    import gated_delta_rule_52_amd as gdn
    log("graph replay of the forward, bf16")
    inp = gi.make_inputs(2, 330, 3, 128, 128, decay="channel", dtype="bf16", seed=31, h0_std=0.1)
    d = to_dev_inputs(inp)
    sc = inp["meta"]["scale"]
    q, k, v, g, beta, h0 = (d[n] for n in ("q", "k", "v", "g", "beta", "h0"))
    sh = gdn.make_shape(q, v, g, sc, 64)
    ws = gdn.workspace(sh, False, q.device)
    o = torch.empty_like(v)
    hT = torch.empty((2, 3, 128, 128), dtype=torch.float32, device="cuda")

    def fwd():
        gdn.gdn_forward(q, k, v, g, beta, h0, scale=sc, chunk=64, o=o, hT=hT, ws=ws)

    want = _replay_checks(fwd, (o, hT))
    o_ref, h_ref = oracle.forward_inputs(inp)
    assert rel_err(host(want[0]), o_ref) <= TOL["bf16"] and rel_err(host(want[1]), h_ref) <= TOL["bf16"]
