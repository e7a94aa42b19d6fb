"""The Python binding rejects mis-shaped tensors before anything is launched
(the C ABI takes bare pointers and cannot check buffer sizes)."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def _inputs(B=1, T=70, H=2, D=64, decay="channel", dtype=torch.bfloat16):
    dev = "cuda"
    q = torch.randn(B, T, H, D, device=dev).to(dtype)
    k = torch.randn(B, T, H, D, device=dev).to(dtype)
    v = torch.randn(B, T, H, D, device=dev).to(dtype)
    g = -torch.rand((B, T, H, D) if decay == "channel" else (B, T, H), device=dev)
    beta = torch.rand(B, T, H, device=dev)
    return q, k, v, g, beta


def test_rejects_bad_input_shapes():
    import gated_delta_rule_52_amd as gdn
    q, k, v, g, beta = _inputs()
    with pytest.raises(ValueError):
        gdn.gdn_forward(q, k[:, :-1], v, g, beta)
    with pytest.raises(ValueError):
        gdn.gdn_forward(q, k, v, g[..., :-1], beta)
    with pytest.raises(ValueError):
        gdn.gdn_forward(q, k, v, g, beta[:, :, :1])
    with pytest.raises(ValueError):
        gdn.gdn_forward(q, k, v, g, beta, torch.zeros(1, 2, 64, 32, device="cuda"))


def test_rejects_bad_output_buffers():
    import gated_delta_rule_52_amd as gdn
    q, k, v, g, beta = _inputs()
    with pytest.raises(ValueError):
        gdn.gdn_forward(q, k, v, g, beta, o=torch.empty_like(v)[:, :-1])
    with pytest.raises(ValueError):
        gdn.gdn_forward(q, k, v, g, beta, hT=torch.empty(1, 2, 64, 63, device="cuda"))
    o, hT, ws = gdn.gdn_forward_train(q, k, v, g, beta)
    dO = torch.randn_like(v)
    good = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(g),
            torch.empty_like(beta), torch.empty(1, 2, 64, 64, device="cuda"))
    bad_dg = good[:3] + (torch.empty(1, 70, 2, device="cuda"),) + good[4:]
    with pytest.raises(ValueError):
        gdn.gdn_backward_train(q, k, v, g, beta, dO, ws, out=bad_dg)
    bad_dtype = (good[0].float(),) + good[1:]
    with pytest.raises(TypeError):
        gdn.gdn_backward_train(q, k, v, g, beta, dO, ws, out=bad_dtype)
    res = gdn.gdn_backward_train(q, k, v, g, beta, dO, ws, out=good)
    torch.cuda.synchronize()
    assert all(a is b for a, b in zip(res, good))
    with pytest.raises(ValueError):
        gdn.gdn_decode_step(q[:, :1], k[:, :1], v[:, :1], g[:, :1], beta[:, :1],
                            torch.zeros(1, 2, 64, 32, device="cuda"))
