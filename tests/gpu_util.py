"""Helpers of the GPU parity tests: move seeded workloads to the device in the
exact bits the oracle sees, and compare with the tolerance the layer's
numerics allow (max|x - y| / max|y|, y the oracle):
  float32 inputs: 1e-5;  bf16 inputs (fp32 state and accumulation): 2e-2."""
import numpy as np
import torch

TOL = {"f32": 1e-5, "bf16": 2e-2}


def dev(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:  # bf16 bits
        return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(x, y) -> float:
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    den = float(np.max(np.abs(y)))
    num = float(np.max(np.abs(x - y)))
    return num / den if den > 0 else num


def to_dev_inputs(inp: dict) -> dict:
    return {k: dev(v) for k, v in inp.items() if isinstance(v, np.ndarray)}


def log(msg: str):
    print(msg, flush=True)
