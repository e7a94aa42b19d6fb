"""Seeded synthetic inputs for the gated delta-rule layer.

This module only draws and rounds numbers.  It holds none of the layer's
arithmetic, so both the CPU oracle (``oracle/``) and the HIP library can be fed
from it without sharing any computation.

Draw order (one ``numpy.random.Generator(PCG64(seed))`` per workload, float64
draws): q, k, v, beta-logits, g-logits, h0, dO, dhT.  Draws that a workload does
not use are skipped.

* q, k: N(0, 1), then divided by their L2 norm over the last axis in float64
  (the inputs arrive normalised, as keys are normalised in practice; the
  gated-deltanet card, "Correctness": stability needs beta*|k|^2 below about 2).
* v: N(0, 1).
* beta = sigmoid(z), z ~ N(0, 1), one value per (b, t, h).
* g = -softplus(z), z ~ N(0, 1), per key channel [B,T,H,Dk] or per head
  [B,T,H]; g <= 0 as the atomic_ops card requires ("Quick start": keep g <= 0).
* optional state wipes: g = wipe_value at every token t with
  t % wipe_period == wipe_period - 1 (all b, h, channels).
* h0 ~ N(0, h0_std) (standard deviation), float32.
* dO ~ N(0, 1) in the input dtype, dhT ~ N(0, 0.01) float32.
* raw q, k (qk_scale set; for the use_qk_l2norm option, which normalises
  inside the layer): the N(0, 1) rows are not normalised but multiplied by
  exp(qk_scale * z), z ~ N(0, 1), one factor per row, drawn last (q's factors,
  then k's), so every other draw is unchanged; meta["qk_l2norm"] is set.

Every tensor is rounded to float32; bf16 tensors (q, k, v, dO in bf16 mode) are
then rounded to nearest-even from the float32 bits.  ``as_f64`` gives the exact
float64 upcast of whatever bits the device receives, so the oracle and the GPU
see the same numbers.
"""
from __future__ import annotations

import numpy as np

BF16_TENSORS = ("q", "k", "v", "dO")


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def as_f64(x: np.ndarray) -> np.ndarray:
    """Exact float64 value of a float32 array or of a bf16 (uint16 bits) array."""
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def _l2n(x: np.ndarray) -> np.ndarray:
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def _softplus(z: np.ndarray) -> np.ndarray:
    # log(1 + e^z) without overflow
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def _sigmoid(z: np.ndarray) -> np.ndarray:
    return 0.5 * (1.0 + np.tanh(0.5 * z))


def make_inputs(B: int, T: int, H: int, Dk: int, Dv: int, *, decay: str = "channel",
                dtype: str = "f32", seed: int = 0, h0_std: float | None = None,
                wipe_period: int | None = None, wipe_value: float = -20.0,
                grads: bool = False, dO_std: float = 1.0, dhT_std: float = 0.01,
                qk_scale: float | None = None, g_scale: float = 1.0) -> dict:
    """Draw one workload.  Returns a dict of numpy arrays in device form
    (float32, or uint16 bf16 bits for q/k/v/dO when dtype == 'bf16') plus the
    shape metadata under 'meta'."""
    assert decay in ("channel", "head") and dtype in ("f32", "bf16")
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk))
    if qk_scale is None:
        q, k = _l2n(q), _l2n(k)
    v = rng.standard_normal((B, T, H, Dv))
    beta = _sigmoid(rng.standard_normal((B, T, H)))
    gshape = (B, T, H, Dk) if decay == "channel" else (B, T, H)
    g = -_softplus(rng.standard_normal(gshape)) * g_scale  # g_scale < 1: weaker decay
    if wipe_period:
        g[:, wipe_period - 1::wipe_period] = wipe_value
    out = {}
    h0 = None
    if h0_std is not None:
        h0 = rng.standard_normal((B, H, Dk, Dv)) * h0_std
    if grads:
        dO = rng.standard_normal((B, T, H, Dv)) * dO_std
        dhT = rng.standard_normal((B, H, Dk, Dv)) * dhT_std
        out["dO"] = dO
        out["dhT"] = dhT
    if qk_scale is not None:
        q = q * np.exp(qk_scale * rng.standard_normal((B, T, H, 1)))
        k = k * np.exp(qk_scale * rng.standard_normal((B, T, H, 1)))
    out.update(q=q, k=k, v=v, beta=beta, g=g)
    if h0 is not None:
        out["h0"] = h0
    res = {}
    for name, x in out.items():
        x32 = x.astype(np.float32)
        if dtype == "bf16" and name in BF16_TENSORS:
            res[name] = f32_to_bf16_bits(x32)
        else:
            res[name] = x32
    res["meta"] = dict(B=B, T=T, H=H, Dk=Dk, Dv=Dv, decay=decay, dtype=dtype, seed=seed,
                       scale=float(np.float32(Dk ** -0.5)), qk_l2norm=qk_scale is not None)
    return res


def f64_inputs(inp: dict) -> dict:
    """Exact float64 copies of every tensor in a workload (for the oracle)."""
    return {k: (as_f64(v) if isinstance(v, np.ndarray) else v) for k, v in inp.items()}


# ---------------------------------------------------------------------------
# The named workloads.  The sizes follow the pages' benchmark shapes (the
# Marin note's "Single-device benchmark": B=4/8, T=4096, H=6, width 128) and the
# gated-deltanet card (2,048-token run with periodic retention-gate wipes).
# ---------------------------------------------------------------------------

def tiny(seed: int = 0, grads: bool = False) -> dict:
    """Per-channel decay, fp32, B=1 T=64 H=2 Dk=Dv=16, chunk 16, zero state."""
    d = make_inputs(1, 64, 2, 16, 16, decay="channel", dtype="f32", seed=seed, grads=grads)
    d["meta"]["chunk"] = 16
    return d


def head_wipe(seed: int = 0) -> dict:
    """Per-head decay, fp32, B=2 T=2048 H=8 128x128, wipes g=-20 at t%256==255,
    h0 ~ N(0, 0.1)."""
    d = make_inputs(2, 2048, 8, 128, 128, decay="head", dtype="f32", seed=seed,
                    h0_std=0.1, wipe_period=256)
    d["meta"]["chunk"] = 64
    return d


def decode(seed: int = 0, B: int = 256, H: int = 16, steps: int = 64) -> dict:
    """Decode: B=256 H=16 128x128, per-channel g, h0 ~ N(0, 0.1); the inputs of
    step t are the [:, t] slices of a T=steps sequence."""
    d = make_inputs(B, steps, H, 128, 128, decay="channel", dtype="f32", seed=seed, h0_std=0.1)
    d["meta"]["chunk"] = 64
    return d


def train(seed: int = 0, B: int = 8, dtype: str = "bf16", grads: bool = False,
          T: int = 4096, H: int = 6, D: int = 128, decay: str = "channel",
          qk_scale: float | None = None) -> dict:
    """Training shape: per-channel decay (or per-head), B=8 (or 4) T=4096 H=6
    128x128, zero state; with grads, dO ~ N(0,1) in the input dtype and
    dhT ~ N(0, 0.01); with qk_scale, raw q, k for use_qk_l2norm."""
    d = make_inputs(B, T, H, D, D, decay=decay, dtype=dtype, seed=seed, grads=grads,
                    qk_scale=qk_scale)
    d["meta"]["chunk"] = 64
    return d
