"""CPU oracle of the gated delta rule (token-serial, float64).

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package.  The HIP library never
does, and this package imports nothing from it.

``forward`` / ``backward`` call the C oracle in ``gdn_oracle.c`` (built with
gcc into ``libgdn_oracle.so`` next to it).  Inputs are converted to their exact
float64 values first (see ``gdn_inputs.as_f64``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "gdn_oracle.c")
LIB = os.path.join(_HERE, "libgdn_oracle.so")
CFLAGS = ["-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=c11"]

_lib = None


LIB_F32 = os.path.join(_HERE, "libgdn_oracle_f32.so")


def build(force: bool = False, src: str = SRC, out: str = LIB, extra: tuple = ()) -> str:
    """Compile the C oracle with gcc (host code only).  Building the float64
    library also builds its float32 instantiation (same source,
    -DORACLE_REAL=float), which only the CPU-baseline timing uses."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp"
        subprocess.run(["gcc", *CFLAGS, *extra, src, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, out)
    if out == LIB and src == SRC and not extra:
        if force or not os.path.exists(LIB_F32) or os.path.getmtime(LIB_F32) < os.path.getmtime(src):
            tmp = LIB_F32 + ".tmp"
            subprocess.run(["gcc", *CFLAGS, "-DORACLE_REAL=float", src, "-o", tmp, "-lm"],
                           check=True)
            os.replace(tmp, LIB_F32)
    return out


def _bind(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    i = ctypes.c_int
    lib.oracle_forward.argtypes = [i, i, i, i, i, i, ctypes.c_double] + [dp] * 8 + [i]
    lib.oracle_forward.restype = i
    lib.oracle_backward.argtypes = [i, i, i, i, i, i, ctypes.c_double] + [dp] * 14 + [i]
    lib.oracle_backward.restype = i
    lib.oracle_max_threads.restype = i
    lib.oracle_l2norm_forward.argtypes = [ctypes.c_long, i, ctypes.c_double, dp, dp]
    lib.oracle_l2norm_forward.restype = i
    lib.oracle_l2norm_backward.argtypes = [ctypes.c_long, i, ctypes.c_double, dp, dp, dp]
    lib.oracle_l2norm_backward.restype = i
    return lib


def load(path: str | None = None):
    """Load (building if needed) the oracle library.  A path loads a variant."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        _lib = _bind(ctypes.CDLL(build()))
    return _lib


def _ptr(x):
    if x is None:
        return None
    assert x.dtype == np.float64 and x.flags.c_contiguous
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


_lib32 = None


def load_f32():
    """The float32 instantiation of the oracle (same source and entry points,
    every value and operation in float32).  Timing use only: the float64
    oracle is the reference."""
    global _lib32
    if _lib32 is None:
        build()
        L = ctypes.CDLL(LIB_F32)
        fp = ctypes.POINTER(ctypes.c_float)
        i = ctypes.c_int
        L.oracle_forward.argtypes = [i, i, i, i, i, i, ctypes.c_float] + [fp] * 8 + [i]
        L.oracle_forward.restype = i
        L.oracle_backward.argtypes = [i, i, i, i, i, i, ctypes.c_float] + [fp] * 14 + [i]
        L.oracle_backward.restype = i
        _lib32 = L
    return _lib32


def _p32(x):
    if x is None:
        return None
    assert x.dtype == np.float32 and x.flags.c_contiguous
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _f32(x):
    if x is None:
        return None
    if x.dtype == np.uint16:  # bf16 bits
        x = (x.astype(np.uint32) << 16).view(np.float32)
    return np.ascontiguousarray(x, dtype=np.float32)


def forward_f32(q, k, v, g, beta, scale, h0=None, nthreads: int = 0):
    """forward() computed by the float32 instantiation; float32 results."""
    L = load_f32()
    q, k, v, g, beta, h0 = map(_f32, (q, k, v, g, beta, h0))
    B, T, H, Dk, Dv, pc = _dims(q, v, g)
    o = np.zeros((B, T, H, Dv), np.float32)
    hT = np.zeros((B, H, Dk, Dv), np.float32)
    if L.oracle_forward(B, T, H, Dk, Dv, pc, float(scale), _p32(q), _p32(k), _p32(v), _p32(g),
                        _p32(beta), _p32(h0), _p32(o), _p32(hT), int(nthreads)):
        raise ValueError("oracle_forward (float32): bad dimensions")
    return o, hT


def backward_f32(q, k, v, g, beta, scale, dO, h0=None, dhT=None, nthreads: int = 0):
    """backward() computed by the float32 instantiation; float32 results."""
    L = load_f32()
    q, k, v, g, beta, h0, dO, dhT = map(_f32, (q, k, v, g, beta, h0, dO, dhT))
    B, T, H, Dk, Dv, pc = _dims(q, v, g)
    out = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v),
               dg=np.zeros_like(g), dbeta=np.zeros_like(beta),
               dh0=np.zeros((B, H, Dk, Dv), np.float32))
    if L.oracle_backward(B, T, H, Dk, Dv, pc, float(scale), _p32(q), _p32(k), _p32(v), _p32(g),
                         _p32(beta), _p32(h0), _p32(dO), _p32(dhT), _p32(out["dq"]),
                         _p32(out["dk"]), _p32(out["dv"]), _p32(out["dg"]), _p32(out["dbeta"]),
                         _p32(out["dh0"]), int(nthreads)):
        raise ValueError("oracle_backward (float32): bad dimensions")
    return out


def _f64(x):
    if x is None:
        return None
    if x.dtype == np.uint16:  # bf16 bits
        x = (x.astype(np.uint32) << 16).view(np.float32)
    return np.ascontiguousarray(x, dtype=np.float64)


def _dims(q, v, g):
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    per_channel = int(g.ndim == 4)
    return B, T, H, Dk, Dv, per_channel


L2NORM_EPS = 1e-6  # the reading taken for use_qk_l2norm's guard (not printed on the pages)


def l2norm(x, eps: float = L2NORM_EPS, lib=None):
    """x / sqrt(sum(x^2) + eps) over the last dimension (float64)."""
    x = _f64(x)
    out = np.zeros_like(x)
    lib = lib or load()
    if lib.oracle_l2norm_forward(x.size // x.shape[-1], x.shape[-1], float(eps), _ptr(x), _ptr(out)):
        raise ValueError("oracle_l2norm_forward: bad dimensions")
    return out


def l2norm_backward(x, dxhat, eps: float = L2NORM_EPS, lib=None):
    """Gradient with respect to the raw rows x given the gradient of l2norm(x)."""
    x, dxhat = _f64(x), _f64(dxhat)
    out = np.zeros_like(x)
    lib = lib or load()
    if lib.oracle_l2norm_backward(x.size // x.shape[-1], x.shape[-1], float(eps), _ptr(x),
                                  _ptr(dxhat), _ptr(out)):
        raise ValueError("oracle_l2norm_backward: bad dimensions")
    return out


def forward(q, k, v, g, beta, scale, h0=None, nthreads: int = 0, lib=None, qk_l2norm=False):
    """Returns (o [B,T,H,Dv], hT [B,H,Dk,Dv]) in float64.  With qk_l2norm the
    q and k rows are L2-normalised first (use_qk_l2norm)."""
    lib = lib or load()
    if qk_l2norm:
        q, k = l2norm(q, lib=lib), l2norm(k, lib=lib)
    q, k, v, g, beta, h0 = map(_f64, (q, k, v, g, beta, h0))
    B, T, H, Dk, Dv, pc = _dims(q, v, g)
    o = np.zeros((B, T, H, Dv))
    hT = np.zeros((B, H, Dk, Dv))
    rc = lib.oracle_forward(B, T, H, Dk, Dv, pc, float(scale), _ptr(q), _ptr(k), _ptr(v),
                            _ptr(g), _ptr(beta), _ptr(h0), _ptr(o), _ptr(hT), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_forward: bad dimensions")
    return o, hT


def backward(q, k, v, g, beta, scale, dO, h0=None, dhT=None, nthreads: int = 0, lib=None,
             qk_l2norm=False):
    """Returns dict of float64 gradients dq, dk, dv, dg, dbeta, dh0 (with
    qk_l2norm: dq, dk with respect to the raw, unnormalised q and k)."""
    lib = lib or load()
    q_raw, k_raw = q, k
    if qk_l2norm:
        q, k = l2norm(q, lib=lib), l2norm(k, lib=lib)
    q, k, v, g, beta, h0, dO, dhT = map(_f64, (q, k, v, g, beta, h0, dO, dhT))
    B, T, H, Dk, Dv, pc = _dims(q, v, g)
    out = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v),
               dg=np.zeros_like(g), dbeta=np.zeros_like(beta), dh0=np.zeros((B, H, Dk, Dv)))
    rc = lib.oracle_backward(B, T, H, Dk, Dv, pc, float(scale), _ptr(q), _ptr(k), _ptr(v),
                             _ptr(g), _ptr(beta), _ptr(h0), _ptr(dO), _ptr(dhT),
                             _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]),
                             _ptr(out["dbeta"]), _ptr(out["dh0"]), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_backward: bad dimensions")
    if qk_l2norm:
        out["dq"] = l2norm_backward(q_raw, out["dq"], lib=lib)
        out["dk"] = l2norm_backward(k_raw, out["dk"], lib=lib)
    return out


def forward_inputs(inp: dict, **kw):
    """forward() on a workload dict from gdn_inputs."""
    kw.setdefault("qk_l2norm", bool(inp["meta"].get("qk_l2norm", False)))
    return forward(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["meta"]["scale"],
                   h0=inp.get("h0"), **kw)


def backward_inputs(inp: dict, **kw):
    kw.setdefault("qk_l2norm", bool(inp["meta"].get("qk_l2norm", False)))
    return backward(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["meta"]["scale"],
                    inp["dO"], h0=inp.get("h0"), dhT=inp.get("dhT"), **kw)


def max_threads() -> int:
    return load().oracle_max_threads()
