"""Python binding of libgdn.so, the gated delta-rule layer for MI355X (gfx950).

Argument marshalling only: torch tensors supply device memory and the current
stream, every computation runs in the library's HIP kernels.  The functions
carry the names of the C entry points in include/gdn.h:

    gdn_new_state(B, H, Dk, Dv)                      -> zeroed fp32 state
    gdn_workspace_bytes(shape, for_backward)
    gdn_forward(q, k, v, g, beta, h0=None, ...)      -> (o, hT)
    gdn_backward(q, k, v, g, beta, dO, h0=None, dhT=None, ...)
                                                     -> (dq, dk, dv, dg, dbeta, dh0)
    gdn_decode_step(q, k, v, g, beta, state, ...)    -> o   (state updated in place)

plus ``new_state`` (the gated-deltanet card's name for gdn_new_state).
Layouts: q, k [B,T,H,Dk]; v [B,T,H,Dv]; g [B,T,H,Dk] or [B,T,H] (fp32);
beta [B,T,H] (fp32); states [B,H,Dk,Dv] fp32.  q, k, v share one dtype
(float32 or bfloat16); outputs take that dtype.  use_qk_l2norm=True has the
library scale every q and k row to unit length, x / sqrt(|x|^2 + 1e-6), inside
the call (the card's option of that name); dq, dk are then the gradients with
respect to the raw rows, and a training pair must pass the same value to both
calls.  The numerical-safety options of the chunked calls (wy_eps damping of
the WY solve, clip at the stage boundaries, diag stage counters read back with
gdn_diag_read) follow include/gdn.h.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")
# the measurement build: the same sources with the launch recorder of
# include/gdn_profile.h compiled in (see use_measurement_build)
PROFILE_LIB_PATH = os.path.join(_HERE, "libgdn_prof.so")

GDN_F32, GDN_BF16 = 0, 1
GDN_DECAY_PER_HEAD, GDN_DECAY_PER_CHANNEL = 0, 1
STATUS = {0: "GDN_OK", 1: "GDN_ERR_INVALID_ARG", 2: "GDN_ERR_UNSUPPORTED", 3: "GDN_ERR_ALIGNMENT",
          4: "GDN_ERR_WORKSPACE", 5: "GDN_ERR_HIP"}
EXPORTS = ("gdn_new_state", "gdn_workspace_bytes", "gdn_forward", "gdn_forward_noalloc",
           "gdn_backward",
           "gdn_forward_train", "gdn_backward_train", "gdn_decode_step", "gdn_diag_read",
           "gdn_replay_buffer_bytes", "gdn_replay_reset", "gdn_replay_step", "gdn_replay_fold",
           "gdn_status_string")
# include/gdn_profile.h: exported by the measurement build only
PROFILE_EXPORTS = ("gdn_profile_begin", "gdn_profile_end", "gdn_profile_launch_name")


class GdnShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int),
                ("Dk", ctypes.c_int), ("Dv", ctypes.c_int), ("dtype", ctypes.c_int),
                ("decay", ctypes.c_int), ("scale", ctypes.c_float), ("chunk", ctypes.c_int),
                ("qk_l2norm", ctypes.c_int), ("wy_eps", ctypes.c_float), ("clip", ctypes.c_float),
                ("diag", ctypes.c_int)]


class GdnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {lib().gdn_status_string(code).decode()}")


_lib = None
_lib_path = LIB_PATH


def use_measurement_build():
    """Bind this process to libgdn_prof.so instead of libgdn.so: the same
    kernels and entry points, plus the launch recorder of include/gdn_profile.h
    (gated_delta_rule_52_amd.profile).  Must be called before the first call
    into the library."""
    global _lib_path
    if _lib is not None and _lib_path != PROFILE_LIB_PATH:
        raise RuntimeError("use_measurement_build() after libgdn.so was loaded")
    _lib_path = PROFILE_LIB_PATH


def lib():
    """The loaded library (libgdn.so, or libgdn_prof.so after
    use_measurement_build()).  Raises if it has not been built: there is no
    other implementation to fall back to."""
    global _lib
    if _lib is None:
        if not os.path.exists(_lib_path):
            raise ImportError(f"{os.path.basename(_lib_path)} is not built ({_lib_path}); run "
                              "`python -m gated_delta_rule_52_amd.build`")
        L = ctypes.CDLL(_lib_path)
        vp, sz, i, fp = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p
        sp = ctypes.POINTER(GdnShape)
        L.gdn_new_state.argtypes = [fp, i, i, i, i, vp]
        L.gdn_new_state.restype = i
        L.gdn_workspace_bytes.argtypes = [sp, i]
        L.gdn_workspace_bytes.restype = sz
        L.gdn_forward.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.gdn_forward.restype = i
        L.gdn_forward_noalloc.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.gdn_forward_noalloc.restype = i
        L.gdn_backward.argtypes = [sp] + [vp] * 15 + [sz, vp]
        L.gdn_backward.restype = i
        L.gdn_forward_train.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.gdn_forward_train.restype = i
        L.gdn_backward_train.argtypes = [sp] + [vp] * 14 + [sz, vp]
        L.gdn_backward_train.restype = i
        L.gdn_decode_step.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.gdn_decode_step.restype = i
        L.gdn_diag_read.argtypes = [sp, vp, ctypes.POINTER(ctypes.c_uint), vp]
        L.gdn_diag_read.restype = i
        L.gdn_replay_buffer_bytes.argtypes = [sp, i]
        L.gdn_replay_buffer_bytes.restype = sz
        L.gdn_replay_reset.argtypes = [sp, vp, i, vp]
        L.gdn_replay_reset.restype = i
        L.gdn_replay_step.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, i, vp, vp]
        L.gdn_replay_step.restype = i
        L.gdn_replay_fold.argtypes = [sp, vp, vp, i, vp]
        L.gdn_replay_fold.restype = i
        L.gdn_status_string.argtypes = [i]
        L.gdn_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return GDN_F32
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    raise TypeError(f"q/k/v must be float32 or bfloat16, got {t.dtype}")


def _check(t, name, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _check_shape(t, name, shape, dtype):
    """A caller-supplied tensor the library reads or writes: device, dense, and
    exactly `shape` (the C ABI takes bare pointers and cannot check sizes)."""
    if t is None:
        return
    _check(t, name, dtype)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


DIAG_STAGES = ("P", "A", "T", "U", "W", "o", "hT")  # GDN_DIAG_* order


def make_shape(q, v, g, scale=None, chunk=None, use_qk_l2norm=False, wy_eps=0.0, clip=0.0,
               diag=False) -> GdnShape:
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    decay = GDN_DECAY_PER_CHANNEL if g.dim() == 4 else GDN_DECAY_PER_HEAD
    return GdnShape(B, T, H, Dk, Dv, _dtype_code(q), decay,
                    0.0 if scale is None else float(scale), 0 if chunk is None else int(chunk),
                    int(bool(use_qk_l2norm)), float(wy_eps), float(clip), int(bool(diag)))


def _call(fn, where, *args):
    rc = fn(*args)
    if rc != 0:
        raise GdnError(rc, where)


def gdn_new_state(B: int, H: int, Dk: int, Dv: int, device="cuda") -> torch.Tensor:
    s = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=device)
    _call(lib().gdn_new_state, "gdn_new_state", _ptr(s), B, H, Dk, Dv, _stream())
    return s


new_state = gdn_new_state


def gdn_workspace_bytes(shape: GdnShape, for_backward: bool = False) -> int:
    return int(lib().gdn_workspace_bytes(ctypes.byref(shape), int(for_backward)))


def workspace(shape: GdnShape, for_backward: bool, device) -> torch.Tensor:
    n = gdn_workspace_bytes(shape, for_backward)
    if n == 0 and shape.T > 0:
        raise GdnError(2, "gdn_workspace_bytes")
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def _check_inputs(q, k, v, g, beta):
    dt = q.dtype
    if q.dim() != 4:
        raise ValueError(f"q must be [B, T, H, Dk], got {tuple(q.shape)}")
    B, T, H, Dk = q.shape
    _check(q, "q", dt)
    _check_shape(k, "k", q.shape, dt)
    if v.dim() != 4 or tuple(v.shape[:3]) != (B, T, H):
        raise ValueError(f"v must be [{B}, {T}, {H}, Dv], got {tuple(v.shape)}")
    _check(v, "v", dt)
    if tuple(g.shape) not in ((B, T, H, Dk), (B, T, H)):
        raise ValueError(f"g must be [{B}, {T}, {H}, {Dk}] or [{B}, {T}, {H}], got {tuple(g.shape)}")
    _check(g, "g", torch.float32)
    _check_shape(beta, "beta", (B, T, H), torch.float32)
    for name, t in (("k", k), ("v", v), ("g", g), ("beta", beta)):
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")


def _state_shape(sh):
    return (sh.B, sh.H, sh.Dk, sh.Dv)


def _check_ws(ws):
    if ws is not None:
        _check(ws, "ws")


def gdn_forward(q, k, v, g, beta, h0=None, *, scale=None, chunk=None, o=None, hT=None,
                want_state=True, ws=None, use_qk_l2norm=False, wy_eps=0.0, clip=0.0, diag=False):
    """Chunked forward.  Returns (o, hT); hT is None when want_state is False.
    Passing hT=h0 carries the state in place."""
    _check_inputs(q, k, v, g, beta)
    sh = make_shape(q, v, g, scale, chunk, use_qk_l2norm, wy_eps, clip, diag)
    _check_shape(h0, "h0", _state_shape(sh), torch.float32)
    _check_shape(o, "o", v.shape, q.dtype)
    _check_shape(hT, "hT", _state_shape(sh), torch.float32)
    _check_ws(ws)
    B, T, H, _ = q.shape
    if o is None:
        o = torch.empty((B, T, H, sh.Dv), dtype=q.dtype, device=q.device)
    if hT is None and want_state:
        hT = torch.empty((B, H, sh.Dk, sh.Dv), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = workspace(sh, False, q.device)
    _call(lib().gdn_forward, "gdn_forward", ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
          _ptr(beta), _ptr(h0), _ptr(o), _ptr(hT), _ptr(ws), ws.numel(), _stream())
    return o, hT


GDN_NOALLOC_SCRATCH_BYTES = 64 << 20  # include/gdn.h


def gdn_forward_noalloc(q, k, v, g, beta, h0=None, *, scale=None, chunk=None, o=None, hT=None,
                        use_qk_l2norm=False, wy_eps=0.0, clip=0.0):
    """gdn_forward whose workspace is the library's static per-device array
    (nothing is allocated for it; the shape's forward workspace must fit in
    GDN_NOALLOC_SCRATCH_BYTES).  Calls overlapping on one device race.
    Pass o and hT to allocate nothing here either.  Returns (o, hT)."""
    _check_inputs(q, k, v, g, beta)
    sh = make_shape(q, v, g, scale, chunk, use_qk_l2norm, wy_eps, clip, False)
    _check_shape(h0, "h0", _state_shape(sh), torch.float32)
    _check_shape(o, "o", v.shape, q.dtype)
    _check_shape(hT, "hT", _state_shape(sh), torch.float32)
    B, T, H, _ = q.shape
    if o is None:
        o = torch.empty((B, T, H, sh.Dv), dtype=q.dtype, device=q.device)
    if hT is None:
        hT = torch.empty((B, H, sh.Dk, sh.Dv), dtype=torch.float32, device=q.device)
    _call(lib().gdn_forward_noalloc, "gdn_forward_noalloc", ctypes.byref(sh), _ptr(q), _ptr(k),
          _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o), _ptr(hT), _stream())
    return o, hT


def gdn_backward(q, k, v, g, beta, dO, h0=None, dhT=None, *, scale=None, chunk=None,
                 want_dh0=True, ws=None, use_qk_l2norm=False, wy_eps=0.0, clip=0.0, diag=False):
    """Gradients (dq, dk, dv, dg, dbeta, dh0) of sum(o*dO) + sum(hT*dhT)."""
    _check_inputs(q, k, v, g, beta)
    sh = make_shape(q, v, g, scale, chunk, use_qk_l2norm, wy_eps, clip, diag)
    _check_shape(dO, "dO", v.shape, q.dtype)
    _check_shape(h0, "h0", _state_shape(sh), torch.float32)
    _check_shape(dhT, "dhT", _state_shape(sh), torch.float32)
    _check_ws(ws)
    dq = torch.empty_like(q); dk = torch.empty_like(k); dv = torch.empty_like(v)
    dg = torch.empty_like(g); dbeta = torch.empty_like(beta)
    dh0 = (torch.empty((sh.B, sh.H, sh.Dk, sh.Dv), dtype=torch.float32, device=q.device)
           if want_dh0 else None)
    if ws is None:
        ws = workspace(sh, True, q.device)
    _call(lib().gdn_backward, "gdn_backward", ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(v),
          _ptr(g), _ptr(beta), _ptr(h0), _ptr(dO), _ptr(dhT), _ptr(dq), _ptr(dk), _ptr(dv),
          _ptr(dg), _ptr(dbeta), _ptr(dh0), _ptr(ws), ws.numel(), _stream())
    return dq, dk, dv, dg, dbeta, dh0


def gdn_forward_train(q, k, v, g, beta, h0=None, *, scale=None, chunk=None, o=None, hT=None,
                      ws=None, use_qk_l2norm=False, wy_eps=0.0, clip=0.0, diag=False):
    """Training forward: as gdn_forward, and leaves residuals in `ws` (a
    backward-sized workspace, returned) for gdn_backward_train.
    Returns (o, hT, ws)."""
    _check_inputs(q, k, v, g, beta)
    sh = make_shape(q, v, g, scale, chunk, use_qk_l2norm, wy_eps, clip, diag)
    _check_shape(h0, "h0", _state_shape(sh), torch.float32)
    _check_shape(o, "o", v.shape, q.dtype)
    _check_shape(hT, "hT", _state_shape(sh), torch.float32)
    _check_ws(ws)
    B, T, H, _ = q.shape
    if o is None:
        o = torch.empty((B, T, H, sh.Dv), dtype=q.dtype, device=q.device)
    if hT is None:
        hT = torch.empty((B, H, sh.Dk, sh.Dv), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = workspace(sh, True, q.device)
    _call(lib().gdn_forward_train, "gdn_forward_train", ctypes.byref(sh), _ptr(q), _ptr(k),
          _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o), _ptr(hT), _ptr(ws), ws.numel(),
          _stream())
    return o, hT, ws


def gdn_backward_train(q, k, v, g, beta, dO, ws, dhT=None, *, scale=None, chunk=None,
                       want_dh0=True, out=None, use_qk_l2norm=False, wy_eps=0.0, clip=0.0,
                       diag=False):
    """Training backward from the residuals gdn_forward_train left in `ws`."""
    _check_inputs(q, k, v, g, beta)
    sh = make_shape(q, v, g, scale, chunk, use_qk_l2norm, wy_eps, clip, diag)
    _check_shape(dO, "dO", v.shape, q.dtype)
    _check_shape(dhT, "dhT", _state_shape(sh), torch.float32)
    _check(ws, "ws")
    if out is not None:
        if len(out) != 6:
            raise ValueError("out must be (dq, dk, dv, dg, dbeta, dh0)")
        for t, name, shape, dt in zip(out, ("dq", "dk", "dv", "dg", "dbeta", "dh0"),
                                      (q.shape, k.shape, v.shape, g.shape, beta.shape,
                                       _state_shape(sh)),
                                      (q.dtype, q.dtype, q.dtype, torch.float32, torch.float32,
                                       torch.float32)):
            if t is None and name != "dh0":
                raise ValueError(f"out: {name} is required")
            _check_shape(t, name, shape, dt)
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(g),
               torch.empty_like(beta),
               torch.empty((sh.B, sh.H, sh.Dk, sh.Dv), dtype=torch.float32, device=q.device)
               if want_dh0 else None)
    dq, dk, dv, dg, dbeta, dh0 = out
    _call(lib().gdn_backward_train, "gdn_backward_train", ctypes.byref(sh), _ptr(q), _ptr(k),
          _ptr(v), _ptr(g), _ptr(beta), _ptr(dO), _ptr(dhT), _ptr(dq), _ptr(dk), _ptr(dv),
          _ptr(dg), _ptr(dbeta), _ptr(dh0), _ptr(ws), ws.numel(), _stream())
    return dq, dk, dv, dg, dbeta, dh0


def gdn_diag_read(shape: GdnShape, ws) -> dict:
    """Stage counters of the last chunked forward pass run in `ws` (shape with
    diag set): {stage: (non-finite, |x| > 1e6)}.  Synchronises the stream."""
    _check(ws, "ws")
    buf = (ctypes.c_uint * (2 * len(DIAG_STAGES)))()
    _call(lib().gdn_diag_read, "gdn_diag_read", ctypes.byref(shape), _ptr(ws), buf, _stream())
    return {st: (int(buf[2 * i]), int(buf[2 * i + 1])) for i, st in enumerate(DIAG_STAGES)}


def gdn_decode_step(q, k, v, g, beta, state, *, scale=None, o=None, use_qk_l2norm=False):
    """One token for every (b, h); q,k [B,1,H,Dk] (or [B,H,Dk]), state updated in place."""
    if q.dim() == 3:
        q, k, v = q.unsqueeze(1), k.unsqueeze(1), v.unsqueeze(1)
        g = g.unsqueeze(1)
        beta = beta.unsqueeze(1)
    _check_inputs(q, k, v, g, beta)
    sh = make_shape(q, v, g, scale, None, use_qk_l2norm)
    _check_shape(state, "state", _state_shape(sh), torch.float32)
    _check_shape(o, "o", (sh.B, 1, sh.H, sh.Dv), q.dtype)
    if o is None:
        o = torch.empty((sh.B, 1, sh.H, sh.Dv), dtype=q.dtype, device=q.device)
    _call(lib().gdn_decode_step, "gdn_decode_step", ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(v),
          _ptr(g), _ptr(beta), _ptr(state), _ptr(o), _stream())
    return o


# ---------------------------------------------------------------------------
# decode from a checkpoint plus a buffer of recent tokens (include/gdn.h)
# ---------------------------------------------------------------------------
def _replay_shape(B, H, Dk, Dv, per_channel, dtype=GDN_F32, scale=None):
    decay = GDN_DECAY_PER_CHANNEL if per_channel else GDN_DECAY_PER_HEAD
    return GdnShape(B, 1, H, Dk, Dv, dtype, decay, 0.0 if scale is None else float(scale), 0)


def gdn_replay_buffer(B: int, H: int, Dk: int, Dv: int, depth: int, *, per_channel=True,
                      device="cuda") -> torch.Tensor:
    """An empty token buffer of the given depth (1..16) for B x H sequences."""
    sh = _replay_shape(B, H, Dk, Dv, per_channel)
    n = int(lib().gdn_replay_buffer_bytes(ctypes.byref(sh), int(depth)))
    if n == 0:
        raise GdnError(1, "gdn_replay_buffer_bytes")
    buf = torch.empty(n, dtype=torch.uint8, device=device)
    _call(lib().gdn_replay_reset, "gdn_replay_reset", ctypes.byref(sh), _ptr(buf), int(depth),
          _stream())
    return buf


def gdn_replay_step(q, k, v, g, beta, ckpt, buf, depth, *, scale=None, o=None):
    """One token for every (b, h) from the checkpoint and the buffer; q,k
    [B,1,H,Dk] (or [B,H,Dk]).  Returns o; ckpt changes only when the buffer
    fills (it is then folded in)."""
    if q.dim() == 3:
        q, k, v = q.unsqueeze(1), k.unsqueeze(1), v.unsqueeze(1)
        g = g.unsqueeze(1)
        beta = beta.unsqueeze(1)
    _check_inputs(q, k, v, g, beta)
    sh = make_shape(q, v, g, scale, None)
    _check_shape(ckpt, "ckpt", _state_shape(sh), torch.float32)
    _check(buf, "buf")
    _check_shape(o, "o", (sh.B, 1, sh.H, sh.Dv), q.dtype)
    if buf.numel() < int(lib().gdn_replay_buffer_bytes(ctypes.byref(sh), int(depth))):
        raise ValueError("buf is smaller than gdn_replay_buffer_bytes for this shape and depth")
    if o is None:
        o = torch.empty((sh.B, 1, sh.H, sh.Dv), dtype=q.dtype, device=q.device)
    _call(lib().gdn_replay_step, "gdn_replay_step", ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(v),
          _ptr(g), _ptr(beta), _ptr(ckpt), _ptr(buf), int(depth), _ptr(o), _stream())
    return o


def gdn_replay_fold(ckpt, buf, depth, *, per_channel=True):
    """Fold the buffer into the checkpoint: ckpt becomes the current state."""
    _check(ckpt, "ckpt", torch.float32)
    _check(buf, "buf")
    B, H, Dk, Dv = ckpt.shape
    sh = _replay_shape(B, H, Dk, Dv, per_channel)
    if buf.numel() < int(lib().gdn_replay_buffer_bytes(ctypes.byref(sh), int(depth))):
        raise ValueError("buf is smaller than gdn_replay_buffer_bytes for this shape and depth")
    _call(lib().gdn_replay_fold, "gdn_replay_fold", ctypes.byref(sh), _ptr(ckpt), _ptr(buf),
          int(depth), _stream())
