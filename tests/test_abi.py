"""The C-ABI library loads and exports every entry point include/gdn.h declares
(no GPU needed: nothing is computed), and the host-side argument checks reject
bad calls before any launch."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_52_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols(header):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_boundary():
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == ["gdn.h", "gdn_profile.h"]
    assert declared_symbols("gdn.h") == sorted(gdn.EXPORTS)
    assert declared_symbols("gdn_profile.h") == sorted(gdn.PROFILE_EXPORTS)


def test_library_exports_every_declared_symbol():
    L = gdn.lib()
    for name in declared_symbols("gdn.h"):
        assert hasattr(L, name), name
    # the library proper keeps no launch recorder
    for name in declared_symbols("gdn_profile.h"):
        assert not hasattr(L, name), name


def test_measurement_build_exports_the_recorder_too():
    P = ctypes.CDLL(gdn.PROFILE_LIB_PATH)
    for name in declared_symbols("gdn.h") + declared_symbols("gdn_profile.h"):
        assert hasattr(P, name), name


def test_status_strings():
    L = gdn.lib()
    for code in range(6):
        s = L.gdn_status_string(code).decode()
        assert s.startswith(gdn.STATUS[code])


def _shape(**kw):
    d = dict(B=2, T=128, H=3, Dk=128, Dv=128, dtype=0, decay=1, scale=0.0, chunk=0)
    d.update(kw)
    return gdn.GdnShape(**d)


def test_workspace_query():
    L = gdn.lib()
    sh = _shape()
    fwd = L.gdn_workspace_bytes(ctypes.byref(sh), 0)
    bwd = L.gdn_workspace_bytes(ctypes.byref(sh), 1)
    assert 0 < fwd < bwd
    assert fwd % 256 == 0 and bwd % 256 == 0
    for bad in (dict(Dk=100, Dv=100), dict(chunk=32), dict(B=0), dict(dtype=7), dict(decay=3),
                dict(Dk=64, Dv=128), dict(qk_l2norm=2), dict(H=32769)):
        assert L.gdn_workspace_bytes(ctypes.byref(_shape(**bad)), 0) == 0, bad
    # the largest head count a chunk's 32-bit row offsets allow at 128 x 128
    assert L.gdn_workspace_bytes(ctypes.byref(_shape(B=1, T=64, H=32768)), 0) > 0
    # token-heads of one call (last chunk counted whole) below 2^27, so every
    # launch's work-item count stays below 2^32
    assert L.gdn_workspace_bytes(ctypes.byref(_shape(B=2 ** 11, T=2 ** 12, H=16)), 0) == 0
    assert L.gdn_workspace_bytes(ctypes.byref(_shape(B=2 ** 11, T=2 ** 12 - 63, H=16)), 0) == 0
    assert L.gdn_workspace_bytes(ctypes.byref(_shape(B=2 ** 11, T=2 ** 12 - 64, H=16)), 0) > 0
    assert L.gdn_workspace_bytes(ctypes.byref(_shape(B=2 ** 20, T=2 ** 14, H=8)), 0) == 0
    # use_qk_l2norm adds the per-row scale table [chunk-heads][2][C] fp32 to both sizes
    sh_n = _shape(qk_l2norm=1)
    n_ch = 2 * 3 * 2
    extra = -(-(n_ch * 2 * 64 * 4) // 256) * 256
    assert L.gdn_workspace_bytes(ctypes.byref(sh_n), 0) == fwd + extra
    assert L.gdn_workspace_bytes(ctypes.byref(sh_n), 1) == bwd + extra


@pytest.mark.parametrize("bad,code", [
    (dict(B=0), 1), (dict(T=-1), 1), (dict(dtype=5), 1), (dict(decay=9), 1),
    (dict(scale=-1.0), 1), (dict(Dk=48, Dv=48), 2), (dict(chunk=32), 2), (dict(qk_l2norm=-1), 1),
    (dict(wy_eps=-0.5), 1), (dict(wy_eps=float("nan")), 1), (dict(clip=-1.0), 1),
    (dict(clip=float("inf")), 1), (dict(diag=2), 1),
])
def test_forward_rejects_bad_shapes_before_launch(bad, code):
    L = gdn.lib()
    sh = _shape(**bad)
    p = ctypes.c_void_p(256)  # never dereferenced: validation fails first
    rc = L.gdn_forward(ctypes.byref(sh), p, p, p, p, p, None, p, None, p, 1 << 40, None)
    assert rc == code


def test_null_and_misaligned_pointers_rejected():
    L = gdn.lib()
    sh = _shape()
    p = ctypes.c_void_p(256)
    mis = ctypes.c_void_p(258)
    assert L.gdn_forward(ctypes.byref(sh), None, p, p, p, p, None, p, None, p, 1 << 40, None) == 1
    assert L.gdn_forward(ctypes.byref(sh), mis, p, p, p, p, None, p, None, p, 1 << 40, None) == 3
    assert L.gdn_forward(ctypes.byref(sh), p, p, p, p, p, None, p, None, p, 16, None) == 4
    d = _shape(T=1)
    assert L.gdn_decode_step(ctypes.byref(_shape(T=2)), p, p, p, p, p, p, p, None) == 1
    assert L.gdn_decode_step(ctypes.byref(d), p, p, p, p, p, None, p, None) == 1
    assert L.gdn_new_state(None, 1, 1, 16, 16, None) == 1
    assert L.gdn_new_state(mis, 1, 1, 16, 16, None) == 3


def test_profile_recorder_arguments():
    L = ctypes.CDLL(gdn.PROFILE_LIB_PATH)
    L.gdn_profile_begin.argtypes = [ctypes.c_void_p, ctypes.c_int]
    assert L.gdn_profile_begin(None, 4) == 1
    ev = (ctypes.c_void_p * 2)()
    assert L.gdn_profile_begin(ev, 0) == 1
    assert L.gdn_profile_begin(ev, 1 << 20) == 1
    assert L.gdn_profile_end() == 0


def test_safety_options_host_checks():
    """The decode step has no stage boundaries: the options are refused there;
    the counters can only be read with diag set; diag adds one 256-byte region
    and clip two tables to the training workspace."""
    L = gdn.lib()
    p = ctypes.c_void_p(256)
    for kw in (dict(wy_eps=0.1), dict(clip=5.0), dict(diag=1)):
        sh = _shape(T=1, **kw)
        assert L.gdn_decode_step(ctypes.byref(sh), p, p, p, p, p, p, p, None) == 2, kw
    buf = (ctypes.c_uint * 14)()
    assert L.gdn_diag_read(ctypes.byref(_shape()), p, buf, None) == 1
    assert L.gdn_diag_read(ctypes.byref(_shape(diag=1)), None, buf, None) == 1
    base = L.gdn_workspace_bytes(ctypes.byref(_shape()), 0)
    assert L.gdn_workspace_bytes(ctypes.byref(_shape(diag=1)), 0) == base + 256
    bwd = L.gdn_workspace_bytes(ctypes.byref(_shape()), 1)
    assert L.gdn_workspace_bytes(ctypes.byref(_shape(wy_eps=0.3)), 1) == bwd
    # clip: the training forward also keeps W (bf16) before clipping
    n_ch = 2 * 3 * 2
    assert L.gdn_workspace_bytes(ctypes.byref(_shape(clip=8.0)), 1) == bwd + n_ch * 64 * 128 * 2


def test_replay_host_checks():
    """The checkpoint-and-buffer decode: depth 1..16, decode shapes only, and
    the buffer size follows the layout (token count, keys, decays, deltas)."""
    L = gdn.lib()
    sh = _shape(T=1)
    assert L.gdn_replay_buffer_bytes(ctypes.byref(sh), 0) == 0
    assert L.gdn_replay_buffer_bytes(ctypes.byref(sh), 17) == 0
    assert L.gdn_replay_buffer_bytes(ctypes.byref(_shape(T=2)), 4) == 0
    a = lambda x: -(-x // 256) * 256
    BH = 2 * 3
    assert L.gdn_replay_buffer_bytes(ctypes.byref(sh), 4) == \
        a(4 * BH) + a(4 * BH * 4 * 128) + a(4 * BH * 4 * 128) + a(4 * BH * 4 * 128)
    assert L.gdn_replay_buffer_bytes(ctypes.byref(_shape(T=1, decay=0)), 4) == \
        a(4 * BH) + a(4 * BH * 4 * 128) + a(4 * BH * 4) + a(4 * BH * 4 * 128)
    p = ctypes.c_void_p(256)
    assert L.gdn_replay_step(ctypes.byref(sh), p, p, p, p, p, p, p, 0, p, None) == 1
    assert L.gdn_replay_step(ctypes.byref(sh), p, p, p, p, p, None, p, 4, p, None) == 1
    assert L.gdn_replay_step(ctypes.byref(_shape(T=1, clip=1.0)), p, p, p, p, p, p, p, 4, p, None) == 2
    assert L.gdn_replay_fold(ctypes.byref(sh), p, None, 4, None) == 1
    assert L.gdn_replay_reset(ctypes.byref(sh), ctypes.c_void_p(258), 4, None) == 3
