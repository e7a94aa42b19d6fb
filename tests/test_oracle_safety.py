"""The chunked oracle with the numerical-safety options against its pins, and
planted mistakes in copies of it that the pins must catch (CPU only)."""
import importlib.util
import os

import pytest

import pins_safety as ps
from oracle import chunked

SRC = chunked.__file__


@pytest.mark.parametrize("pin", ps.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(chunked)


MUTANTS = {
    "damping_dropped": ("M = (1.0 + wy_eps) * eye + A", "M = eye + A"),
    "damping_sign": ("M = (1.0 + wy_eps) * eye + A", "M = (1.0 - wy_eps) * eye + A"),
    "damping_on_A": ("M = (1.0 + wy_eps) * eye + A", "M = eye + (1.0 + wy_eps) * A"),
    "A_with_diagonal": ("A = torch.where(low_strict,", "A = torch.where(low_incl,"),
    "P_without_diagonal": ("P = torch.where(low_incl, qk", "P = torch.where(low_strict, qk"),
    "W_without_gamma": ("W = Tm @ (b_[..., None] * k_ * Gam)", "W = Tm @ (b_[..., None] * k_)"),
    "decay_transposed": ("diff = G[:, :, :, None, :] - G[:, :, None, :, :]",
                         "diff = G[:, :, None, :, :] - G[:, :, :, None, :]"),
    "state_decay_dropped": ("S = torch.exp(Gl_last[:, :, 0, :, None]) * S +", "S = S +"),
    "nan_kept": ("nan=0.0, posinf=c, neginf=-c", "posinf=c, neginf=-c, nan=float('nan')"),
    "U_not_clipped": ('U = _boundary(U, "U", clip, counts)', "U = U"),
    "o_not_clipped": ('o = _boundary(o, "o", clip, counts)', "o = o"),
    "counts_after_clip": ('    if counts is not None:\n        xv = x.detach()',
                          '    if counts is not None:\n        x = _Clip.apply(x, clip) if clip else x\n'
                          '        xv = x.detach()'),
    "large_threshold_inclusive": ("xv.abs() > DIAG_LARGE", "xv.abs() >= 0.5 * DIAG_LARGE"),
}


def _load_variant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, name
    src = src.replace(old, new).replace("from . import _f64", "from oracle import _f64")
    path = os.path.join(tmp_path, f"chunked_{name}.py")
    with open(path, "w") as fh:
        fh.write(src)
    spec = importlib.util.spec_from_file_location(f"chunked_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_caught(tmp_path, name):
    mod = _load_variant(str(tmp_path), name, *MUTANTS[name])
    for pin in ps.ALL_PINS:
        try:
            pin(mod)
        except Exception:
            return
    pytest.fail(f"planted mistake {name} passed every pin")
