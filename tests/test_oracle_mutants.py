"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins catch every one: a dropped term, a wrong sign, a wrong index, a
transposed operand, a wrong order of the steps.  The real oracle source is
never modified; each mutant is compiled from a temporary copy."""
import os

import pytest

import oracle
import pins

MUTANTS = {
    # forward
    "decay_columns_not_rows": ("S[i * Dv + j] *= a[i];", "S[i * Dv + j] *= a[j % d->Dk];"),
    "delta_sign": ("dd[j] = bt * (vt[j] - m[j]);", "dd[j] = bt * (vt[j] + m[j]);"),
    "delta_dropped": ("dd[j] = bt * (vt[j] - m[j]);", "dd[j] = bt * vt[j];"),
    "beta_dropped": ("dd[j] = bt * (vt[j] - m[j]);", "dd[j] = (vt[j] - m[j]);"),
    "read_transposed": ("s += kt[i] * S[i * Dv + j];", "s += kt[i] * S[j * Dv + i];"),
    "read_before_write": ("step(d, S, a, k + r * Dk, v + r * Dv, beta[r], m, dd);\n"
                          "        read_out(d, S, q + r * Dk, o + r * Dv);",
                          "read_out(d, S, q + r * Dk, o + r * Dv);\n"
                          "        step(d, S, a, k + r * Dk, v + r * Dv, beta[r], m, dd);"),
    "per_channel_collapsed": ("a[i] = exp(gp[i]);", "a[i] = exp(gp[0]);"),
    "scale_dropped": ("ot[j] = d->scale * s;", "ot[j] = s;"),
    "h0_ignored": ("if (h0) memcpy(S, h0 + sidx, sizeof(real) * Dk * Dv);", ""),
    "decay_after_read": ("for (int i = 0; i < Dk; ++i)\n        for (int j = 0; j < Dv; ++j) S[i * Dv + j] *= a[i];\n"
                         "    for (int j = 0; j < Dv; ++j) {\n        real s = 0.0;\n        for (int i = 0; i < Dk; ++i) s += kt[i] * S[i * Dv + j];\n        m[j] = s;\n    }",
                         "for (int j = 0; j < Dv; ++j) {\n        real s = 0.0;\n        for (int i = 0; i < Dk; ++i) s += kt[i] * S[i * Dv + j];\n        m[j] = s;\n    }\n"
                         "    for (int i = 0; i < Dk; ++i)\n        for (int j = 0; j < Dv; ++j) S[i * Dv + j] *= a[i];"),
    # backward
    "dbeta_sign": ("dbeta[r] = db;", "dbeta[r] = -db;"),
    "dg_uses_undecayed_state": ("s2 += dS[i * Dv + j] * Sp[i * Dv + j];",
                                "s2 += dS[i * Dv + j] * Sm1[i * Dv + j];"),
    "dk_read_term_dropped": ("dk[r * Dk + i] += s2;", "dk[r * Dk + i] += 0.0 * s2;"),
    "dS_wrong_cotangent": ("dS[i * Dv + j] += kt[i] * dm[j];", "dS[i * Dv + j] += kt[i] * ddv[j];"),
    "dq_scale_dropped": ("dq[r * Dk + i] = d->scale * s2;", "dq[r * Dk + i] = s2;"),
    "dS_not_decayed": ("for (int j = 0; j < Dv; ++j) dS[i * Dv + j] *= a[i];", ""),
    "dv_beta_dropped": ("dv[r * Dv + j] = bt * ddv[j];", "dv[r * Dv + j] = ddv[j];"),
    "dh0_not_carried": ("if (dh0) memcpy(dh0 + sidx, dS, sizeof(real) * SS);",
                        "if (dh0) memset(dh0 + sidx, 0, sizeof(real) * SS);"),
    # use_qk_l2norm prologue
    "l2norm_projection_dropped": ("inv * (dxhat[r * D + c] - x[r * D + c] * inv * dot)",
                                  "inv * dxhat[r * D + c]"),
    "l2norm_sqrt_dropped": ("const real inv = 1.0 / sqrt(s + eps);\n        for (int c = 0; c < D; ++c) xhat",
                            "const real inv = 1.0 / (s + eps);\n        for (int c = 0; c < D; ++c) xhat"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    with open(oracle.SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new, 1)
    path = os.path.join(tmp_path, "mutant.c")
    with open(path, "w") as f:
        f.write(mutated)
    so = oracle.build(force=True, src=path, out=os.path.join(tmp_path, "libmutant.so"))
    lib = oracle.load(so)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            if pin in (pins.pin_fd_gradients, pins.pin_l2norm_fd):
                pin(lib, seeds=(0,))
            else:
                pin(lib)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name}"
