"""The benchmark reports nothing unless its correctness checks pass (atomic_ops
card, "Reproduce": rows that do not match are rejected).  CPU only: the gate is
one function of bench.py, fed here with made-up check results."""
import json

import pytest

import bench


def test_failed_check_prints_no_line_and_exits_nonzero(capsys):
    line = {"metric": "tokens/s", "value": 123.0}
    with pytest.raises(SystemExit) as exc:
        bench.emit(line, {"fwd+bwd B=8 bf16": True, "variant f32": False})
    assert exc.value.code not in (0, None)
    out = capsys.readouterr()
    assert out.out == ""
    assert "variant f32" in out.err


def test_gate_alone_exits_on_any_failure(capsys):
    with pytest.raises(SystemExit) as exc:
        bench.parity_gate({"decode": False})
    assert exc.value.code == 3
    assert capsys.readouterr().out == ""


def test_passing_checks_print_one_line(capsys):
    line = {"metric": "tokens/s", "value": 123.0}
    bench.emit(line, {"fwd+bwd B=8 bf16": True, "decode": True})
    out = capsys.readouterr().out.strip().splitlines()
    assert len(out) == 1 and json.loads(out[0])["value"] == 123.0


def test_method_bytes_follow_the_method():
    """Step bytes per token-head: each input read once, each output written
    once (bf16 128x128 per channel: 1,540 forward, 4,364 forward + backward;
    fp32: 2,564 and 7,180)."""
    assert bench.method_step_bytes(128, 2, backward=False) == 1540
    assert bench.method_step_bytes(128, 2) == 4364
    assert bench.method_step_bytes(128, 4, backward=False) == 2564
    assert bench.method_step_bytes(128, 4) == 7180
