"""Planted mistakes in the oracle (on the CPU) must each fail at least one pin.

Each mutant is the oracle's C source with one plausible slip applied
textually (a flipped sign, a dropped term, a wrong operand, a misplaced gate,
an off-by-one range, a transposed read), built with gcc into a temporary
library and run through every pin.  A mutant that passes all pins would mean
the pins cannot tell that slip from the definition.
"""
import functools
import os
import subprocess
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import oracle_pins as P  # noqa: E402

MUTANTS = {
    "delta_sign": [("be * (vt[r] - p)", "be * (vt[r] + p)")],
    "beta_dropped": [(": be * (vt[r] - p)", ": (vt[r] - p)")],
    "gate_after_predict": [("row[c] *= ga[c]; p += row[c] * kt[c];", "p += row[c] * kt[c]; row[c] *= ga[c];")],
    "gate_after_write": [("row[c] *= ga[c]; p += row[c] * kt[c];", "p += row[c] * kt[c];"),
                         ("row[c] += e * kt[c];", "row[c] = ga[c] * (row[c] + e * kt[c]);")],
    "gate_ignored": [("exp(j->log_alpha[x])", "1.0")],
    "gate_squared": [("exp(j->log_alpha[x])", "exp(2.0 * j->log_alpha[x])")],
    "write_dropped": [("const double e = j->no_erase", "const double e = 0.0 * (j->no_erase"),
                      ("be * (vt[r] - p);", "be * (vt[r] - p));")],
    "read_with_key": [("o += row[c] * qt[c];", "o += row[c] * kt[c];")],
    "write_along_query": [("row[c] += e * kt[c];", "row[c] += e * qt[c];")],
    "read_transposed_state": [("o += row[c] * qt[c];", "o += S[(c % Dv) * Dk + (r % Dk)] * qt[c];")],
    "initial_state_ignored": [("if (j->S0) memcpy", "if (0) memcpy")],
    "sequence_end_off_by_one": [("t1 = j->cu[n + 1]; }", "t1 = j->cu[n + 1] - (j->cu[n + 1] > j->cu[n]); }")],
    # per-channel gate
    "vector_gate_ignored": [("ga[c] = exp(j->log_alpha[x * Dk + c]);", "ga[c] = 1.0;")],
    "vector_gate_channels_reversed": [("exp(j->log_alpha[x * Dk + c])", "exp(j->log_alpha[x * Dk + (Dk - 1 - c)])")],
    "vector_gate_on_value_side": [("row[c] *= ga[c];", "row[c] *= ga[r % Dk];")],
    "vector_gate_first_channel_only": [("exp(j->log_alpha[x * Dk + c])", "exp(j->log_alpha[x * Dk])")],
}


@pytest.fixture(scope="module")
def oracle_src(oracle_mod):
    with open(oracle_mod._SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, oracle_src, oracle_mod, tmp_path):
    src = oracle_src
    for old, new in MUTANTS[name]:
        assert old in src, f"mutation site {old!r} not found"
        src = src.replace(old, new)
    c = tmp_path / f"m_{name}.c"
    so = tmp_path / f"m_{name}.so"
    c.write_text(src)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-w",
                           "-o", str(so), str(c), "-lm"])
    lib = oracle_mod._bind(str(so))
    fwd = functools.partial(oracle_mod.forward, lib=lib)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(forward=fwd, wy_vectors=oracle_mod.wy_vectors, u_vectors=oracle_mod.u_vectors)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
