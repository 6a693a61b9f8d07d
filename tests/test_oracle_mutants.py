"""Planted mistakes in the C oracle must fail at least one pin.

Each mutant is the oracle source with one plausible mistake (a dropped term, a
wrong sign, a wrong index, a skipped read or write), compiled with gcc into a
temporary directory.  This shows the pins are strong enough to catch such a
mistake in the oracle itself.  CPU only; the real oracle is never modified.
"""
import os
import tempfile

import pytest

import pins
from oracle.build import SRC, compile_oracle
from oracle.recurrent import OracleLib

MUTANTS = {
    "decay_sign": ("const double d = exp(g[i]);", "const double d = exp(-g[i]);"),
    "decay_on_value_channel": ("for (int64_t j = 0; j < dv; ++j) row[j] *= d;",
                               "for (int64_t j = 0; j < dv; ++j) row[j] *= exp(g[j % dk]);"),
    "no_erase": ("u[j] = beta * (v[j] - u[j]);", "u[j] = beta * v[j];"),
    "erase_sign": ("u[j] = beta * (v[j] - u[j]);", "u[j] = beta * (v[j] + u[j]);"),
    "no_beta": ("u[j] = beta * (v[j] - u[j]);", "u[j] = (v[j] - u[j]);"),
    "erase_uses_query": ("const double ki = k[i];\n    const double* row = S + i * dv;\n"
                         "    for (int64_t j = 0; j < dv; ++j) u[j] += row[j] * ki;",
                         "const double ki = q[i];\n    const double* row = S + i * dv;\n"
                         "    for (int64_t j = 0; j < dv; ++j) u[j] += row[j] * ki;"),
    "read_with_key": ("const double qi = q[i];", "const double qi = k[i];"),
    "no_scale": ("o[j] *= scale;", "o[j] *= 1.0;"),
    "h0_ignored": ("if (h0)\n", "if (0)\n"),
    "ht_not_written": ("if (ht) memcpy", "if (0) memcpy"),
    "no_sequence_reset": ("for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t)",
                          "for (int64_t t = 0; t < cu_seqlens[n + 1]; ++t)"),
    "decay_dropped": ("  /* decay: row i of S is multiplied by exp(g_i) */\n  for (int64_t i = 0; i < dk; ++i) {",
                          "  for (int64_t i = 0; i < dk && 0; ++i) {"),
    "read_before_write": ("  /* S += k u^T */", "  for (int64_t j = 0; j < dv; ++j) o[j] = 0.0;\n"
                          "  for (int64_t i = 0; i < dk; ++i) for (int64_t j = 0; j < dv; ++j)"
                          " o[j] += S[i * dv + j] * q[i] * scale;\n  return;\n  /* S += k u^T */"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found in the oracle source"
    with tempfile.TemporaryDirectory() as td:
        path = os.path.join(td, "mut.c")
        open(path, "w").write(src.replace(old, new, 1))
        lib = OracleLib(compile_oracle(path, os.path.join(td, "libmut.so"), werror=False))
        failed = []
        for pin in pins.ALL_PINS:
            try:
                pin(lib)
            except (AssertionError, RuntimeError, ValueError, FloatingPointError):
                failed.append(pin.__name__)
        assert failed, f"mutant {name} passed every pin"
