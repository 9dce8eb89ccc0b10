"""Planted mistakes in the oracle are caught by its pins.

Each case copies ``oracle/lao.c``, plants one plausible bug in the copy
(a dropped decay term, a transposed operand, a wrong index), compiles it with
gcc into a temporary directory and swaps it in for the real oracle; at least
one pin of ``test_oracle_pins`` must then fail.  Runs on the CPU only.
"""
import ctypes
import os
import subprocess

import pytest

from oracle import lao
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(lao.__file__), "lao.c")

MUTATIONS = [
    ("decay dropped in the forward state update",
     "S[i * w + j] = l * S[i * w + j] + ki * v[t * dv + c0 + j];",
     "S[i * w + j] = S[i * w + j] + ki * v[t * dv + c0 + j];",
     [lambda: pins.test_recurrence_equals_quadratic_form(77, 16, 24)]),
    ("initial state read transposed",
     "S[i * w + j] = S0 ? S0[(n * dk + i) * dv + c0 + j] : 0.0;",
     "S[i * w + j] = S0 ? S0[(n * dv + c0 + j) * dk + i] : 0.0;",
     [pins.test_hand_example_forward,
      lambda: pins.test_recurrence_equals_quadratic_form(300, 64, 64)]),
    ("query read at the mirrored token",
     "acc += q[t * dk + i] * S[i * w + j];",
     "acc += q[(Ls - 1 - t) * dk + i] * S[i * w + j];",
     [pins.test_hand_example_forward]),
    ("decay dropped in the backward reverse sweep (dk)",
     "U[i * dv + j] = l * G;",
     "U[i * dv + j] = G;",
     [pins.test_backward_closed_forms]),
    ("dv contracted with q instead of k",
     "acc[j] += G * ki;",
     "acc[j] += G * qi;",
     [pins.test_backward_closed_forms]),
    ("dq contracted with v instead of dO",
     "acc += S[i * dv + j] * g[t * dv + j];",
     "acc += S[i * dv + j] * v[t * dv + j];",
     [pins.test_backward_finite_differences]),
    ("segment decay dropped in the scan",
     "X = a * X + dS[(bh * P + s) * E + e];",
     "X = X + dS[(bh * P + s) * E + e];",
     [pins.test_hand_example_scan]),
    ("initial state under-decayed in the sampled rows",
     "const double w0 = lao_pow(l, t + 1);",
     "const double w0 = lao_pow(l, t);",
     [pins.test_hand_example_rows]),
    ("gate applied after the new token is added",
     "S[i * w + j] = a * S[i * w + j] + ki * v[t * dv + c0 + j];",
     "S[i * w + j] = a * (S[i * w + j] + ki * v[t * dv + c0 + j]);",
     [pins.test_gated_hand_example,
      lambda: pins.test_gated_recurrence_equals_quadratic_form(77, 16, 24)]),
    ("initial state skipped in the gated recurrence",
     "S[i * w + j] = s0 ? s0[i * dv + c0 + j] : 0.0;",
     "S[i * w + j] = 0.0;",
     [pins.test_gated_hand_example,
      lambda: pins.test_gated_recurrence_equals_quadratic_form(77, 16, 24)]),
    ("gate of the previous token",
     "const double a = exp(g[t]);",
     "const double a = exp(g[t > 0 ? t - 1 : 0]);",
     [pins.test_gated_hand_example,
      lambda: pins.test_gated_recurrence_equals_quadratic_form(300, 64, 64)]),
    ("segment decay of the neighbouring segment in the gated scan",
     "X = exp(LD[bh * P + s]) * X + dS[(bh * P + s) * E + e];",
     "X = exp(LD[bh * P + (s + 1) % P]) * X + dS[(bh * P + s) * E + e];",
     [pins.test_gated_hand_example_scan, pins.test_gated_segments_with_scanned_starts_equal_monolithic]),
    ("gate of the wrong token in the gated reverse sweep (dv)",
     """      for (int64_t t = Ls - 1; t >= 0; --t) {
        const double a = exp(gl[t]);
        for (int64_t j = 0; j < w; ++j) acc[j] = 0.0;""",
     """      for (int64_t t = Ls - 1; t >= 0; --t) {
        const double a = exp(gl[t > 0 ? t - 1 : 0]);
        for (int64_t j = 0; j < w; ++j) acc[j] = 0.0;""",
     [lambda: pins.test_gated_backward_finite_differences(150)]),
    ("gate factor dropped from the log-gate gradient",
     "dG[n * Ls + t] = exp(Gl[n * Ls + t]) * sum;",
     "dG[n * Ls + t] = sum;",
     [lambda: pins.test_gated_backward_finite_differences(65), pins.test_gated_log_gate_gradient_identity]),
    ("state after the token instead of before it in the log-gate gradient",
     "const double* Sprev = run + (size_t)(t - t0) * blk; /* S_{t-1} */",
     "const double* Sprev = run + (size_t)(t - t0 + (t + 1 < t1 ? 1 : 0)) * blk; /* S_{t-1} */",
     [lambda: pins.test_gated_backward_finite_differences(150)]),
]


@pytest.mark.parametrize("name,old,new,checks", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, monkeypatch, name, old, new, checks):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site not unique: {old}"
    mutated = tmp_path / "lao_mut.c"
    mutated.write_text(src.replace(old, new))
    so = tmp_path / "liblao_mut.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                           "-ffp-contract=off", str(mutated), "-o", str(so), "-lm"])
    monkeypatch.setattr(lao, "_lib", lao.bind(ctypes.CDLL(str(so))))
    caught = 0
    for check in checks:
        try:
            check()
        except AssertionError:
            caught += 1
    assert caught == len(checks), f"planted mistake '{name}' went unnoticed"
