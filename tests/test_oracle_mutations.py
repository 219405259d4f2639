"""Planted mistakes in the oracle must be caught by the pins.

Each case compiles a copy of ``oracle/oracle.c`` with one plausible mistake
(a dropped term, a wrong sign, a wrong index, a transposed operand, a wrong
order of update and readout), points the oracle wrapper at that copy, and
checks that at least one pin in ``test_oracle_pins.py`` fails.  The copies live
in pytest's tmp_path; the real oracle is untouched.
"""
import inspect
import os
import subprocess

import pytest

import oracle
import test_oracle_pins as P

MUTATIONS = {
    "drop_skip_term": ("double out = acc + Dd * x;", "double out = acc;"),
    "bias_after_softplus": ("oracle_softplus(dr[l] + bias)", "(oracle_softplus(dr[l]) + bias)"),
    "readout_before_update": (
        "      h[n] = abar * h[n] + bbar * x;\n      acc += Cb[n * L + l] * h[n];",
        "      acc += Cb[n * L + l] * h[n];\n      h[n] = abar * h[n] + bbar * x;"),
    "wrong_sign_bbar": ("return expm1(delta * a) / a;", "return -expm1(delta * a) / a;"),
    "C_used_as_B": ("* Bb[n * L + l];", "* Cb[n * L + l];"),
    "transposed_B_index": ("Bb[n * L + l]", "Bb[l * N + n]"),
    "skip_outside_gate": (
        "    double out = acc + Dd * x;\n    if (z) out *= silu(z[l]);",
        "    double out = acc;\n    if (z) out *= silu(z[l]);\n    out += Dd * x;"),
    "delta_b_instead_of_zoh": ("return expm1(delta * a) / a;", "return delta;"),
    "ignores_initial_state": ("h[n] = j->h0 ? j->h0[ch * N + n] : 0.0;", "h[n] = 0.0;"),
    "sigmoid_not_silu": ("return z / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(-z));"),
    "abar_wrong_sign": ("const double abar = exp(delta * a);", "const double abar = exp(-delta * a);"),
    "conv_taps_reversed": ("acc += wd[i] * ORACLE_CONV_IN(s);", "acc += wd[K - 1 - i] * ORACLE_CONV_IN(s);"),
    "conv_reads_future": ("const int64_t s = t - i;", "const int64_t s = (t + i < L) ? t + i : t;"),
    "conv_drops_bias": ("double acc = bias ? bias[d] : 0.0;", "double acc = 0.0;"),
    "conv_state_off_by_one": ("(s0 ? s0[K + (s)] : 0.0)", "(s0 ? s0[K - 1 + (s) + ((s) == -K)] : 0.0)"),
    "conv_final_state_shifted": ("const int64_t s = L - K + k;", "const int64_t s = L - K + k - 1;"),
    "bwd_drops_state_carry": ("const double gn = dyc * Cb[n * L + l] + anext[n] * g[n];",
                              "const double gn = dyc * Cb[n * L + l];"),
    "bwd_dcoef_ddelta_wrong": ("ddelta += dabar * a * abar + dcoef * abar;", "ddelta += dabar * a * abar + dcoef;"),
    "bwd_dA_misses_coef_term": ("j->dA[d * N + n] += dabar * delta * abar + dcoef * delta * delta * phi_coef(delta * a);",
                                "j->dA[d * N + n] += dabar * delta * abar;"),
    "bwd_softplus_grad_dropped": ("const double dr_l = ddelta * sigmoid(dr[l] + bias);", "const double dr_l = ddelta;"),
    "bwd_dB_misses_coef": ("j->dBt[b * N * L + n * L + l] += gn * coef * x;", "j->dBt[b * N * L + n * L + l] += gn * x;"),
    "bwd_dC_uses_previous_state": ("j->dCt[b * N * L + n * L + l] += dyc * H[(l + 1) * N + n];",
                                   "j->dCt[b * N * L + n * L + l] += dyc * H[l * N + n];"),
    "bwd_dsilu_incomplete": ("s * (1.0 + z[l] * (1.0 - s))", "s"),
    "bwd_phi_series_wrong": ("double term = 0.5, sum = 0.0;", "double term = 1.0, sum = 0.0;"),
}


def _run_pins():
    failed = []
    for name in sorted(n for n in dir(P) if n.startswith("test_")):
        fn = getattr(P, name)
        params = inspect.signature(fn).parameters
        try:
            if "shape" in params:
                fn(6, (2, 3, 7, 41), True)
            elif "seed" in params:
                fn(3)
            else:
                fn()
        except Exception:
            failed.append(name)
    return failed


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path, monkeypatch):
    before, after = MUTATIONS[name]
    src = open(oracle._SRC, encoding="utf-8").read()
    assert before in src, "mutation anchor not found; update the mutation list"
    mut_c = tmp_path / "oracle_mut.c"
    mut_so = tmp_path / "liboracle_mut.so"
    mut_c.write_text(src.replace(before, after), encoding="utf-8")
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-o", str(mut_so), str(mut_c), "-lm", "-lpthread"],
                   check=True)
    monkeypatch.setattr(oracle, "_LIB", str(mut_so))
    monkeypatch.setattr(oracle, "_SRC", str(mut_c))
    monkeypatch.setattr(oracle, "_lib", None)
    failed = _run_pins()
    monkeypatch.setattr(oracle, "_lib", None)
    assert failed, "planted mistake %r passed every pin" % name
