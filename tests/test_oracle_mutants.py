"""Plant plausible mistakes in copies of the C oracle (on the CPU) and check that the pins catch
every one.  The real oracle source is never modified: each mutant is a text edit of a temporary
copy, compiled with gcc into a temporary directory."""
import functools
import os
import subprocess

import pytest

import oracle
from tests import oracle_pins as P
from tests.test_oracle_pins import oracle_api

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")

_UPDATE = """    /* S <- S + u k_t^T */
    for (int32_t i = 0; i < dv; ++i)
      for (int32_t j = 0; j < dk; ++j) S[(int64_t)i * dk + j] += u[i] * kt[j];
"""
_READOUT = """    /* o_t = S q_t */
    double *ot = o + (t * Hv + h) * dv;
    for (int32_t i = 0; i < dv; ++i) {
      double acc = 0.0;
      for (int32_t j = 0; j < dk; ++j) acc += S[(int64_t)i * dk + j] * qt[j];
      ot[i] = acc;
    }
"""
_DECAY = """    /* S <- exp(g_t) S */
    for (int64_t e = 0; e < (int64_t)dv * dk; ++e) S[e] *= decay;
"""
_DELTA = """    /* u = beta_t (v_t - S k_t) */
    for (int32_t i = 0; i < dv; ++i) {
      double sk = 0.0;
      for (int32_t j = 0; j < dk; ++j) sk += S[(int64_t)i * dk + j] * kt[j];
      u[i] = bt * (vt[i] - sk);
    }
"""

MUTANTS = {
    "dropped_decay": [("S[e] *= decay;", "S[e] *= 1.0;")],
    "decay_sign": [("const double decay = exp(gt);", "const double decay = exp(-gt);")],
    "delta_sign": [("u[i] = bt * (vt[i] - sk);", "u[i] = bt * (vt[i] + sk);")],
    "dropped_beta": [("u[i] = bt * (vt[i] - sk);", "u[i] = (vt[i] - sk);")],
    "beta_squared": [("u[i] = bt * (vt[i] - sk);", "u[i] = bt * bt * (vt[i] - sk);")],
    "h0_transposed": [("h0_nh ? h0_nh[(int64_t)j * dv + i]", "h0_nh ? h0_nh[(int64_t)i * dk + j]")],
    "hT_transposed": [("hT_nh[(int64_t)j * dv + i] = S", "hT_nh[(int64_t)i * dk + j] = S")],
    "readout_with_key": [("acc += S[(int64_t)i * dk + j] * qt[j];", "acc += S[(int64_t)i * dk + j] * kt[j];")],
    "readout_before_update": [(_UPDATE + _READOUT, _READOUT + _UPDATE)],
    "delta_on_undecayed_state": [(_DECAY + _DELTA, _DELTA + _DECAY)],
    "gqa_modulo_map": [("const int32_t hk = h / group;", "const int32_t hk = h % Hk;")],
    "sequence_start_ignored": [("recur_one(cu[n], cu[n + 1],", "recur_one(n ? cu[n] - 1 : 0, cu[n + 1],")],
    "conv_crosses_sequences": [("if (src >= cu[n]) c +=", "if (src >= 0) c +=")],
    "conv_tap_reversed": [("c += w[(int64_t)ch * taps + j] * x[src", "c += w[(int64_t)ch * taps + (taps - 1 - j)] * x[src")],
    "rmsnorm_sum_not_mean": [("sqrt(ms / dv + eps_norm)", "sqrt(ms + eps_norm)")],
    "gate_without_silu": [("norm_w[j] * zs[j] * sigmoid(zs[j])", "norm_w[j] * sigmoid(zs[j])")],
    "l2norm_missing_on_k": [("k[(t * Hk + hh) * dk + j] = ks[j] * rk;", "k[(t * Hk + hh) * dk + j] = ks[j];")],
    "bf16_ties_away": [("(diff == 0.5 && fmod(r, 2.0) != 0.0)", "(diff == 0.5)")],
    "bf16_truncates": [("if (diff > 0.5 ||", "if (0 &&")],
    "state_index_ignored": [("const int64_t r = h0_index ? h0_index[n] : n;", "const int64_t r = n;")],
    "out_of_range_index_reads_row_0": [("(h0 && r >= 0 && r < num_h0) ? h0 + (r * Hv + h) * state",
                                        "h0 ? h0 + ((r >= 0 && r < num_h0) ? r : 0) * Hv * state + h * state")],
    "window_index_ignored": [("const int64_t r = state_index ? state_index[n] : n;", "const int64_t r = n;")],
    "window_ignored": [("else if (win) c +=", "else if (0) c +=")],
    "window_reversed": [("win[(src - cu[n] + taps - 1) * C + ch];", "win[(cu[n] - 1 - src) * C + ch];")],
    "window_out_shifted": [("const int64_t p = cu[n + 1] - (taps - 1) + j;", "const int64_t p = cu[n + 1] - taps + j;")],
    "window_out_drops_carried": [("else if (win) val =", "else if (0) val =")],
    "bf16_point_on_o_missing": [("for (int64_t e = 0; e < T * Cv; ++e) o[e] = oracle_round_bf16(o[e]);", ";")],
    "gate_sign": [("g[i] = -exp(A_log[h]) *", "g[i] = exp(A_log[h]) *")],
    "gate_A_log_not_exponentiated": [("g[i] = -exp(A_log[h]) *", "g[i] = -A_log[h] *")],
    "gate_dt_bias_dropped": [("softplus(a[i] + dt_bias[h])", "softplus(a[i])")],
    "gate_softplus_as_exp": [("return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x));", "return exp(x);")],
    "beta_not_sigmoid": [("beta[i] = sigmoid(b[i]);", "beta[i] = b[i];")],
}


def _build(tmp_path, name, edits):
    src = open(SRC).read()
    for old, new in edits:
        assert src.count(old) == 1, f"mutant {name}: anchor not found exactly once"
        src = src.replace(old, new)
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"{name}.so"
    c.write_text(src)
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", str(c), "-o", str(so), "-lm"],
                   check=True)
    return oracle.load_library(str(so))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    lib = _build(tmp_path, name, MUTANTS[name])
    fwd = functools.partial(oracle.gdn_fwd, lib=lib)
    conv = functools.partial(oracle.conv_silu, lib=lib)
    mixer = functools.partial(oracle.mixer_fwd, lib=lib)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(fwd)
        except (AssertionError, RuntimeError, ValueError):
            caught.append(pin.__name__)
    for pin in P.MIXER_PINS:
        try:
            pin(conv, mixer, fwd)
        except (AssertionError, RuntimeError, ValueError):
            caught.append(pin.__name__)
    for pin in P.CONT_PINS:
        try:
            pin(oracle_api(lib))
        except (AssertionError, RuntimeError, ValueError):
            caught.append(pin.__name__)
    for pin in P.GATE_PINS:
        try:
            pin(functools.partial(oracle.gates, lib=lib))
        except (AssertionError, RuntimeError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"


def test_unmutated_copy_passes(tmp_path):
    lib = _build(tmp_path, "identity", [])
    fwd = functools.partial(oracle.gdn_fwd, lib=lib)
    for pin in P.ALL_PINS:
        pin(fwd)
    for pin in P.MIXER_PINS:
        pin(functools.partial(oracle.conv_silu, lib=lib), functools.partial(oracle.mixer_fwd, lib=lib), fwd)
    for pin in P.CONT_PINS:
        pin(oracle_api(lib))
    for pin in P.GATE_PINS:
        pin(functools.partial(oracle.gates, lib=lib))
