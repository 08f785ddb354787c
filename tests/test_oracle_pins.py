"""CPU tests: the fp64 oracle against its pins, and planted-mistake controls.

Every pin in ``oracle_pins`` must pass on the real oracle.  Each mutant below
is the oracle's C source with one plausible mistake planted textually (a
dropped term, a wrong sign or index, a transposed operand, a wrong head map,
a wrong norm epsilon...), compiled into a temporary library; at least one pin
must fail on it, which shows the pins can see that kind of mistake.
"""
import json
import os
import subprocess
import sys
import tempfile

import numpy as np
import pytest

import oracle
from oracle import build as oracle_build
import oracle_pins as P

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(lib, pin):
    pin(lib)


def test_block_inverse_and_newton_schulz():
    err2, err3 = P.check_inverse_and_newton_schulz()
    assert err3 < err2


# (name, text in oracle.c, replacement, pins expected to catch it)
MUTANTS = [
    ("gqa_mod_map", "const int32_t h = hv / group;\n            prepare_qk(y",
     "const int32_t h = hv % H;\n            prepare_qk(y", ["pin_decode_split"]),
    ("gqa_mod_map_prefill", "const int32_t h = hv / group;\n            double* S",
     "const int32_t h = hv % H;\n            double* S", ["pin_gqa_map"]),
    ("predict_with_undecayed_state", "const double delta = beta * (v[i] - u);",
     "const double delta = beta * (v[i] - u / alpha);", ["pin_delta_rule_unit_key"]),
    ("drop_beta", "const double delta = beta * (v[i] - u);",
     "const double delta = (v[i] - u);", ["pin_brute_force_matrix_form"]),
    ("wrong_sign_update", "row[j] = row[j] + delta * k[j];",
     "row[j] = row[j] - delta * k[j];", ["pin_delta_rule_unit_key"]),
    ("transposed_state_in_prediction", "u += row[j] * k[j];",
     "u += S[(size_t)j * dk + i] * k[j];", ["pin_brute_force_matrix_form"]),
    ("output_before_update", "for (int32_t j = 0; j < dk; ++j) acc += row[j] * q[j];",
     "for (int32_t j = 0; j < dk; ++j) acc += (row[j] - delta * k[j]) * q[j];",
     ["pin_brute_force_matrix_form"]),
    ("no_decay", "const double alpha = exp(g);", "const double alpha = 1.0 + 0.0 * g;",
     ["pin_decay"]),
    ("eps_outside_sqrt", "qn = 1.0 / sqrt(sq + 1e-6);", "qn = 1.0 / (sqrt(sq) + 1e-6);",
     ["pin_qk_norm"]),
    ("k_scaled_too", "k[j] = kin[j] * kn;", "k[j] = kin[j] * kn * scale;",
     ["pin_qk_norm"]),
    ("no_k_norm", "kn = 1.0 / sqrt(sk + 1e-6);", "kn = 1.0 + 0.0 * sk;", ["pin_qk_norm"]),
    ("conv_taps_reversed", "y += weight[(size_t)c * width + j] * X[t + j];",
     "y += weight[(size_t)c * width + (width - 1 - j)] * X[t + j];",
     ["pin_conv_sliding_window"]),
    ("roll_off_by_one", "state[(size_t)c * W1 + j] = X[L + j];",
     "state[(size_t)c * W1 + j] = X[L + j - (j > 0)];", ["pin_conv_sliding_window"]),
    ("bias_dropped", "double y = bias ? bias[c] : 0.0;", "double y = 0.0;",
     ["pin_conv_sliding_window"]),
    ("silu_wrong", "return y / (1.0 + exp(-y));", "return y / (1.0 + exp(y));", ["pin_silu"]),
    ("inactive_not_zeroed",
     "memset(ob, 0, sizeof(double) * (size_t)HV * dv);\n            continue;",
     "continue;", ["pin_slot_contract"]),
    ("no_repeat_check", "if (slot_idx[j] == s) err |= ORACLE_ERR_SLOT_REPEAT;",
     "(void)j;", ["pin_slot_contract"]),
    ("range_check_off_by_one", "if (s >= num_slots) err |= ORACLE_ERR_SLOT_RANGE;",
     "if (s > num_slots) err |= ORACLE_ERR_SLOT_RANGE;", ["pin_slot_contract"]),
    ("zero_slot_active", "if (s <= 0) continue;                 /* inactive row */",
     "if (s < 0) continue;", ["pin_slot_contract"]),
    ("split_k_offset", "y + (size_t)H * dk + (size_t)h * dk, q, k,",
     "y + (size_t)h * dk, q, k,", ["pin_decode_split"]),
    ("state_not_carried_across_tokens",
     "for (int64_t t = start; t < end; ++t) {\n                prepare_qk",
     "for (int64_t t = start; t < end; ++t) {\n                if (t > start) memset(S, 0, sizeof(double) * (size_t)dv * dk);\n                prepare_qk",
     ["pin_brute_force_matrix_form", "pin_chunked_equals_token"]),
    ("gating_no_threshold", "return (x <= 20.0) ? log1p(exp(x)) : x;",
     "return log(exp(x));", ["pin_gating"]),
    ("gating_threshold_branch_swapped", "return (x <= 20.0) ? log1p(exp(x)) : x;",
     "return (x > 20.0) ? log1p(exp(x)) : x;", ["pin_gating"]),
    ("gating_dt_bias_dropped", "softplus_thresholded(a[i] + dt_bias[h])",
     "softplus_thresholded(a[i])", ["pin_gating"]),
    ("gating_A_log_not_exponentiated", "g[i] = -exp(A_log[h]) *",
     "g[i] = -A_log[h] *", ["pin_gating"]),
    ("gating_head_index_by_row", "g[i] = -exp(A_log[h]) * softplus_thresholded(a[i] + dt_bias[h]);",
     "g[i] = -exp(A_log[r % num_v_heads]) * softplus_thresholded(a[i] + dt_bias[r % num_v_heads]);",
     ["pin_gating"]),
    ("gating_beta_sign", "beta[i] = 1.0 / (1.0 + exp(-b[i]));",
     "beta[i] = 1.0 / (1.0 + exp(b[i]));", ["pin_gating"]),
    ("rmsnorm_sum_not_mean", "const double rms = sqrt(ss / dim + eps);",
     "const double rms = sqrt(ss + eps);", ["pin_gated_rmsnorm"]),
    ("rmsnorm_no_sqrt", "const double rms = sqrt(ss / dim + eps);",
     "const double rms = ss / dim + eps;", ["pin_gated_rmsnorm"]),
    ("rmsnorm_eps_outside_root", "const double rms = sqrt(ss / dim + eps);",
     "const double rms = sqrt(ss / dim) + eps;", ["pin_gated_rmsnorm"]),
    ("rmsnorm_gate_swapped", "gate = (flags & ORACLE_NORM_GATE_SIGMOID) ? sig : zj * sig;",
     "gate = (flags & ORACLE_NORM_GATE_SIGMOID) ? zj * sig : sig;", ["pin_gated_rmsnorm"]),
    ("rmsnorm_offset_dropped", "? weight[j] + 1.0 : weight[j];", "? weight[j] : weight[j];",
     ["pin_gated_rmsnorm"]),
    ("rmsnorm_weight_by_row", "? weight[j] + 1.0 : weight[j];",
     "? weight[j] + 1.0 : weight[r % dim];", ["pin_gated_rmsnorm"]),
]


def _build_mutant(tmpdir, name, old, new):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    assert src.count(old) == 1, f"mutation site for {name} must occur exactly once"
    path = os.path.join(tmpdir, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    return oracle_build.build(out=os.path.join(tmpdir, f"lib{name}.so"), source=path,
                              extra_cflags=["-w"])


@pytest.mark.parametrize("name,old,new,catchers", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, catchers):
    # A mutant may corrupt memory (e.g. an off-by-one range check lets a write
    # run past the cache), so its pins run in a child process; a crash there
    # counts as the mistake being caught.
    here = os.path.dirname(os.path.abspath(__file__))
    with tempfile.TemporaryDirectory() as d:
        so = _build_mutant(d, name, old, new)
        code = ("import json, sys; sys.path[:0] = [%r, %r]; import oracle, oracle_pins as P; "
                "print(json.dumps(P.run_all(oracle.load(%r))))"
                % (here, os.path.dirname(here), so))
        r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                           timeout=300)
    if r.returncode != 0:
        return                                   # crashed: caught
    failed = json.loads(r.stdout.strip().splitlines()[-1])
    assert failed, f"planted mistake {name} passed every pin"
    assert any(c in failed for c in catchers), (name, failed)
