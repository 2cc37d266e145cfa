"""Plant plausible mistakes in copies of the oracle source (CPU only) and
check that every one of them fails at least one pin.  This shows the pins
constrain each term, sign, index and operand of the recurrence (scalar and
per-channel decay), of the prologue and of the output epilogue."""
import os
import shutil
import subprocess
import tempfile

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, exact text in oracle.c, replacement)
MUTANTS = [
    ("no_decay", "S[(size_t)i * dk + j] *= a;", "(void)a;"),
    ("error_sign", "e[i] = (double)v[i] - pred;", "e[i] = (double)v[i] + pred;"),
    ("error_vs_undecayed_state",
     "pred += S[(size_t)i * dk + j] * (double)k[j];",
     "pred += S[(size_t)i * dk + j] / a * (double)k[j];"),
    ("transposed_prediction",
     "pred += S[(size_t)i * dk + j] * (double)k[j];",
     "pred += S[(size_t)j * dk + i] * (double)k[j];"),
    ("write_without_beta", "S[(size_t)i * dk + j] += b * e[i] * (double)k[j];",
     "S[(size_t)i * dk + j] += e[i] * (double)k[j];"),
    ("write_value_not_error", "S[(size_t)i * dk + j] += b * e[i] * (double)k[j];",
     "S[(size_t)i * dk + j] += b * (double)v[i] * (double)k[j];"),
    ("write_with_query", "S[(size_t)i * dk + j] += b * e[i] * (double)k[j];",
     "S[(size_t)i * dk + j] += b * e[i] * (double)q[j];"),
    ("readout_with_key", "acc += S[(size_t)i * dk + j] * (double)q[j];",
     "acc += S[(size_t)i * dk + j] * (double)k[j];"),
    ("readout_transposed", "acc += S[(size_t)i * dk + j] * (double)q[j];",
     "acc += S[(size_t)j * dk + i] * (double)q[j];"),
    ("ignore_S0", "if (S0) memcpy(S, S0 + (size_t)u * dd, dd * sizeof(double));",
     "if (S0 && 0) memcpy(S, S0, dd * sizeof(double));"),
    ("skip_first_token", "const int64_t t0 = cu ? cu[n] : 0;",
     "const int64_t t0 = (cu ? cu[n] : 0) + 1;"),
    ("wrong_head", "const size_t th = (size_t)t * H + h;",
     "const size_t th = (size_t)t * H + (H - 1 - h);"),
    ("decode_state_of_head0", "oracle_token(S + (size_t)u * dd, e,",
     "oracle_token(S + (size_t)(u - u % H) * dd, e,"),
    ("norm_sum_not_mean", "ms /= dv;", "(void)0;"),
    ("norm_without_eps", "const double inv = 1.0 / sqrt(ms + eps);",
     "const double inv = 1.0 / sqrt(ms);"),
    ("norm_rms_not_inverse", "const double inv = 1.0 / sqrt(ms + eps);",
     "const double inv = sqrt(ms + eps);"),
    ("gate_sign", "const double sig = 1.0 / (1.0 + exp(-x));",
     "const double sig = 1.0 / (1.0 + exp(x));"),
    ("silu_is_sigmoid", "gate = act == 0 ? sig : x * sig;", "gate = sig;"),
    ("weight_ignored", "* (w ? (double)w[c] : 1.0) * gate;", "* gate;"),
    ("gate_of_first_channel", "const double x = (double)g[(size_t)r * dv + c];",
     "const double x = (double)g[(size_t)r * dv];"),
    ("conv_taps_reversed", "acc += (double)w[(((size_t)x * H + h) * d + c) * K + i] * xr;",
     "acc += (double)w[(((size_t)x * H + h) * d + c) * K + (K - 1 - i)] * xr;"),
    ("conv_history_ignored", "} else if (hist_in) {", "} else if (0) {"),
    ("history_out_not_shifted", "val = hist_in[(((size_t)n * 3 + x) * (K - 1) + (m + len)) * hd + e];",
     "val = hist_in[(((size_t)n * 3 + x) * (K - 1) + m) * hd + e];"),
    ("write_gate_inverted", "const double wgate = (1.0 / (1.0 + exp(-(br + dl)))) / sig_b;",
     "const double wgate = sig_b / (1.0 / (1.0 + exp(-(br + dl))));"),
    ("decay_floor_missing", "a[tkh] = exp(fmax((double)g_log[tkh], floor_log));",
     "a[tkh] = exp((double)g_log[tkh]);"),
    ("beta_without_sigmoid", "b[tkh] = sig_b;", "b[tkh] = br;"),
    ("l2_norm_without_sqrt", "const double scale = x < 2 ? 1.0 / sqrt(ss + l2_eps) : wgate;",
     "const double scale = x < 2 ? 1.0 / (ss + l2_eps) : wgate;"),
    ("value_normalised_too", "const double scale = x < 2 ? 1.0 / sqrt(ss + l2_eps) : wgate;",
     "const double scale = x < 3 ? 1.0 / sqrt(ss + l2_eps) : wgate;"),
    ("silu_sign", "if (act == 1) acc = acc / (1.0 + exp(-acc));",
     "if (act == 1) acc = acc / (1.0 + exp(acc));"),
    ("diag_decay_of_wrong_channel", "row[c] = row[c] * (double)alpha[c];",
     "row[c] = row[c] * (double)alpha[dk - 1 - c];"),
    ("diag_decay_on_value_channel", "row[c] = row[c] * (double)alpha[c];",
     "row[c] = row[c] * (double)alpha[r % dk];"),
    ("diag_error_before_decay",
     "row[c] = row[c] * (double)alpha[c];\n            pr += row[c] * (double)kv[c];",
     "pr += row[c] * (double)kv[c];\n            row[c] = row[c] * (double)alpha[c];"),
    ("diag_decay_of_head0", "alpha + row * dk, (double)b[row], o + row * dv);",
     "alpha + ((size_t)t * H) * dk, (double)b[row], o + row * dv);"),
    ("diag_write_without_beta", "const double be = beta * err[r];", "const double be = err[r];"),
]


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="oracle_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def test_mutations_apply_exactly():
    src = open(SRC).read()
    for name, old, new in MUTANTS:
        assert src.count(old) == 1, f"mutation {name}: pattern found {src.count(old)} times"


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_fails_a_pin(workdir, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1
    msrc = os.path.join(workdir, f"{name}.c")
    with open(msrc, "w") as f:
        f.write(src.replace(old, new))
    lib = os.path.join(workdir, f"lib_{name}.so")
    oracle.build(force=True, src=msrc, out=lib)
    orc = oracle.Oracle(lib)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
