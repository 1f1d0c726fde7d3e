"""Mutation check of the pins: copies of the C oracle with one planted mistake
each (a dropped term, a wrong sign, index or operand) must each fail at least
one pin.  Runs on the CPU; nothing here touches the GPU library."""
import pytest

import oracle
import oracle_pins

SRC = oracle.SOURCE.read_text()

MUTANTS = {
    "no_decay": ("S[c * V + j] *= a;", "(void)a;"),
    "delta_sign": ("(vt[j] - r[j])", "(vt[j] + r[j])"),
    "retrieval_uses_query": ("r[j] += S[c * V + j] * kn[c];", "r[j] += S[c * V + j] * qn[c];"),
    "output_uses_key": ("ot[j] += S[c * V + j] * qn[c];", "ot[j] += S[c * V + j] * kn[c];"),
    "no_floor": ("log_a[c] = fmax(lower_bound, a);", "log_a[c] = a;"),
    "floor_hardcoded": ("log_a[c] = fmax(lower_bound, a);", "log_a[c] = fmax(-5.0, a);"),
    "no_dt_bias": ("softplus(g[row * K + c] + dt_bias_h[c])", "softplus(g[row * K + c])"),
    "dt_bias_head_offset": ("dt_bias + h * K", "dt_bias"),
    "no_sigmoid": ("b = sigmoid(beta[row]);", "b = beta[row];"),
    "gdn_sigmoid": ("            b = beta[row];\n", "            b = sigmoid(beta[row]);\n"),
    "rate_not_exp": ("gdn ? 0.0 : exp(A_log[h])", "gdn ? 0.0 : A_log[h]"),
    "rate_sign": ("double a = -decay_rate *", "double a = decay_rate *"),
    "no_normalise": ("out[c] = x[c] * inv;", "out[c] = x[c];"),
    "eps_wrong": ("#define ORACLE_NORM_EPS 1e-6", "#define ORACLE_NORM_EPS 1e-3"),
    "beta_dropped": ("+= b * kn[c] * (vt[j] - r[j])", "+= kn[c] * (vt[j] - r[j])"),
    "decay_channel_index": ("double a = exp(log_a[c]);", "double a = exp(log_a[0]);"),
    "state_head_offset": ("h0 + (n * H + h) * K * V", "h0 + n * K * V"),
    "no_scale": ("ot[j] *= scale;", "ot[j] *= 1.0;"),
    "gdn_decay_sign": ("log_a[c] = g[row];", "log_a[c] = -g[row];"),
    "gdn_decay_index": ("log_a[c] = g[row];", "log_a[c] = g[t];"),
    "varlen_start": ("const int64_t t0 = cu ? cu[n] : 0;", "const int64_t t0 = 0;"),
    "softplus_sign": ("log1p(exp(-fabs(x)))", "log1p(exp(fabs(x)))"),
    "o_before_update": ("ot[j] += S[c * V + j] * qn[c];",
                        "ot[j] += (S[c * V + j] - b * kn[c] * (vt[j] - r[j])) * qn[c];"),
    "batch_offset": ("const int64_t off = b * T * H;", "const int64_t off = 0 * b;"),
}


def _failing_pins(orc):
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
        except ValueError:
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, f"mutation site for {name} not unique"
    src = tmp_path / "mutant.c"
    src.write_text(SRC.replace(old, new))
    lib = oracle.build(src, tmp_path / "libmutant.so")
    failed = _failing_pins(oracle.Oracle(lib))
    assert failed, f"mutant {name} passed every pin"
