"""The backward oracle against its pins, and copies of it with one planted
mistake each (a dropped term, a wrong sign, operand or index), each of which
must fail at least one pin.  CPU only."""
import types

import pytest

import oracle_bwd_pins
from oracle import backward

SRC = open(backward.__file__).read()

MUTANTS = {
    "no_w_dr_term": ('dk = dk + np.einsum("pkv,pv->pk", w, dr)', "dk = dk"),
    "dr_sign": ("dr = -b[:, t, None] * du", "dr = b[:, t, None] * du"),
    "no_decay_on_state_grad": ("dS = a[:, t, :, None] * dw", "dS = dw"),
    "dla_without_a": ("np.sum(dw * Sp, axis=-1) * a[:, t]", "np.sum(dw * Sp, axis=-1)"),
    "dq_from_old_state": ('np.einsum("pkv,pv->pk", Sn, do[:, t])',
                          'np.einsum("pkv,pv->pk", Sp, do[:, t])'),
    "dbeta_without_sigmoid": ("db * b * (1.0 - b)", "db"),
    "clamp_inverted": ("a_pre >= lower_bound", "a_pre <= lower_bound"),
    "norm_grad_no_projection": ("(dxh - xh * np.sum(xh * dxh, axis=-1, keepdims=True)) / n",
                                "dxh / n"),
    "dA_log_without_a": ("(da * a_pre).sum(axis=(0, 1, 3))", "da.sum(axis=(0, 1, 3))"),
    "gdn_dg_mean": ('out["dg"] = dla.sum(axis=-1)', 'out["dg"] = dla.mean(axis=-1)'),
    "dv_without_beta": ("dv[:, t] = b[:, t, None] * du", "dv[:, t] = du"),
    "dbeta_uses_v": ("db[:, t] = np.sum(du * (v[:, t] - r), axis=-1)",
                     "db[:, t] = np.sum(du * v[:, t], axis=-1)"),
    "dfinal_ignored": ("else dST.copy()", "else 0.0 * dST"),
    "no_output_term": ("dS = dS + scale * qh[:, t, :, None] * do[:, t, None, :]",
                       "dS = dS + 0.0 * do[:, t, None, :]"),
    "gate_sigmoid_sign": ("dx = da * (-rate * _sigmoid(x))", "dx = da * (-rate * _sigmoid(-x))"),
    "dk_uses_q": ('du = np.einsum("pkv,pk->pv", dS, kh[:, t])',
                  'du = np.einsum("pkv,pk->pv", dS, qh[:, t])'),
    "dw_key_term_dropped": ("dw = dS + kh[:, t, :, None] * dr[:, None, :]", "dw = dS"),
    "recompute_skips_token": ("for t in range(seg, end - 1):", "for t in range(seg + 1, end - 1):"),
}


@pytest.mark.parametrize("pin", oracle_bwd_pins.ALL_PINS, ids=lambda f: f.__name__[4:])
def test_pin(pin):
    pin(backward)


def _mutant(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, f"mutation site for {name} not unique"
    mod = types.ModuleType(f"backward_{name}")
    exec(compile(SRC.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(name)
    for pin in oracle_bwd_pins.ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError, KeyError):
            return
    pytest.fail(f"mutant {name} passed every pin")
