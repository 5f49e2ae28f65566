"""Plant plausible mistakes in the oracle (on the CPU, by monkeypatching) and
check that the pins catch every one of them."""
import math

import numpy as np
import pytest

from oracle import kda_oracle as ko
from tests import test_oracle_pins as pins


def _all_pins():
    runs = [
        (pins.test_hand_worked_dk2_golden, {}),
        (pins.test_l2_normalize_closed_form, {}),
        (pins.test_softplus_and_sigmoid_against_library_forms, {}),
        (pins.test_gate_special_values_fix_a_log_placement, {}),
        (pins.test_pass_through_beta0_g0, {"mode": "softplus"}),
        (pins.test_pass_through_beta0_g0, {"mode": "lb0"}),
        (pins.test_delta_property_unit_key, {}),
        (pins.test_beta0_closed_form_decay, {}),
        (pins.test_orthonormal_keys_recall_exactly, {}),
        (pins.test_round_to_bf16_ties_and_library_agreement, {}),
        (pins.test_silu_values, {}),
        (pins.test_short_conv_matches_library_correlation, {}),
        (pins.test_short_conv_tap_order_and_window_roll, {}),
        (pins.test_decode_conv_windows_follow_requests, {}),
    ]
    for gm in (ko.GATE_SOFTPLUS, ko.GATE_LOWER_BOUND):
        for shape in ((3, 2, 4), (5, 7, 3), (1, 4, 2)):
            runs.append((pins.test_bruteforce_affine_form,
                         {"gate_mode": gm, "dk": shape[0], "dv": shape[1], "n": shape[2]}))
    return runs


def _caught():
    for fn, kw in _all_pins():
        try:
            fn(**kw)
        except Exception:  # an assertion, or a shape error the slip provokes
            return True
    return False


MUTANTS = {
    "decay_wrong_axis": ("decay", lambda S, g: S * np.exp(g)[:S.shape[1]][None, :] if S.shape[0] >= S.shape[1]
                         else S * np.resize(np.exp(g), S.shape[1])[None, :]),
    "decay_sign": ("decay", lambda S, g: np.exp(-g)[:, None] * S),
    "write_sign": ("delta_write", lambda S, k, v, b: S - np.outer(b * k, v - k @ S)),
    "write_no_beta": ("delta_write", lambda S, k, v, b: S + np.outer(k, v - k @ S)),
    "write_no_correction": ("delta_write", lambda S, k, v, b: S + np.outer(b * k, v)),
    "write_correction_sign": ("delta_write", lambda S, k, v, b: S + np.outer(b * k, v + k @ S)),
    "write_outer_transposed": ("delta_write", lambda S, k, v, b: S + np.outer(v - k @ S, b * k).T
                               if S.shape[0] == S.shape[1] else S + np.outer(b * k[::-1], v - k @ S)),
    "read_wrong_vector": ("read", lambda S, q: (S.sum(axis=0) * q.sum())),
    "read_transposed": ("read", lambda S, q: (S @ q[:S.shape[1]]) if S.shape[0] == S.shape[1]
                        else q[::-1] @ S),
    "gate_a_log_inside_softplus": ("gate", None),
    "gate_lb_without_a_log": ("gate", None),
    "gate_dt_bias_subtracted": ("gate", None),
    "sigmoid_sign": ("sigmoid", lambda x: 1.0 / (1.0 + np.exp(np.asarray(x, dtype=np.float64)))),
    "softplus_plain_relu": ("softplus", lambda x: np.maximum(np.asarray(x, dtype=np.float64), 0.0)),
    "l2_no_sqrt": ("l2_normalize", lambda x, eps: np.asarray(x, np.float64) /
                   (np.sum(np.asarray(x, np.float64) ** 2, axis=-1, keepdims=True) + eps)),
    "bf16_round_half_up": ("round_to_bf16", None),
    "conv_taps_reversed": ("short_conv", None),
    "conv_window_not_rolled": ("short_conv", None),
    "conv_without_silu": ("short_conv", None),
    "silu_as_sigmoid": ("silu", lambda x: ko.sigmoid(x)),
}


def _gate_mutant(kind):
    orig = ko.gate

    def g(raw_gate, dt_bias, a_log, gate_mode=ko.GATE_SOFTPLUS, lower_bound=None):
        x = np.asarray(raw_gate, np.float64) + np.asarray(dt_bias, np.float64)
        amp = math.exp(a_log)
        if kind == "gate_a_log_inside_softplus" and gate_mode == ko.GATE_SOFTPLUS:
            return -ko.softplus(amp * x)
        if kind == "gate_lb_without_a_log" and gate_mode == ko.GATE_LOWER_BOUND:
            return lower_bound * ko.sigmoid(x)
        if kind == "gate_dt_bias_subtracted":
            return orig(np.asarray(raw_gate) - 2 * np.asarray(dt_bias), dt_bias, a_log, gate_mode, lower_bound)
        return orig(raw_gate, dt_bias, a_log, gate_mode, lower_bound)
    return g


def _conv_mutant(kind):
    orig = ko.short_conv

    def conv(x, window, w):
        w = np.asarray(w, dtype=np.float64)
        if kind == "conv_taps_reversed":
            return orig(x, window, w[::-1])
        y, new_win = orig(x, window, w)
        if kind == "conv_window_not_rolled":
            return y, np.asarray(window, dtype=np.float64)
        xx = np.concatenate([np.asarray(window, np.float64), np.asarray(x, np.float64)])
        raw = np.stack([np.sum(w * xx[t:t + w.shape[0]], axis=0) for t in range(len(x))])
        return raw, new_win
    return conv


def _bf16_half_up(x):
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    qe = np.maximum(e - 8, -133)
    return np.ldexp(np.floor(np.ldexp(x, -qe) + 0.5), qe)


def test_unmutated_oracle_passes_every_pin():
    assert not _caught()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    if attr == "gate":
        fn = _gate_mutant(name)
    elif attr == "round_to_bf16":
        fn = _bf16_half_up
    elif attr == "short_conv":
        fn = _conv_mutant(name)
    monkeypatch.setattr(ko, attr, fn)
    assert _caught(), f"no pin catches mutant {name}"
