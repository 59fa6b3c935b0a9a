"""The oracle pins must catch plausible mistakes planted in the oracle (CPU only).

Each case monkeypatches one oracle function or constant with a wrong variant
and checks that at least one pin of tests/test_oracle_pins.py then fails.
"""

import math

import numpy as np
import pytest

from oracle import muon_oracle as mo
from tests import test_oracle_pins as pins


def _ns_variant(transposed_gram=False, spectral_norm=False, forget_transpose_back=False,
                eps_in_sqrt=False, poly_right=False):
    def ns(update, ns_steps):
        rows, cols = update.shape
        tall = rows > cols
        x = np.ascontiguousarray(update.T if tall else update, dtype=np.float64)
        if spectral_norm:
            x = x / (np.linalg.norm(x, 2) + mo.NORM_EPS)
        elif eps_in_sqrt:
            x = x / math.sqrt(np.sum(x * x) + mo.NORM_EPS)
        else:
            x = x / (np.linalg.norm(x) + mo.NORM_EPS)
        a, b, c = mo.NS_COEFFS
        for _ in range(ns_steps):
            gram = x.T @ x if transposed_gram else x @ x.T
            poly = b * gram + c * (gram @ gram)
            x = a * x + (x @ poly if poly_right else poly @ x)
        out = x if forget_transpose_back else (np.ascontiguousarray(x.T) if tall else x)
        return mo.shape_scale(rows, cols) * out
    return ns


def _left_factor_variant(gram_once=False, no_norm=False):
    def lf(gram, ns_steps):
        scale = 1.0 if no_norm else 1.0 / (math.sqrt(np.trace(gram)) + mo.NORM_EPS)
        p = np.eye(gram.shape[0]) * scale
        a, b, c = mo.NS_COEFFS
        for _ in range(ns_steps):
            gx = p @ gram if gram_once else p @ gram @ p.T
            p = a * p + (b * gx + c * (gx @ gx)) @ p
        return p
    return lf


PIN_TESTS = [
    lambda: pins.test_momentum_constant_gradient_closed_form(True),
    lambda: pins.test_momentum_constant_gradient_closed_form(False),
    pins.test_zero_gradient_is_pure_decay_over_steps,
    pins.test_update_direction_opposes_gradient_1x1,
    pins.test_decay_then_update_order_exact_1x1,
    pins.test_hyperparameters_are_float32_values,
    lambda: pins.test_newton_schulz_1x1_exact(1e-7),
    lambda: pins.test_newton_schulz_singular_value_closed_form((6, 10), 5),
    lambda: pins.test_newton_schulz_singular_value_closed_form((10, 6), 5),
    lambda: pins.test_newton_schulz_singular_value_closed_form((17, 3), 1),
    pins.test_rank_one_input,
    pins.test_orthogonal_input,
    lambda: pins.test_transposition((13, 4)),
    pins.test_sharded_scatter_equals_contiguous,
    pins.test_bf16_params_step_uses_exact_widening,
    lambda: pins.test_left_factor_closed_form((6, 10), 5),
]


def _some_pin_fails():
    for t in PIN_TESTS:
        try:
            t()
        except Exception:  # a failed assertion, or the mutated code blowing up
            return True
    return False


MUTATIONS = {
    "wrong_sign_b": ("NS_COEFFS", (3.4445, 4.7750, 2.0315)),
    "swapped_a_c": ("NS_COEFFS", (2.0315, -4.7750, 3.4445)),
    "eps_large": ("NORM_EPS", 1e-3),
    "scale_inverted": ("shape_scale", lambda r, c: math.sqrt(max(1.0, c / r))),
    "scale_missing": ("shape_scale", lambda r, c: 1.0),
    "ema_momentum": ("momentum_update", lambda g, m, b: b * m + (1 - b) * g),
    "nesterov_without_beta": ("orthogonalization_input",
                              lambda g, m, b, n: g + m if n else m.copy()),
    "decay_without_lr": ("apply_update", lambda w, o, lr, wd: w * (1 - wd) - lr * o),
    "update_sign": ("apply_update", lambda w, o, lr, wd: w * (1 - lr * wd) + lr * o),
    "decay_after_update": ("apply_update", lambda w, o, lr, wd: (w - lr * o) * (1 - lr * wd)),
    "decay_on_update_not_weight": ("apply_update", lambda w, o, lr, wd: w - lr * o * (1 - lr * wd)),
    "hyper_not_f32_rounded": ("as_f32_value", lambda x: float(x)),
    "transposed_gram": ("newton_schulz", _ns_variant(transposed_gram=True)),
    "poly_on_right_of_square_gram": ("newton_schulz", _ns_variant(poly_right=True)),
    "spectral_norm": ("newton_schulz", _ns_variant(spectral_norm=True)),
    "no_transpose_back": ("newton_schulz", _ns_variant(forget_transpose_back=True)),
    "eps_in_sqrt": ("newton_schulz", _ns_variant(eps_in_sqrt=True)),
    "scatter_ignores_stride": ("scatter_param", None),
    "left_factor_gram_once": ("newton_schulz_left_factor", _left_factor_variant(gram_once=True)),
    "left_factor_unnormalized": ("newton_schulz_left_factor", _left_factor_variant(no_norm=True)),
    "bf16_truncating_widen": ("bf16_bits_to_f64",
                              lambda b: (b.astype(np.uint32) << 15).view(np.float32)
                              .astype(np.float64)),
}


def _bad_scatter(params64, d, weight):
    flat = weight.reshape(-1)
    per = flat.size // d.n_shards
    for k in range(d.n_shards):
        dst = d.param_offset + k * per
        params64[dst:dst + per] = flat[k * per:(k + 1) * per]


def test_pins_pass_unmutated():
    assert not _some_pin_fails()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, monkeypatch):
    attr, value = MUTATIONS[name]
    if name == "scatter_ignores_stride":
        value = _bad_scatter
    monkeypatch.setattr(mo, attr, value)
    assert _some_pin_fails(), f"no pin caught mutation {name}"
