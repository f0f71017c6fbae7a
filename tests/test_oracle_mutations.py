"""The oracle's pins must catch plausible mistakes: each case below plants one
slip in a function of the CPU oracle (monkeypatched for the duration of the
test, never on disk) and checks that at least one pin then fails.

A mutant that no pin notices would mean the pins do not constrain that part
of the oracle, and parity against it would prove less than it claims.
CPU only.
"""
import numpy as np
import pytest

import oracle as orc
import oracle.muon_oracle as om
import test_oracle_pins as pins

# mutants overflow or produce NaN on purpose; their warnings are noise here
pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

_scale = om.scale_factor   # the unmutated rule, for the rules a mutant leaves alone


def _ns(X, schedule, *, drop_c=False, minus=False, right=False, untranspose=True, swap=False,
        linear_a=False):
    """Newton-Schulz with one planted mistake selected by a flag."""
    X = np.asarray(X, np.float64)
    tr = X.shape[0] > X.shape[1]
    if tr:
        X = X.T
    for (a, b, c) in schedule:
        if swap:
            a, c = c, a
        A = X @ X.T
        A2 = A if linear_a else A @ A
        B = b * A + (0.0 if drop_c else c) * A2
        BX = X @ B if (right and X.shape[0] == X.shape[1]) else B @ X
        X = a * X - BX if minus else a * X + BX
    if tr and untranspose:
        X = X.T
    return np.ascontiguousarray(X)


MUTANTS = {
    # Newton-Schulz
    "ns_drops_c_term": ("newton_schulz", lambda X, s: _ns(X, s, drop_c=True)),
    "ns_subtracts_BX": ("newton_schulz", lambda X, s: _ns(X, s, minus=True)),
    "ns_multiplies_on_the_right": ("newton_schulz", lambda X, s: _ns(X, s, right=True)),
    "ns_forgets_to_transpose_back": ("newton_schulz", lambda X, s: _ns(X, s, untranspose=False)),
    "ns_swaps_a_and_c": ("newton_schulz", lambda X, s: _ns(X, s, swap=True)),
    "ns_uses_A_for_A_squared": ("newton_schulz", lambda X, s: _ns(X, s, linear_a=True)),
    # normalization
    "norm_spectral": ("frobenius_normalize",
                      lambda U, eps: np.asarray(U, np.float64) / (np.linalg.norm(U, 2) + eps)),
    "norm_without_eps": ("frobenius_normalize",
                         lambda U, eps: np.asarray(U, np.float64) / np.sqrt(np.sum(np.square(U)))),
    "norm_eps_under_root": ("frobenius_normalize",
                            lambda U, eps: np.asarray(U, np.float64) / np.sqrt(np.sum(np.square(U)) + eps)),
    # momentum
    "momentum_ema": ("momentum_update",
                     lambda M, G, beta: beta * np.asarray(M, np.float64) + (1 - beta) * np.asarray(G, np.float64)),
    "momentum_scales_gradient": ("momentum_update",
                                 lambda M, G, beta: beta * (np.asarray(M, np.float64) + np.asarray(G, np.float64))),
    # decay and apply
    "decay_without_lr": ("apply_update",
                         lambda W, O, lr, wd, s: (1 - wd) * np.asarray(W) - lr * s * np.asarray(O)),
    "apply_adds_update": ("apply_update",
                          lambda W, O, lr, wd, s: (1 - lr * wd) * np.asarray(W) + lr * s * np.asarray(O)),
    "apply_forgets_scale": ("apply_update",
                            lambda W, O, lr, wd, s: (1 - lr * wd) * np.asarray(W) - lr * np.asarray(O)),
    # scale rules
    "moonlight_uses_min": ("scale_factor",
                           lambda r, c, rule: 0.2 * np.sqrt(min(r, c)) if rule == "moonlight"
                           else _scale(r, c, rule)),
    "kellerjordan_inverted": ("scale_factor",
                              lambda r, c, rule: float(np.sqrt(max(1.0, c / r))) if rule == "kellerjordan"
                              else _scale(r, c, rule)),
    "mup_inverted": ("scale_factor",
                     lambda r, c, rule: float(np.sqrt(c / r)) if rule == "mup" else _scale(r, c, rule)),
    # the scalar map the closed-form pins use
    "phi_wrong_power": ("phi", lambda x, a, b, c: a * np.asarray(x) + b * np.asarray(x) ** 3
                        + c * np.asarray(x) ** 4),
    "phi_drops_b": ("phi", lambda x, a, b, c: a * np.asarray(x) + c * np.asarray(x) ** 5),
}


def _pin_calls():
    calls = [
        lambda: pins.test_printed_coefficients_match_oracle_constants(),
        lambda: pins.test_taylor_triple_from_series_of_inverse_sqrt(),
        lambda: pins.test_kj_fixed_points_bracket_one(),
        lambda: pins.test_kj_band_after_five_steps_matches_page_claim(),
        lambda: pins.test_ns_closed_form_where_eps_matters(),
        lambda: pins.test_orthogonal_input_is_a_fixed_direction(16),
        lambda: pins.test_orthonormal_rows_rectangular(),
        lambda: pins.test_transpose_equivariance((20, 36)),
        lambda: pins.test_converged_ns_equals_jacobi_msign((8, 5)),
        lambda: pins.test_converged_ns_equals_jacobi_msign((6, 16)),
        lambda: pins.test_nuclear_norm_identity(),
        lambda: pins.test_scale_rules_worked_example(),
        lambda: pins.test_moonlight_update_rms_is_point_two(),
        lambda: pins.test_momentum_geometric_series(),
        lambda: pins.test_weight_decay_only_when_gradient_is_zero(),
        lambda: pins.test_nesterov_closed_form(),
    ]
    for shape in [(24, 40), (40, 24), (32, 32)]:
        for sched in ("kj5", "mixed"):
            calls.append(lambda shape=shape, sched=sched: pins.test_ns_closed_form_on_constructed_svd(shape, sched))
    for rule in orc.SCALE_RULES:
        calls.append(lambda rule=rule: pins.test_step_closed_form_and_descent_direction(rule))
    return calls


def _failing_pins():
    n = 0
    for call in _pin_calls():
        try:
            call()
        except (AssertionError, ValueError):
            n += 1
    return n


def test_unmutated_oracle_passes_every_pin_used_here():
    assert _failing_pins() == 0


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(om, attr, fn)
    if hasattr(orc, attr):
        monkeypatch.setattr(orc, attr, fn)
    assert _failing_pins() > 0, f"no pin notices the mutant {name}"
