"""Pins for the fp64 oracle: closed forms, invariants, printed values, brute force.

Each test checks the oracle against something other than itself, chosen so
that a plausible slip (dropped term, wrong sign, wrong side of a product,
wrong norm, EMA instead of plain momentum, swapped coefficients) fails at
least one of them.  CPU only.
"""
import json
import os

import numpy as np
import pytest

import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _printed():
    with open(os.path.join(GOLDEN, "pages_printed_values.json")) as f:
        return json.load(f)


def _orthonormal(rng, n, k):
    q, r = np.linalg.qr(rng.standard_normal((n, k)))
    return q * np.sign(np.diag(r))


def _svd_built(rng, rows, cols, sigma):
    """M = U diag(sigma) V^T with seeded orthonormal factors (k = len(sigma))."""
    k = len(sigma)
    U = _orthonormal(rng, rows, k)
    V = _orthonormal(rng, cols, k)
    return U, np.asarray(sigma, np.float64), V, (U * sigma) @ V.T


SCHEDULES = {
    "kj5": [orc.KJ_COEFFS] * 5,
    "hybrid8+2": orc.hybrid_schedule(8, 2),
    "taylor5": [orc.TAYLOR_COEFFS] * 5,
    "mixed": [orc.KJ_COEFFS, orc.TAYLOR_COEFFS, (2.0, -1.5, 0.5), orc.KJ_COEFFS],
}


# ----------------------------------------------------------------------------
# Printed coefficients and the scalar map
# ----------------------------------------------------------------------------

def test_printed_coefficients_match_oracle_constants():
    p = _printed()
    assert tuple(p["kj_coefficients"]["value"]) == orc.KJ_COEFFS
    assert np.allclose(p["taylor_coefficients"]["value"], orc.TAYLOR_COEFFS, rtol=0, atol=0)


def test_taylor_triple_from_series_of_inverse_sqrt():
    # t^(-1/2) = 1 - (t-1)/2 + 3/8 (t-1)^2 + ...; x * that polynomial in t = x^2 has
    # coefficients (15/8, -10/8, 3/8).  Check by sampling: phi(x)/x must equal the
    # second-order Taylor polynomial of t^(-1/2) at t = x^2.
    x = np.linspace(0.05, 1.3, 41)
    t = x * x
    taylor = 1 - (t - 1) / 2 + 3.0 / 8.0 * (t - 1) ** 2
    assert np.allclose(orc.phi(x, *orc.TAYLOR_COEFFS) / x, taylor, rtol=0, atol=1e-14)
    # fixed point at 1 with zero slope
    h = 1e-6
    assert abs(orc.phi(1.0, *orc.TAYLOR_COEFFS) - 1.0) < 1e-15
    slope = (orc.phi(1 + h, *orc.TAYLOR_COEFFS) - orc.phi(1 - h, *orc.TAYLOR_COEFFS)) / (2 * h)
    assert abs(slope) < 1e-9


def test_kj_fixed_points_bracket_one():
    # The page parameterizes the map as x + kappa x (x^2 - x1^2)(x^2 - x2^2) with
    # fixed points x1 < 1 < x2.  The positive fixed points of the oracle's map with
    # the KJ triple must therefore be two numbers bracketing 1, and kappa = c.
    a, b, c = orc.KJ_COEFFS
    # phi(x) = x  <=>  (a - 1) + b t + c t^2 = 0 with t = x^2
    roots = np.roots([c, b, a - 1.0])
    assert np.all(np.isreal(roots)) and np.all(roots.real > 0)
    x1, x2 = np.sort(np.sqrt(roots.real))
    assert x1 < 1.0 < x2
    assert abs(x1 - 0.8680) < 5e-4 and abs(x2 - 1.2637) < 5e-4
    for x in (x1, x2):
        assert abs(orc.phi(x, a, b, c) - x) < 1e-12
    # the product form reproduces the map
    xs = np.linspace(0, 1.5, 31)
    prod = xs + c * xs * (xs ** 2 - x1 ** 2) * (xs ** 2 - x2 ** 2)
    assert np.allclose(orc.phi(xs, a, b, c), prod, atol=1e-12)


def test_kj_band_after_five_steps_matches_page_claim():
    lo, hi = _printed()["kj_band_after_5_steps"]["value"]
    sig = np.geomspace(1e-2, 1.0, 200)
    D = np.diag(sig)  # already has top singular value 1; run the matrix iteration
    out = np.diag(orc.newton_schulz(D, SCHEDULES["kj5"]))
    assert np.all(out >= lo) and np.all(out <= hi)
    assert np.all(out > 0.68) and np.all(out < 1.135)


def test_hybrid_schedule_holds_singular_values_at_one():
    sig = np.geomspace(1e-3, 1.0, 200)
    out = np.diag(orc.newton_schulz(np.diag(sig), orc.hybrid_schedule(8, 2)))
    assert np.all(np.abs(out - 1.0) < 1e-3)


# ----------------------------------------------------------------------------
# Newton-Schulz: closed form through an independent decomposition
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(24, 40), (40, 24), (32, 32), (1, 17), (17, 1)])
@pytest.mark.parametrize("sched", sorted(SCHEDULES))
def test_ns_closed_form_on_constructed_svd(shape, sched):
    rng = np.random.default_rng(11)
    k = min(shape)
    sigma = np.geomspace(1.0, 1e-3, k)
    U, s, V, M = _svd_built(rng, *shape, sigma)
    eps = 1e-7
    O = orc.muon_ns(M, SCHEDULES[sched], eps=eps)
    e32 = orc.as_f32(eps)
    sch32 = [tuple(orc.as_f32(v) for v in t) for t in SCHEDULES[sched]]
    xhat = s / (np.sqrt(np.sum(s * s)) + e32)     # ||M||_F = ||sigma||_2
    expect = (U * orc.phi_schedule(xhat, sch32)) @ V.T
    assert O.shape == M.shape
    assert np.max(np.abs(O - expect)) < 1e-12


def test_ns_closed_form_where_eps_matters():
    # ||M||_F = 1e-6, so eps = 1e-7 changes the normalized singular values by ~9 %.
    rng = np.random.default_rng(5)
    U, s, V, M = _svd_built(rng, 12, 20, np.geomspace(1.0, 0.1, 12))
    M = M * (1e-6 / np.linalg.norm(s))
    s = s * (1e-6 / np.linalg.norm(s))
    O = orc.muon_ns(M, SCHEDULES["kj5"], eps=1e-7)
    xhat = s / (1e-6 + orc.as_f32(1e-7))
    sch32 = [tuple(orc.as_f32(v) for v in t) for t in SCHEDULES["kj5"]]
    expect = (U * orc.phi_schedule(xhat, sch32)) @ V.T
    assert np.max(np.abs(O - expect)) < 1e-12
    # and it is measurably different from the eps-free value
    no_eps = (U * orc.phi_schedule(s / 1e-6, sch32)) @ V.T
    assert np.max(np.abs(O - no_eps)) > 1e-3


def test_rank_deficient_null_directions_stay_zero():
    rng = np.random.default_rng(9)
    U, s, V, M = _svd_built(rng, 16, 30, [1.0, 0.5, 0.25])
    O = orc.muon_ns(M, SCHEDULES["hybrid8+2"])
    # O maps the orthogonal complement of span(V) to zero.  fp64 rounding noise
    # in those directions is multiplied by about a^8 ~ 2e4 over the fast steps.
    P = np.eye(30) - V @ V.T
    assert np.max(np.abs(O @ P)) < 1e-10


# ----------------------------------------------------------------------------
# Invariants the pages fix
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("n", [16, 128])
def test_orthogonal_input_is_a_fixed_direction(n):
    rng = np.random.default_rng(n)
    Q = _orthonormal(rng, n, n)
    O = orc.muon_ns(Q, SCHEDULES["kj5"])
    sch32 = [tuple(orc.as_f32(v) for v in t) for t in SCHEDULES["kj5"]]
    gamma = orc.phi_schedule(1.0 / (np.sqrt(n) + orc.as_f32(1e-7)), sch32)
    assert np.max(np.abs(O - gamma * Q)) < 1e-12
    # a converging schedule returns Q itself: msign(Q) = Q
    conv = [orc.KJ_COEFFS] * 8 + [orc.TAYLOR_COEFFS] * 6
    assert np.max(np.abs(orc.muon_ns(Q, conv) - Q)) < 1e-12


def test_orthonormal_rows_rectangular():
    rng = np.random.default_rng(3)
    Q = _orthonormal(rng, 40, 16).T      # 16 x 40, orthonormal rows, ||Q||_F = 4
    O = orc.muon_ns(Q, SCHEDULES["kj5"])
    sch32 = [tuple(orc.as_f32(v) for v in t) for t in SCHEDULES["kj5"]]
    gamma = orc.phi_schedule(1.0 / (4.0 + orc.as_f32(1e-7)), sch32)
    assert np.max(np.abs(O - gamma * Q)) < 1e-12


@pytest.mark.parametrize("shape", [(20, 36), (36, 20), (25, 25)])
def test_transpose_equivariance(shape):
    rng = np.random.default_rng(21)
    M = rng.standard_normal(shape)
    O = orc.muon_ns(M, SCHEDULES["hybrid8+2"])
    Ot = orc.muon_ns(M.T.copy(), SCHEDULES["hybrid8+2"])
    assert np.max(np.abs(Ot - O.T)) < 1e-13


@pytest.mark.parametrize("c", [1e-6, 1e-2, 37.0, 1e3])
def test_scale_invariance_without_eps(c):
    rng = np.random.default_rng(22)
    M = rng.standard_normal((18, 30))
    O1 = orc.muon_ns(M, SCHEDULES["kj5"], eps=0.0)
    O2 = orc.muon_ns(c * M, SCHEDULES["kj5"], eps=0.0)
    assert np.max(np.abs(O1 - O2)) < 1e-12


# ----------------------------------------------------------------------------
# Hand-written Jacobi SVD (pinned to numpy's LAPACK SVD), then msign agreement
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(8, 5), (12, 12), (6, 16)])
def test_jacobi_svd_pinned_to_library(shape):
    rng = np.random.default_rng(31)
    M = rng.standard_normal(shape)
    U, s, V = orc.jacobi_svd(M)
    k = min(shape)
    assert U.shape == (shape[0], k) and V.shape == (shape[1], k)
    assert np.max(np.abs((U * s) @ V.T - M)) < 1e-13
    assert np.max(np.abs(U.T @ U - np.eye(k))) < 1e-13
    assert np.max(np.abs(V.T @ V - np.eye(k))) < 1e-13
    assert np.max(np.abs(s - np.linalg.svd(M, compute_uv=False))) < 1e-13


@pytest.mark.parametrize("shape", [(8, 5), (12, 12), (6, 16)])
def test_converged_ns_equals_jacobi_msign(shape):
    rng = np.random.default_rng(32)
    k = min(shape)
    _, _, _, M = _svd_built(rng, *shape, np.linspace(1.0, 0.1, k))
    target = orc.msign_via_svd(M)
    conv = [orc.KJ_COEFFS] * 5 + [orc.TAYLOR_COEFFS] * 5
    O = orc.muon_ns(M, conv)
    assert np.max(np.abs(O - target)) < 1e-12
    # KJ x 5 alone stops short, as the page says (band, not exactly 1)
    O5 = orc.muon_ns(M, SCHEDULES["kj5"])
    assert np.max(np.abs(O5 - target)) > 0.05


def test_nuclear_norm_identity():
    # msign(M) is the best orthogonal approximation, so <M, msign(M)> = sum(sigma).
    rng = np.random.default_rng(33)
    M = rng.standard_normal((10, 7)) + 3 * np.eye(10, 7)
    _, s, _ = orc.jacobi_svd(M)
    conv = [orc.KJ_COEFFS] * 8 + [orc.TAYLOR_COEFFS] * 6
    O = orc.muon_ns(M, conv)
    assert abs(np.sum(M * O) - np.sum(s)) < 1e-11


def test_msign_matches_best_orthogonal_approximation_by_brute_force():
    # 2x2: search over all rotations/reflections for argmin ||M - O||_F.
    rng = np.random.default_rng(34)
    M = rng.standard_normal((2, 2))
    best, best_err = None, np.inf
    for th in np.linspace(0, 2 * np.pi, 200001):
        c, s = np.cos(th), np.sin(th)
        for O in (np.array([[c, -s], [s, c]]), np.array([[c, s], [s, -c]])):
            err = np.sum((M - O) ** 2)
            if err < best_err:
                best, best_err = O, err
    conv = [orc.KJ_COEFFS] * 10 + [orc.TAYLOR_COEFFS] * 6
    assert np.max(np.abs(orc.muon_ns(M, conv) - best)) < 1e-4


# ----------------------------------------------------------------------------
# Scale rules: the page's worked example and the RMS alignment claim
# ----------------------------------------------------------------------------

def test_scale_rules_worked_example():
    ex = _printed()["scale_worked_example"]
    r, c = ex["shape"]
    assert orc.scale_factor(r, c, "kellerjordan") == pytest.approx(ex["kellerjordan"], abs=1e-12)
    assert orc.scale_factor(r, c, "moonlight") == pytest.approx(ex["moonlight"], abs=1e-12)
    assert orc.scale_factor(r, c, "mup") == pytest.approx(0.5, abs=1e-12)
    assert orc.scale_factor(r, c, "naive") == 1.0
    # tall version: the expansion case of the KJ rule
    assert orc.scale_factor(c, r, "kellerjordan") == pytest.approx(2.0, abs=1e-12)
    assert orc.scale_factor(c, r, "mup") == pytest.approx(2.0, abs=1e-12)
    assert orc.scale_factor(c, r, "moonlight") == pytest.approx(12.8, abs=1e-12)


def test_moonlight_update_rms_is_point_two():
    rng = np.random.default_rng(35)
    G = rng.standard_normal((256, 1024))
    conv = [orc.KJ_COEFFS] * 10 + [orc.TAYLOR_COEFFS] * 6
    O = orc.muon_ns(G, conv)
    rms = np.sqrt(np.mean(O * O))
    assert rms == pytest.approx(1.0 / np.sqrt(1024), rel=1e-9)
    s = orc.scale_factor(256, 1024, "moonlight")
    assert s * rms == pytest.approx(_printed()["update_rms_alignment"]["adamw_update_rms_over_lr"], rel=1e-9)


# ----------------------------------------------------------------------------
# Momentum, weight decay, apply: closed forms over several steps
# ----------------------------------------------------------------------------

def test_momentum_geometric_series():
    rng = np.random.default_rng(36)
    G = rng.standard_normal((5, 7))
    M0 = rng.standard_normal((5, 7))
    beta = 0.9
    M = M0.copy()
    for k in range(1, 13):
        M = orc.momentum_update(M, G, beta)
        closed = beta ** k * M0 + G * (1 - beta ** k) / (1 - beta)
        assert np.max(np.abs(M - closed)) < 1e-12


def test_weight_decay_only_when_gradient_is_zero():
    rng = np.random.default_rng(37)
    W = rng.standard_normal((6, 9))
    Z = np.zeros_like(W)
    lr, wd = 0.05, 0.3
    cur = W.copy()
    for k in range(1, 6):
        out = orc.muon_step(cur, Z, Z, lr=lr, beta=0.95, weight_decay=wd,
                            schedule=SCHEDULES["kj5"], scale_rule="moonlight")
        assert np.all(out["O"] == 0.0)
        cur = out["W"]
        f = 1.0 - orc.as_f32(lr) * orc.as_f32(wd)
        assert np.max(np.abs(cur - f ** k * W)) < 1e-12


@pytest.mark.parametrize("rule", orc.SCALE_RULES)
def test_step_closed_form_and_descent_direction(rule):
    # Build G and M on shared singular vectors so every stage has a closed form.
    rng = np.random.default_rng(38)
    rows, cols = 14, 22
    U = _orthonormal(rng, rows, rows)
    V = _orthonormal(rng, cols, rows)
    sg = np.geomspace(2.0, 0.05, rows)
    sm = np.geomspace(1.0, 0.3, rows)
    G = (U * sg) @ V.T
    M = (U * sm) @ V.T
    W = rng.standard_normal((rows, cols)) / np.sqrt(cols)
    lr, beta, wd = 0.02, 0.9, 0.1
    out = orc.muon_step(W, G, M, lr=lr, beta=beta, weight_decay=wd,
                        schedule=SCHEDULES["hybrid8+2"], scale_rule=rule)
    b32, lr32, wd32 = orc.as_f32(beta), orc.as_f32(lr), orc.as_f32(wd)
    sch32 = [tuple(orc.as_f32(v) for v in t) for t in SCHEDULES["hybrid8+2"]]
    s_new = b32 * sm + sg
    xhat = s_new / (np.linalg.norm(s_new) + orc.as_f32(1e-7))
    O = (U * orc.phi_schedule(xhat, sch32)) @ V.T
    scale = orc.as_f32(orc.scale_factor(rows, cols, rule))
    assert np.max(np.abs(out["M"] - (U * s_new) @ V.T)) < 1e-12
    assert np.max(np.abs(out["O"] - O)) < 1e-12
    assert np.max(np.abs(out["W"] - ((1 - lr32 * wd32) * W - lr32 * scale * O))) < 1e-12
    # the step (without decay) opposes the momentum
    step = out["W"] - (1 - lr32 * wd32) * W
    assert np.sum(step * out["M"]) < 0


def test_nesterov_closed_form():
    rng = np.random.default_rng(39)
    rows, cols = 10, 16
    U = _orthonormal(rng, rows, rows)
    V = _orthonormal(rng, cols, rows)
    sg = np.geomspace(1.0, 0.1, rows)
    sm = np.geomspace(0.5, 0.4, rows)
    G, M = (U * sg) @ V.T, (U * sm) @ V.T
    W = np.zeros((rows, cols))
    out = orc.muon_step(W, G, M, lr=1.0, beta=0.8, weight_decay=0.0,
                        schedule=SCHEDULES["kj5"], nesterov=True)
    b = orc.as_f32(0.8)
    s_u = b * (b * sm + sg) + sg
    xhat = s_u / (np.linalg.norm(s_u) + orc.as_f32(1e-7))
    sch32 = [tuple(orc.as_f32(v) for v in t) for t in SCHEDULES["kj5"]]
    assert np.max(np.abs(out["O"] - (U * orc.phi_schedule(xhat, sch32)) @ V.T)) < 1e-12
    assert np.max(np.abs(out["M"] - (U * (b * sm + sg)) @ V.T)) < 1e-12


def test_zero_momentum_and_gradient_give_zero_update():
    W = np.arange(12, dtype=np.float64).reshape(3, 4)
    Z = np.zeros_like(W)
    out = orc.muon_step(W, Z, Z, lr=0.1, beta=0.95, weight_decay=0.0,
                        schedule=SCHEDULES["kj5"])
    assert np.all(out["O"] == 0) and np.all(out["W"] == W)


# ----------------------------------------------------------------------------
# Rounding to the storage dtype
# ----------------------------------------------------------------------------

def test_rne_bf16_matches_torch_on_fp32_values():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(40)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-80, 80, 200000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = orc.rne(x.astype(np.float64), "bf16")
    assert np.array_equal(got, ref)


def test_rne_bf16_ties_and_edges():
    u = 2.0 ** -7   # bf16 ulp at 1
    cases = {
        1.0 + u / 2: 1.0,                  # tie, round to even (1.0)
        1.0 + 3 * u / 2: 1.0 + 2 * u,      # tie, round to even (1 + 2u)
        1.0 + u / 2 + 2 ** -40: 1.0 + u,   # just above the tie (fp64-only bit)
        -(1.0 + u / 2 + 2 ** -40): -(1.0 + u),
        2.0 ** -133: 2.0 ** -133,          # smallest subnormal
        2.0 ** -134: 0.0,                  # tie to even (zero)
        3e38 * 1.2: np.inf,
    }
    for x, want in cases.items():
        assert orc.rne(np.array([x]), "bf16")[0] == np.float32(want), x
