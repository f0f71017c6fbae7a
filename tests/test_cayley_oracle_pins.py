"""Pins for the fp64 Muon-Cayley oracle (CPU only).

* 2 x 1 closed form: W = e1, V = v e2 gives a plane rotation,
  W' = ((1 - t^2), -2 t) / (1 + t^2) with t = lr v / 2.
* Orthogonality: W'^T W' = I to rounding for any lr (the page's section 3.1).
* Tangent space (section 1.3): W^T V + V^T W = 0; the projection is idempotent
  and leaves tangent vectors unchanged.
* First order: (W'(lr) - W) / lr -> -(V - W V^T W) as lr -> 0, which fixes the
  sign of A and c = lr / 2.
* The 2k x 2k (low-rank, Woodbury) form of section 6.2 equals the n x n solve.
* Momentum of centered constant gradients: M_t = (1 - beta^t) G_centered.
* The leading block C11 = I + c W^T V of the 2k system (section 6.2): on the
  manifold W^T V is skew, so C11's symmetric part is I and elimination without
  pivoting meets pivots of magnitude >= 1; off it (W = 2 Q) a pivot can fall
  below 1/2.  The GPU path inverts C11 unpivoted and pivots when that happens.
* The Schur complement S = C22 - C21 C11^-1 C12 of the same system: its symmetric
  part is at least C's, whose smallest eigenvalue on the manifold is
  1 - (c / 2) max |1 - sigma(V)^2|; on the benchmark's inputs that bound is near 1,
  so S too is inverted without pivoting, and W = 2 Q drives its fallback as well.
* Planted mistakes are each caught.
"""
import numpy as np
import pytest

import oracle as orc
import oracle.cayley_oracle as co


def _stiefel(rng, n, k):
    q, r = np.linalg.qr(rng.standard_normal((n, k)))
    return q * np.sign(np.diag(r))


def test_two_by_one_is_a_plane_rotation():
    W = np.array([[1.0], [0.0]])
    for v, lr in [(0.3, 0.1), (2.0, 0.5), (-1.5, 2.0)]:
        V = np.array([[0.0], [v]])
        t = lr * v / 2
        expect = np.array([[(1 - t * t)], [-2 * t]]) / (1 + t * t)
        assert np.max(np.abs(orc.cayley_retraction(W, V, lr) - expect)) < 1e-15


@pytest.mark.parametrize("lr", [1e-3, 0.1, 3.0])
def test_retraction_keeps_columns_orthonormal(lr):
    rng = np.random.default_rng(1)
    W = _stiefel(rng, 40, 7)
    V = orc.project_tangent(W, rng.standard_normal((40, 7)))
    assert orc.orthogonality_error(orc.cayley_retraction(W, V, lr)) < 1e-13


def test_projection_is_onto_the_tangent_space():
    rng = np.random.default_rng(2)
    W = _stiefel(rng, 30, 6)
    X = rng.standard_normal((30, 6))
    V = orc.project_tangent(W, X)
    assert np.max(np.abs(W.T @ V + V.T @ W)) < 1e-14
    assert np.max(np.abs(orc.project_tangent(W, V) - V)) < 1e-14
    # a tangent vector with a nonzero skew part W^T T is left unchanged
    S = rng.standard_normal((6, 6))
    T = W @ (S - S.T) + (np.eye(30) - W @ W.T) @ rng.standard_normal((30, 6))
    assert np.max(np.abs(orc.project_tangent(W, T) - T)) < 1e-13


def test_first_order_direction():
    rng = np.random.default_rng(3)
    W = _stiefel(rng, 25, 5)
    V = orc.project_tangent(W, rng.standard_normal((25, 5)))
    lr = 1e-7
    d = (orc.cayley_retraction(W, V, lr) - W) / lr
    assert np.max(np.abs(d + (V - W @ (V.T @ W)))) < 1e-5


@pytest.mark.parametrize("shape", [(64, 16), (33, 5), (8, 8)])
def test_lowrank_form_equals_direct_solve(shape):
    rng = np.random.default_rng(4)
    W = _stiefel(rng, *shape)
    V = orc.project_tangent(W, rng.standard_normal(shape))
    for lr in (1e-3, 0.3, 2.0):
        a = orc.cayley_retraction(W, V, lr)
        b = orc.cayley_retraction_lowrank(W, V, lr)
        assert np.max(np.abs(a - b)) < 1e-12


def test_centering_and_momentum_closed_form():
    rng = np.random.default_rng(5)
    W = _stiefel(rng, 20, 4)
    G = rng.standard_normal((20, 4)) + 3.0
    Gc = orc.center_columns(G)
    assert np.max(np.abs(Gc.mean(axis=0))) < 1e-15
    M = np.zeros_like(G)
    beta = orc.as_f32(0.9)
    for t in range(1, 6):
        out = orc.cayley_step(W, G, M, lr=0.0, beta=0.9)
        M = out["M"]
        assert np.max(np.abs(M - (1 - beta ** t) * Gc)) < 1e-14
        assert np.max(np.abs(out["W"] - W)) < 1e-15      # lr = 0 leaves W


def test_wide_matrix_uses_the_transposed_problem():
    rng = np.random.default_rng(6)
    W = _stiefel(rng, 24, 6).T                      # 6 x 24, orthonormal rows
    G = rng.standard_normal((6, 24))
    M = rng.standard_normal((6, 24))
    out = orc.cayley_step(W, G, M, lr=0.2, beta=0.9)
    ref = orc.cayley_step(W.T, G.T, M.T, lr=0.2, beta=0.9)
    assert np.max(np.abs(out["W"] - ref["W"].T)) == 0.0
    assert np.max(np.abs(out["W"] @ out["W"].T - np.eye(6))) < 1e-13


# ----------------------------------------------------------------------------
# Planted mistakes
# ----------------------------------------------------------------------------

def _retr(sign=1.0, cfac=0.5):
    def r(W, V, lr):
        c = lr * cfac
        A = sign * (V @ W.T - W @ V.T)
        eye = np.eye(W.shape[0])
        return np.linalg.solve(eye + c * A, (eye - c * A) @ W)
    return r


def _pins_fail(monkeypatch, **patches):
    for name, fn in patches.items():
        monkeypatch.setattr(co, name, fn)
        monkeypatch.setattr(orc, name, fn)
    checks = [test_two_by_one_is_a_plane_rotation, test_projection_is_onto_the_tangent_space,
              test_first_order_direction, test_centering_and_momentum_closed_form,
              lambda: test_retraction_keeps_columns_orthonormal(0.1)]
    failed = 0
    for chk in checks:
        try:
            chk()
        except AssertionError:
            failed += 1
    return failed


@pytest.mark.parametrize("kind", ["flipped_A", "c_equals_lr", "projection_without_sym", "centering_rows",
                                  "plain_momentum"])
def test_pins_catch_planted_mistake(kind, monkeypatch):
    if kind == "flipped_A":
        n = _pins_fail(monkeypatch, cayley_retraction=_retr(sign=-1.0))
    elif kind == "c_equals_lr":
        n = _pins_fail(monkeypatch, cayley_retraction=_retr(cfac=1.0))
    elif kind == "projection_without_sym":
        n = _pins_fail(monkeypatch, project_tangent=lambda W, X: X - W @ (W.T @ X))
    elif kind == "centering_rows":
        n = _pins_fail(monkeypatch, center_columns=lambda G: G - np.asarray(G).mean(axis=1, keepdims=True))
    else:
        orig = co.cayley_step

        def plain(W, G, M, *, lr, beta, retraction=co.cayley_retraction):
            W, G, M = (np.asarray(x, np.float64) for x in (W, G, M))
            b = orc.as_f32(beta)
            Mn = b * M + co.center_columns(G)
            V = co.project_tangent(W, Mn)
            return {"W": retraction(W, V, lr), "M": Mn, "V": V}
        n = _pins_fail(monkeypatch, cayley_step=plain)
        assert co.cayley_step is not orig
    assert n > 0, kind


def _unpivoted_pivots(C):
    C = np.array(C, np.float64)
    piv = []
    for j in range(C.shape[0]):
        piv.append(C[j, j])
        C[j + 1:, :] -= np.outer(C[j + 1:, j] / C[j, j], C[j, :])
    return np.array(piv)


def _c11(W, M, lr):
    V = co.project_tangent(W, M)
    return np.eye(W.shape[1]) + (lr / 2.0) * (W.T @ V)


@pytest.mark.parametrize("lr", [0.05, 1.0, 10.0])
def test_leading_block_needs_no_pivoting_on_the_manifold(lr):
    rng = np.random.default_rng(21)
    for n, k in [(300, 24), (64, 64), (1000, 128)]:
        W = _stiefel(rng, n, k)
        M = 3.0 * rng.standard_normal((n, k))
        C11 = _c11(W, M, lr)
        assert np.abs(0.5 * (C11 + C11.T) - np.eye(k)).max() < 1e-9      # symmetric part I
        assert np.abs(_unpivoted_pivots(C11)).min() >= 1.0 - 1e-9


def test_leading_block_off_the_manifold_can_need_pivoting():
    # the input of the GPU test that exercises the pivoting fallback
    import workloads as wk
    h = wk.cayley_host_matrix(300, 24, seed=7, momentum_std=1.0)
    W = 2.0 * h["W"].astype(np.float64)
    M = 0.9 * h["M"].astype(np.float64) + 0.1 * co.center_columns(h["G"])
    assert np.abs(_unpivoted_pivots(_c11(W, M, 1.0))).min() < 0.5


def _schur(W, V, lr):
    # the 2k system C = I + c B U with B = [W^T; -V^T], U = [V, W], built whole
    c, k = lr / 2.0, W.shape[1]
    C = np.eye(2 * k) + c * np.vstack([W.T, -V.T]) @ np.hstack([V, W])
    return C[k:, k:] - C[k:, :k] @ np.linalg.solve(C[:k, :k], C[:k, k:]), C


@pytest.mark.parametrize("lr,std", [(1e-3, 1e-2), (0.05, 1e-2), (0.05, 1.0), (1.0, 0.1)])
def test_schur_complement_pivots_are_bounded_on_the_manifold(lr, std):
    rng = np.random.default_rng(22)
    for n, k in [(300, 24), (1000, 100), (4096, 128)]:
        W = _stiefel(rng, n, k)
        V = co.project_tangent(W, std * rng.standard_normal((n, k)))
        S, C = _schur(W, V, lr)
        # C's symmetric part: I + (c / 2) [0, I - V^T V; I - V^T V, 0]
        mu = 1.0 - (lr / 4.0) * np.abs(np.linalg.eigvalsh(np.eye(k) - V.T @ V)).max()
        assert np.linalg.eigvalsh(0.5 * (C + C.T)).min() >= mu - 1e-9
        assert np.linalg.eigvalsh(0.5 * (S + S.T)).min() >= mu - 1e-9
        assert _unpivoted_pivots(S).min() >= mu - 1e-9


def test_schur_complement_needs_no_pivoting_on_the_benchmark_inputs():
    import workloads as wk
    for seed in range(3):
        h = wk.cayley_host_matrix(4096, 128, seed=seed)
        W = h["W"].astype(np.float64)
        M = 0.9 * h["M"].astype(np.float64) + 0.1 * co.center_columns(h["G"].astype(np.float64))
        V = co.project_tangent(W, M)
        for lr in (1e-3, 0.05, 1.0):
            mu = 1.0 - (lr / 4.0) * np.abs(np.linalg.eigvalsh(np.eye(128) - V.T @ V)).max()
            assert mu >= 0.5
            assert np.abs(_unpivoted_pivots(_schur(W, V, lr)[0])).min() >= 0.5


def test_schur_complement_off_the_manifold_can_need_pivoting():
    import workloads as wk
    h = wk.cayley_host_matrix(300, 24, seed=7, momentum_std=1.0)
    W = 2.0 * h["W"].astype(np.float64)
    M = 0.9 * h["M"].astype(np.float64) + 0.1 * co.center_columns(h["G"])
    assert np.abs(_unpivoted_pivots(_schur(W, co.project_tangent(W, M), 1.0)[0])).min() < 0.5
