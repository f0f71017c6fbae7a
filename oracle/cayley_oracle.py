"""Muon-Cayley on the Stiefel manifold in fp64: the closed-form retraction update.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Source: [Muon在Stiefel流形上的精确闭式更新解析] (mlqm.cn/news/1339166):
* section 1.3: the tangent space of the Stiefel manifold at W (W^T W = I) holds
  the X with X^T W + W^T X = 0; a gradient G is projected onto it as
  G - W sym(W^T G), sym(S) = (S + S^T) / 2;
* section 3.1: for a skew-symmetric A, Q = (I + c A)^(-1) (I - c A) is
  orthogonal, so Q W keeps W^T W = I;
* section 3.2: with V the projected direction, A = V W^T - W V^T and c = lr / 2,
  W' = (I + c A)^(-1) (I - c A) W;
* section 3.3: the order of one step is: center the gradient, update the
  momentum as M = beta M + (1 - beta) G_centered, project M onto the tangent
  space at W to get V, apply the Cayley update;
* section 6.2: the same update reduces to a 2k x 2k linear system, because A
  has rank at most 2k (see cayley_retraction_lowrank for the derivation used
  here).

Readings where the pages leave a choice:
* centering subtracts each column's mean over the rows (the page's code takes
  the mean over dimension 0; its text only says the mean is removed);
* matrices with more columns than rows are handled as their transposes (the
  page's row-orthogonal mirror); the momentum state is stored untransposed;
* there is no weight decay on this path (the page's Cayley branch has none).
"""
from __future__ import annotations

import numpy as np

from .muon_oracle import as_f32


def center_columns(G):
    """G minus the mean of each column (taken over the rows)."""
    G = np.asarray(G, np.float64)
    return G - G.mean(axis=0, keepdims=True)


def sym(S):
    return 0.5 * (S + S.T)


def project_tangent(W, X):
    """X - W sym(W^T X): the tangent-space component at W (W^T W = I)."""
    W = np.asarray(W, np.float64)
    X = np.asarray(X, np.float64)
    return X - W @ sym(W.T @ X)


def cayley_retraction(W, V, lr):
    """(I + c A)^(-1) (I - c A) W with A = V W^T - W V^T and c = lr / 2, as an n x n solve."""
    W = np.asarray(W, np.float64)
    V = np.asarray(V, np.float64)
    c = np.float64(lr) / 2.0
    A = V @ W.T - W @ V.T
    n = W.shape[0]
    eye = np.eye(n)
    return np.linalg.solve(eye + c * A, (eye - c * A) @ W)


def cayley_retraction_lowrank(W, V, lr):
    """The same update through a 2k x 2k solve instead of an n x n one.

    Derivation (section 6.2 states that the n x n system reduces to 2k x 2k):
    A = V W^T - W V^T factors as A = L R with L = [V, W] (n x 2k) and
    R = [W^T; -V^T] (2k x n).  Since I - cA = 2I - (I + cA), the Cayley factor
    is (I + cA)^(-1) (I - cA) = 2 (I + cA)^(-1) - I.  The Woodbury identity
    gives (I + c L R)^(-1) = I - c L (I_2k + c R L)^(-1) R, hence
        W' = 2 (I + cA)^(-1) W - W = W - 2c L (I_2k + c R L)^(-1) (R W).
    """
    W = np.asarray(W, np.float64)
    V = np.asarray(V, np.float64)
    c = np.float64(lr) / 2.0
    left = np.hstack([V, W])
    right = np.vstack([W.T, -V.T])
    inner = np.eye(left.shape[1]) + c * (right @ left)
    return W - 2.0 * c * (left @ np.linalg.solve(inner, right @ W))


def cayley_step(W, G, M, *, lr, beta, retraction=cayley_retraction):
    """One Muon-Cayley step for one matrix.  Returns W', M' and V (fp64).

    Inputs hold fp32 values; lr and beta are rounded to fp32 first (they cross
    the C boundary as float).
    """
    W = np.asarray(W, np.float64)
    G = np.asarray(G, np.float64)
    M = np.asarray(M, np.float64)
    if W.ndim != 2 or W.shape != G.shape or W.shape != M.shape:
        raise ValueError("W, G and M must be 2-D with equal shapes")
    lr, beta = as_f32(lr), as_f32(beta)
    if W.shape[0] < W.shape[1]:   # row-orthogonal mirror: work on the transposes
        out = cayley_step(W.T, G.T, M.T, lr=lr, beta=beta, retraction=retraction)
        return {"W": out["W"].T, "M": out["M"].T, "V": out["V"].T}
    M_new = beta * M + (1.0 - beta) * center_columns(G)
    V = project_tangent(W, M_new)
    return {"W": retraction(W, V, lr), "M": M_new, "V": V}


def orthogonality_error(W):
    """||W^T W - I||_F (the page's section 5.1 check), for n >= k."""
    W = np.asarray(W, np.float64)
    if W.shape[0] < W.shape[1]:
        W = W.T
    return float(np.linalg.norm(W.T @ W - np.eye(W.shape[1])))
