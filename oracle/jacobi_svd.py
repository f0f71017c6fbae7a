"""Hand-written one-sided Jacobi SVD (Hestenes' method) in fp64.

TEST INFRASTRUCTURE ONLY.  Used by the pins to check the Newton-Schulz oracle
against the definition msign(M) = U V^T ([Muon优化器], section
"Muon 的核心思想——谱均衡化": msign sets every nonzero singular value to 1;
[Adam vs Muon essay]: the update is U V^T of the momentum's SVD).  Meant for
tiny, well-conditioned matrices; it is slow by design.

Method: orthogonalize pairs of columns of A (m >= n) by plane rotations,
sweeping cyclically over all pairs, until every pair is orthogonal to a
relative tolerance.  The column norms are then the singular values, the
normalized columns are the left singular vectors and the accumulated rotations
are the right singular vectors.
"""
from __future__ import annotations

import numpy as np


def jacobi_svd(M, tol=1e-15, max_sweeps=100):
    """Return (U, s, V) with M = U @ diag(s) @ V.T, s descending, thin form."""
    M = np.array(M, dtype=np.float64)
    transposed = M.shape[0] < M.shape[1]
    A = M.T.copy() if transposed else M.copy()
    m, n = A.shape
    V = np.eye(n)
    for _ in range(max_sweeps):
        rotated = False
        for i in range(n - 1):
            for j in range(i + 1, n):
                alpha = float(A[:, i] @ A[:, i])
                beta = float(A[:, j] @ A[:, j])
                gamma = float(A[:, i] @ A[:, j])
                if abs(gamma) <= tol * np.sqrt(alpha * beta) or gamma == 0.0:
                    continue
                rotated = True
                zeta = (beta - alpha) / (2.0 * gamma)
                t = np.copysign(1.0, zeta) / (abs(zeta) + np.sqrt(1.0 + zeta * zeta))
                c = 1.0 / np.sqrt(1.0 + t * t)
                s = c * t
                ai, aj = A[:, i].copy(), A[:, j].copy()
                A[:, i] = c * ai - s * aj
                A[:, j] = s * ai + c * aj
                vi, vj = V[:, i].copy(), V[:, j].copy()
                V[:, i] = c * vi - s * vj
                V[:, j] = s * vi + c * vj
        if not rotated:
            break
    s = np.sqrt(np.sum(A * A, axis=0))
    order = np.argsort(-s)
    s = s[order]
    A = A[:, order]
    V = V[:, order]
    U = np.zeros_like(A)
    nz = s > 0
    U[:, nz] = A[:, nz] / s[nz]
    if transposed:
        return V, s, U
    return U, s, V


def msign_via_svd(M, rank_tol=1e-12):
    """msign(M) = sum over nonzero singular values of u_i v_i^T."""
    U, s, V = jacobi_svd(M)
    keep = s > rank_tol * (s[0] if s.size else 0.0)
    return U[:, keep] @ V[:, keep].T
