"""The Muon optimizer step in fp64, written step by step from the pages.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Precision and input conventions (readings where the pages are silent):

* Every input array holds values that are exactly representable in the
  caller's dtype (bf16 or fp32); they are upcast to fp64 without change.
* Scalars that cross the C boundary as ``float`` (lr, beta, weight decay,
  eps and every Newton-Schulz coefficient) are rounded to fp32 first, with
  :func:`as_f32`, so both sides see the same numbers.  The oracle then
  computes in fp64.
* The method's result is the fp64 value; :func:`rne` rounds it once
  (round-to-nearest-even) to the storage dtype when a stored tensor is
  compared.
"""
from __future__ import annotations

import numpy as np

# [Muon优化器], section "Newton-Schulz 迭代——高效实现与系数优化": the empirically
# tuned quintic coefficients (a, b, c) for five iterations on square matrices.
KJ_COEFFS = (3.4445, -4.7750, 2.0315)

# Same section: the Taylor expansion of t^(-1/2) about t = 1 to second order,
# (15 - 10 t + 3 t^2) / 8, gives the "theoretical" triple.  Its scalar map has
# a fixed point at 1 with zero slope, which is why it serves as the "stable"
# triple of the hybrid schedule (see hybrid_schedule).
TAYLOR_COEFFS = (15.0 / 8.0, -10.0 / 8.0, 3.0 / 8.0)

# [Muon优化器], section "缩放因子：从初始化到更新尺度": the four update-scale rules.
SCALE_RULES = ("naive", "kellerjordan", "mup", "moonlight")


def as_f32(x) -> float:
    """Round a Python scalar to the nearest fp32 value, returned as fp64."""
    return float(np.float32(x))


def hybrid_schedule(n_fast: int, n_stable: int, fast=KJ_COEFFS, stable=TAYLOR_COEFFS):
    """Coefficient schedule: ``n_fast`` fast triples, then ``n_stable`` stable ones.

    [DeepSeek V4 summary], section "Muon的训练效率与DeepSeek V4的混合优化策略":
    the first 8 iterations use coefficients that push singular values towards 1
    quickly, the last 2 use more stable coefficients that hold them at 1.  The
    page prints no stable triple; the reading used here is the Taylor triple,
    the only triple on the pages whose map has a fixed point at exactly 1.
    """
    return [tuple(fast)] * n_fast + [tuple(stable)] * n_stable


# --------------------------------------------------------------------------
# Scalar maps (used by the pins: each NS step acts on every singular value
# through this odd quintic).
# --------------------------------------------------------------------------

def phi(x, a, b, c):
    """One step's action on a singular value: a*x + b*x^3 + c*x^5.

    [Muon优化器], section "Newton-Schulz 迭代——高效实现与系数优化": with
    A = X X^T, B = bA + cA^2 and X <- aX + BX, a singular value x of X maps to
    a x + b x^3 + c x^5.
    """
    x = np.asarray(x, dtype=np.float64)
    x2 = x * x
    return x * (a + x2 * (b + c * x2))


def phi_schedule(x, schedule):
    """Compose :func:`phi` over a schedule of (a, b, c) triples, first to last."""
    y = np.asarray(x, dtype=np.float64)
    for (a, b, c) in schedule:
        y = phi(y, a, b, c)
    return y


# --------------------------------------------------------------------------
# The step, in the order the industrial Muon class of [Muon优化器] runs it.
# --------------------------------------------------------------------------

def momentum_update(M, G, beta):
    """M' = beta * M + G, no dampening.

    [Muon优化器], the ``Muon.step`` listing: the buffer is multiplied by the
    momentum coefficient and the gradient is added.  [Adam vs Muon essay]
    writes the same recurrence.  (The Stiefel page's EMA form
    beta*M + (1 - beta)*G is not this method's reading.)
    """
    return np.float64(beta) * np.asarray(M, np.float64) + np.asarray(G, np.float64)


def frobenius_normalize(U, eps):
    """X = U / (||U||_F + eps).

    [Muon优化器], ``zeropower_via_newtonschulz``: divide by the (Frobenius)
    norm plus eps so that the top singular value is at most 1.  The norm is
    written out as the square root of the sum of squares.
    """
    U = np.asarray(U, np.float64)
    nrm = np.sqrt(np.sum(U * U))
    return U / (nrm + np.float64(eps))


def newton_schulz(X, schedule):
    """Odd-quintic Newton-Schulz iteration on an already normalized X.

    [Muon优化器], ``zeropower_via_newtonschulz``: if the matrix has more rows
    than columns it is transposed so that the Gram matrix is formed on the
    smaller side (square matrices are not transposed); then for each step
    A = X X^T, B = b A + c A A, X = a X + B X; finally the transpose is undone.
    The coefficients may change from step to step (hybrid schedule).
    """
    X = np.asarray(X, np.float64)
    transpose = X.shape[0] > X.shape[1]
    if transpose:
        X = X.T
    for (a, b, c) in schedule:
        a, b, c = np.float64(a), np.float64(b), np.float64(c)
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    if transpose:
        X = X.T
    return np.ascontiguousarray(X)


def scale_factor(rows: int, cols: int, rule: str) -> float:
    """Shape-dependent update scale for a rows x cols weight (rows = d_out).

    [Muon优化器], section "缩放因子：从初始化到更新尺度" and ``get_scale`` in the
    class listing: with the PyTorch Linear layout d_out x d_in,
      naive        1
      kellerjordan sqrt(max(1, d_out / d_in))
      mup          sqrt(d_out / d_in)
      moonlight    0.2 * sqrt(max(d_out, d_in))
    """
    d_out, d_in = float(rows), float(cols)
    if rule == "naive":
        return 1.0
    if rule == "kellerjordan":
        return float(np.sqrt(max(1.0, d_out / d_in)))
    if rule == "mup":
        return float(np.sqrt(d_out / d_in))
    if rule == "moonlight":
        return float(0.2 * np.sqrt(max(d_out, d_in)))
    raise ValueError(f"unknown scale rule {rule!r}")


def apply_update(W, O, lr, wd, scale):
    """W' = (1 - lr*wd) W - lr*scale*O  (decoupled weight decay, then the step).

    [Muon优化器], the last two lines of ``Muon.step``: the parameter is
    multiplied by (1 - lr*weight_decay), then lr times the scaled orthogonalized
    update is subtracted.  Written here as one exact fp64 expression.
    """
    lr, wd, scale = np.float64(lr), np.float64(wd), np.float64(scale)
    return (1.0 - lr * wd) * np.asarray(W, np.float64) - (lr * scale) * np.asarray(O, np.float64)


def muon_ns(X_in, schedule, eps=1e-7):
    """Normalize then orthogonalize: the ``zeropower_via_newtonschulz`` contract."""
    sched = [tuple(as_f32(v) for v in t) for t in schedule]
    return newton_schulz(frobenius_normalize(X_in, as_f32(eps)), sched)


def muon_step(W, G, M, *, lr, beta, weight_decay, schedule, scale_rule="naive",
              eps=1e-7, nesterov=False, dtype="f32"):
    """One Muon step for one 2-D weight.  Returns a dict of fp64 and rounded results.

    Order of operations ([Muon优化器], ``Muon.step``):
      1. M' = beta*M + G
      2. U = M' (or, with Nesterov, U = beta*M' + G)
      3-6. O = NS(U / (||U||_F + eps)) with the caller's coefficient schedule
      7. s = scale_factor(rows, cols, rule)
      8. W' = (1 - lr*wd) W - lr*s*O
    Scalars are rounded to fp32 first (see :func:`as_f32`).
    """
    W = np.asarray(W, np.float64)
    G = np.asarray(G, np.float64)
    M = np.asarray(M, np.float64)
    if W.ndim != 2 or W.shape != G.shape or W.shape != M.shape:
        raise ValueError("W, G and M must be 2-D with equal shapes")
    lr, beta, wd, eps = as_f32(lr), as_f32(beta), as_f32(weight_decay), as_f32(eps)
    sched = [tuple(as_f32(v) for v in t) for t in schedule]

    M_new = momentum_update(M, G, beta)
    U = momentum_update(M_new, G, beta) if nesterov else M_new
    O = newton_schulz(frobenius_normalize(U, eps), sched)
    rows, cols = W.shape
    s = as_f32(scale_factor(rows, cols, scale_rule))
    W_new = apply_update(W, O, lr, wd, s)
    return {
        "W": W_new,
        "M": M_new,
        "O": O,
        "scale": s,
        "W_rounded": rne(W_new, dtype),
        "M_rounded": rne(M_new, dtype),
    }


# --------------------------------------------------------------------------
# Rounding to the storage dtype.
# --------------------------------------------------------------------------

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def rne(x, dtype: str):
    """Round fp64 values once, to nearest-even, to ``dtype`` ('f32' or 'bf16').

    Returned as float32 arrays (bf16 values are exactly representable in fp32).
    bf16 has an 8-bit significand and fp32's exponent range; subnormals have a
    quantum of 2^-133.
    """
    x = np.asarray(x, np.float64)
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype != "bf16":
        raise ValueError(dtype)
    m, e = np.frexp(x)                       # x = m * 2^e, 0.5 <= |m| < 1
    q = np.ldexp(np.rint(m * 256.0), e - 8)  # keep 8 significant bits, ties to even
    sub = np.abs(x) < 2.0 ** -126
    if np.any(sub):
        q_sub = np.ldexp(np.rint(np.ldexp(x, 133)), -133)
        q = np.where(sub, q_sub, q)
    over = np.abs(q) > _BF16_MAX
    if np.any(over):
        q = np.where(over, np.copysign(np.inf, x), q)
    q = np.where(np.isfinite(x), q, x)
    return q.astype(np.float32)
