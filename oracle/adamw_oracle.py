"""The AdamW step in fp64, for the non-matrix parameters of a Muon training step.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Sources (by page title and section):

* [Muon优化器], section "AdamW的问题": per-parameter first and second moments
  m = beta1 m + (1 - beta1) g and v = beta2 v + (1 - beta2) g^2, bias
  corrections m / (1 - beta1^t) and v / (1 - beta2^t), and the step
  lr * m_hat / (sqrt(v_hat) + eps).
* [DeepSeek V4 summary], section "Adam优化器的机制与AdamW的改进": AdamW applies
  weight decay apart from the gradient-based update.
* [Muon在Stiefel流形上的精确闭式更新解析], section 4.3: the parameter is first
  multiplied by (1 - lr * weight_decay), then the corrected step is
  subtracted; the moments start at zero and t counts calls.

Readings where the pages leave a choice: the moments are kept in fp32
whatever the parameter dtype; the decay uses the same lr as the step; t is
the step count after this call's increment (t >= 1).  Scalars are rounded to
fp32 first, as they cross the C boundary as float; the bias corrections are
formed from them in fp64.
"""
from __future__ import annotations

import numpy as np

from .muon_oracle import as_f32, rne


def adamw_step(p, g, m, v, *, lr, beta1, beta2, eps, weight_decay, step, dtype="f32"):
    """One AdamW step for one tensor.  Returns fp64 results and their stored roundings.

    p and g hold values of the parameter dtype, m and v fp32 values; all are
    upcast exactly.  Order of operations:
      1. m' = beta1 m + (1 - beta1) g
      2. v' = beta2 v + (1 - beta2) g^2
      3. m_hat = m' / (1 - beta1^t), v_hat = v' / (1 - beta2^t)
      4. p' = (1 - lr wd) p - lr m_hat / (sqrt(v_hat) + eps)
    """
    if int(step) < 1:
        raise ValueError("step counts calls and starts at 1")
    p = np.asarray(p, np.float64)
    g = np.asarray(g, np.float64)
    m = np.asarray(m, np.float64)
    v = np.asarray(v, np.float64)
    lr, b1, b2 = as_f32(lr), as_f32(beta1), as_f32(beta2)
    eps, wd = as_f32(eps), as_f32(weight_decay)
    t = int(step)
    m_new = b1 * m + (1.0 - b1) * g
    v_new = b2 * v + (1.0 - b2) * g * g
    m_hat = m_new / (1.0 - b1 ** t)
    v_hat = v_new / (1.0 - b2 ** t)
    p_new = (1.0 - lr * wd) * p - lr * m_hat / (np.sqrt(v_hat) + eps)
    return {
        "p": p_new,
        "m": m_new,
        "v": v_new,
        "p_rounded": rne(p_new, dtype),
        "m_rounded": rne(m_new, "f32"),
        "v_rounded": rne(v_new, "f32"),
    }
