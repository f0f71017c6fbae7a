"""fp64 CPU oracle for the Muon optimizer step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code,
header, helper or constant with the HIP implementation; the only thing both
sides share is the seeded input generator in ``workloads/``.

Sources (cited by page title and section; the page text is Chinese):

* [Muon优化器] -- linsight.cn/f25d614e.html, the technical page on Muon:
  sections "Muon 的核心思想——谱均衡化" (msign), "Newton-Schulz 迭代——高效实现
  与系数优化" (the iteration, its coefficients and the Taylor derivation),
  "缩放因子：从初始化到更新尺度" (the four update-scale rules and the
  1024x4096 worked example) and the closing industrial ``Muon`` class
  (momentum, Nesterov flag, decoupled weight decay and apply).
* [DeepSeek V4 summary] -- prism.simon-ai.net/article/8795, section
  "Muon的训练效率与DeepSeek V4的混合优化策略": the hybrid schedule of 8 fast
  iterations followed by 2 stable ones.
* [Adam vs Muon essay] -- guanweilu.cn/article/354.html: the step is named
  ``muon_step(weight, grad, momentum, lr, beta)``; update = U V^T of the
  momentum.
* [Muon在Stiefel流形上的精确闭式更新解析] -- mlqm.cn/news/1339166: the AdamW
  half of a training step (section 4.3) and the Muon-Cayley update on the
  Stiefel manifold (sections 1.3, 3.1-3.3, 6.2).

Modules: ``muon_oracle`` (the Muon step), ``jacobi_svd`` (a pin for it),
``adamw_oracle`` (AdamW for the non-matrix parameters), ``cayley_oracle``
(Muon-Cayley on the Stiefel manifold).

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
against closed forms, invariants, a hand-written Jacobi SVD, library routines
on special cases, or the pages' worked examples.  No function is
"parity unpinned".
"""
from .muon_oracle import (  # noqa: F401
    KJ_COEFFS,
    TAYLOR_COEFFS,
    SCALE_RULES,
    as_f32,
    momentum_update,
    frobenius_normalize,
    newton_schulz,
    scale_factor,
    apply_update,
    muon_step,
    muon_ns,
    phi,
    phi_schedule,
    rne,
    hybrid_schedule,
)
from .jacobi_svd import jacobi_svd, msign_via_svd  # noqa: F401
from .adamw_oracle import adamw_step  # noqa: F401
from .cayley_oracle import (  # noqa: F401
    cayley_retraction,
    cayley_retraction_lowrank,
    cayley_step,
    center_columns,
    orthogonality_error,
    project_tangent,
)
