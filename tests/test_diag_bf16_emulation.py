"""CPU check of the precision plan with the bf16 emulation diagnostic.

On a low-rank input (the pages' late-training gradients), storing the
Newton-Schulz iterate in bf16 misses the fp64 oracle by far more than the
bf16 tolerance of 3e-2, while an fp32 iterate with bf16 operand copies (the
kernels' plan) stays well inside it.
"""
import numpy as np

import diag_bf16_emulation as diag
import oracle as orc


def test_fp32_iterate_needed_on_low_rank_input():
    rng = np.random.default_rng(7)
    G = diag.lowrank(rng, 256, 384, 8, 1e-3)
    r = diag.compare(G, [orc.KJ_COEFFS] * 5)
    assert r["fp32_iterate"][0] < 1e-2
    assert r["fp32_iterate"][1] < 0.05
    assert r["bf16_storage"][0] > 3e-2
