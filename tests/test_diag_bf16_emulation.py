"""CPU check of the precision plan with the bf16 emulation diagnostic.

On a low-rank input (the pages' late-training gradients), storing the
Newton-Schulz iterate as a single bf16 value misses the fp64 oracle by far
more than the bf16 tolerance of 3e-2.  The kernels' plan keeps the iterate as
the pair hi + lo (hi = bf16(X), the MFMA operand; lo = bf16(X - hi)), about 16
significant bits, with bf16 operands and fp32 sums; that plan stays well
inside the tolerance and tracks an fp32 iterate.
"""
import numpy as np

import diag_bf16_emulation as diag
import oracle as orc


def test_bf16_pair_iterate_needed_on_low_rank_input():
    rng = np.random.default_rng(7)
    G = diag.lowrank(rng, 256, 384, 8, 1e-3)
    r = diag.compare(G, [orc.KJ_COEFFS] * 5)
    pair_err, pair_band = r["bf16_pair"]
    f32_err, f32_band = r["fp32_iterate"]
    # the kernels' plan: within the bf16 tolerance with a wide margin, and the
    # singular values inside the oracle's band
    assert pair_err < 1e-2
    assert pair_band < 0.05
    # it is as good as an fp32 iterate (the pair carries ~16 bits; the operands are bf16 in both)
    assert pair_err < 1.5 * f32_err + 1e-4
    # a single bf16 iterate is not enough on this input
    assert r["bf16_storage"][0] > 3e-2
