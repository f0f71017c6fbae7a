"""DIAGNOSTIC, NOT THE ORACLE: why the GPU path keeps about 16 bits of the Newton-Schulz iterate.

Emulates a bf16-MFMA Newton-Schulz on the CPU (operands rounded to bf16,
products accumulated in fp32) under three storage plans and compares each with
the fp64 oracle on the same bf16 inputs:

* "bf16 storage": X is rounded to bf16 between steps (what a plain bf16
  implementation of the pages' listing does);
* "fp32 iterate": X stays fp32, and only the operand copies of X, A and B are
  rounded to bf16;
* "bf16 pair": X is stored as hi + lo with hi = bf16(X) and lo = bf16(X - hi)
  (about 16 significant bits) and hi serves as the MFMA operand.  This is the
  plan the bf16 kernels follow (fp32 matrices keep an fp32 iterate).

Each step multiplies small singular values by about a = 3.4445
([Muon优化器], Newton-Schulz coefficient section), so rounding noise in those
directions is amplified with them; storing X in bf16 re-injects that noise
every step.  Run as a script for the table at sizes shaped like the workloads:

    python tests/diag_bf16_emulation.py [--seeds N]

``tests/test_diag_bf16_emulation.py`` runs one small case in the CPU suite.
"""
from __future__ import annotations

import argparse
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import oracle as orc  # noqa: E402


def bf16(x):
    """Round to bf16 (nearest-even), returned as float32."""
    return orc.rne(np.asarray(x, np.float64), "bf16").astype(np.float32)


def mm_bf16(P, Q):
    """bf16 operands, fp32 accumulation (emulated: exact products of bf16 values summed in fp32)."""
    return bf16(P) @ bf16(Q)


def bf16_pair(x):
    """x stored as hi + lo, hi = bf16(x), lo = bf16(x - hi) (about 16 significant bits)."""
    x = np.asarray(x, np.float32)
    hi = bf16(x)
    return (hi + bf16(x - hi)).astype(np.float32)


def emulated_ns(U, schedule, eps=1e-7, store_bf16=False, store_pair=False):
    """Normalize and iterate with bf16 operands; X kept in fp32 unless store_bf16 (X rounded
    to bf16 between steps) or store_pair (X rounded to a bf16 hi + lo pair between steps)."""
    U = np.asarray(U, np.float32)
    tr = U.shape[0] > U.shape[1]
    if tr:
        U = U.T
    X = (U / (np.sqrt(np.sum(U.astype(np.float64) ** 2)) + eps)).astype(np.float32)
    store = bf16 if store_bf16 else (bf16_pair if store_pair else (lambda v: v))
    X = store(X)
    for (a, b, c) in schedule:
        A = mm_bf16(X, X.T)
        B = (b * A + c * mm_bf16(A, A.T)).astype(np.float32)
        X = store((a * X + mm_bf16(B, X)).astype(np.float32))
    return X.T if tr else X


def compare(G, schedule):
    """Relative Frobenius error and singular-value band excess of both plans against fp64."""
    ref = orc.muon_ns(G.astype(np.float64), schedule)
    s_ref = np.linalg.svd(ref, compute_uv=False)
    out = {}
    for name, kw in (("bf16_storage", dict(store_bf16=True)), ("fp32_iterate", {}),
                     ("bf16_pair", dict(store_pair=True))):
        got = emulated_ns(G, schedule, **kw).astype(np.float64)
        err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        s = np.linalg.svd(got, compute_uv=False)
        band = max(0.0, s_ref.min() - s.min(), s.max() - s_ref.max())
        out[name] = (float(err), float(band))
    return out


def lowrank(rng, rows, cols, rank, noise):
    G = rng.standard_normal((rows, rank)) @ rng.standard_normal((cols, rank)).T + noise * rng.standard_normal((rows, cols))
    return bf16(G)


CASES = {
    # name: (rows, cols, kind, rank, noise, schedule)
    "square low rank (like 4096^2 rank 64, scaled)": (1024, 1024, "lowrank", 16, 1e-3, [orc.KJ_COEFFS] * 5),
    "tall low rank (like 28672x8192 rank 256, scaled)": (1792, 512, "lowrank", 16, 1e-2, [orc.KJ_COEFFS] * 5),
    "square Gaussian, hybrid 8+2": (1024, 1024, "gauss", 0, 0.0, orc.hybrid_schedule(8, 2)),
    "wide Gaussian 1:4, hybrid 8+2": (512, 2048, "gauss", 0, 0.0, orc.hybrid_schedule(8, 2)),
}


def make(case, seed):
    rows, cols, kind, rank, noise, sched = CASES[case]
    rng = np.random.default_rng(seed)
    G = lowrank(rng, rows, cols, rank, noise) if kind == "lowrank" else bf16(1e-3 * rng.standard_normal((rows, cols)))
    return G, sched


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--seeds", type=int, default=2)
    args = ap.parse_args()
    print(f"{'case':52s} {'seed':>4s}  {'bf16 storage err / band':>24s}  {'fp32 iterate err / band':>24s}"
          f"  {'bf16 pair err / band':>24s}")
    for case in CASES:
        for seed in range(args.seeds):
            G, sched = make(case, seed)
            r = compare(G, sched)
            b, f, h = r["bf16_storage"], r["fp32_iterate"], r["bf16_pair"]
            print(f"{case:52s} {seed:4d}  {b[0]:12.3e} / {b[1]:9.3e}  {f[0]:12.3e} / {f[1]:9.3e}"
                  f"  {h[0]:12.3e} / {h[1]:9.3e}", flush=True)


if __name__ == "__main__":
    main()
