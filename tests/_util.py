"""Helpers shared by the GPU tests (comparison metrics; no method arithmetic)."""
from __future__ import annotations

import numpy as np


def rel_frob(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    if den == 0.0:
        return float(np.linalg.norm(got))
    return float(np.linalg.norm(got - ref) / den)


def _ordered_int(x, dtype):
    """Map float values to integers whose difference counts ulps."""
    x = np.ascontiguousarray(x, np.float32)
    bits = x.view(np.int32).astype(np.int64)
    if dtype == "bf16":
        assert np.all((bits & 0xFFFF) == 0), "values are not bf16"
        bits = bits >> 16
        sign_mask = 1 << 15
    else:
        sign_mask = 1 << 31
    neg = bits < 0 if dtype != "bf16" else (bits & sign_mask) != 0
    mag = bits & (sign_mask - 1)
    return np.where(neg, -mag, mag)


def ulp_distance(got, ref, dtype):
    """Elementwise distance in units of the storage dtype's last place."""
    return np.abs(_ordered_int(got, dtype) - _ordered_int(ref, dtype))


def singular_values(x):
    """Singular values of a 2-D array (fp64, descending), via the smaller Gram."""
    x = np.asarray(x, np.float64)
    g = x @ x.T if x.shape[0] <= x.shape[1] else x.T @ x
    ev = np.linalg.eigvalsh(g)
    return np.sqrt(np.clip(ev[::-1], 0.0, None))


def to_numpy_f32(t):
    import torch
    return t.detach().to(device="cpu", dtype=torch.float32).numpy()


def record_parity(**fields):
    """Append one parity record (a JSON line) to the file named by the
    MUON_PARITY_LOG environment variable, if it is set.  The records are the
    margins of the GPU parity checks (O error, singular-value range against
    the band, M' and W' ulps); tests/parity_summary.py tabulates them."""
    import json
    import os
    path = os.environ.get("MUON_PARITY_LOG")
    if not path:
        return
    clean = {}
    for k, v in fields.items():
        if isinstance(v, (np.floating, np.integer)):
            v = v.item()
        elif isinstance(v, tuple):
            v = list(v)
        clean[k] = v
    with open(path, "a") as fh:
        fh.write(json.dumps(clean) + "\n")
