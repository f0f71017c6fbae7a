"""Tabulate the parity margins recorded by the GPU tests.

The GPU parity tests append one JSON line per checked matrix to the file named
by MUON_PARITY_LOG (see tests/_util.py, ``record_parity``).  This script turns
such a log into the markdown summary kept under profiles/:

    MUON_PARITY_LOG=gpurun_out/parity.jsonl python -m pytest tests -m gpu -x -q
    python tests/parity_summary.py gpurun_out/parity.jsonl profiles/parity_margins.md "<command>"

No GPU is needed for the second step.
"""
from __future__ import annotations

import json
import sys


def fmt_range(r):
    return "—" if not r else f"[{r[0]:.4f}, {r[1]:.4f}]"


def main(log_path, out_path, command):
    rows = [json.loads(line) for line in open(log_path) if line.strip()]
    # keep the first record per (config, matrix): the named workload checks
    seen, keep = set(), []
    for r in rows:
        key = (r["config"], r["matrix"], tuple(r["shape"]))
        if key in seen:
            continue
        seen.add(key)
        keep.append(r)
    lines = [
        "# Parity margins of the GPU path against the fp64 oracle",
        "",
        "One line per matrix checked by the GPU parity tests (`tests/test_gpu_parity.py`), on the",
        "seeded host draws the oracle reads.  Bars: O relative Frobenius error <= 3e-2 (bf16) or",
        "1e-5 (fp32); for bf16 every singular value of O inside the oracle's [min - 0.05, max + 0.05];",
        "stored M' within 1 ulp of the once-rounded oracle value; W' within 1 ulp plus the share",
        "of O's own error.  'W' bound' is the largest |W'_gpu - W'_oracle| / (1 ulp + O's share) over",
        "the matrix (the test requires <= 1; for fp32 the relative Frobenius error of W' is listed).",
        "'spectrum' is the largest deviation of the sorted singular values of O from the schedule's",
        "scalar map of the input's (28672x8192 only; bar 0.05).",
        "",
        "Command (from the repository root):",
        "",
        f"    {command}",
        "",
        "| case | matrix | shape | dtype | O rel err | bar | margin | sigma(O_gpu) | oracle band | M' max ulp | W' bound | spectrum |",
        "|---|---|---|---|---|---|---|---|---|---|---|---|",
    ]
    for r in keep:
        err, tol = r["o_rel_err"], r["tol"]
        w = f"{r['w_bound_ratio']:.3f}" if "w_bound_ratio" in r else "—"
        if "w_rel_err" in r:
            w = f"rel {r['w_rel_err']:.1e}"
        m = r.get("m_ulp_max", "—")
        sp = f"{r['spectrum_dev']:.4f}" if "spectrum_dev" in r else "—"
        lines.append(
            f"| {r['config']} | {r['matrix']} | {r['shape'][0]}x{r['shape'][1]} | {r['dtype']} | {err:.3e} | "
            f"{tol:.0e} | {tol / max(err, 1e-300):.1f}x | {fmt_range(r.get('sigma'))} | {fmt_range(r.get('band'))} | "
            f"{m} | {w} | {sp} |")
    lines.append("")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines))
    print(f"wrote {out_path} ({len(keep)} matrices)")


if __name__ == "__main__":
    main(sys.argv[1], sys.argv[2], sys.argv[3] if len(sys.argv) > 3 else "(not given)")
