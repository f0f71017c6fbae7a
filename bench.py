#!/usr/bin/env python3
"""Benchmark: one grouped Muon step over a synthetic parameter set on one MI355X.

A "step" is one muon_step call: momentum + norm, the Newton-Schulz schedule
(Gram, polynomial and update per iteration) and scale / weight decay / apply,
over every matrix of the workload, with inputs already resident in HBM.

Default workload: the d=2048, 24-layer transformer parameter set in bf16
(per layer Q, K, V, O 2048x2048, MLP up 8192x2048 and down 2048x8192:
144 matrices), hybrid schedule of 8 fast + 2 stable iterations, Moonlight
scale, lr 3e-4, weight decay 0.01, beta 0.95.

Prints ONE JSON line.  `value` is matrices per second of whole steps.  The
Newton-Schulz FLOP count is algorithmic, 3 m^2 n + m^3 per iteration with
m = min(rows, cols), n = max(rows, cols) (half Gram, half polynomial, full
update).  `roofline` is for the dominant kernel (the update, 2 m^2 n per
matrix per launch), timed with HIP events recorded on the launch stream over
the timed region.  `cpu_baseline` times the fp64 oracle on a bounded sample
of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2516.6     # MI355X dense bf16 MFMA
F32_PEAK_TFLOPS = 157.3       # MI355X fp32 matrix
HBM_PEAK_GBS = 8000.0


# The rocprofv3 session the profiles/ summaries come from (run from the repository root).
PROFILE_COMMANDS = [
    "cd /tmp && export TMPDIR=/tmp",
    "rocprofv3 --kernel-trace --stats --output-format csv -d $R/gpurun_out/prof/trace -o transformer "
    "-- python3 $R/bench.py --steps 5 --warmup 2 --only --no-cpu-baseline",
    "rocprofv3 --pmc FETCH_SIZE --kernel-include-regex muon:: --output-format csv "
    "-d $R/gpurun_out/prof/fetch -o fetch -- python3 $R/bench.py --steps 1 --warmup 1 --only --no-cpu-baseline",
    "rocprofv3 --pmc WRITE_SIZE --kernel-include-regex muon:: --output-format csv "
    "-d $R/gpurun_out/prof/write -o write -- python3 $R/bench.py --steps 1 --warmup 1 --only --no-cpu-baseline",
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $R/gpurun_out/prof/cfetch -o copy "
    "-- python3 $R/bench.py --calibrate-copy",
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d $R/gpurun_out/prof/cwrite -o copy "
    "-- python3 $R/bench.py --calibrate-copy",
    "rocprofv3 --kernel-trace --pmc GRBM_COUNT GRBM_GUI_ACTIVE --kernel-include-regex \"ns_gemm_kernel\" "
    "--output-format csv -d $R/gpurun_out/prof/clock -o clk -- python3 $R/bench.py --steps 1 --warmup 1 --only --no-cpu-baseline",
    "python3 bench.py --summarize-profiles gpurun_out/prof",
]

KERNEL_SOURCES = ("matrix_aware_optimizer_amd/csrc/ns_gemm.hip", "matrix_aware_optimizer_amd/csrc/muon_internal.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "update_kernel_transformer_traffic.json")


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload_id):
    """HBM bytes per update launch from the committed counter runs, if they
    were taken on the current kernel source; otherwise None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash() or t.get("workload_id") != workload_id:
        return None
    return t.get("bytes_per_launch")


def calibrate_copy(nbytes=1 << 30, reps=5):
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    x = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    x.fill_(1.0)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "reps": reps}), flush=True)


def _counter_rows(path, name_part=None):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(path, "*counter_collection.csv"))):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if name_part is None or name_part in r["Kernel_Name"]:
                    rows.append(r)
    return rows


UPDATE_KERNEL = "ns_gemm_kernel<unsigned short, 2>"


def _engine_clock(path):
    """Average engine clock per kernel from a --kernel-trace --pmc GRBM_COUNT run."""
    import csv
    import glob
    traces = sorted(glob.glob(os.path.join(path, "*kernel_trace.csv")))
    if not traces:
        return {}
    dur = {}
    with open(traces[0]) as fh:
        for r in csv.DictReader(fh):
            dur[r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    acc = {}
    for r in _counter_rows(path):
        if r["Counter_Name"] != "GRBM_COUNT" or r["Dispatch_Id"] not in dur:
            continue
        ghz = float(r["Counter_Value"]) / 8.0 / dur[r["Dispatch_Id"]]
        n, tot = acc.get(r["Kernel_Name"], (0, 0.0))
        acc[r["Kernel_Name"]] = (n + 1, tot + ghz)
    def short(k):
        return k.replace("void ", "").replace("muon::(anonymous namespace)::", "").split("(")[0]
    return {short(k): (n, tot / n) for k, (n, tot) in acc.items()}


def summarize_profiles(prof_dir, workload_id, commands):
    """Turn one rocprofv3 session (kernel trace, FETCH_SIZE and WRITE_SIZE runs of
    the update kernel, and the same two counters on a 1 GiB device copy) into
    the text summaries kept under profiles/."""
    import csv
    import glob
    stats = sorted(glob.glob(os.path.join(prof_dir, "trace", "*_kernel_stats.csv")))[0]
    with open(stats) as fh:
        krows = list(csv.DictReader(fh))
    copy_bytes = 1 << 30
    cf = [float(r["Counter_Value"]) for r in _counter_rows(os.path.join(prof_dir, "cfetch"), "copyBuffer")]
    cw = [float(r["Counter_Value"]) for r in _counter_rows(os.path.join(prof_dir, "cwrite"), "copyBuffer")]
    fetch_factor = copy_bytes / (sum(cf) / len(cf) * 1024.0)
    write_factor = copy_bytes / (sum(cw) / len(cw) * 1024.0)
    uf = [float(r["Counter_Value"]) for r in _counter_rows(os.path.join(prof_dir, "fetch"), UPDATE_KERNEL)]
    uw = [float(r["Counter_Value"]) for r in _counter_rows(os.path.join(prof_dir, "write"), UPDATE_KERNEL)]
    # the counted kernel runs ns_steps - 1 times per step: the last update of a
    # step is the kernel that also applies the step to W
    import workloads as wk
    wl = wk.WORKLOADS[workload_id]
    T = len(wl.hp["schedule"])
    read_b = sum(uf) / len(uf) * 1024.0 * fetch_factor
    write_b = sum(uw) / len(uw) * 1024.0 * write_factor
    traffic = {
        "workload_id": workload_id,
        "kernel": UPDATE_KERNEL,
        "source_hash": kernel_source_hash(),
        "dispatches": len(uf),
        "fetch_kib_per_dispatch_raw": round(sum(uf) / len(uf), 1),
        "write_kib_per_dispatch_raw": round(sum(uw) / len(uw), 1),
        "fetch_scale": round(fetch_factor, 4),
        "write_scale": round(write_factor, 4),
        "read_bytes_per_launch": int(read_b),
        "write_bytes_per_launch": int(write_b),
        "bytes_per_launch": int(read_b + write_b),
        "note": f"average over the update launches that write the iterate, {T - 1} per step",
        "commands": commands,
    }
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(traffic, fh, indent=1)
        fh.write("\n")
    lines = [f"# Kernel time per launch, {wl.name}", "",
             "rocprofv3 --kernel-trace --stats summary (`*_kernel_stats.csv`), library kernels only.", "",
             "Commands (from the repository root; `R` is its absolute path):", ""]
    lines += [f"    {c}" for c in commands] + [""]
    lines += ["| kernel | calls | avg ms | min ms | max ms | % of GPU time |", "|---|---|---|---|---|---|"]
    for r in krows:
        if "muon::" not in r["Name"]:
            continue
        nm = r["Name"].replace("void ", "").replace("muon::(anonymous namespace)::", "").split("(")[0]
        lines.append(f"| `{nm}` | {r['Calls']} | {float(r['AverageNs']) / 1e6:.4f} | {float(r['MinNs']) / 1e6:.4f} | "
                     f"{float(r['MaxNs']) / 1e6:.4f} | {float(r['Percentage']):.2f} |")
    lines += ["", f"Update kernel HBM traffic per launch (FETCH_SIZE x {fetch_factor:.3f}, WRITE_SIZE x "
              f"{write_factor:.3f}, factors from a 1 GiB device copy): read {read_b / 1e9:.3f} GB, "
              f"write {write_b / 1e9:.3f} GB.", ""]
    clock = _engine_clock(os.path.join(prof_dir, "clock"))
    if clock:
        lines += ["Engine clock during the Newton-Schulz GEMMs: GRBM_COUNT (summed over the 8 XCDs) / 8 / dispatch",
                  "duration, averaged over the dispatches of one step.", "",
                  "| kernel | dispatches | avg GHz |", "|---|---|---|"]
        lines += [f"| `{k}` | {n} | {ghz:.3f} |" for k, (n, ghz) in sorted(clock.items())]
        lines += [""]
    out = os.path.join(ROOT, "profiles", f"kernels_{wk.short_name(workload_id)}.md")
    with open(out, "w") as fh:
        fh.write("\n".join(lines))
    print(json.dumps({"written": [os.path.relpath(out, ROOT), os.path.relpath(TRAFFIC_FILE, ROOT)]}))


COUNTER_COMMANDS = [
    "cd /tmp && export TMPDIR=/tmp",
    "rocprofv3 --kernel-trace --stats --output-format csv -d $R/gpurun_out/prof/trace -o transformer "
    "-- python3 $R/bench.py --steps 5 --warmup 2 --only --no-cpu-baseline",
    "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_BUSY_CU_CYCLES GRBM_COUNT --kernel-include-regex muon:: "
    "--output-format csv -d $R/gpurun_out/prof/mfma -o mfma -- python3 $R/bench.py --steps 1 --warmup 1 --only --no-cpu-baseline",
    "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE; then TD_TD_BUSY_sum TA_TA_BUSY_sum GRBM_GUI_ACTIVE; then "
    "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS SQ_WAIT_INST_LDS) with the same options, directories "
    "fetch, write, tdta, lds",
    "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -d $R/gpurun_out/prof/cfetch (cwrite) -o copy "
    "-- python3 $R/bench.py --calibrate-copy",
    "python3 bench.py --summarize-counters gpurun_out/prof",
]

# Library kernels by their rocprofv3 names, with the algorithmic work of one launch on a
# workload: ('flop', n) for the matrix-core kernels, ('bytes', n) for the HBM-bound ones.
def _kernel_table(wl):
    shapes = wl.shapes
    elem = sum(r * c for r, c in shapes)
    es = 2 if wl.dtype == "bf16" else 4
    gram = sum(min(r, c) ** 2 * max(r, c) for r, c in shapes)
    poly = sum(min(r, c) ** 3 for r, c in shapes)
    upd = sum(2 * min(r, c) ** 2 * max(r, c) for r, c in shapes)
    t = "unsigned short" if wl.dtype == "bf16" else "float"
    return [
        (f"momentum_norm_kernel<{t}, false>", "K1 momentum + norm", ("bytes", 3 * es * elem)),
        ("norm_finalize_kernel", "norm finalize", None),
        (f"rescale_kernel<{t}>", "norm shift (no-op here)", None),
        (f"ns_gemm_kernel<{t}, 0>", "K2 Gram", ("flop", gram)),
        (f"ns_gemm_kernel<{t}, 3>", "K3 polynomial", ("flop", poly)),
        (f"ns_gemm_kernel<{t}, 2>", "K4 update", ("flop", upd)),
        (f"ns_gemm_kernel<{t}, 4>", "K4 last update + apply", ("flop", upd)),
    ]


def summarize_counters(prof_dir, workload_id, commands):
    """Per-kernel counter table from one rocprofv3 session (see COUNTER_COMMANDS):
    time, engine clock, MFMA busy, TD / TA busy, HBM bytes, LDS conflicts."""
    import csv
    import glob
    import workloads as wk
    wl = wk.WORKLOADS[workload_id]

    def short(k):
        return k.replace("void ", "").replace("muon::(anonymous namespace)::", "").split("(")[0]

    stats = sorted(glob.glob(os.path.join(prof_dir, "trace", "*_kernel_stats.csv")))[0]
    avg_ns = {}
    with open(stats) as fh:
        for r in csv.DictReader(fh):
            avg_ns[short(r["Name"])] = float(r["AverageNs"])
    cnt = {}
    for sub in ("mfma", "fetch", "write", "tdta", "lds"):
        for r in _counter_rows(os.path.join(prof_dir, sub)):
            k = short(r["Kernel_Name"])
            cnt.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))

    def avg(k, c):
        v = cnt.get(k, {}).get(c)
        return sum(v) / len(v) if v else None

    cf = [float(r["Counter_Value"]) for r in _counter_rows(os.path.join(prof_dir, "cfetch"), "copyBuffer")]
    cw = [float(r["Counter_Value"]) for r in _counter_rows(os.path.join(prof_dir, "cwrite"), "copyBuffer")]
    fetch_factor = (1 << 30) / (sum(cf) / len(cf) * 1024.0)
    write_factor = (1 << 30) / (sum(cw) / len(cw) * 1024.0)
    CUS, SIMDS, XCDS = 256, 4, 8
    lines = [f"# Counters per kernel, {wl.name}", "",
             "One rocprofv3 session on the library's kernels (`bench.py --only`, one step after one warm-up",
             "for the counter passes; five steps for the kernel trace).  Each counter pass is its own run.", "",
             "Commands (from the repository root; `R` is its absolute path):", ""]
    lines += [f"    {c}" for c in commands] + [""]
    lines += [
        "How the columns are formed:",
        "",
        "- `ms`: average duration per launch from the kernel trace.",
        "- `GHz`: GRBM_GUI_ACTIVE / 8 (the counter is summed over the 8 XCDs) / the dispatch's duration.",
        "- `MFMA busy`: SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 256 CUs x 4 SIMDs).  The counter",
        "  sums busy cycles over the SIMDs: one 32x32x16 bf16 MFMA (32768 FLOP) keeps a SIMD's matrix core",
        "  busy 32 cycles, so its per-launch value equals the executed FLOP / 1024 (the update: 4.83e9 =",
        "  4.948e12 / 1024).  This is utilization at the clock the kernel ran at, executed work (diagonal",
        "  Gram and polynomial tiles are computed whole), not the published-peak fraction.",
        "- `alg. frac`: algorithmic FLOP (or bytes) per launch / duration / published peak (2516.6 TFLOP/s",
        "  bf16, 8 TB/s HBM), as the benchmark reports it.",
        "- `TD busy`, `TA busy`: TD_TD_BUSY_sum, TA_TA_BUSY_sum / (GRBM_GUI_ACTIVE / 8 x 256).  TD returns",
        "  the operand data to the CU (here mostly direct-to-LDS loads).",
        f"- `HBM read / write`: FETCH_SIZE x {fetch_factor:.3f} and WRITE_SIZE x {write_factor:.3f} (KiB per dispatch;",
        "  factors from a 1 GiB device copy, which reads 0.5 GiB and writes 1 GiB by these counters).",
        "- `LDS conflict`: SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE (cycles stalled on bank conflicts per",
        "  active LDS cycle).",
        "",
        "| kernel | ms | GHz | MFMA busy | alg. frac | TD busy | TA busy | HBM read GB | HBM write GB | LDS conflict |",
        "|---|---|---|---|---|---|---|---|---|---|",
    ]
    for name, label, work in _kernel_table(wl):
        ms = avg_ns.get(name, 0.0) / 1e6
        gui = avg(name, "GRBM_GUI_ACTIVE")
        if not ms or not gui:
            continue
        cyc = gui / XCDS
        ghz = cyc / (ms * 1e6)
        mb = avg(name, "SQ_VALU_MFMA_BUSY_CYCLES")
        mfma = f"{100 * mb / (cyc * CUS * SIMDS):.1f}%" if mb else "—"
        td = avg(name, "TD_TD_BUSY_sum")
        ta = avg(name, "TA_TA_BUSY_sum")
        fr = avg(name, "FETCH_SIZE")
        wr = avg(name, "WRITE_SIZE")
        bc, ia = avg(name, "SQ_LDS_BANK_CONFLICT"), avg(name, "SQ_LDS_IDX_ACTIVE")
        if work is None:
            alg = "—"
        elif work[0] == "flop":
            alg = f"{work[1] / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS * 100:.1f}%"
        else:
            alg = f"{work[1] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS * 100:.1f}% HBM"
        ghz_s = f"{ghz:.2f}" if ms >= 0.05 else "—"   # launch overhead dominates tiny kernels
        lines.append(
            f"| {label} `{name}` | {ms:.4f} | {ghz_s} | {mfma} | {alg} | "
            f"{100 * td / (cyc * CUS):.1f}% | {100 * ta / (cyc * CUS):.1f}% | "
            f"{fr * 1024 * fetch_factor / 1e9:.3f} | {wr * 1024 * write_factor / 1e9:.3f} | "
            f"{(100 * bc / ia) if ia else 0:.1f}% |")
    lines.append("")
    out = os.path.join(ROOT, "profiles", f"counters_{wk.short_name(workload_id)}.md")
    with open(out, "w") as fh:
        fh.write("\n".join(lines))
    print(json.dumps({"written": os.path.relpath(out, ROOT)}))


def measure_adamw(dev, steps, dtype="bf16"):
    """The AdamW half of the step: the transformer's non-matrix parameters (token
    embedding and head, 32000 x 2048 each, and 49 norm vectors of 2048), timed with
    the library's HIP events.  Algorithmic bytes per element: read p, g and the two
    fp32 moments, write p and the moments = 3 es + 16."""
    import torch
    import matrix_aware_optimizer_amd as mao
    import workloads as wk
    sizes = wk.transformer_adamw_sizes()
    td = wk.torch_dtype(dtype)
    g = torch.Generator(device=dev)
    g.manual_seed(4242)
    P = [(0.02 * torch.randn(n, generator=g, device=dev)).to(td) for n in sizes]
    G = [(1e-3 * torch.randn(n, generator=g, device=dev)).to(td) for n in sizes]
    M = [torch.zeros(n, dtype=torch.float32, device=dev) for n in sizes]
    V = [torch.zeros(n, dtype=torch.float32, device=dev) for n in sizes]
    kw = dict(lr=1e-3, betas=(0.9, 0.95), eps=1e-8, weight_decay=0.1)
    ws = mao.allocate_workspace(mao.muon_adamw_workspace_bytes(P, G, M, V, step=1, **kw), dev)
    for t in range(1, 3):
        mao.muon_adamw_step(P, G, M, V, step=t, workspace=ws, **kw)
    torch.cuda.synchronize()
    mao.muon_profile_enable(True)
    mao.muon_profile_read()
    for t in range(3, 3 + steps):
        mao.muon_adamw_step(P, G, M, V, step=t, workspace=ws, **kw)
    torch.cuda.synchronize()
    prof = mao.muon_profile_read()["adamw"]
    mao.muon_profile_enable(False)
    ms = prof["ms"] / max(1, prof["launches"])
    es = 2 if dtype == "bf16" else 4
    elems = sum(sizes)
    gbs = (3 * es + 16) * elems / (ms * 1e-3) / 1e9
    return {"workload": f"transformer non-matrix parameters ({len(sizes)} tensors, {elems} elements, {dtype})",
            "ms_per_step": round(ms, 4), "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_element": 3 * es + 16}


def measure_cayley(dev, steps):
    """The Muon-Cayley row: 32 matrices of 4096 x 128 in fp32, all of its kernels per
    step, timed with the library's HIP events.  Algorithmic FLOPs per matrix:
    16 N K^2 (the K x K products W^T G, W^T M, W^T W, W^T V, V^T V over N and the
    N x K products W S, V Y1, W Y2), against the fp32 peak: those products run on the
    fp32 matrix cores, whose published peak equals the vector one."""
    import torch
    import matrix_aware_optimizer_amd as mao
    import workloads as wk
    shapes = wk.CAYLEY_SET
    g = torch.Generator(device=dev)
    g.manual_seed(777)
    W, G, M = [], [], []
    for (r, c) in shapes:
        q, _ = torch.linalg.qr(torch.randn(r, c, generator=g, device=dev))
        W.append(q.contiguous())
        G.append(1e-2 * torch.randn(r, c, generator=g, device=dev))
        M.append(torch.zeros(r, c, device=dev))
    ws = mao.allocate_workspace(mao.muon_cayley_workspace_bytes(W, G, M), dev)
    for _ in range(2):
        mao.muon_cayley_step(W, G, M, lr=1e-3, beta=0.9, workspace=ws)
    torch.cuda.synchronize()
    mao.muon_profile_enable(True)
    mao.muon_profile_read()
    for _ in range(steps):
        mao.muon_cayley_step(W, G, M, lr=1e-3, beta=0.9, workspace=ws)
    torch.cuda.synchronize()
    prof = mao.muon_profile_read()["cayley"]
    mao.muon_profile_enable(False)
    ms = prof["ms"] / steps
    flops = sum(16.0 * max(r, c) * min(r, c) ** 2 for r, c in shapes)
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": f"{len(shapes)} x {shapes[0][0]}x{shapes[0][1]} fp32 on the Stiefel manifold",
            "ms_per_step": round(ms, 4), "matrices_per_s": round(len(shapes) / (ms * 1e-3), 1),
            "bound": "mfma", "achieved": round(tf, 2), "peak": F32_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / F32_PEAK_TFLOPS, 4), "flops_per_step": flops}


def ns_flops(shapes, steps):
    tot = 0
    for r, c in shapes:
        m, n = min(r, c), max(r, c)
        tot += (3 * m * m * n + m ** 3) * steps
    return tot


def update_flops_per_launch(shapes):
    return sum(2 * min(r, c) ** 2 * max(r, c) for r, c in shapes)


def cpu_baseline(wl, budget_s=20.0):
    """Time the fp64 oracle on a bounded sample of the workload's matrices."""
    import oracle as orc
    import workloads as wk
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    # workload order keeps the shape mix (per layer: Q, K, V, O, up, down; per expert: gate, up, down)
    total = len(wl.shapes)
    order = range(total)
    hp = wl.hp
    done, t_used, names = 0, 0.0, []
    for i in order:
        h = wk.host_matrix(wl, i)
        t0 = time.perf_counter()
        orc.muon_step(h["W"], h["G"], h["M"], lr=hp["lr"], beta=hp["beta"], weight_decay=hp["weight_decay"],
                      schedule=hp["schedule"], scale_rule=hp["scale_rule"], eps=hp["eps"], dtype=wl.dtype)
        t_used += time.perf_counter() - t0
        done += 1
        names.append("x".join(map(str, wl.shapes[i])))
        if t_used > budget_s:
            break
    shapes = {}
    for nm in names:
        shapes[nm] = shapes.get(nm, 0) + 1
    return {
        "value": done / t_used,
        "unit": "matrices/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"first {done} of {total} matrices in workload order "
                  f"({', '.join(f'{c} x {k}' for k, c in shapes.items())}), full muon_step each, "
                  f"fp64 numpy, {t_used:.1f} s",
    }


def time_workload(wid, steps, warmup, dev):
    """Whole muon_step calls on one workload, inputs resident in HBM: wall time
    between two device synchronizations, and per-kernel time from the library's
    HIP events recorded on the launch stream."""
    import torch
    import matrix_aware_optimizer_amd as mao
    import workloads as wk
    wl = wk.WORKLOADS[wid]
    hp = wl.hp
    print(f"# workload {wid}: generating {wl.n} matrices on the device ({wl.name})", file=sys.stderr, flush=True)
    W, G, M = [], [], []
    for i in range(wl.n):
        d = wk.device_matrix(wl, i, dev)
        W.append(d["W"]); G.append(d["G"]); M.append(d["M"])
    torch.cuda.synchronize()
    kw = dict(lr=hp["lr"], beta=hp["beta"], weight_decay=hp["weight_decay"], schedule=hp["schedule"],
              scale_rule=hp["scale_rule"], eps=hp["eps"])
    ws = mao.allocate_workspace(mao.muon_workspace_bytes(W, G, M, **kw), dev)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        mao.muon_step(W, G, M, workspace=ws, stream=stream, **kw)
    torch.cuda.synchronize()
    print(f"# workload {wid}: warmup done, timing {steps} steps", file=sys.stderr, flush=True)
    mao.muon_profile_enable(True)
    mao.muon_profile_read()          # reset counters
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        mao.muon_step(W, G, M, workspace=ws, stream=stream, **kw)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    prof = mao.muon_profile_read()
    mao.muon_profile_enable(False)
    del W, G, M, ws
    torch.cuda.empty_cache()

    ms_per_step = (t1 - t0) * 1e3 / steps
    steps_ns = len(hp["schedule"])
    flops_ns = ns_flops(wl.shapes, steps_ns)
    ns_ms = (prof["gram"]["ms"] + prof["poly"]["ms"] + prof["update"]["ms"] + prof["update_apply"]["ms"]) / steps
    # the roofline kernel: the update launches that write the iterate (all but the
    # last of a step, whose kernel also applies the step to W and is timed apart)
    upd = prof["update"] if prof["update"]["launches"] else prof["update_apply"]
    upd_ms = upd["ms"] / max(1, upd["launches"])
    upd_tflops = update_flops_per_launch(wl.shapes) / (upd_ms * 1e-3) / 1e12
    bf16 = wl.dtype == "bf16"
    peak = BF16_PEAK_TFLOPS if bf16 else F32_PEAK_TFLOPS
    elem = sum(r * c for r, c in wl.shapes)
    es = 2 if bf16 else 4
    k1_ms = prof["momentum_norm"]["ms"] / max(1, prof["momentum_norm"]["launches"])
    # muon_step's apply runs inside its last update launch; a separate apply launch
    # only happens for muon_ns and for ns_steps = 0
    k5_ms = prof["apply"]["ms"] / prof["apply"]["launches"] if prof["apply"]["launches"] else None
    gram_ms = prof["gram"]["ms"] / max(1, prof["gram"]["launches"])
    poly_ms = prof["poly"]["ms"] / max(1, prof["poly"]["launches"])
    gram_fl = sum(min(r, c) ** 2 * max(r, c) for r, c in wl.shapes)
    poly_fl = sum(min(r, c) ** 3 for r, c in wl.shapes)
    return {
        "wl": wl,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "matrices_per_s": wl.n / (ms_per_step * 1e-3),
        "ns_steps": steps_ns,
        "flops_ns": flops_ns,
        "ns_ms": ns_ms,
        "peak": peak,
        "prof": prof,
        "upd": upd,
        "upd_ms": upd_ms,
        "upd_tflops": upd_tflops,
        "gram_ms": gram_ms,
        "gram_tflops": gram_fl / (gram_ms * 1e-3) / 1e12,
        "poly_ms": poly_ms,
        "poly_tflops": poly_fl / (poly_ms * 1e-3) / 1e12,
        "elem": elem,
        "es": es,
        "k1_ms": k1_ms,
        "k5_ms": k5_ms,
    }


def workload_summary(r):
    """The per-workload object of the bench line."""
    ns_tf = r["flops_ns"] / (r["ns_ms"] * 1e-3) / 1e12
    return {
        "workload": r["wl"].name,
        "dtype": r["wl"].dtype,
        "matrices": r["wl"].n,
        "ns_steps": r["ns_steps"],
        "steps_timed": r["steps"],
        "ms_per_step": round(r["ms_per_step"], 4),
        "matrices_per_s": round(r["matrices_per_s"], 2),
        "ns_ms_per_step": round(r["ns_ms"], 4),
        "ns_tflops_algorithmic": round(ns_tf, 2),
        "ns_frac_of_peak": round(ns_tf / r["peak"], 4),
        "peak_tflops": r["peak"],
        "update_frac_of_peak": round(r["upd_tflops"] / r["peak"], 4),
        "gram_frac_of_peak": round(r["gram_tflops"] / r["peak"], 4),
        "poly_frac_of_peak": round(r["poly_tflops"] / r["peak"], 4),
        "momentum_norm_gbs": round(3 * r["es"] * r["elem"] / (r["k1_ms"] * 1e-3) / 1e9, 1),
    }


# The pages' own figure for the method, with no hardware stated: context, not a target.
PAGES_CONTEXT = {
    "figure": "Muon reaches AdamW's loss with about 52% of AdamW's training FLOPs (16B-parameter MoE, 5.7T tokens)",
    "source": "[DeepSeek V4 summary] prism.simon-ai.net/article/8795, section on Muon's training efficiency",
    "hardware": "not stated",
    "role": "context only; not comparable with a per-step throughput",
}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=3, help="workload id (1-5) of the headline line")
    ap.add_argument("--only", action="store_true", help="time the headline workload only (no other workloads, "
                    "no AdamW / Cayley rows)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write the profiles/ summaries from a rocprofv3 session under DIR (no GPU)")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="write the per-kernel counter table from a rocprofv3 counter session under DIR (no GPU)")
    args = ap.parse_args()

    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, args.workload, PROFILE_COMMANDS)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.workload, COUNTER_COMMANDS)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the multi-GPU sharding of the "
              "step is described in the design notes and not built here.", file=sys.stderr)
        sys.exit(2)

    import torch
    import matrix_aware_optimizer_amd as mao
    import workloads as wk

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    mao.load()
    r = time_workload(args.workload, args.steps, args.warmup, dev)
    wl = r["wl"]
    hp = wl.hp
    prof = r["prof"]
    peak = r["peak"]
    out = {
        "metric": "Muon step matrices/s and NS TFLOP/s as % of MI355X bf16 MFMA peak",
        "value": round(r["matrices_per_s"], 3),
        "unit": "matrices/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "matrices": wl.n,
            "ns_steps": r["ns_steps"],
            "schedule": "8 fast + 2 stable" if args.workload == 3 else f"{r['ns_steps']} fast",
            "scale_rule": hp["scale_rule"],
        },
        "ns_tflops_algorithmic": round(r["flops_ns"] / (r["ns_ms"] * 1e-3) / 1e12, 2),
        "ns_frac_of_peak": round(r["flops_ns"] / (r["ns_ms"] * 1e-3) / 1e12 / peak, 4),
        "ns_ms_per_step": round(r["ns_ms"], 4),
        "step_tflops_algorithmic": round(r["flops_ns"] / (r["ms_per_step"] * 1e-3) / 1e12, 2),
        "kernel_ms_per_step": {k: round(v["ms"] / args.steps, 4) for k, v in prof.items()},
        "elementwise_gbs": {
            "momentum_norm": round(3 * r["es"] * r["elem"] / (r["k1_ms"] * 1e-3) / 1e9, 1),
            "apply": round((2 * r["es"] + 4) * r["elem"] / (r["k5_ms"] * 1e-3) / 1e9, 1) if r["k5_ms"]
            else "fused into the last update",
        },
        "roofline": {
            "kernel": "update (X <- aX + BX)",
            "bound": "mfma",
            "achieved": round(r["upd_tflops"], 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(r["upd_tflops"] / peak, 4),
            "traffic": measured_traffic(args.workload),
            "avg_launch_ms": round(r["upd_ms"], 4),
            "launches_per_step": round(r["upd"]["launches"] / args.steps, 2),
            "flops_per_launch": update_flops_per_launch(wl.shapes),
        },
        "pages_context": PAGES_CONTEXT,
    }
    if not args.only:
        # the other workloads (parity cases of the same path), fewer steps each
        others = {}
        plan = {1: (50, 5), 2: (10, 2), 3: (args.steps, args.warmup), 4: (10, 2), 5: (3, 1)}
        for wid in (1, 2, 3, 4, 5):
            if wid == args.workload:
                others[str(wid)] = workload_summary(r)
                continue
            st, wu = plan[wid]
            others[str(wid)] = workload_summary(time_workload(wid, st, wu, dev))
        out["workloads"] = others
        # the other rows of the optimizer step, timed after the headline region
        out["adamw"] = measure_adamw(dev, 10)
        out["cayley"] = measure_cayley(dev, 5)

    if not args.no_cpu_baseline:
        print("# timing the fp64 oracle on a sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
