"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances (from the method's arithmetic and the stated bounds):
  * O (the orthogonalized update): relative Frobenius error <= 1e-5 for fp32,
    <= 3e-2 for bf16, and for bf16 every singular value of O inside
    [min sigma(O_oracle) - 0.05, max sigma(O_oracle) + 0.05];
  * M' (stored momentum): within 1 ulp of the oracle's value rounded once to
    the storage dtype (the kernel rounds fma(beta, M, G) from fp32);
  * W' (stored weight): fp32 relative Frobenius <= 1e-6 plus the share of O's
    own error, lr * s * |dO|_F / |W'|_F; bf16 within 1 ulp of the rounded oracle
    value, plus the share of O's own error that lr * s * |dO| can carry into an
    element.
Small cases run the oracle in full; the full-size workloads compare sampled
matrices of the grouped call (the 28672x8192 set through sampled elements and
the singular-value map, which the oracle computes at any size).
"""
from __future__ import annotations

import time

import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wk
from tests._util import record_parity, rel_frob, singular_values, to_numpy_f32, ulp_distance

pytestmark = pytest.mark.gpu

KJ5 = [wk.FAST] * 5
DEV = "cuda:0"
TOL = {"f32": 1e-5, "bf16": 3e-2}


def _say(*a):
    print(*a, flush=True)


def _ns_gpu(mao, mats, dtype, schedule, eps=1e-7):
    ins = [wk.upload(m, dtype, DEV) for m in mats]
    outs = [torch.empty(m.shape, dtype=torch.float32, device=DEV) for m in mats]
    mao.muon_ns(ins, outs, schedule=schedule, eps=eps)
    torch.cuda.synchronize()
    return [to_numpy_f32(o).astype(np.float64) for o in outs]


def _check_band(o_gpu, o_ref, tag):
    s_ref = singular_values(o_ref)
    s_gpu = singular_values(o_gpu)
    lo, hi = s_ref.min() - 0.05, s_ref.max() + 0.05
    assert s_gpu.min() >= lo and s_gpu.max() <= hi, (tag, s_gpu.min(), s_gpu.max(), lo, hi)
    return (float(s_gpu.min()), float(s_gpu.max())), (float(lo), float(hi))


# ----------------------------------------------------------------------------
# Single Newton-Schulz products through muon_ns: isolate Gram, polynomial and update
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("coeffs", [(1.0, 0.0, 0.0), (0.0, 1.0, 0.0), (0.0, 0.0, 1.0), (0.5, -0.25, 0.125)])
def test_single_step_products(gpu_lib, dtype, coeffs):
    shapes = [(128, 256), (200, 130), (300, 517), (64, 64)]
    wl = wk.custom_workload(shapes, dtype=dtype, wid=201)
    mats = [wk.host_matrix(wl, i, need=("G",))["G"] for i in range(len(shapes))]
    _say("single step", dtype, coeffs)
    got = _ns_gpu(gpu_lib, mats, dtype, [coeffs])
    for i, m in enumerate(mats):
        ref = orc.muon_ns(m, [coeffs])
        err = rel_frob(got[i], ref)
        tol = 2e-6 if dtype == "f32" else 1e-2
        assert err <= tol, (shapes[i], err)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_steps_is_normalized_input(gpu_lib, dtype):
    wl = wk.custom_workload([(33, 70), (70, 33)], dtype=dtype, wid=202)
    mats = [wk.host_matrix(wl, i, need=("G",))["G"] for i in range(2)]
    got = _ns_gpu(gpu_lib, mats, dtype, [])
    for i, m in enumerate(mats):
        ref = orc.muon_ns(m, [])
        assert rel_frob(got[i], ref) <= 1e-6


# ----------------------------------------------------------------------------
# Full orthogonalization, several shapes in one grouped call (tiles + ragged tails)
# ----------------------------------------------------------------------------

RAGGED = [(300, 517), (517, 300), (256, 256), (1, 200), (200, 1), (1024, 768), (77, 1100)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("sched_name", ["kj5", "hybrid8+2"])
def test_ns_grouped_ragged(gpu_lib, dtype, sched_name):
    sched = KJ5 if sched_name == "kj5" else wk.WORKLOADS[3].hp["schedule"]
    wl = wk.custom_workload(RAGGED, dtype=dtype, wid=203)
    mats = [wk.host_matrix(wl, i, need=("G",))["G"] for i in range(len(RAGGED))]
    _say("ns grouped", dtype, sched_name)
    got = _ns_gpu(gpu_lib, mats, dtype, sched)
    for i, m in enumerate(mats):
        ref = orc.muon_ns(m, sched)
        err = rel_frob(got[i], ref)
        assert err <= TOL[dtype], (RAGGED[i], err)
        if dtype == "bf16" and min(m.shape) > 1:
            _check_band(got[i], ref, RAGGED[i])


# A seeded sweep of shapes around the tile edges (256 for bf16, 128 for fp32), thin
# and single-row or single-column matrices, in one grouped call.
def _sweep_shapes(seed, count):
    rng = np.random.default_rng(seed)
    edges = [1, 2, 31, 127, 128, 129, 255, 256, 257, 383, 511, 512, 513, 640, 767, 769, 1024]
    shapes = []
    for _ in range(count):
        r = int(rng.choice(edges)) if rng.random() < 0.6 else int(rng.integers(1, 1100))
        c = int(rng.choice(edges)) if rng.random() < 0.6 else int(rng.integers(1, 1100))
        shapes.append((r, c))
    return shapes


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ns_shape_sweep(gpu_lib, dtype):
    shapes = _sweep_shapes(2024 if dtype == "bf16" else 2025, 24)
    wl = wk.custom_workload(shapes, dtype=dtype, wid=230)
    mats = [wk.host_matrix(wl, i, need=("G",))["G"] for i in range(len(shapes))]
    _say("ns shape sweep", dtype, shapes)
    got = _ns_gpu(gpu_lib, mats, dtype, KJ5)
    for i, m in enumerate(mats):
        ref = orc.muon_ns(m, KJ5)
        err = rel_frob(got[i], ref)
        assert err <= TOL[dtype], (shapes[i], err)
        if dtype == "bf16" and min(m.shape) > 1:
            _check_band(got[i], ref, shapes[i])


def test_lowrank_ill_conditioned_bf16(gpu_lib):
    # rank-32 + 1e-3 noise, condition number far above 1e4
    wl = wk.custom_workload([(1024, 1024), (768, 1536)], dtype="bf16", grad="lowrank", rank=32,
                            noise_std=1e-3, wid=204)
    mats = [wk.host_matrix(wl, i, need=("G",))["G"] for i in range(2)]
    got = _ns_gpu(gpu_lib, mats, "bf16", KJ5)
    for i, m in enumerate(mats):
        ref = orc.muon_ns(m, KJ5)
        assert rel_frob(got[i], ref) <= TOL["bf16"]
        _check_band(got[i], ref, i)


# ----------------------------------------------------------------------------
# Invariants
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_transpose_equivariance_is_bitwise(gpu_lib, dtype):
    wl = wk.custom_workload([(300, 517), (128, 1024)], dtype=dtype, wid=205)
    mats = [wk.host_matrix(wl, i, need=("G",))["G"] for i in range(2)]
    a = _ns_gpu(gpu_lib, mats, dtype, KJ5)
    b = _ns_gpu(gpu_lib, [np.ascontiguousarray(m.T) for m in mats], dtype, KJ5)
    for x, y in zip(a, b):
        assert np.array_equal(x, y.T)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_orthogonal_input(gpu_lib, dtype):
    rng = np.random.default_rng(7)
    n = 256
    q, r = np.linalg.qr(rng.standard_normal((n, n)))
    q = q * np.sign(np.diag(r))
    q = wk.to_bf16_bits_f32(q.astype(np.float32)) if dtype == "bf16" else q.astype(np.float32)
    got = _ns_gpu(gpu_lib, [q], dtype, KJ5)[0]
    ref = orc.muon_ns(q, KJ5)
    assert rel_frob(got, ref) <= TOL[dtype]
    # a converging schedule returns (nearly) the orthogonal input itself
    conv = [wk.FAST] * 8 + [wk.STABLE] * 4
    got2 = _ns_gpu(gpu_lib, [q], dtype, conv)[0]
    assert rel_frob(got2, q.astype(np.float64)) <= (1e-5 if dtype == "f32" else 2e-2)


def test_scale_invariance_across_expert_scales(gpu_lib):
    rng = np.random.default_rng(8)
    base = rng.standard_normal((384, 640))
    mats = [wk.to_bf16_bits_f32((base * c).astype(np.float32)) for c in (1e-4, 1e-2, 1.0, 1e2)]
    got = _ns_gpu(gpu_lib, mats, "bf16", KJ5)
    for g in got[1:]:
        assert rel_frob(g, got[0]) <= 2e-2


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_extreme_magnitudes_against_oracle(gpu_lib, dtype):
    """Scale invariance against the oracle itself, over the storage dtype's range.

    From c = 1e-30 (where eps dominates the norm and the iteration acts almost
    linearly) to c = 1e18 (squares near fp32's limit; 1e30 for fp32 inputs):
    the library shifts the stored iterate by an exact power of two when the norm
    is outside its plain range, so no product overflows or underflows."""
    rng = np.random.default_rng(9)
    base = rng.standard_normal((384, 640))
    scales = (1e-30, 1e-10, 1e-3, 1e10, 1e15, 1e18) + ((1e30,) if dtype == "f32" else ())
    if dtype == "bf16":
        mats = [wk.to_bf16_bits_f32((base * c).astype(np.float32)) for c in scales]
    else:
        mats = [(base * c).astype(np.float32) for c in scales]
    got = _ns_gpu(gpu_lib, mats, dtype, KJ5)
    for c, m, g in zip(scales, mats, got):
        ref = orc.muon_ns(m, KJ5)
        err = rel_frob(g, ref)
        _say(f"scale {c:.0e} {dtype}: O rel err {err:.3e}")
        assert np.all(np.isfinite(g)), c
        tol = TOL[dtype] + (2e-7 if dtype == "f32" else 0.0)
        assert err <= tol, (c, err)
        sig = band = None
        if dtype == "bf16":
            sig, band = _check_band(g, ref, c)
        record_parity(config=f"muon_ns, input scaled by {c:.0e}", matrix=0, shape=m.shape, dtype=dtype,
                      o_rel_err=err, tol=tol, sigma=sig, band=band)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_eps_tiny_input(gpu_lib, dtype):
    # eps = 0: X0 = U / ||U||_F exactly, for norms far below fp32's squared range
    rng = np.random.default_rng(10)
    base = rng.standard_normal((200, 300))
    mats = [(base * c).astype(np.float32) for c in (1e-25, 1e-3, 1e25)]
    if dtype == "bf16":
        mats = [wk.to_bf16_bits_f32(m) for m in mats]
    got = _ns_gpu(gpu_lib, mats, dtype, KJ5, eps=0.0)
    for m, g in zip(mats, got):
        ref = orc.muon_ns(m, KJ5, eps=0.0)
        assert np.all(np.isfinite(g))
        assert rel_frob(g, ref) <= TOL[dtype] + (2e-7 if dtype == "f32" else 0.0)


def test_step_with_huge_gradients(gpu_lib):
    # the whole step (momentum in bf16 at 1e18, state rounding, the shifted
    # iterate, decay and apply) against the oracle
    # 256x512 and 512x512 read the first step's operand from the caller's momentum
    # buffer; the shifted copy must go to the workspace and leave the state intact
    shapes = [(256, 384), (384, 256), (256, 512), (512, 512)]
    wl = wk.custom_workload(shapes, dtype="bf16", wid=213, grad_std=1e18,
                            lr=3e-4, weight_decay=0.01, scale_rule="moonlight")
    host = [wk.host_matrix(wl, i) for i in range(len(shapes))]
    _check_step(gpu_lib, wl, range(len(shapes)), host, label="step with gradients of 1e18")


@pytest.mark.parametrize("scale", [1e-30, 1.0, 1e18])
def test_ns_input_operand_and_shift_leave_input_intact(gpu_lib, scale):
    # tile-multiple shapes: the first step reads the caller's bf16 input as its operand
    rng = np.random.default_rng(11)
    mats = [wk.to_bf16_bits_f32((rng.standard_normal(sh) * scale).astype(np.float32))
            for sh in ((256, 512), (512, 512), (768, 256))]
    ins = [wk.upload(m, "bf16", DEV) for m in mats]
    keep = [t.clone() for t in ins]
    outs = [torch.empty(m.shape, dtype=torch.float32, device=DEV) for m in mats]
    gpu_lib.muon_ns(ins, outs, schedule=KJ5)
    torch.cuda.synchronize()
    for x, k in zip(ins, keep):
        assert torch.equal(x, k)
    for m, o in zip(mats, outs):
        ref = orc.muon_ns(m, KJ5)
        g = to_numpy_f32(o).astype(np.float64)
        assert rel_frob(g, ref) <= TOL["bf16"]
        _check_band(g, ref, m.shape)


def test_deterministic_bitwise(gpu_lib):
    wl = wk.custom_workload([(300, 517), (517, 300), (256, 1024)], dtype="bf16", wid=206)
    mats = [wk.host_matrix(wl, i, need=("G",))["G"] for i in range(3)]
    a = _ns_gpu(gpu_lib, mats, "bf16", KJ5)
    b = _ns_gpu(gpu_lib, mats, "bf16", KJ5)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# ----------------------------------------------------------------------------
# The whole step
# ----------------------------------------------------------------------------

def _step_gpu(mao, host, dtype, hp, zero_w=False, lr=None, skip=()):
    Ws, Gs, Ms = [], [], []
    for i, h in enumerate(host):
        W = torch.zeros(h["W"].shape, dtype=wk.torch_dtype(dtype), device=DEV) if zero_w \
            else wk.upload(h["W"], dtype, DEV)
        Ws.append(W)
        Gs.append(None if i in skip else wk.upload(h["G"], dtype, DEV))
        Ms.append(wk.upload(h["M"], dtype, DEV))
    mao.muon_step(Ws, Gs, Ms, lr=hp["lr"] if lr is None else lr, beta=hp["beta"],
                  weight_decay=hp["weight_decay"], schedule=hp["schedule"], scale_rule=hp["scale_rule"],
                  eps=hp["eps"], nesterov=hp.get("nesterov", False))
    torch.cuda.synchronize()
    return [to_numpy_f32(w) for w in Ws], [to_numpy_f32(m) for m in Ms]


def _oracle_step(h, dtype, hp, zero_w=False, lr=None):
    W = np.zeros_like(h["W"]) if zero_w else h["W"]
    return orc.muon_step(W, h["G"], h["M"], lr=hp["lr"] if lr is None else lr, beta=hp["beta"],
                         weight_decay=hp["weight_decay"], schedule=hp["schedule"],
                         scale_rule=hp["scale_rule"], eps=hp["eps"], nesterov=hp.get("nesterov", False),
                         dtype=dtype)


def _check_step(mao, wl, indices, host, label=None):
    """Full step on all of `host` (one grouped call); oracle checks on `indices`.
    Returns the first pass's W' and M' (real weights) for every matrix."""
    dtype, hp = wl.dtype, wl.hp
    # pass 1: real weights -> M' and W'
    Wg, Mg = _step_gpu(mao, host, dtype, hp)
    # pass 2: W = 0, lr = 1 -> W' = -s * O exactly rounded once, so O is observable
    Wo, _ = _step_gpu(mao, host, dtype, hp, zero_w=True, lr=1.0)
    for i in indices:
        h = host[i]
        ref = _oracle_step(h, dtype, hp)
        rows, cols = h["W"].shape
        s = ref["scale"]
        # M'
        du = ulp_distance(Mg[i], ref["M_rounded"], dtype)
        assert du.max() <= 1, (i, "M'", du.max())
        # O
        o_gpu = -Wo[i].astype(np.float64) / s
        err = rel_frob(o_gpu, ref["O"])
        tol = TOL[dtype] if dtype == "bf16" else TOL[dtype] + 2e-7
        assert err <= tol, (i, (rows, cols), "O", err)
        sig = band = None
        if dtype == "bf16" and min(rows, cols) > 1:
            sig, band = _check_band(o_gpu, ref["O"], i)
        rec = dict(config=label or wl.name, matrix=int(i), shape=(rows, cols), dtype=dtype, o_rel_err=err,
                   tol=tol, sigma=sig, band=band, m_ulp_max=int(du.max()))
        # W'
        if dtype == "f32":
            e = rel_frob(Wg[i], ref["W"])
            # the apply's own fp32 rounding, plus the share of O's (already bounded) error that
            # W' = decay W - lr s O carries: it dominates when lr s |O| outweighs |W|
            share = orc.as_f32(hp["lr"]) * s * np.linalg.norm(o_gpu - ref["O"]) / max(np.linalg.norm(ref["W"]), 1e-300)
            assert e <= 1e-6 + share, (i, "W'", e, share)
            record_parity(**rec, w_rel_err=e)
        else:
            du = ulp_distance(Wg[i], ref["W_rounded"], dtype)
            lr32 = orc.as_f32(hp["lr"])
            # what O's own (already bounded) error can move an element by
            slack = lr32 * s * (np.abs(o_gpu - ref["O"]) + 0.01 * np.abs(ref["O"]))
            ulp = np.abs(ref["W_rounded"].astype(np.float64)) * 2.0 ** -7 + 2.0 ** -133
            dev_ = np.abs(Wg[i].astype(np.float64) - ref["W"])
            assert np.all(dev_ <= ulp + slack), (i, "W'", float(np.max(dev_ - ulp - slack)))
            # where that share is negligible the apply arithmetic itself must be within 1 ulp
            exact = slack < 0.25 * ulp
            assert np.all(du[exact] <= 1), (i, "W' ulp", int(du[exact].max()))
            assert exact.any()
            record_parity(**rec, w_bound_ratio=float(np.max(dev_ / (ulp + slack))),
                          w_ulp_max_where_o_negligible=int(du[exact].max()))
    return Wg, Mg


def test_step_fp32_single_matrix_workload(gpu_lib):
    wl = wk.WORKLOADS[1]
    host = [wk.host_matrix(wl, 0)]
    _say("step fp32 128x256")
    _check_step(gpu_lib, wl, [0], host, label="c1 single fp32 128x256")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rule", ["naive", "kellerjordan", "mup", "moonlight"])
def test_step_grouped_ragged(gpu_lib, dtype, rule):
    shapes = [(300, 517), (517, 300), (256, 256), (1, 200), (200, 1), (1024, 768)]
    wl = wk.custom_workload(shapes, dtype=dtype, wid=207, lr=0.02, weight_decay=0.1, scale_rule=rule)
    host = [wk.host_matrix(wl, i) for i in range(len(shapes))]
    _say("step grouped", dtype, rule)
    _check_step(gpu_lib, wl, range(len(shapes)), host, label=f"ragged grouped step, {rule} scale")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_step_maximum_dimension(gpu_lib, dtype):
    """MUON_MAX_DIM (2^20) columns, and 2^20 rows: the widest padded row (2 MB in bf16,
    4 MB in fp32), 4096 update tiles and 16384 elementwise tiles in one tile row, the
    tall transpose at that length, and a half-padded tile row (m = 40)."""
    big = 1 << 20
    shapes = [(40, big), (big, 3)]
    wl = wk.custom_workload(shapes, dtype=dtype, wid=232, lr=0.02, weight_decay=0.1, scale_rule="moonlight")
    host = [wk.host_matrix(wl, i) for i in range(len(shapes))]
    _say("step at the maximum dimension", dtype, shapes)
    _check_step(gpu_lib, wl, range(len(shapes)), host, label="maximum dimension 2^20")


def test_step_maximum_matrix_count(gpu_lib):
    """MUON_MAX_MATRICES (65536) matrices in one grouped call: the descriptor table, the tile
    prefix sums and the run lookup at their largest.  Every matrix's stored momentum within
    1 ulp of its rounding and every W' finite; 16 sampled matrices against the oracle in full.
    fp32, whose 1e-5 bar is tight at any size: small Gaussian matrices in bf16 carry an O
    error of 2-3 % under any bf16-operand plan (tests/diag_bf16_emulation.py), at the 3e-2 bar."""
    n = 1 << 16
    base = [(1, 1), (3, 7), (16, 24), (40, 9), (64, 64), (100, 31), (5, 256), (256, 2)]
    shapes = [base[i % len(base)] for i in range(n)]
    wl = wk.custom_workload(shapes, dtype="f32", wid=233, lr=0.02, weight_decay=0.1, scale_rule="kellerjordan")
    _say("step with the maximum matrix count", n)
    host = [wk.host_matrix(wl, i) for i in range(n)]
    sample = sorted({0, 1, 2, 3, 4, 5, 6, 7, n // 2, n // 2 + 3, n - 6, n - 5, n - 4, n - 3, n - 2, n - 1})
    Wg, Mg = _check_step(gpu_lib, wl, sample, host, label="65536 matrices in one call (sampled)")
    beta = orc.as_f32(wl.hp["beta"])   # beta crosses the C boundary as a float, as in the oracle's step
    for i in range(n):
        h = host[i]
        want = orc.rne(orc.momentum_update(h["M"], h["G"], beta), "f32")
        assert ulp_distance(Mg[i], want, "f32").max() <= 1, (i, "M'")
        assert np.all(np.isfinite(Wg[i])), (i, "W'")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_step_shape_sweep(gpu_lib, dtype):
    # the sweep of NS shapes through the whole step: K1's row groups with and without
    # 16-byte accesses (cols % 8), the tall transposes, and the fused apply at the edges
    shapes = _sweep_shapes(2026 if dtype == "bf16" else 2027, 24)
    wl = wk.custom_workload(shapes, dtype=dtype, wid=231, lr=0.02, weight_decay=0.1, scale_rule="kellerjordan")
    host = [wk.host_matrix(wl, i) for i in range(len(shapes))]
    _say("step shape sweep", dtype, shapes)
    _check_step(gpu_lib, wl, range(len(shapes)), host, label="shape sweep, Keller Jordan scale")


def test_step_nesterov(gpu_lib):
    wl = wk.custom_workload([(256, 384), (384, 256)], dtype="bf16", wid=208, nesterov=True,
                            scale_rule="moonlight", lr=3e-4, weight_decay=0.01)
    host = [wk.host_matrix(wl, i) for i in range(2)]
    _check_step(gpu_lib, wl, [0, 1], host, label="Nesterov step")


def test_step_zero_gradient_and_skip(gpu_lib):
    shapes = [(128, 300), (300, 128), (64, 64)]
    wl = wk.custom_workload(shapes, dtype="bf16", wid=209, lr=0.1, weight_decay=0.5)
    host = [wk.host_matrix(wl, i) for i in range(3)]
    host[0]["G"] = np.zeros_like(host[0]["G"])
    host[0]["M"] = np.zeros_like(host[0]["M"])
    Wg, Mg = _step_gpu(gpu_lib, host, "bf16", wl.hp, skip=(2,))
    # zero momentum and gradient: O = 0, W' = (1 - lr*wd) W, M' = 0
    ref0 = _oracle_step(host[0], "bf16", wl.hp)
    assert np.all(ref0["O"] == 0)
    assert ulp_distance(Wg[0], ref0["W_rounded"], "bf16").max() <= 1
    assert np.all(Mg[0] == 0)
    # skipped matrix: weight and momentum untouched
    assert np.array_equal(Wg[2], host[2]["W"]) and np.array_equal(Mg[2], host[2]["M"])
    # the other matrix is unaffected by its neighbours
    ref1 = _oracle_step(host[1], "bf16", wl.hp)
    assert ulp_distance(Mg[1], ref1["M_rounded"], "bf16").max() <= 1


def test_nan_stays_in_its_matrix(gpu_lib):
    shapes = [(128, 256), (128, 256)]
    wl = wk.custom_workload(shapes, dtype="bf16", wid=210)
    host = [wk.host_matrix(wl, i) for i in range(2)]
    host[0]["G"] = host[0]["G"].copy()
    host[0]["G"][3, 5] = np.nan
    Wg, Mg = _step_gpu(gpu_lib, host, "bf16", wl.hp)
    assert np.isnan(Wg[0]).any()
    assert np.all(np.isfinite(Wg[1])) and np.all(np.isfinite(Mg[1]))
    ref1 = _oracle_step(host[1], "bf16", wl.hp)
    assert ulp_distance(Mg[1], ref1["M_rounded"], "bf16").max() <= 1


def test_two_steps_match_resumed_steps(gpu_lib):
    # the step is a pure function of (W, G, M): running step 2 from restored
    # state gives the same bits as running it straight after step 1
    wl = wk.custom_workload([(256, 512)], dtype="bf16", wid=211)
    h = wk.host_matrix(wl, 0)
    W = wk.upload(h["W"], "bf16", DEV)
    M = wk.upload(h["M"], "bf16", DEV)
    G = wk.upload(h["G"], "bf16", DEV)
    kw = dict(lr=0.02, beta=0.95, weight_decay=0.01, schedule=KJ5, scale_rule="moonlight")
    gpu_lib.muon_step([W], [G], [M], **kw)
    W1, M1 = W.clone(), M.clone()
    gpu_lib.muon_step([W], [G], [M], **kw)
    W2, M2 = W.clone(), M.clone()
    gpu_lib.muon_step([W1], [G], [M1], **kw)
    torch.cuda.synchronize()
    assert torch.equal(W1, W2) and torch.equal(M1, M2)


# ----------------------------------------------------------------------------
# Full-size workloads (the launch configuration the benchmark times)
# ----------------------------------------------------------------------------

def _full_host(wl, indices):
    """Host draws for `indices`, device draws (uploaded back) for the rest."""
    host = []
    for i in range(wl.n):
        if i in indices:
            host.append(wk.host_matrix(wl, i))
        else:
            d = wk.device_matrix(wl, i, DEV)
            host.append({k: to_numpy_f32(v) for k, v in d.items()})
    return host


def test_full_single_4096_lowrank(gpu_lib):
    wl = wk.WORKLOADS[2]
    host = [wk.host_matrix(wl, 0)]
    _say("full 4096^2 low-rank")
    _check_step(gpu_lib, wl, [0], host, label="c2 single bf16 4096^2 low rank")


def _full_workload_check(mao, wl, sample, label):
    """The whole workload in one grouped call (as the benchmark runs it);
    oracle checks on the host-drawn `sample` matrices."""
    dtype, hp = wl.dtype, wl.hp
    host = {i: wk.host_matrix(wl, i) for i in sample}
    W, G, M = [], [], []
    for i in range(wl.n):
        if i in host:
            W.append(wk.upload(host[i]["W"], dtype, DEV))
            G.append(wk.upload(host[i]["G"], dtype, DEV))
            M.append(wk.upload(host[i]["M"], dtype, DEV))
        else:
            d = wk.device_matrix(wl, i, DEV)
            W.append(d["W"]); G.append(d["G"]); M.append(d["M"])
    M0 = [m.clone() for m in M]
    kw = dict(beta=hp["beta"], weight_decay=hp["weight_decay"], schedule=hp["schedule"],
              scale_rule=hp["scale_rule"], eps=hp["eps"])
    ws = mao.muon_step(W, G, M, lr=hp["lr"], **kw)
    torch.cuda.synchronize()
    Wg = {i: to_numpy_f32(W[i]) for i in sample}
    Mg = {i: to_numpy_f32(M[i]) for i in sample}
    # second call from the same state with W = 0 and lr = 1: W' = -s * O
    for i in range(wl.n):
        W[i].zero_()
        M[i].copy_(M0[i])
    del M0
    mao.muon_step(W, G, M, lr=1.0, workspace=ws, **kw)
    torch.cuda.synchronize()
    Wo = {i: to_numpy_f32(W[i]) for i in sample}
    del W, G, M, ws
    torch.cuda.empty_cache()
    for i in sample:
        h = host[i]
        ref = _oracle_step(h, dtype, hp)
        s = ref["scale"]
        mu = ulp_distance(Mg[i], ref["M_rounded"], dtype).max()
        assert mu <= 1, (i, "M'")
        o_gpu = -Wo[i].astype(np.float64) / s
        err = rel_frob(o_gpu, ref["O"])
        _say(f"matrix {i} {wl.shapes[i]}: O rel err {err:.3e}")
        assert err <= TOL[dtype], (i, err)
        sig, band = _check_band(o_gpu, ref["O"], i)
        lr32 = orc.as_f32(hp["lr"])
        slack = lr32 * s * (np.abs(o_gpu - ref["O"]) + 0.01 * np.abs(ref["O"]))
        ulp = np.abs(ref["W_rounded"].astype(np.float64)) * 2.0 ** -7 + 2.0 ** -133
        dev_ = np.abs(Wg[i].astype(np.float64) - ref["W"])
        assert np.all(dev_ <= ulp + slack), (i, "W'")
        record_parity(config=label, matrix=int(i), shape=wl.shapes[i], dtype=dtype, o_rel_err=err, tol=TOL[dtype],
                      sigma=sig, band=band, m_ulp_max=int(mu), w_bound_ratio=float(np.max(dev_ / (ulp + slack))))


def test_full_transformer_parameter_set(gpu_lib):
    wl = wk.WORKLOADS[3]
    _say("full transformer set, 144 matrices")
    # layer 0: Q (square), up (tall), down (wide); layer 23: down
    _full_workload_check(gpu_lib, wl, [0, 4, 5, 143], "c3 transformer d=2048 x 24 layers (144 matrices)")


def test_full_moe_expert_set(gpu_lib):
    wl = wk.WORKLOADS[4]
    _say("full MoE set, 192 matrices")
    # expert 0 gate, expert 7 down, expert 63 up (different per-expert scales)
    _full_workload_check(gpu_lib, wl, [0, 23, 190], "c4 MoE 64 experts (192 matrices)")


def _gram_eigs(x):
    """Eigenvalues (ascending, fp64) of x^T x for a tall matrix x (host array or
    device tensor): the Gram is formed in fp64 on the device with torch, its
    eigenvalues on the host in fp64."""
    xd = (torch.from_numpy(np.ascontiguousarray(x)).to(DEV) if isinstance(x, np.ndarray) else x).to(torch.float64)
    g = (xd.T @ xd).cpu().numpy()
    del xd
    return np.linalg.eigvalsh(g)


LARGE_SAMPLE = (0, 15)


@pytest.fixture(scope="module")
def large_mlp_run(gpu_lib):
    """16 x 28672x8192 in one grouped call, as the benchmark launches it.
    Matrices 0 and 15 are drawn on the host (the bits the oracle reads), the
    other 14 on the device.  Two calls from the same state: real weights
    (-> W', M'), then W = 0 and lr = 1, which gives W' = -s O rounded once."""
    wl = wk.WORKLOADS[5]
    hp = wl.hp
    _say("large MLP set: host draws of matrices", LARGE_SAMPLE)
    host = {i: wk.host_matrix(wl, i) for i in LARGE_SAMPLE}
    W, G, M = [], [], []
    for i in range(wl.n):
        if i in host:
            W.append(wk.upload(host[i]["W"], "bf16", DEV))
            G.append(wk.upload(host[i]["G"], "bf16", DEV))
            M.append(wk.upload(host[i]["M"], "bf16", DEV))
        else:
            d = wk.device_matrix(wl, i, DEV)
            W.append(d["W"]); G.append(d["G"]); M.append(d["M"])
    M0 = {i: M[i].clone() for i in LARGE_SAMPLE}
    kw = dict(beta=hp["beta"], weight_decay=hp["weight_decay"], schedule=hp["schedule"],
              scale_rule=hp["scale_rule"], eps=hp["eps"])
    _say("step 1 (real weights)")
    ws = gpu_lib.muon_step(W, G, M, lr=hp["lr"], **kw)
    torch.cuda.synchronize()
    Wg = {i: to_numpy_f32(W[i]) for i in LARGE_SAMPLE}
    Mg = {i: to_numpy_f32(M[i]) for i in LARGE_SAMPLE}
    for i in range(wl.n):
        W[i].zero_()
        if i in M0:
            M[i].copy_(M0[i])   # the others start from zero momentum and are only timed here
    _say("step 2 (W = 0, lr = 1)")
    gpu_lib.muon_step(W, G, M, lr=1.0, workspace=ws, **kw)
    torch.cuda.synchronize()
    Wo = {i: to_numpy_f32(W[i]) for i in LARGE_SAMPLE}
    del W, G, M, M0, ws
    torch.cuda.empty_cache()
    return {"wl": wl, "host": host, "Wg": Wg, "Mg": Mg, "Wo": Wo}


@pytest.mark.parametrize("index", LARGE_SAMPLE)
def test_full_large_mlp_set(gpu_lib, large_mlp_run, index):
    """Matrix `index` of the 16 x 28672x8192 call against the fp64 oracle run in full:
      * O: relative Frobenius error <= 3e-2 and every singular value inside the
        band [min - 0.05, max + 0.05] of the oracle's;
      * M' within 1 ulp of the once-rounded oracle value;
      * W' within 1 ulp plus the share of O's own error;
      * the singular values of O against the oracle's scalar map of the input's
        (the iteration acts on each singular value through the schedule's odd
        polynomials), sorted, to 0.05."""
    wl, run = large_mlp_run["wl"], large_mlp_run
    hp = wl.hp
    h = run["host"][index]
    t0 = time.time()
    ref = _oracle_step(h, "bf16", hp)
    _say(f"oracle for matrix {index}: {time.time() - t0:.1f}s")
    s = ref["scale"]
    mu = ulp_distance(run["Mg"][index], ref["M_rounded"], "bf16").max()
    assert mu <= 1, (index, "M'", mu)
    o_gpu = -run["Wo"][index].astype(np.float64) / s
    err = rel_frob(o_gpu, ref["O"])
    _say(f"matrix {index}: O rel err {err:.3e}")
    assert err <= TOL["bf16"], (index, err)
    lr32 = orc.as_f32(hp["lr"])
    slack = lr32 * s * (np.abs(o_gpu - ref["O"]) + 0.01 * np.abs(ref["O"]))
    ulp = np.abs(ref["W_rounded"].astype(np.float64)) * 2.0 ** -7 + 2.0 ** -133
    dev_ = np.abs(run["Wg"][index].astype(np.float64) - ref["W"])
    assert np.all(dev_ <= ulp + slack), (index, "W'")
    w_ratio = float(np.max(dev_ / (ulp + slack)))
    del dev_
    o_ref = ref["O"]
    m_new = ref["M"]
    del ref
    # singular values (tall: through the 8192 x 8192 Gram)
    s_ref = np.sqrt(np.clip(_gram_eigs(o_ref), 0.0, None))
    s_gpu = np.sqrt(np.clip(_gram_eigs(o_gpu), 0.0, None))
    lo, hi = s_ref.min() - 0.05, s_ref.max() + 0.05
    _say(f"sigma(O) in [{s_gpu.min():.4f}, {s_gpu.max():.4f}], oracle band [{lo:.4f}, {hi:.4f}]")
    assert s_gpu.min() >= lo and s_gpu.max() <= hi
    ev_in = np.clip(_gram_eigs(m_new), 0.0, None)
    x = np.sqrt(ev_in) / (np.sqrt(ev_in.sum()) + orc.as_f32(hp["eps"]))
    s_map = orc.phi_schedule(x, hp["schedule"])
    dev_map = float(np.abs(np.sort(s_gpu) - np.sort(s_map)).max())
    dev_ref = float(np.abs(np.sort(s_ref) - np.sort(s_map)).max())
    _say(f"max sorted deviation from the scalar map: gpu {dev_map:.4f}, oracle {dev_ref:.2e}, "
         f"{time.time() - t0:.1f}s")
    assert dev_map <= 0.05
    record_parity(config="c5 16 x 28672x8192 low rank", matrix=int(index), shape=wl.shapes[index], dtype="bf16",
                  o_rel_err=err, tol=TOL["bf16"], sigma=(float(s_gpu.min()), float(s_gpu.max())),
                  band=(float(lo), float(hi)), m_ulp_max=int(mu), w_bound_ratio=w_ratio, spectrum_dev=dev_map)


def test_bf16_state_rounding_is_round_to_nearest_even(gpu_lib):
    # beta = 1: M' = M + G is exact in fp32 for bf16 inputs of similar magnitude,
    # so the stored bf16 state must equal the once-rounded exact sum bit for bit
    # (ties included: sums of two bf16 values hit exact halfway points often).
    wl = wk.custom_workload([(96, 160)], dtype="bf16", wid=212)
    h = wk.host_matrix(wl, 0)
    _, Mg = _step_gpu(gpu_lib, [h], "bf16", dict(wl.hp, beta=1.0, lr=0.0))
    exact = h["M"].astype(np.float64) + h["G"].astype(np.float64)
    assert np.array_equal(Mg[0], orc.rne(exact, "bf16"))
