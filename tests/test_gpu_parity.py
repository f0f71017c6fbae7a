"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances (from the method's arithmetic and the stated bounds):
  * O (the orthogonalized update): relative Frobenius error <= 1e-5 for fp32,
    <= 3e-2 for bf16, and for bf16 every singular value of O inside
    [min sigma(O_oracle) - 0.05, max sigma(O_oracle) + 0.05];
  * M' (stored momentum): within 1 ulp of the oracle's value rounded once to
    the storage dtype (the kernel rounds fma(beta, M, G) from fp32);
  * W' (stored weight): fp32 relative Frobenius <= 1e-6; bf16 within 1 ulp of
    the rounded oracle value, plus the share of O's own error that
    lr * s * |dO| can carry into an element.
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
from tests._util import rel_frob, singular_values, to_numpy_f32, ulp_distance

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


def _check_step(mao, wl, indices, host):
    """Full step on all of `host` (one grouped call); oracle checks on `indices`."""
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
        if dtype == "bf16" and min(rows, cols) > 1:
            _check_band(o_gpu, ref["O"], i)
        # W'
        if dtype == "f32":
            e = rel_frob(Wg[i], ref["W"])
            assert e <= 1e-6, (i, "W'", e)
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


def test_step_fp32_single_matrix_workload(gpu_lib):
    wl = wk.WORKLOADS[1]
    host = [wk.host_matrix(wl, 0)]
    _say("step fp32 128x256")
    _check_step(gpu_lib, wl, [0], host)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rule", ["naive", "kellerjordan", "mup", "moonlight"])
def test_step_grouped_ragged(gpu_lib, dtype, rule):
    shapes = [(300, 517), (517, 300), (256, 256), (1, 200), (200, 1), (1024, 768)]
    wl = wk.custom_workload(shapes, dtype=dtype, wid=207, lr=0.02, weight_decay=0.1, scale_rule=rule)
    host = [wk.host_matrix(wl, i) for i in range(len(shapes))]
    _say("step grouped", dtype, rule)
    _check_step(gpu_lib, wl, range(len(shapes)), host)


def test_step_nesterov(gpu_lib):
    wl = wk.custom_workload([(256, 384), (384, 256)], dtype="bf16", wid=208, nesterov=True,
                            scale_rule="moonlight", lr=3e-4, weight_decay=0.01)
    host = [wk.host_matrix(wl, i) for i in range(2)]
    _check_step(gpu_lib, wl, [0, 1], host)


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
    _check_step(gpu_lib, wl, [0], host)


def _full_workload_check(mao, wl, sample):
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
        assert ulp_distance(Mg[i], ref["M_rounded"], dtype).max() <= 1, (i, "M'")
        o_gpu = -Wo[i].astype(np.float64) / s
        err = rel_frob(o_gpu, ref["O"])
        _say(f"matrix {i} {wl.shapes[i]}: O rel err {err:.3e}")
        assert err <= TOL[dtype], (i, err)
        _check_band(o_gpu, ref["O"], i)
        lr32 = orc.as_f32(hp["lr"])
        slack = lr32 * s * (np.abs(o_gpu - ref["O"]) + 0.01 * np.abs(ref["O"]))
        ulp = np.abs(ref["W_rounded"].astype(np.float64)) * 2.0 ** -7 + 2.0 ** -133
        assert np.all(np.abs(Wg[i].astype(np.float64) - ref["W"]) <= ulp + slack), (i, "W'")


def test_full_transformer_parameter_set(gpu_lib):
    wl = wk.WORKLOADS[3]
    _say("full transformer set, 144 matrices")
    # layer 0: Q (square), up (tall), down (wide); layer 23: down
    _full_workload_check(gpu_lib, wl, [0, 4, 5, 143])


def test_full_moe_expert_set(gpu_lib):
    wl = wk.WORKLOADS[4]
    _say("full MoE set, 192 matrices")
    # expert 0 gate, expert 7 down, expert 63 up (different per-expert scales)
    _full_workload_check(gpu_lib, wl, [0, 23, 190])


def _gram_eigs(x):
    """Eigenvalues (ascending, fp64) of x^T x for a tall device matrix x."""
    xd = x.to(torch.float64)
    g = (xd.T @ xd).cpu().numpy()
    del xd
    return np.linalg.eigvalsh(g)


def test_full_large_mlp_set(gpu_lib):
    """16 x 28672x8192 in one grouped call.  The oracle cannot run the iteration
    at this size inside a test, so it checks what it computes at any size:
      * M' at sampled positions, to 1 ulp of the once-rounded oracle value;
      * W' at sampled positions against the oracle's apply with the observed O;
      * the singular values of O: in exact arithmetic the iteration maps each
        singular value x of M' / (||M'||_F + eps) through the schedule's odd
        polynomials (oracle ``phi_schedule``), so sigma(O) must lie inside
        [min - 0.05, max + 0.05] of that map, and the sorted spectra must agree
        to 0.05 (the bf16 band).
    The two 8192 x 8192 Gram matrices are formed in fp64 with torch on the
    device; their eigenvalues are taken on the host in fp64."""
    wl = wk.WORKLOADS[5]
    hp = wl.hp
    sample = 0
    t0 = time.time()
    _say("full large MLP set, 16 x 28672x8192: drawing inputs")
    W, G, M = [], [], []
    for i in range(wl.n):
        d = wk.device_matrix(wl, i, DEV)
        W.append(d["W"]); G.append(d["G"]); M.append(d["M"])
    W0 = W[sample].clone()
    M0 = M[sample].clone()
    kw = dict(beta=hp["beta"], weight_decay=hp["weight_decay"], schedule=hp["schedule"],
              scale_rule=hp["scale_rule"], eps=hp["eps"])
    _say("step 1 (real weights)")
    ws = gpu_lib.muon_step(W, G, M, lr=hp["lr"], **kw)
    torch.cuda.synchronize()
    rows, cols = wl.shapes[sample]
    rng = np.random.default_rng(5)
    pos = rng.choice(rows * cols, size=8192, replace=False)

    def at(t):
        return to_numpy_f32(t.reshape(-1)[torch.from_numpy(pos).to(DEV)]).astype(np.float64)

    Wp, Mp = at(W[sample]), at(M[sample])
    # second call from the same state: W = 0, lr = 1 gives W' = -s O
    for i in range(wl.n):
        W[i].zero_()
    M[sample].copy_(M0)
    _say("step 2 (W = 0, lr = 1)")
    gpu_lib.muon_step(W, G, M, lr=1.0, workspace=ws, **kw)
    torch.cuda.synchronize()
    del ws
    s = orc.scale_factor(rows, cols, hp["scale_rule"])
    O = W[sample].to(torch.float32) / (-s)
    Gs = G[sample]
    for i in range(wl.n):
        if i != sample:
            W[i] = G[i] = M[i] = None
    torch.cuda.empty_cache()

    # M' at sampled positions
    g_at, m0_at = at(Gs), at(M0)
    m_ref = orc.rne(orc.momentum_update(m0_at, g_at, orc.as_f32(hp["beta"])), "bf16")
    assert ulp_distance(Mp.astype(np.float32), m_ref, "bf16").max() <= 1

    # W' at sampled positions: the oracle's apply with the observed O (itself
    # rounded once to bf16 in the second call, hence the 2^-8 |O| slack)
    o_at, w0_at = at(O), at(W0)
    lr32, wd32 = orc.as_f32(hp["lr"]), orc.as_f32(hp["weight_decay"])
    w_ref = orc.apply_update(w0_at, o_at, lr32, wd32, s)
    ulp = np.abs(orc.rne(w_ref, "bf16").astype(np.float64)) * 2.0 ** -7 + 2.0 ** -133
    slack = lr32 * s * np.abs(o_at) * 2.0 ** -8
    assert np.all(np.abs(Wp - w_ref) <= ulp + slack)

    # singular values: input through the oracle's scalar map vs the GPU's O
    _say("spectra", f"{time.time() - t0:.1f}s")
    # the iteration starts from the unrounded M' = beta M + G (exact in fp64 here)
    M1 = orc.as_f32(hp["beta"]) * M0.to(torch.float64) + Gs.to(torch.float64)
    ev_in = np.clip(_gram_eigs(M1), 0.0, None)
    del M1
    x = np.sqrt(ev_in) / (np.sqrt(ev_in.sum()) + hp["eps"])
    s_exp = orc.phi_schedule(x, hp["schedule"])
    s_gpu = np.sqrt(np.clip(_gram_eigs(O), 0.0, None))
    lo, hi = s_exp.min() - 0.05, s_exp.max() + 0.05
    dev = np.abs(np.sort(s_gpu) - np.sort(s_exp)).max()
    _say(f"sigma(O) in [{s_gpu.min():.4f}, {s_gpu.max():.4f}], band [{lo:.4f}, {hi:.4f}], "
         f"max sorted deviation {dev:.4f}, {time.time() - t0:.1f}s")
    assert s_gpu.min() >= lo and s_gpu.max() <= hi
    assert dev <= 0.05


def test_bf16_state_rounding_is_round_to_nearest_even(gpu_lib):
    # beta = 1: M' = M + G is exact in fp32 for bf16 inputs of similar magnitude,
    # so the stored bf16 state must equal the once-rounded exact sum bit for bit
    # (ties included: sums of two bf16 values hit exact halfway points often).
    wl = wk.custom_workload([(96, 160)], dtype="bf16", wid=212)
    h = wk.host_matrix(wl, 0)
    _, Mg = _step_gpu(gpu_lib, [h], "bf16", dict(wl.hp, beta=1.0, lr=0.0))
    exact = h["M"].astype(np.float64) + h["G"].astype(np.float64)
    assert np.array_equal(Mg[0], orc.rne(exact, "bf16"))
