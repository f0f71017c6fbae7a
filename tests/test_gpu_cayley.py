"""GPU parity of the Muon-Cayley step against the fp64 oracle (through the C ABI).

The GPU forms the K x K products over N in fp32 (row-block partials summed in
fp64) and solves the 2K x 2K system in fp64, so W' must match the oracle
within a relative Frobenius error of 1e-5 (the fp32 bound), the step W' - W
within 1e-3 of its own size, and M' within 1e-5; W' keeps orthonormal columns
to 3e-5, and over many chained steps well inside the Stiefel page's 1e-2
acceptance level (its section 5.1).
"""
import numpy as np
import pytest

import oracle as orc
import workloads as wk

pytestmark = pytest.mark.gpu

SHAPES = [(64, 16), (300, 37), (1100, 130), (40, 200), (256, 256), (5000, 8), (8, 3), (700, 1)]


def _say(*a):
    print("[cayley]", *a, flush=True)


def _rel(a, b):
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / max(np.linalg.norm(b), 1e-300))


def _run(mao, hosts, lr, beta, skip=()):
    import torch
    dev = torch.device("cuda:0")
    W = [torch.from_numpy(h["W"]).to(dev) for h in hosts]
    G = [None if i in skip else torch.from_numpy(h["G"]).to(dev) for i, h in enumerate(hosts)]
    M = [torch.from_numpy(h["M"]).to(dev) for h in hosts]
    mao.muon_cayley_step(W, G, M, lr=lr, beta=beta)
    torch.cuda.synchronize()
    return [w.cpu().numpy() for w in W], [m.cpu().numpy() for m in M]


def _check(h, w, m, lr, beta, retraction=orc.cayley_retraction):
    ref = orc.cayley_step(h["W"], h["G"], h["M"], lr=lr, beta=beta, retraction=retraction)
    assert _rel(w, ref["W"]) <= 1e-5, _rel(w, ref["W"])
    assert _rel(w.astype(np.float64) - h["W"], ref["W"] - h["W"]) <= 1e-3
    assert _rel(m, ref["M"]) <= 1e-5
    assert orc.orthogonality_error(w) <= 3e-5


@pytest.mark.parametrize("lr", [0.05, 1.0])
def test_cayley_grouped_ragged_matches_oracle(gpu_lib, lr):
    hosts = [wk.cayley_host_matrix(r, c, seed=i) for i, (r, c) in enumerate(SHAPES)]
    _say("ragged lr", lr)
    Ws, Ms = _run(gpu_lib, hosts, lr, 0.9)
    for h, w, m in zip(hosts, Ws, Ms):
        _check(h, w, m, lr, 0.9)


def test_cayley_large_gradients_move_far_and_stay_orthonormal(gpu_lib):
    hosts = [wk.cayley_host_matrix(512, 64, seed=3, grad_std=10.0, momentum_std=0.0)]
    _say("large steps")
    Ws, Ms = _run(gpu_lib, hosts, 0.5, 0.0)
    _check(hosts[0], Ws[0], Ms[0], 0.5, 0.0)
    assert np.linalg.norm(Ws[0] - hosts[0]["W"]) > 0.1      # a real rotation happened


def test_cayley_chained_steps_keep_the_manifold(gpu_lib):
    import torch
    dev = torch.device("cuda:0")
    h = wk.cayley_host_matrix(1024, 96, seed=11, momentum_std=0.0)
    W = torch.from_numpy(h["W"]).to(dev)
    M = torch.from_numpy(h["M"]).to(dev)
    _say("chain")
    for t in range(50):
        g = wk.cayley_host_matrix(1024, 96, seed=100 + t)["G"]
        before_w, before_m = W.cpu().numpy(), M.cpu().numpy()
        gpu_lib.muon_cayley_step([W], [torch.from_numpy(g).to(dev)], [M], lr=0.1, beta=0.9)
        torch.cuda.synchronize()
        if t % 10 == 0:   # each step on the GPU's own state matches the oracle's step
            _check({"W": before_w, "G": g, "M": before_m}, W.cpu().numpy(), M.cpu().numpy(), 0.1, 0.9)
    assert orc.orthogonality_error(W.cpu().numpy()) < 1e-4


def test_cayley_zero_lr_and_skipped_matrices(gpu_lib):
    hosts = [wk.cayley_host_matrix(200, 20, seed=5), wk.cayley_host_matrix(90, 30, seed=6)]
    _say("lr 0 and skip")
    Ws, Ms = _run(gpu_lib, hosts, 0.0, 0.9, skip=(1,))
    assert np.array_equal(Ws[0], hosts[0]["W"])
    assert _rel(Ms[0], orc.cayley_step(hosts[0]["W"], hosts[0]["G"], hosts[0]["M"], lr=0.0, beta=0.9)["M"]) <= 1e-5
    assert np.array_equal(Ws[1], hosts[1]["W"]) and np.array_equal(Ms[1], hosts[1]["M"])


def test_cayley_full_width_blocks(gpu_lib):
    # K = 128 fills every column block of the in-register inverse and the 128-wide product
    # tiles; K = 100 pads the last block; the wide 128 x 2000 goes through the transposed frame
    shapes = [(4096, 128), (1000, 100), (128, 2000)]
    hosts = [wk.cayley_host_matrix(r, c, seed=40 + i) for i, (r, c) in enumerate(shapes)]
    _say("full width", shapes)
    Ws, Ms = _run(gpu_lib, hosts, 0.05, 0.9)
    for h, w, m in zip(hosts, Ws, Ms):
        _check(h, w, m, 0.05, 0.9)


def test_cayley_maximum_dimension(gpu_lib):
    # MUON_MAX_DIM (2^20) rows, and 2^20 columns through the transposed frame: the K x K
    # products over N = 2^20 (row-block partials).  The oracle takes its 2K x 2K form here
    # (pinned equal to the n x n solve); an n x n system of that size cannot be formed.
    big = 1 << 20
    shapes = [(big, 8), (16, big)]
    hosts = [wk.cayley_host_matrix(r, c, seed=60 + i) for i, (r, c) in enumerate(shapes)]
    _say("maximum dimension", shapes)
    Ws, Ms = _run(gpu_lib, hosts, 0.05, 0.9)
    for h, w, m in zip(hosts, Ws, Ms):
        _check(h, w, m, 0.05, 0.9, retraction=orc.cayley_retraction_lowrank)


def test_cayley_benchmark_set(gpu_lib):
    # the grouped set the benchmark times, in one call: four sampled matrices against the
    # oracle (about a second each in fp64), orthonormal columns for all of them
    hosts = [wk.cayley_host_matrix(r, c, seed=200 + i) for i, (r, c) in enumerate(wk.CAYLEY_SET)]
    _say("benchmark set", len(hosts), "matrices")
    Ws, Ms = _run(gpu_lib, hosts, 1e-3, 0.9)
    n = len(hosts)
    for i in sorted({0, n // 3, (2 * n) // 3, n - 1}):
        _check(hosts[i], Ws[i], Ms[i], 1e-3, 0.9)
    for w in Ws:
        assert orc.orthogonality_error(w) <= 3e-5


def test_cayley_off_manifold_falls_back_to_pivoting(gpu_lib):
    # W = 2 x orthonormal: C11 = I + c W^T V has an unpivoted pivot below 1/2 (pinned on the
    # CPU), so the GPU's unpivoted inverse hands over to the pivoting one
    h = wk.cayley_host_matrix(300, 24, seed=7, momentum_std=1.0)
    h = dict(h, W=(2.0 * h["W"]).astype(np.float32))
    _say("off the manifold")
    Ws, Ms = _run(gpu_lib, [h], 1.0, 0.9)
    ref = orc.cayley_step(h["W"], h["G"], h["M"], lr=1.0, beta=0.9)
    assert _rel(Ws[0], ref["W"]) <= 1e-5, _rel(Ws[0], ref["W"])
    assert _rel(Ms[0], ref["M"]) <= 1e-5
