"""muon_step_noalloc (the entry point that allocates nothing) against muon_step.

Both run the same kernels on the same inputs; only the workspace differs (the
library's per-GPU device array against a caller's buffer), and nothing in the
workspace is read before it is written, so W' and M' must agree bit for bit.
Two calls in a row, the second with a smaller list, show that contents left in
the shared array by one call do not leak into the next.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import matrix_aware_optimizer_amd as mao
import oracle as orc
import workloads as wk
from tests._util import rel_frob, to_numpy_f32, ulp_distance

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _inputs(wl):
    host = [wk.host_matrix(wl, i) for i in range(wl.n)]
    def up(key):
        return [wk.upload(h[key], wl.dtype, DEV) for h in host]
    return host, up


def _run_both(wl):
    hp = wl.hp
    kw = dict(lr=hp["lr"], beta=hp["beta"], weight_decay=hp["weight_decay"], schedule=hp["schedule"],
              scale_rule=hp["scale_rule"], eps=hp["eps"])
    host, up = _inputs(wl)
    G = up("G")
    W1, M1 = up("W"), up("M")
    W2, M2 = up("W"), up("M")
    mao.muon_step(W1, G, M1, **kw)
    mao.muon_step_noalloc(W2, G, M2, **kw)
    torch.cuda.synchronize()
    return host, [to_numpy_f32(w) for w in W1], [to_numpy_f32(m) for m in M1], \
        [to_numpy_f32(w) for w in W2], [to_numpy_f32(m) for m in M2]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_muon_step_twice(gpu_lib, dtype):
    big = wk.custom_workload([(2048, 2048), (300, 517), (517, 300), (1, 200)], dtype=dtype, wid=301,
                             lr=0.02, weight_decay=0.1, scale_rule="moonlight")
    small = wk.custom_workload([(130, 200), (64, 64)], dtype=dtype, wid=302,
                               lr=0.02, weight_decay=0.1, scale_rule="kellerjordan")
    for wl in (big, small):   # the second call is smaller: stale contents of the first must not matter
        host, Wa, Ma, Wb, Mb = _run_both(wl)
        for i in range(wl.n):
            assert np.array_equal(Wa[i], Wb[i]), (wl.shapes[i], "W'")
            assert np.array_equal(Ma[i], Mb[i]), (wl.shapes[i], "M'")
        # and against the oracle, on the M' bar (the O and W' bars are those of muon_step's tests)
        ref = orc.muon_step(host[0]["W"], host[0]["G"], host[0]["M"], lr=wl.hp["lr"], beta=wl.hp["beta"],
                            weight_decay=wl.hp["weight_decay"], schedule=wl.hp["schedule"],
                            scale_rule=wl.hp["scale_rule"], eps=wl.hp["eps"], dtype=dtype)
        assert ulp_distance(Mb[0], ref["M_rounded"], dtype).max() <= 1
        assert rel_frob(Wb[0], ref["W"]) <= 1e-2


def test_noalloc_rejects_a_list_beyond_its_scratch(gpu_lib):
    # 4 x 2048x8192 bf16 needs about 4 x 117 MB of workspace, more than the 128 MiB array
    shapes = [(2048, 8192)] * 4
    W = [torch.zeros(s, dtype=torch.bfloat16, device=DEV) for s in shapes]
    G = [torch.ones(s, dtype=torch.bfloat16, device=DEV) for s in shapes]
    M = [torch.zeros(s, dtype=torch.bfloat16, device=DEV) for s in shapes]
    need = mao.muon_workspace_bytes(W, G, M, schedule=[wk.FAST] * 5)
    assert need > mao.NOALLOC_SCRATCH_BYTES
    with pytest.raises(mao.MuonError) as ei:
        mao.muon_step_noalloc(W, G, M, lr=0.1, schedule=[wk.FAST] * 5)
    assert ei.value.status == mao.MUON_ERR_WORKSPACE
    torch.cuda.synchronize()
    # nothing was enqueued: the state is untouched
    assert all(int(torch.count_nonzero(m)) == 0 for m in M)
    assert all(int(torch.count_nonzero(w)) == 0 for w in W)


def test_noalloc_step_replays_from_a_captured_graph(gpu_lib):
    # The callers this entry is for capture it in a graph.  One call is captured after an
    # eager warm-up (which sets up the library's per-GPU array); the graph is replayed three
    # times, each time after eager work that resets the state to the same inputs, and every
    # replay must give the eager call's bits.
    wl = wk.custom_workload([(512, 768), (300, 517), (1024, 256)], dtype="bf16", wid=303,
                            lr=0.02, weight_decay=0.1, scale_rule="moonlight")
    hp = wl.hp
    kw = dict(lr=hp["lr"], beta=hp["beta"], weight_decay=hp["weight_decay"], schedule=hp["schedule"],
              scale_rule=hp["scale_rule"], eps=hp["eps"])
    host, up = _inputs(wl)
    G, W0, M0 = up("G"), up("W"), up("M")
    We, Me = [w.clone() for w in W0], [m.clone() for m in M0]
    mao.muon_step_noalloc(We, G, Me, **kw)
    torch.cuda.synchronize()
    Wg, Mg = [w.clone() for w in W0], [m.clone() for m in M0]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mao.muon_step_noalloc([w.clone() for w in W0], G, [m.clone() for m in M0], **kw)   # warm-up
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mao.muon_step_noalloc(Wg, G, Mg, **kw)
    for replay in range(3):
        for w, w0 in zip(Wg, W0):
            w.copy_(w0)
        for m, m0 in zip(Mg, M0):
            m.copy_(m0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i in range(wl.n):
            assert torch.equal(Wg[i], We[i]), (replay, wl.shapes[i], "W'")
            assert torch.equal(Mg[i], Me[i]), (replay, wl.shapes[i], "M'")
