"""GPU parity of the grouped AdamW step against the fp64 oracle (through the C ABI).

Tolerances follow from the kernel's fp32 arithmetic: each stored moment is
within a few fp32 ulps of the magnitudes of its terms (m' may cancel, so the
bound is absolute); the fp32 parameter within a few ulps of its two terms plus
the moment's error carried through lr / (1 - beta1^t) / (sqrt(v_hat) + eps);
a bf16 parameter within one bf16 ulp of the oracle's rounded result.
"""
import numpy as np
import pytest

import oracle as orc
import workloads as wk

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)
SIZES = [1, 3, 4, 5, 4095, 4096, 4097, 3 * 4096 + 7, 65536 + 1, 1 << 20]
U32 = 2.0 ** -24


def _say(*a):
    print("[adamw]", *a, flush=True)


def _upload(arr, dtype, dev):
    return wk.upload(arr, dtype, dev)


def _gpu_step(mao, host, dtype, step, dev, skip=()):
    import torch
    P = [_upload(h["p"], dtype, dev) for h in host]
    Gs = [None if i in skip else _upload(h["g"], dtype, dev) for i, h in enumerate(host)]
    M = [torch.from_numpy(h["m"]).to(dev) for h in host]
    V = [torch.from_numpy(h["v"]).to(dev) for h in host]
    mao.muon_adamw_step(P, Gs, M, V, lr=HP["lr"], betas=(HP["beta1"], HP["beta2"]), eps=HP["eps"],
                        weight_decay=HP["weight_decay"], step=step)
    torch.cuda.synchronize()
    return ([p.float().cpu().numpy() for p in P], [m.cpu().numpy() for m in M], [v.cpu().numpy() for v in V])


def _check(h, p_gpu, m_gpu, v_gpu, step, dtype):
    out = orc.adamw_step(h["p"], h["g"], h["m"], h["v"], step=step, dtype=dtype, **HP)
    b1, b2 = orc.as_f32(HP["beta1"]), orc.as_f32(HP["beta2"])
    g = h["g"].astype(np.float64)
    m_scale = np.abs(b1 * h["m"]) + np.abs((1 - b1) * g)
    v_scale = np.abs(b2 * h["v"]) + (1 - b2) * g * g
    assert np.all(np.abs(m_gpu - out["m"]) <= 4 * U32 * m_scale + 1e-37)
    assert np.all(np.abs(v_gpu - out["v"]) <= 4 * U32 * v_scale + 1e-37)
    if dtype == "f32":
        # p' = decay p - s m' / d: a few ulps of both terms, plus the stored m' error
        # (absolute, up to 4 ulps of its terms' magnitudes) carried through s / d
        lr, wd = orc.as_f32(HP["lr"]), orc.as_f32(HP["weight_decay"])
        upd = out["p"] - (1 - lr * wd) * h["p"]
        s_over_d = lr / (1 - b1 ** step) / (np.sqrt(out["v"] / (1 - b2 ** step)) + orc.as_f32(HP["eps"]))
        p_tol = 8 * U32 * (np.abs((1 - lr * wd) * h["p"]) + np.abs(upd)) + s_over_d * 4 * U32 * m_scale
        assert np.all(np.abs(p_gpu - out["p"]) <= p_tol + 1e-37), np.max(np.abs(p_gpu - out["p"]) / (p_tol + 1e-37))
    else:
        ref = out["p_rounded"]
        ulp = np.abs(ref) * 2.0 ** -7 + 2.0 ** -133
        assert np.all(np.abs(p_gpu - ref) <= ulp), np.max(np.abs(p_gpu - ref) / ulp)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("step", [1, 5])
def test_adamw_ragged_group_matches_oracle(gpu_lib, dtype, step):
    import torch
    dev = torch.device("cuda:0")
    host = wk.adamw_host_tensors(SIZES, dtype=dtype, seed=1, step=step)
    _say("ragged", dtype, "step", step)
    P, M, V = _gpu_step(gpu_lib, host, dtype, step, dev)
    for i, h in enumerate(host):
        _check(h, P[i], M[i], V[i], step, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_adamw_three_steps_chain_gpu_state(gpu_lib, dtype):
    import torch
    dev = torch.device("cuda:0")
    sizes = [777, 4096 * 5 + 3]
    host = wk.adamw_host_tensors(sizes, dtype=dtype, seed=2, step=1)
    _say("chain", dtype)
    for t in (1, 2, 3):
        if t > 1:   # fresh gradients, GPU-stored state
            fresh = wk.adamw_host_tensors(sizes, dtype=dtype, seed=2 + t, step=1)
            for h, f in zip(host, fresh):
                h["g"] = f["g"]
        P, M, V = _gpu_step(gpu_lib, host, dtype, t, dev)
        for i, h in enumerate(host):
            _check(h, P[i], M[i], V[i], t, dtype)
            h["p"], h["m"], h["v"] = P[i].astype(np.float32), M[i], V[i]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_adamw_unaligned_tensors_take_the_element_path(gpu_lib, dtype):
    import torch
    dev = torch.device("cuda:0")
    n = 4096 + 11
    host = wk.adamw_host_tensors([n], dtype=dtype, seed=7, step=3)[0]
    td = wk.torch_dtype(dtype)
    # views one element into larger buffers: not 4-element aligned
    pb = torch.zeros(n + 1, dtype=td, device=dev)
    gb = torch.zeros(n + 1, dtype=td, device=dev)
    mb = torch.zeros(n + 1, dtype=torch.float32, device=dev)
    vb = torch.zeros(n + 1, dtype=torch.float32, device=dev)
    p, g, m, v = pb[1:], gb[1:], mb[1:], vb[1:]
    p.copy_(_upload(host["p"], dtype, dev))
    g.copy_(_upload(host["g"], dtype, dev))
    m.copy_(torch.from_numpy(host["m"]).to(dev))
    v.copy_(torch.from_numpy(host["v"]).to(dev))
    _say("unaligned", dtype)
    gpu_lib.muon_adamw_step([p], [g], [m], [v], lr=HP["lr"], betas=(HP["beta1"], HP["beta2"]), eps=HP["eps"],
                            weight_decay=HP["weight_decay"], step=3)
    torch.cuda.synchronize()
    _check(host, p.float().cpu().numpy(), m.cpu().numpy(), v.cpu().numpy(), 3, dtype)
    assert float(pb[0].float()) == 0.0 and float(mb[0]) == 0.0   # the element before is untouched


def test_adamw_null_gradient_skips_tensor(gpu_lib):
    import torch
    dev = torch.device("cuda:0")
    host = wk.adamw_host_tensors([1000, 2000], dtype="bf16", seed=5, step=2)
    _say("skip")
    P, M, V = _gpu_step(gpu_lib, host, "bf16", 2, dev, skip=(0,))
    assert np.array_equal(P[0], host[0]["p"]) and np.array_equal(M[0], host[0]["m"])
    assert np.array_equal(V[0], host[0]["v"])
    _check(host[1], P[1], M[1], V[1], 2, "bf16")
