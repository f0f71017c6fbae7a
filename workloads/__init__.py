"""Seeded synthetic inputs for the Muon step (shared by tests, smoke and bench).

This module only draws random numbers and rounds them to a storage dtype.  It
holds none of the optimizer's arithmetic, so both the HIP path and the CPU
oracle can read the same input bits from it.

Weights are stored row-major as rows x cols = d_out x d_in (the PyTorch Linear
layout the pages use).  The workload table below names each configuration by
what it is, with its sizes; the recipes follow the pages:

* Gaussian gradients have Marchenko-Pastur singular values, and late-training
  gradients are low rank with a numerical rank of 1-10 % of the nominal size
  ([Muon优化器], sections on the low rank of gradient matrices and on the
  Marchenko-Pastur distribution), so the low-rank cases use a Gaussian factor
  product plus small Gaussian noise;
* weights start from Xavier/Kaiming, W_ij ~ N(0, 1/d_in) ([Muon优化器],
  section on why initialization is scaled).

Every array is drawn in fp64 from numpy's PCG64 seeded with
(workload id, matrix index, tensor id), then rounded to fp32 and, for bf16,
once more to bf16 with round-to-nearest-even.  Large workloads can instead be
drawn on the device with torch's seeded generator (``device_matrix``): timing
does not depend on the values, and parity checks always use host draws.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# Coefficient triples the caller passes in (inputs to both sides).
# [Muon优化器], "Newton-Schulz 迭代——高效实现与系数优化": the tuned triple and the
# Taylor triple (15/8, -10/8, 3/8).
FAST = (3.4445, -4.7750, 2.0315)
STABLE = (1.875, -1.25, 0.375)

TENSOR_W, TENSOR_G, TENSOR_M = 0, 1, 2


@dataclass
class Workload:
    wid: int
    name: str
    dtype: str                       # 'f32' or 'bf16'
    shapes: list                     # [(rows, cols), ...]
    grad: str                        # 'gauss' | 'lowrank'
    grad_std: float = 1.0
    rank: int = 0
    noise_std: float = 0.0
    expert_scale: bool = False       # per-expert log-uniform scale on G (and M)
    momentum: str = "same"           # 'same' recipe as G, or 'zero'
    hp: dict = field(default_factory=dict)

    @property
    def n(self):
        return len(self.shapes)


def _sched(n_fast, n_stable=0):
    return [FAST] * n_fast + [STABLE] * n_stable


def _transformer_shapes(layers=24, d=2048, ffn=8192):
    # per layer: Q, K, V, O (d x d); MLP up d -> ffn stored ffn x d; down ffn -> d stored d x ffn
    one = [(d, d)] * 4 + [(ffn, d), (d, ffn)]
    return one * layers


def _moe_shapes(experts=64, d=2048, f=1408):
    # per expert: gate and up d -> f stored f x d; down f -> d stored d x f
    return [(f, d), (f, d), (d, f)] * experts


WORKLOADS = {
    1: Workload(1, "single fp32 128x256 (N(0,1) grad and momentum)", "f32", [(128, 256)],
                grad="gauss", grad_std=1.0,
                hp=dict(lr=0.02, beta=0.95, weight_decay=0.0, eps=1e-7,
                        scale_rule="naive", schedule=_sched(5))),
    2: Workload(2, "single bf16 4096x4096 (rank-64 + 1e-3 noise)", "bf16", [(4096, 4096)],
                grad="lowrank", rank=64, noise_std=1e-3,
                hp=dict(lr=3e-4, beta=0.95, weight_decay=0.1, eps=1e-7,
                        scale_rule="moonlight", schedule=_sched(5))),
    3: Workload(3, "transformer d=2048 x 24 layers bf16 (QKVO 2048^2, up 8192x2048, "
                   "down 2048x8192; 144 matrices)", "bf16", _transformer_shapes(),
                grad="gauss", grad_std=1e-3,
                hp=dict(lr=3e-4, beta=0.95, weight_decay=0.01, eps=1e-7,
                        scale_rule="moonlight", schedule=_sched(8, 2))),
    4: Workload(4, "MoE 64 experts bf16 (gate/up 1408x2048, down 2048x1408; 192 matrices)",
                "bf16", _moe_shapes(), grad="gauss", grad_std=1e-3, expert_scale=True,
                hp=dict(lr=3e-4, beta=0.95, weight_decay=0.01, eps=1e-7,
                        scale_rule="moonlight", schedule=_sched(5))),
    5: Workload(5, "16 x bf16 28672x8192 (rank-256 + 1e-2 noise)", "bf16", [(28672, 8192)] * 16,
                grad="lowrank", rank=256, noise_std=1e-2, momentum="zero",
                hp=dict(lr=3e-4, beta=0.95, weight_decay=0.1, eps=1e-7,
                        scale_rule="moonlight", schedule=_sched(5))),
}


SHORT_NAMES = {1: "single_f32_128x256", 2: "single_bf16_4096_lowrank", 3: "transformer_d2048_24l",
               4: "moe_64_experts", 5: "mlp_16x28672x8192"}


def short_name(wid):
    """File-name friendly label of a workload."""
    return SHORT_NAMES.get(wid, f"workload{wid}")


def custom_workload(shapes, dtype="bf16", grad="gauss", grad_std=1.0, rank=0, noise_std=0.0,
                    momentum="same", wid=100, **hp):
    """A workload with arbitrary shapes (tests use it for ragged and edge cases)."""
    base = dict(lr=0.02, beta=0.95, weight_decay=0.0, eps=1e-7, scale_rule="naive",
                schedule=_sched(5))
    base.update(hp)
    return Workload(wid, "custom", dtype, list(shapes), grad=grad, grad_std=grad_std, rank=rank,
                    noise_std=noise_std, momentum=momentum, hp=base)


# --------------------------------------------------------------------------
# Rounding (storage representation only).
# --------------------------------------------------------------------------

def to_bf16_bits_f32(x):
    """Round float32 values to bf16 (nearest-even on the fp32 bit pattern).

    Returns float32 arrays whose values are exactly representable in bf16.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    out = rounded.astype(np.uint32).view(np.float32)
    return np.where(np.isnan(x), x, out)


def _store(x64, dtype):
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    return to_bf16_bits_f32(x32) if dtype == "bf16" else x32


# --------------------------------------------------------------------------
# Host draws (numpy PCG64).
# --------------------------------------------------------------------------

def _rng(wid, index, tensor):
    return np.random.Generator(np.random.PCG64([wid, index, tensor]))


def _expert_scale(wl, index):
    if not wl.expert_scale:
        return 1.0
    expert = index // 3
    u = np.random.Generator(np.random.PCG64([wl.wid, expert, 99])).uniform(-1.0, 1.0)
    return float(10.0 ** u)


def _draw_grad_like(wl, index, tensor, rows, cols):
    rng = _rng(wl.wid, index, tensor)
    if wl.grad == "gauss":
        g = rng.standard_normal((rows, cols)) * wl.grad_std
    elif wl.grad == "lowrank":
        P = rng.standard_normal((rows, wl.rank))
        Q = rng.standard_normal((cols, wl.rank))
        g = P @ Q.T + wl.noise_std * rng.standard_normal((rows, cols))
    else:
        raise ValueError(wl.grad)
    return g * _expert_scale(wl, index)


def host_matrix(wl: Workload, index: int, need=("W", "G", "M")):
    """Draw matrix ``index`` of a workload on the host as float32 arrays."""
    rows, cols = wl.shapes[index]
    out = {}
    if "W" in need:
        rng = _rng(wl.wid, index, TENSOR_W)
        out["W"] = _store(rng.standard_normal((rows, cols)) / np.sqrt(cols), wl.dtype)
    if "G" in need:
        out["G"] = _store(_draw_grad_like(wl, index, TENSOR_G, rows, cols), wl.dtype)
    if "M" in need:
        if wl.momentum == "zero":
            out["M"] = np.zeros((rows, cols), np.float32)
        else:
            out["M"] = _store(_draw_grad_like(wl, index, TENSOR_M, rows, cols), wl.dtype)
    return out


# --------------------------------------------------------------------------
# Device draws (torch's seeded generator; for timing-only matrices).
# --------------------------------------------------------------------------

def torch_dtype(dtype):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def upload(arr_f32, dtype, device):
    """Copy a host float32 array (already rounded) to a device tensor of ``dtype``."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(arr_f32))
    return t.to(device=device, dtype=torch_dtype(dtype)).contiguous()


def device_matrix(wl: Workload, index: int, device):
    """Draw matrix ``index`` directly on ``device`` with torch (same recipe, other bits)."""
    import torch
    rows, cols = wl.shapes[index]
    g = torch.Generator(device=device)
    g.manual_seed(1_000_003 * wl.wid + 7919 * index + 17)
    td = torch_dtype(wl.dtype)

    def gauss(r, c):
        return torch.randn((r, c), generator=g, device=device, dtype=torch.float32)

    def grad_like():
        if wl.grad == "gauss":
            x = gauss(rows, cols) * wl.grad_std
        else:
            x = gauss(rows, wl.rank) @ gauss(cols, wl.rank).T
            x += wl.noise_std * gauss(rows, cols)
        return x * _expert_scale(wl, index)

    W = (gauss(rows, cols) / float(np.sqrt(cols))).to(td)
    G = grad_like().to(td)
    M = torch.zeros((rows, cols), device=device, dtype=td) if wl.momentum == "zero" else grad_like().to(td)
    return {"W": W.contiguous(), "G": G.contiguous(), "M": M.contiguous()}


# --------------------------------------------------------------------------
# AdamW tensors (the parameters Muon does not take).
# --------------------------------------------------------------------------

def transformer_adamw_sizes(d=2048, layers=24, vocab=32000):
    """Non-matrix parameters of the d=2048, 24-layer transformer: token embedding and
    output head (vocab x d each; the pages route both to AdamW), two norm weight
    vectors per layer and a final norm.  The pages give no vocabulary size; 32000 is
    a stated stand-in."""
    return [vocab * d, vocab * d] + [d] * (2 * layers + 1)


def adamw_host_tensors(sizes, dtype="bf16", seed=0, step=1):
    """Seeded host arrays p, g (dtype values as float32) and m, v (float32) per tensor.

    p ~ N(0, 0.02^2), g ~ N(0, 1e-3^2) times a per-tensor scale 10^U(-1, 1); the
    moments are those of a run already under way when step > 1: m ~ N(0, 1e-3^2),
    v ~ U(0, 2e-6); zero when step == 1.
    """
    out = []
    for i, n in enumerate(sizes):
        rng = np.random.default_rng([9000 + seed, i])
        scale = 10.0 ** rng.uniform(-1.0, 1.0)
        p = _store(0.02 * rng.standard_normal(n), dtype)
        g = _store(1e-3 * scale * rng.standard_normal(n), dtype)
        if step > 1:
            m = (1e-3 * rng.standard_normal(n)).astype(np.float32)
            v = rng.uniform(0.0, 2e-6, n).astype(np.float32)
        else:
            m = np.zeros(n, np.float32)
            v = np.zeros(n, np.float32)
        out.append({"p": p, "g": g, "m": m, "v": v})
    return out


# --------------------------------------------------------------------------
# Muon-Cayley inputs (points on the Stiefel manifold).
# --------------------------------------------------------------------------

def cayley_host_matrix(rows, cols, seed=0, grad_std=1e-2, momentum_std=1e-2):
    """Seeded float32 W with orthonormal columns (orthonormal rows when rows < cols),
    taken from the QR factor of a Gaussian draw, and Gaussian G and M."""
    rng = np.random.default_rng([7000 + seed, rows, cols])
    n, k = max(rows, cols), min(rows, cols)
    q, r = np.linalg.qr(rng.standard_normal((n, k)))
    q = q * np.sign(np.diag(r))
    W = q if rows >= cols else q.T
    G = grad_std * rng.standard_normal((rows, cols))
    M = momentum_std * rng.standard_normal((rows, cols))
    return {"W": np.ascontiguousarray(W, np.float32), "G": G.astype(np.float32), "M": M.astype(np.float32)}


CAYLEY_SET = [(4096, 128)] * 32
"""Timing workload for the Muon-Cayley row: 32 matrices of 4096 x 128 (the Stiefel
page discusses a hidden size of 4096 with k much smaller than n)."""
