"""Pins for the fp64 AdamW oracle (CPU only).

* torch.optim.AdamW, run in fp64 on the CPU, implements exactly the method the
  pages state (decoupled decay, bias-corrected moments); several steps must
  agree with the oracle to rounding.
* Closed forms: a constant gradient from zero state gives m_hat = g and
  v_hat = g^2 at every step, so each step is lr * g / (|g| + eps) plus decay;
  a zero gradient with zero state only decays the parameter.
* Planted mistakes in a copy of the step are each caught by these pins.
"""
import numpy as np
import pytest

import oracle as orc
import oracle.adamw_oracle as ao

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)


def _f32(hp):
    return {k: orc.as_f32(v) for k, v in hp.items()}


def _torch_reference(p0, grads, hp):
    torch = pytest.importorskip("torch")
    h = _f32(hp)
    p = torch.nn.Parameter(torch.tensor(p0, dtype=torch.float64))
    opt = torch.optim.AdamW([p], lr=h["lr"], betas=(h["beta1"], h["beta2"]), eps=h["eps"],
                            weight_decay=h["weight_decay"], foreach=False)
    for g in grads:
        p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
    st = opt.state[p]
    return p.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


def _run_oracle(p0, grads, hp, step_fn=None):
    step_fn = step_fn or orc.adamw_step
    p, m, v = np.array(p0, np.float64), np.zeros_like(p0), np.zeros_like(p0)
    for t, g in enumerate(grads, start=1):
        out = step_fn(p, g, m, v, step=t, **hp)
        p, m, v = out["p"], out["m"], out["v"]
    return p, m, v


@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_matches_torch_adamw_in_fp64(wd):
    rng = np.random.default_rng(1)
    p0 = rng.standard_normal(257)
    grads = [rng.standard_normal(257) * 10.0 ** rng.uniform(-4, 1) for _ in range(7)]
    hp = dict(HP, weight_decay=wd)
    p, m, v = _run_oracle(p0, grads, hp)
    tp, tm, tv = _torch_reference(p0, grads, hp)
    assert np.max(np.abs(m - tm)) <= 1e-15 * np.max(np.abs(tm)) + 1e-300
    assert np.max(np.abs(v - tv) / tv) < 1e-14
    assert np.max(np.abs(p - tp)) < 1e-14


def test_constant_gradient_closed_form():
    rng = np.random.default_rng(2)
    p0 = rng.standard_normal(64)
    g = rng.standard_normal(64)
    h = _f32(HP)
    T = 9
    p, m, v = _run_oracle(p0, [g] * T, HP)
    f = 1.0 - h["lr"] * h["weight_decay"]
    stepv = h["lr"] * g / (np.abs(g) + h["eps"])
    expect = f ** T * p0 - stepv * sum(f ** s for s in range(T))
    assert np.max(np.abs(p - expect)) < 1e-13
    b1, b2 = h["beta1"], h["beta2"]
    assert np.max(np.abs(m - g * (1 - b1 ** T))) < 1e-15
    assert np.max(np.abs(v - g * g * (1 - b2 ** T))) < 1e-15


def test_zero_gradient_only_decays():
    p0 = np.arange(-5.0, 6.0)
    z = np.zeros_like(p0)
    out = orc.adamw_step(p0, z, z, z, step=1, **HP)
    h = _f32(HP)
    assert np.all(out["m"] == 0) and np.all(out["v"] == 0)
    assert np.max(np.abs(out["p"] - (1 - h["lr"] * h["weight_decay"]) * p0)) == 0.0


def test_step_must_count_from_one():
    z = np.zeros(3)
    with pytest.raises(ValueError):
        orc.adamw_step(z, z, z, z, step=0, **HP)


def test_rounding_of_stored_results():
    rng = np.random.default_rng(3)
    p0 = orc.rne(rng.standard_normal(100), "bf16").astype(np.float64)
    g = orc.rne(rng.standard_normal(100), "bf16").astype(np.float64)
    out = orc.adamw_step(p0, g, np.zeros(100), np.zeros(100), step=1, dtype="bf16", **HP)
    assert np.array_equal(out["p_rounded"], orc.rne(out["p"], "bf16"))
    assert out["m_rounded"].dtype == np.float32


# ----------------------------------------------------------------------------
# Planted mistakes
# ----------------------------------------------------------------------------

def _mutant(kind):
    def step(p, g, m, v, *, lr, beta1, beta2, eps, weight_decay, step, dtype="f32"):
        lr, b1, b2 = orc.as_f32(lr), orc.as_f32(beta1), orc.as_f32(beta2)
        eps, wd = orc.as_f32(eps), orc.as_f32(weight_decay)
        t = step
        gg = g + wd * p if kind == "coupled_decay" else g
        m2 = b1 * m + (1 - b1) * gg if kind != "swapped_beta" else (1 - b1) * m + b1 * gg
        v2 = b2 * v + (1 - b2) * gg * gg
        mh = m2 if kind == "no_bias_correction" else m2 / (1 - b1 ** t)
        vh = v2 if kind == "no_bias_correction" else v2 / (1 - b2 ** t)
        den = np.sqrt(vh + eps) if kind == "eps_under_root" else np.sqrt(vh) + eps
        decay = 1.0 if kind == "coupled_decay" else (1 - wd if kind == "decay_without_lr" else 1 - lr * wd)
        p2 = decay * p - lr * mh / den
        return {"p": p2, "m": m2, "v": v2}
    return step


@pytest.mark.parametrize("kind", ["coupled_decay", "swapped_beta", "no_bias_correction", "eps_under_root",
                                  "decay_without_lr"])
def test_pins_catch_planted_mistake(kind):
    rng = np.random.default_rng(4)
    p0 = rng.standard_normal(257)
    grads = [rng.standard_normal(257) * 10.0 ** rng.uniform(-4, 1) for _ in range(7)]
    p, m, v = _run_oracle(p0, grads, HP, step_fn=_mutant(kind))
    tp, tm, tv = _torch_reference(p0, grads, HP)
    caught = np.max(np.abs(p - tp)) > 1e-12 or np.max(np.abs(m - tm)) > 1e-12
    assert caught, kind
