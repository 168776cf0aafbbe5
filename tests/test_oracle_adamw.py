"""Pins of the AdamW oracle (oracle/adamw.py) against an independent
implementation of the same published algorithm (torch.optim.AdamW on the
CPU) and against closed forms (the first step of bias-corrected Adam moves
every parameter by lr * sign(g) when eps = 0).  Source of the step's role:
"QLoRA Paper Breakdown ..." section 5, "QLoRA, explained." step 6."""
import numpy as np
import torch

from oracle import adamw

HP = dict(lr=2e-4, b1=0.9, b2=0.999, eps=1e-8, wd=0.01)


def _torch_steps(p0, grads, **hp):
    p = torch.nn.Parameter(torch.tensor(p0, dtype=torch.float64))
    opt = torch.optim.AdamW([p], lr=hp["lr"], betas=(hp["b1"], hp["b2"]), eps=hp["eps"], weight_decay=hp["wd"])
    for g in grads:
        p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
    st = opt.state[p]
    return p.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


def test_matches_torch_adamw_over_several_steps():
    rng = np.random.default_rng(1)
    p0 = rng.standard_normal(1000) * 0.05
    p = p0
    m = np.zeros(1000)
    v = np.zeros(1000)
    grads = [rng.standard_normal(1000) * 10.0 ** rng.uniform(-4, 0) for _ in range(5)]
    for t, g in enumerate(grads, start=1):
        p, m, v = adamw.adamw_step(p, g, m, v, t, **HP)
    tp, tm, tv = _torch_steps(p0, grads, **HP)
    np.testing.assert_allclose(p, tp, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(m, tm, rtol=1e-12, atol=1e-18)
    np.testing.assert_allclose(v, tv, rtol=1e-12, atol=1e-22)


def test_first_step_is_a_signed_lr_step_without_eps_and_decay():
    g = np.array([3.0, -0.25, 1e-6, -7.0])
    p = np.array([0.5, -0.5, 0.0, 2.0])
    pt, mt, vt = adamw.adamw_step(p, g, np.zeros(4), np.zeros(4), 1, lr=0.01, b1=0.9, b2=0.99, eps=0.0, wd=0.0)
    np.testing.assert_allclose(pt, p - 0.01 * np.sign(g), rtol=0, atol=1e-15)
    np.testing.assert_allclose(mt, 0.1 * g)
    np.testing.assert_allclose(vt, 0.01 * g * g)


def test_decay_alone_shrinks_the_parameter():
    p = np.array([1.0, -2.0])
    pt, _, _ = adamw.adamw_step(p, np.zeros(2), np.zeros(2), np.zeros(2), 3, lr=0.1, b1=0.9, b2=0.999, eps=1e-8, wd=0.5)
    np.testing.assert_allclose(pt, p * (1 - 0.1 * 0.5))
