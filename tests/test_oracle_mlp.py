"""Pins of the MLP-block oracle (oracle/mlp.py): closed-form SwiGLU values,
central finite differences of the block's forward against its backward,
and linearity of the adapters' gradients.  Sources: "QLoRA, explained."
all-linear placement; "QLoRA Explained ... Part 2/6" (checkpointed block)."""
import numpy as np

from oracle import mlp


def test_silu_closed_forms():
    assert mlp.silu(0.0) == 0.0
    assert np.isclose(mlp.silu(1.0), 1.0 / (1.0 + np.exp(-1.0)))
    assert np.isclose(mlp.silu(-50.0), 0.0, atol=1e-20) and np.isclose(mlp.silu(50.0), 50.0)
    dg, du = mlp.swiglu_bwd(np.array([0.0]), np.array([2.0]), np.array([1.0]))
    assert dg[0] == 1.0 and du[0] == 0.0            # silu'(0) = 1/2, times u = 2


def test_swiglu_bwd_matches_finite_differences():
    rng = np.random.default_rng(1)
    g, u, dh = rng.standard_normal(50) * 3, rng.standard_normal(50), rng.standard_normal(50)
    eps = 1e-6
    dg, du = mlp.swiglu_bwd(g, u, dh)
    num_g = dh * (mlp.swiglu_fwd(g + eps, u) - mlp.swiglu_fwd(g - eps, u)) / (2 * eps)
    num_u = dh * (mlp.swiglu_fwd(g, u + eps) - mlp.swiglu_fwd(g, u - eps)) / (2 * eps)
    np.testing.assert_allclose(dg, num_g, rtol=1e-7, atol=1e-9)
    np.testing.assert_allclose(du, num_u, rtol=1e-7, atol=1e-9)


def _tiny_block(seed):
    rng = np.random.default_rng(seed)
    M, k, n, r = 3, 8, 12, 2
    t = lambda *s: rng.standard_normal(s) * 0.3
    return dict(X=t(M, k), Wg=t(n, k), Wu=t(n, k), Wd=t(k, n), Ag=t(r, k), Bg=t(n, r), Au=t(r, k), Bu=t(n, r),
                Ad=t(r, n), Bd=t(k, r)), t(M, k)


def test_block_backward_matches_finite_differences():
    p, dY = _tiny_block(2)
    alpha = 4.0
    grads = mlp.block_bwd(p["X"], dY, p["Wg"], p["Wu"], p["Wd"], p["Ag"], p["Bg"], p["Au"], p["Bu"], p["Ad"],
                          p["Bd"], alpha)
    loss = lambda q: float(np.sum(dY * mlp.block_fwd(q["X"], q["Wg"], q["Wu"], q["Wd"], q["Ag"], q["Bg"], q["Au"],
                                                      q["Bu"], q["Ad"], q["Bd"], alpha)[0]))
    eps = 1e-6
    for name, key in (("X", "dX"), ("Ag", "dAg"), ("Bg", "dBg"), ("Au", "dAu"), ("Bu", "dBu"), ("Ad", "dAd"),
                      ("Bd", "dBd")):
        num = np.zeros_like(p[name])
        for idx in np.ndindex(p[name].shape):
            a, b = dict(p), dict(p)
            a[name] = p[name].copy(); a[name][idx] += eps
            b[name] = p[name].copy(); b[name][idx] -= eps
            num[idx] = (loss(a) - loss(b)) / (2 * eps)
        np.testing.assert_allclose(grads[key], num, rtol=1e-6, atol=1e-8, err_msg=name)
