"""Pins of the decoder-layer oracle (oracle/layer.py): central finite
differences of its forward against its backward for the input and every
adapter (the gradient a training step uses), and the closed form of a layer
whose projections are all zero (both residuals pass X through, so Y = X and
dX = dY).  Sources: "QLoRA, explained." all-linear placement; "QLoRA
Explained ... Part 2/6" (App. G's checkpointed LLaMA layer)."""
import numpy as np

from oracle import layer


def _params(hidden, inter, r, seed, zero=False):
    rng = np.random.default_rng(seed)
    shapes = {"q": (hidden, hidden), "k": (hidden, hidden), "v": (hidden, hidden), "o": (hidden, hidden),
              "gate": (inter, hidden), "up": (inter, hidden), "down": (hidden, inter)}
    out = {}
    for name, (n, k) in shapes.items():
        W, A, B = rng.standard_normal((n, k)) * 0.4, rng.standard_normal((r, k)) * 0.3, rng.standard_normal((n, r)) * 0.3
        out[name] = (0 * W, 0 * A, 0 * B) if zero else (W, A, B)
    return out


def test_layer_backward_matches_finite_differences():
    batch, seq, heads, d, inter, r, alpha = 1, 3, 2, 2, 6, 2, 3.0
    hidden = heads * d
    rng = np.random.default_rng(7)
    X, dY = rng.standard_normal((batch * seq, hidden)), rng.standard_normal((batch * seq, hidden))
    P = _params(hidden, inter, r, 8)
    dX, grads = layer.bwd(X, dY, P, alpha, batch, seq, heads, d)
    loss = lambda x, p: float((layer.fwd(x, p, alpha, batch, seq, heads, d)[0] * dY).sum())
    eps = 1e-6

    def fd(get, set_):
        base = get()
        num = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            vals = []
            for sgn in (1, -1):
                t = base.copy()
                t[idx] += sgn * eps
                vals.append(set_(t))
            num[idx] = (vals[0] - vals[1]) / (2 * eps)
        return num

    np.testing.assert_allclose(dX, fd(lambda: X, lambda t: loss(t, P)), rtol=1e-6, atol=1e-7)
    for name in layer.PROJ:
        W, A, B = P[name]
        numA = fd(lambda: A, lambda t: loss(X, {**P, name: (W, t, B)}))
        numB = fd(lambda: B, lambda t: loss(X, {**P, name: (W, A, t)}))
        np.testing.assert_allclose(grads[name][0], numA, rtol=1e-6, atol=1e-7, err_msg=f"dA {name}")
        np.testing.assert_allclose(grads[name][1], numB, rtol=1e-6, atol=1e-7, err_msg=f"dB {name}")


def test_zero_projections_pass_the_input_through():
    batch, seq, heads, d, inter, r = 2, 5, 2, 4, 12, 2
    rng = np.random.default_rng(9)
    X, dY = rng.standard_normal((batch * seq, heads * d)), rng.standard_normal((batch * seq, heads * d))
    P = _params(heads * d, inter, r, 10, zero=True)
    Y, _ = layer.fwd(X, P, 16.0, batch, seq, heads, d)
    np.testing.assert_array_equal(Y, X)
    dX, grads = layer.bwd(X, dY, P, 16.0, batch, seq, heads, d)
    np.testing.assert_array_equal(dX, dY)
    # with A = B = 0 both adapter gradients vanish (dA carries B, dB carries X A^T)
    assert all(not g[0].any() and not g[1].any() for g in grads.values())
