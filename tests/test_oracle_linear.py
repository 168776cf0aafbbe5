"""Pins of the oracle's float64 forward / backward of the frozen-base
linear layer with LoRA adapters.

Pins used (none re-types the oracle's matrix expressions):
  * brute-force scalar loops on tiny shapes (the teardown's section-4
    forward formula written elementwise, with its row-vector factors
    L_1 = A^T, L_2 = B^T);
  * the merged-weight identity X (W + s B A)^T;
  * central finite differences of the scalar <dY, Y> for every gradient;
  * the adjoint identity <dY, J v> = <J^T dY, v>;
  * special cases: B = 0 or A = 0 switch the adapter path off.
"""
import itertools

import numpy as np
import pytest

from oracle import linear

RNG = np.random.default_rng(11)


def _case(M=3, K=5, N=4, r=2):
    X = RNG.standard_normal((M, K))
    W = RNG.standard_normal((N, K)) * 0.3
    A = RNG.uniform(-0.5, 0.5, (r, K))
    B = RNG.uniform(-0.5, 0.5, (N, r))
    dY = RNG.standard_normal((M, N))
    return X, W, A, B, dY


def test_fwd_brute_force_loops():
    X, W, A, B, _ = _case()
    alpha = 16.0
    M, K = X.shape
    N, r = B.shape
    L1, L2 = A.T, B.T                       # k x r and r x n factors
    Y, H = linear.fwd(X, W, A, B, alpha)
    for m, n in itertools.product(range(M), range(N)):
        base = sum(X[m, k] * W[n, k] for k in range(K))
        lora = sum(X[m, k] * L1[k, j] * L2[j, n] for k in range(K) for j in range(r))
        assert Y[m, n] == pytest.approx(base + alpha / r * lora, rel=1e-13, abs=1e-13)
    for m, j in itertools.product(range(M), range(r)):
        assert H[m, j] == pytest.approx(sum(X[m, k] * A[j, k] for k in range(K)), rel=1e-13, abs=1e-13)


def test_fwd_equals_merged_weight():
    X, W, A, B, _ = _case(7, 64, 9, 3)
    Y, _ = linear.fwd(X, W, A, B, 16.0)
    merged = W + (16.0 / 3) * np.einsum("nj,jk->nk", B, A)
    ref = np.einsum("mk,nk->mn", X, merged)
    assert np.allclose(Y, ref, rtol=1e-12, atol=1e-12)


def test_adapters_off():
    X, W, A, B, dY = _case(4, 8, 6, 2)
    Y, _ = linear.fwd(X, W, A, np.zeros_like(B), 16.0)
    assert np.allclose(Y, np.einsum("mk,nk->mn", X, W), rtol=1e-13, atol=1e-13)
    dX, dA, dB, G = linear.bwd(X, dY, W, np.zeros_like(A), B, 16.0)
    assert np.all(dB == 0)
    assert np.allclose(dX, np.einsum("mn,nk->mk", dY, W) + np.einsum("mj,jk->mk", G, 0 * A))


def _fd_grad(f, x, eps=1e-6):
    g = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += eps
        xm[idx] -= eps
        g[idx] = (f(xp) - f(xm)) / (2 * eps)
    return g


@pytest.mark.parametrize("shape", [(3, 64, 5, 2), (4, 128, 3, 8)])
def test_bwd_matches_finite_differences(shape):
    X, W, A, B, dY = _case(*shape)
    alpha = 16.0

    def loss(X_=X, A_=A, B_=B):
        return float(np.sum(dY * linear.fwd(X_, W, A_, B_, alpha)[0]))

    dX, dA, dB, G = linear.bwd(X, dY, W, A, B, alpha)
    assert np.allclose(dX, _fd_grad(lambda v: loss(X_=v), X), rtol=1e-7, atol=1e-8)
    assert np.allclose(dA, _fd_grad(lambda v: loss(A_=v), A), rtol=1e-7, atol=1e-8)
    assert np.allclose(dB, _fd_grad(lambda v: loss(B_=v), B), rtol=1e-7, atol=1e-8)
    # G is the gradient reaching H = X A^T
    H0 = X @ A.T
    lossH = lambda Hv: float(np.sum(dY * (X @ W.T + alpha / A.shape[0] * Hv @ B.T)))
    assert np.allclose(G, _fd_grad(lossH, H0), rtol=1e-7, atol=1e-8)


def test_bwd_with_given_H_equals_recomputed():
    X, W, A, B, dY = _case(5, 64, 6, 4)
    _, H = linear.fwd(X, W, A, B, 8.0)
    a = linear.bwd(X, dY, W, A, B, 8.0, H=H)
    b = linear.bwd(X, dY, W, A, B, 8.0)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_adjoint_identity():
    X, W, A, B, dY = _case(6, 128, 7, 4)
    alpha = 16.0
    vX = RNG.standard_normal(X.shape)
    # J v for the map X -> Y (linear in X)
    JvX = linear.fwd(vX, W, A, B, alpha)[0]
    dX, _, _, _ = linear.bwd(X, dY, W, A, B, alpha)
    assert np.sum(dY * JvX) == pytest.approx(np.sum(dX * vX), rel=1e-12)
