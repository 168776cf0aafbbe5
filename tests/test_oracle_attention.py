"""Pins of the attention oracle (oracle/attention.py) against things other
than itself: PyTorch's CPU scaled-dot-product attention in float64 with
autograd (a second implementation of the same definition), central finite
differences of the forward against the backward, the closed form for Q = 0
(a causal prefix mean of V), causality, independence of the sequences and
heads, and the one-token case.  Sources: "QLoRA, explained." all-linear
placement (q, k, v, o hold adapters); "QLoRA Explained ... Part 2/6" (the
decoder layer of App. G)."""
import numpy as np
import torch

from oracle import attention as at


def _qkvo(batch, seq, heads, d, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((batch * seq, heads * d)) for _ in range(4)]


def _heads(X, batch, seq, heads, d):
    return torch.from_numpy(X).reshape(batch, seq, heads, d).transpose(1, 2)


def test_matches_torch_sdpa_and_autograd():
    b, s, h, d = 2, 13, 3, 8
    Q, K, V, dO = _qkvo(b, s, h, d, 1)
    O, lse = at.fwd(Q, K, V, b, s, h, d)
    dQ, dK, dV = at.bwd(Q, K, V, dO, b, s, h, d)
    tq, tk, tv = (_heads(t, b, s, h, d).clone().requires_grad_(True) for t in (Q, K, V))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    to.backward(_heads(dO, b, s, h, d))
    merge = lambda t: t.detach().transpose(1, 2).reshape(b * s, h * d).numpy()
    np.testing.assert_allclose(O, merge(to), rtol=1e-12, atol=1e-12)
    for got, ref in ((dQ, tq.grad), (dK, tk.grad), (dV, tv.grad)):
        np.testing.assert_allclose(got, merge(ref), rtol=1e-11, atol=1e-12)
    # lse against a direct log-sum-exp of the causal scores
    Sc = (_heads(Q, b, s, h, d) @ _heads(K, b, s, h, d).transpose(-1, -2)) / np.sqrt(d)
    Sc = Sc.masked_fill(~torch.ones(s, s, dtype=torch.bool).tril(), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(Sc, dim=-1).numpy(), rtol=1e-13)


def test_backward_matches_finite_differences():
    b, s, h, d = 1, 5, 2, 4
    Q, K, V, dO = _qkvo(b, s, h, d, 2)
    grads = at.bwd(Q, K, V, dO, b, s, h, d)
    loss = lambda q, k, v: float((at.fwd(q, k, v, b, s, h, d)[0] * dO).sum())
    eps = 1e-6
    args = [Q, K, V]
    for which, g in enumerate(grads):
        num = np.zeros_like(g)
        for idx in np.ndindex(g.shape):
            up = [a.copy() for a in args]
            dn = [a.copy() for a in args]
            up[which][idx] += eps
            dn[which][idx] -= eps
            num[idx] = (loss(*up) - loss(*dn)) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


def test_zero_queries_give_causal_prefix_means():
    b, s, h, d = 2, 9, 2, 4
    _, K, V, _ = _qkvo(b, s, h, d, 3)
    O, lse = at.fwd(np.zeros_like(K), K, V, b, s, h, d)
    Vs = V.reshape(b, s, h * d)
    want = np.cumsum(Vs, axis=1) / np.arange(1, s + 1)[None, :, None]
    np.testing.assert_allclose(O, want.reshape(b * s, h * d), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(np.arange(1, s + 1)), (b, h, s)), rtol=1e-14)


def test_causality_and_independence():
    b, s, h, d = 3, 7, 2, 4
    Q, K, V, _ = _qkvo(b, s, h, d, 4)
    O, _ = at.fwd(Q, K, V, b, s, h, d)
    K2, V2 = K.copy(), V.copy()
    K2[s + 4:2 * s] += 5.0          # later tokens of sequence 1
    V2[s + 4:2 * s] -= 3.0
    K2[2 * s:, :d] *= 2.0           # sequence 2, head 0 only
    O2, _ = at.fwd(Q, K2, V2, b, s, h, d)
    np.testing.assert_array_equal(O2[:s + 4], O[:s + 4])          # sequence 0 and tokens 0..3 of sequence 1
    assert not np.allclose(O2[s + 4:2 * s], O[s + 4:2 * s])
    np.testing.assert_array_equal(O2[2 * s:, d:], O[2 * s:, d:])  # head 1 of sequence 2
    assert not np.allclose(O2[2 * s + 1:, :d], O[2 * s + 1:, :d])


def test_one_token_sequences():
    b, s, h, d = 4, 1, 2, 8
    Q, K, V, dO = _qkvo(b, s, h, d, 5)
    O, lse = at.fwd(Q, K, V, b, s, h, d)
    np.testing.assert_array_equal(O, V)
    own = (Q * K).reshape(b, s, h, d).sum(axis=-1).transpose(0, 2, 1) / np.sqrt(d)   # the only score
    np.testing.assert_allclose(lse, own, rtol=1e-14, atol=1e-15)
    dQ, dK, dV = at.bwd(Q, K, V, dO, b, s, h, d)
    assert not dQ.any() and not dK.any()
    np.testing.assert_array_equal(dV, dO)
