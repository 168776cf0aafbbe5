"""Oracle for the attention core between the q/k/v projections and the o
projection of the decoder layer the adapters sit in.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
  [explainer] "QLoRA, explained." step 4 / the reading note's 'Conditions':
              adapters go on every linear layer of the block, so the layer's
              backward runs the frozen-base backward of the seven projections
              (q, k, v, o, gate, up, down) with the attention core and the
              SwiGLU gate between them.
  [video]     "QLoRA Explained ... Part 2/6": App. G's estimate is for a
              LLaMA decoder with batch 1, sequence 512, gradient checkpointing.

The pages do not write the attention itself out.  Reading: the plain causal
scaled dot-product attention of a decoder-only LLaMA layer, per sequence and
per head:
    S = Q K^T / sqrt(d),  S[i, j] = -inf for j > i   (a token sees itself and
                                                       earlier tokens only)
    P = row softmax(S),  O = P V,  lse[i] = log sum_j exp(S[i, j])
and its exact gradient through the softmax Jacobian
    dV = P^T dO,  dP = dO V^T,  dS[i, j] = P[i, j] (dP[i, j] - sum_l P[i, l] dP[i, l]),
    dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d).
Rotary position embedding is left out: it is a fixed rotation of Q and K
that holds no adapter.

Layout (the projections' outputs as they come): Q, K, V, O are
[batch * seq, heads * d] row-major; sequence b holds rows b*seq .. b*seq+seq-1
and head h holds columns h*d .. h*d+d-1.  lse is [batch, heads, seq].
Everything is float64.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def _split(X, batch, seq, heads, d):
    """[batch*seq, heads*d] -> [batch, heads, seq, d]."""
    return np.asarray(X, F64).reshape(batch, seq, heads, d).transpose(0, 2, 1, 3)


def _merge(Z):
    """[batch, heads, seq, d] -> [batch*seq, heads*d]."""
    b, h, s, d = Z.shape
    return Z.transpose(0, 2, 1, 3).reshape(b * s, h * d)


def _probs(Qh, Kh):
    """Causal softmax probabilities and log-sum-exp for [b, h, s, d] inputs."""
    d = Qh.shape[-1]
    s = Qh.shape[2]
    S = Qh @ np.swapaxes(Kh, -1, -2) / np.sqrt(F64(d))
    S = np.where(np.tril(np.ones((s, s), bool)), S, -np.inf)
    m = S.max(axis=-1, keepdims=True)
    e = np.exp(S - m)
    z = e.sum(axis=-1, keepdims=True)
    return e / z, (m + np.log(z))[..., 0]


def fwd(Q, K, V, batch, seq, heads, d):
    """(O, lse): O [batch*seq, heads*d], lse [batch, heads, seq]."""
    Qh, Kh, Vh = (_split(t, batch, seq, heads, d) for t in (Q, K, V))
    P, lse = _probs(Qh, Kh)
    return _merge(P @ Vh), lse


def bwd(Q, K, V, dO, batch, seq, heads, d):
    """(dQ, dK, dV), each [batch*seq, heads*d]."""
    Qh, Kh, Vh, dOh = (_split(t, batch, seq, heads, d) for t in (Q, K, V, dO))
    P, _ = _probs(Qh, Kh)
    dV = np.swapaxes(P, -1, -2) @ dOh
    dP = dOh @ np.swapaxes(Vh, -1, -2)
    dS = P * (dP - (P * dP).sum(axis=-1, keepdims=True))
    c = 1.0 / np.sqrt(F64(d))
    dQ = c * (dS @ Kh)
    dK = c * (np.swapaxes(dS, -1, -2) @ Qh)
    return _merge(dQ), _merge(dK), _merge(dV)
