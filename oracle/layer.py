"""Oracle for the whole decoder layer whose seven linears carry adapters:
attention sublayer (q, k, v -> causal attention -> o, plus the residual)
and MLP sublayer (gate, up -> SwiGLU -> down, plus the residual).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
  [explainer] "QLoRA, explained." step 4 / the reading note's 'Conditions':
              adapters on every linear layer; the backward runs each
              projection's frozen-base backward and updates only adapters.
  [video]     "QLoRA Explained ... Part 2/6": App. G's LLaMA layer, batch 1,
              sequence 512, gradient checkpointing (the layer's activations
              are recomputed from its input in the backward pass).

Readings: the pages name neither the normalisation nor the positional
encoding.  Both are frozen maps that hold no adapter, so the layer here keeps
what the adapted path runs through: the seven projections, the attention
core (oracle.attention), SwiGLU (oracle.mlp) and the two residual additions.

``rnd`` (identity by default) is applied to every tensor that a bf16
implementation stores between steps, so a test can take the same roundings
at the same places; the arithmetic between them stays float64.
"""
from __future__ import annotations

import numpy as np

from . import attention, linear, mlp

PROJ = ("q", "k", "v", "o", "gate", "up", "down")


def _same(x):
    return x


def fwd(X, params, alpha, batch, seq, heads, d, rnd=_same):
    """params[name] = (W_hat, A, B) for each name in PROJ.  Returns (Y, acts)."""
    X = np.asarray(X, np.float64)
    lin = lambda name, x: rnd(linear.fwd(x, *params[name], alpha)[0])
    Q, K, V = lin("q", X), lin("k", X), lin("v", X)
    O = rnd(attention.fwd(Q, K, V, batch, seq, heads, d)[0])
    Y1 = rnd(X + lin("o", O))
    G, U = lin("gate", Y1), lin("up", Y1)
    Hh = rnd(mlp.swiglu_fwd(G, U))
    Y = rnd(Y1 + lin("down", Hh))
    return Y, {"Q": Q, "K": K, "V": V, "O": O, "Y1": Y1, "G": G, "U": U, "H": Hh}


def bwd(X, dY, params, alpha, batch, seq, heads, d, rnd=_same):
    """Gradients (dX, {name: (dA, dB)}) with the activations recomputed from X."""
    X, dY = np.asarray(X, np.float64), np.asarray(dY, np.float64)
    _, a = fwd(X, params, alpha, batch, seq, heads, d, rnd)
    grads = {}

    def back(name, x, dy):
        dx, dA, dB, _ = linear.bwd(x, dy, *params[name], alpha)
        grads[name] = (dA, dB)
        return rnd(dx)

    dH = back("down", a["H"], dY)
    dG, dU = (rnd(t) for t in mlp.swiglu_bwd(a["G"], a["U"], dH))
    dY1 = rnd(dY + rnd(back("gate", a["Y1"], dG) + back("up", a["Y1"], dU)))
    dO = back("o", a["O"], dY1)
    dQ, dK, dV = (rnd(t) for t in attention.bwd(a["Q"], a["K"], a["V"], dO, batch, seq, heads, d))
    dX = rnd(dY1 + rnd(rnd(back("q", X, dQ) + back("k", X, dK)) + back("v", X, dV)))
    return dX, grads
