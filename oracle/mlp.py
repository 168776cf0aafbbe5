"""Oracle for the LLaMA MLP block the adapters sit in: gate and up
projections, the SwiGLU gate between them and the down projection.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
  [explainer] "QLoRA, explained." step 4 / the reading note's 'Conditions':
              adapters go on every linear layer of the block (all-linear
              placement), so a block's backward runs the frozen-base
              backward of each projection in turn.
  [video]     "QLoRA Explained ... Part 2/6": App. G's memory estimate uses
              batch 1, sequence 512 and gradient checkpointing (activations
              recomputed in the backward pass).

The pages give no activation function.  Reading: SwiGLU, the gate of the
LLaMA MLP whose shapes (hidden 4096, intermediate 11008) the workloads use:
h = silu(g) * u with silu(x) = x / (1 + exp(-x)).  Everything here is
float64 on exactly representable inputs.
"""
from __future__ import annotations

import numpy as np

from . import linear

F64 = np.float64


def silu(x):
    x = np.asarray(x, F64)
    return x / (1.0 + np.exp(-x))


def swiglu_fwd(g, u):
    """h = silu(g) * u."""
    return silu(g) * np.asarray(u, F64)


def swiglu_bwd(g, u, dh):
    """(dg, du) for h = silu(g) u: du = dh silu(g); dg = dh u silu'(g),
    silu'(x) = sigma(x) (1 + x (1 - sigma(x)))."""
    g, u, dh = (np.asarray(t, F64) for t in (g, u, dh))
    sig = 1.0 / (1.0 + np.exp(-g))
    return dh * u * sig * (1.0 + g * (1.0 - sig)), dh * g * sig


def block_fwd(X, Wg, Wu, Wd, Ag, Bg, Au, Bu, Ad, Bd, alpha):
    """Y = down( swiglu( gate(X), up(X) ) ), each projection the frozen-base
    layer with its own adapters (oracle.linear.fwd)."""
    Yg, _ = linear.fwd(X, Wg, Ag, Bg, alpha)
    Yu, _ = linear.fwd(X, Wu, Au, Bu, alpha)
    h = swiglu_fwd(Yg, Yu)
    Y, _ = linear.fwd(h, Wd, Ad, Bd, alpha)
    return Y, {"Yg": Yg, "Yu": Yu, "h": h}


def block_bwd(X, dY, Wg, Wu, Wd, Ag, Bg, Au, Bu, Ad, Bd, alpha):
    """Gradients of the block: dX and each projection's dA, dB (no dW).
    The gate and up outputs are recomputed from X (checkpointing)."""
    Yg, _ = linear.fwd(X, Wg, Ag, Bg, alpha)
    Yu, _ = linear.fwd(X, Wu, Au, Bu, alpha)
    h = swiglu_fwd(Yg, Yu)
    dh, dAd, dBd, _ = linear.bwd(h, dY, Wd, Ad, Bd, alpha)
    dg, du = swiglu_bwd(Yg, Yu, dh)
    dXg, dAg, dBg, _ = linear.bwd(X, dg, Wg, Ag, Bg, alpha)
    dXu, dAu, dBu, _ = linear.bwd(X, du, Wu, Au, Bu, alpha)
    return {"dX": dXg + dXu, "dAg": dAg, "dBg": dBg, "dAu": dAu, "dBu": dBu, "dAd": dAd, "dBd": dBd,
            "dh": dh, "dg": dg, "du": du}
