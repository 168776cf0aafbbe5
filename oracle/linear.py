"""Oracle for the frozen-base linear layer with LoRA adapters, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
  [teardown]  "QLoRA Paper Breakdown ..." section 4 'QLoRA Dual-Precision
              Storage vs. Computation Contract': the forward pass
              Y = X * dequant(W) + (alpha/r) * (X * L_1 * L_2), and that the
              backward pass needs dY/dX through the dequantized W while the
              gradient of W is never materialized.
  [explainer] "QLoRA, explained." method step 5: BF16 adapters are the only
              trainable parameters; gradients pass through the dequantized
              base but no update is applied to it.
  [reading note] "What the method actually is": gradients flow back through
              the dequantized base but are computed only for the LoRA
              parameters.

Layout (PyTorch nn.Linear convention): W_hat [n, k] (out, in); X [M, k];
A [r, k]; B [n, r]; Y, dY [M, n].  The teardown's row-vector factors are
L_1 = A^T (k x r) and L_2 = B^T (r x n).  s = alpha / r: the explainer notes
that the paper's own equation leaves the scale out; the teardown includes it
(reading: include it).

Every product is an exact-input float64 product: the inputs are the BF16
values the GPU path consumes (exactly representable in float64), and the
outputs are float64 references for the tolerance comparison.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def lora_scale(alpha: float, r: int) -> float:
    """s = alpha / r  [teardown sec. 4 forward pass]."""
    return float(alpha) / float(r)


def fwd(X, W_hat, A, B, alpha: float):
    """Forward pass.  Returns (Y [M, n], H [M, r]) in float64.

    H = X A^T is the adapter's down-projection (kept for the backward pass);
    Y = X W_hat^T + s * H B^T.
    """
    X, W_hat, A, B = (np.asarray(t, dtype=F64) for t in (X, W_hat, A, B))
    s = lora_scale(alpha, A.shape[0])
    H = X @ A.T
    Y = X @ W_hat.T + s * (H @ B.T)
    return Y, H


def bwd(X, dY, W_hat, A, B, alpha: float, H=None):
    """Backward pass.  Returns (dX [M, k], dA [r, k], dB [n, r], G [M, r]).

    Chain rule on Y = X W_hat^T + s (X A^T) B^T, with W_hat frozen (no dW):
      G  = s * dY B            gradient reaching H = X A^T
      dX = dY W_hat + G A      input gradient through the dequantized base
      dB = s * dY^T H          H = X A^T (recomputed here when not given)
      dA = G^T X
    """
    X, dY, W_hat, A, B = (np.asarray(t, dtype=F64) for t in (X, dY, W_hat, A, B))
    s = lora_scale(alpha, A.shape[0])
    if H is None:
        H = X @ A.T
    H = np.asarray(H, dtype=F64)
    G = s * (dY @ B)
    dX = dY @ W_hat + G @ A
    dB = s * (dY.T @ H)
    dA = G.T @ X
    return dX, dA, dB, G
