"""Oracle for one AdamW step on the LoRA adapters.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
  [teardown]  "QLoRA Paper Breakdown ..." section 5 'Paged Optimizers via
              CUDA Unified Memory': the adapters' Adam states m_t, v_t are
              the paged tensors; an optimizer step reads them back on demand.
  [explainer] "QLoRA, explained." method step 6: Adam's states live in
              memory the driver may move to host RAM; the step is the same.

The pages name the optimizer (paged AdamW) but print no update rule.
Reading: AdamW as published (Loshchilov & Hutter, decoupled weight decay,
bias-corrected moments), with the decay applied to the parameter before
the moment step:
  m_t = b1 m + (1 - b1) g;   v_t = b2 v + (1 - b2) g^2
  p_t = p (1 - lr wd) - (lr / (1 - b1^t)) * m_t / (sqrt(v_t) / sqrt(1 - b2^t) + eps)
computed here in float64 from the float32 / bf16 inputs (the plain
definition; the GPU computes in float32 and is compared with a tolerance).
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def adamw_step(p, g, m, v, step: int, lr: float, b1: float, b2: float, eps: float, wd: float):
    """One step; returns (p_t, m_t, v_t) in float64.  p, m, v are float32
    values, g the bf16 gradient values (all exactly representable in
    float64); ``step`` is t >= 1, the number of this update."""
    if step < 1:
        raise ValueError("step counts from 1")
    p, g, m, v = (np.asarray(x, F64) for x in (p, g, m, v))
    m_t = b1 * m + (1.0 - b1) * g
    v_t = b2 * v + (1.0 - b2) * g * g
    bc1 = 1.0 - b1 ** step
    bc2 = 1.0 - b2 ** step
    p_t = p * (1.0 - lr * wd) - (lr / bc1) * m_t / (np.sqrt(v_t) / np.sqrt(bc2) + eps)
    return p_t, m_t, v_t
