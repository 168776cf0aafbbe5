"""Oracle for folding trained LoRA adapters back into the frozen base.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
  [teardown]  "QLoRA Paper Breakdown ..." section 'Limitations': full-rank
              weight updates need the adapters dequantized and merged into
              16-bit precision.
  [video]     "QLoRA Explained: What Actually Trains in 4 Bits? | Part 2/6":
              adapter merging / requantization is a deployment step the
              paper does not evaluate.
  [teardown]  section 4 forward pass: the layer computes
              X W_hat^T + s X A^T B^T, so the merged weight is
              W_hat + s B A (n x k), s = alpha / r.

The pages fix no arithmetic for the merge.  Reading, chosen so that the
result is one defined float32 tensor:
  t[n, k] = sum over j = 0 .. r-1, in that order, of B[n, j] * A[j, k]
            in float64 (each product of two bf16 values is exact);
  u[n, k] = float64(W_hat[n, k]) + float64(s) * t[n, k]   (two roundings);
  W'[n, k] = float32(u[n, k]),   s = float32(alpha) / float32(r) in float32
(the same s the layer's forward pass uses).  The merged 16-bit weight is
bf16_rne(W'); requantization is the storage encoding applied to W'.
"""
from __future__ import annotations

import numpy as np

from . import nf4_dq

F32, F64 = np.float32, np.float64


def merged_f32(W_hat_bits, A_bits, B_bits, alpha: float) -> np.ndarray:
    """W' = float32(W_hat + s * B A) [n, k] with the rounding order above."""
    What = nf4_dq.bf16_bits_to_f64(W_hat_bits)
    A = nf4_dq.bf16_bits_to_f64(A_bits)
    B = nf4_dq.bf16_bits_to_f64(B_bits)
    r = A.shape[0]
    s = F64(F32(alpha) / F32(r))
    t = np.zeros(What.shape, F64)
    for j in range(r):                       # sequential in j, float64
        t = t + B[:, j:j + 1] * A[j:j + 1, :]
    u = What + s * t
    return u.astype(F32)


def merge_and_requantize(W_hat_bits, A_bits, B_bits, alpha: float, codebook: str = "nf4") -> dict:
    """The merged float32 weight, its bf16 copy and its NF4+DQ re-encoding."""
    Wm = merged_f32(W_hat_bits, A_bits, B_bits, alpha)
    enc = nf4_dq.quantize_nf4_dq(Wm, codebook)
    return {"merged_f32": Wm, "merged_bf16": nf4_dq.bf16_rne_bits(Wm), "encoding": enc}
