"""Shared plumbing for the GPU parity tests: device upload/download, the
library round trips, and the tolerance check stated for the fwd/bwd outputs
(relative Frobenius error <= 5e-3 and max |diff| <= 2e-2 * max |ref|)."""
from __future__ import annotations

import sys

import numpy as np
import torch

REL_FRO = 5e-3
REL_MAX = 2e-2


def note(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16).cuda()


def host_bf16(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gpu_quantize(q, W: np.ndarray, codebook: str = "nf4", scales: str = "dq"):
    n, k = W.shape
    w = q.NF4Weight.empty(n, k, codebook=q.CODEBOOKS[codebook],
                          scales=q.QLORA_SCALES_FP32 if scales == "fp32" else q.QLORA_SCALES_DQ)
    ws = torch.empty(q.qlora_quantize_workspace_bytes(n, k), dtype=torch.uint8, device="cuda")
    q.qlora_quantize_nf4_dq(dev_f32(W), w, ws)
    return w


def encoding_to_host(w) -> dict:
    torch.cuda.synchronize()
    return {"packed": w.packed.cpu().numpy(), "scale_code": w.scale_code.cpu().numpy(),
            "group_amax": w.group_amax.cpu().numpy(), "offset": np.float32(w.offset.cpu().numpy()[0])}


def assert_encoding_equal(got: dict, ref: dict, ctx: str = "") -> None:
    for key in ("packed", "scale_code"):
        g, r = got[key], ref[key]
        bad = np.flatnonzero(g != r)
        assert bad.size == 0, f"{ctx} {key}: {bad.size} bytes differ, first at {bad[:5]}: {g[bad[:5]]} vs {r[bad[:5]]}"
    assert np.array_equal(got["group_amax"].view(np.uint32), ref["group_amax"].view(np.uint32)), f"{ctx} group_amax"
    assert np.float32(got["offset"]).view(np.uint32) == np.float32(ref["offset"]).view(np.uint32), \
        f"{ctx} offset {got['offset']!r} vs {ref['offset']!r}"


def assert_close(got, ref, name: str) -> None:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} vs {ref.shape}"
    assert np.isfinite(got).all(), f"{name}: non-finite output"
    scale = np.abs(ref).max()
    if scale == 0:
        assert np.all(got == 0), f"{name}: expected zeros"
        return
    err = got - ref
    fro = np.linalg.norm(err) / np.linalg.norm(ref)
    mx = np.abs(err).max() / scale
    assert fro <= REL_FRO and mx <= REL_MAX, f"{name}: rel_fro={fro:.3e} (<= {REL_FRO}) rel_max={mx:.3e} (<= {REL_MAX})"


class Linear:
    """One layer's device tensors and library calls."""

    def __init__(self, q, w, X: np.ndarray, A: np.ndarray, B: np.ndarray, r: int, alpha: float):
        self.q, self.w, self.r, self.alpha = q, w, r, alpha
        self.M = X.shape[0]
        self.X, self.A, self.B = dev_bf16(X), dev_bf16(A), dev_bf16(B)
        nbytes = q.qlora_linear_workspace_bytes(self.M, w.n, w.k, r)
        self.ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")

    def fwd(self):
        Y = torch.empty(self.M, self.w.n, dtype=torch.bfloat16, device="cuda")
        H = torch.empty(self.M, self.r, dtype=torch.float32, device="cuda")
        self.q.qlora_linear_fwd(self.w, self.X, self.A, self.B, self.r, self.alpha, Y, H, self.ws)
        return Y, H

    def bwd(self, dY: np.ndarray, H=None, want_dx=True):
        dYd = dev_bf16(dY)
        dX = torch.empty(self.M, self.w.k, dtype=torch.bfloat16, device="cuda") if want_dx else None
        dA = torch.empty(self.r, self.w.k, dtype=torch.bfloat16, device="cuda")
        dB = torch.empty(self.w.n, self.r, dtype=torch.bfloat16, device="cuda")
        self.q.qlora_linear_bwd(self.w, self.X, dYd, self.A, self.B, self.r, self.alpha, H, dX, dA, dB, self.ws)
        return dX, dA, dB
