"""The decoder layer whose seven linears carry adapters ("QLoRA, explained.",
all-linear placement; the LLaMA layer of "QLoRA Explained ... Part 2/6",
App. G), as an ordered sequence of libqlora calls.

    Q, K, V = q(X), k(X), v(X);  O = causal_attention(Q, K, V)
    Y1 = X + o(O);  Y = Y1 + down(swiglu(gate(Y1), up(Y1)))

Normalisation and positional rotation are frozen maps without adapters and
are not part of the layer here.  The backward recomputes from X the
activations it needs (checkpointing at layer granularity: everything up to
the SwiGLU output, with the adapter products H = x A^T of q, k, v, o, gate
and up; the down projection's output and the final sum are not needed, and
the down projection's H is recomputed by its own backward call), then runs
each projection's frozen-base backward (dX, dA, dB; no weight gradient),
the attention and SwiGLU backwards and the residual gradient sums.  Nothing
the backward reads is left over from an earlier forward call.

This module holds buffers and orders calls; every step runs in the library's
kernels on the current stream.
"""
from __future__ import annotations

import torch

from . import qlora as Q

PROJ = ("q", "k", "v", "o", "gate", "up", "down")


class DecoderLayer:
    """weights[name]: NF4Weight; adapters[name]: (A [r, k], B [n, r]) bf16 device tensors."""

    def __init__(self, weights: dict, adapters: dict, r: int, alpha: float, batch: int, seq: int, heads: int,
                 head_dim: int, device="cuda"):
        self.w, self.ad, self.r, self.alpha = weights, adapters, r, alpha
        self.batch, self.seq, self.heads, self.d = batch, seq, heads, head_dim
        hidden, inter = heads * head_dim, weights["gate"].n
        for name in ("q", "k", "v", "o"):
            if (weights[name].n, weights[name].k) != (hidden, hidden):
                raise ValueError(f"{name} must be [{hidden}, {hidden}]")
        if (weights["up"].n, weights["up"].k) != (inter, hidden) or (weights["down"].n, weights["down"].k) != \
                (hidden, inter) or weights["gate"].k != hidden:
            raise ValueError("gate/up must be [inter, hidden] and down [hidden, inter]")
        M = self.M = batch * seq
        bf = lambda n: torch.empty(M, n, dtype=torch.bfloat16, device=device)
        self.act = {k: bf(hidden) for k in ("q", "k", "v", "attn", "o_out", "y1", "down_out")}
        self.act.update({k: bf(inter) for k in ("gate", "up", "h")})
        self.lse = torch.empty(batch, heads, seq, dtype=torch.float32, device=device)
        self.H = {n: torch.empty(M, r, dtype=torch.float32, device=device) for n in PROJ}
        self.grad = {k: bf(hidden) for k in ("dq", "dk", "dv", "dattn", "dxg", "dxu", "dy1", "dxq", "dxk", "dxv")}
        self.grad.update({k: bf(inter) for k in ("dh", "dgate", "dup")})
        self.dA = {n: torch.empty_like(adapters[n][0]) for n in PROJ}
        self.dB = {n: torch.empty_like(adapters[n][1]) for n in PROJ}
        need = max([Q.qlora_linear_workspace_bytes(M, weights[n].n, weights[n].k, r) for n in PROJ] +
                   [Q.qlora_attention_workspace_bytes(batch, seq, heads, head_dim), 16])
        self.ws = torch.empty(need, dtype=torch.uint8, device=device)

    def _fwd(self, name, X, Y):
        A, B = self.ad[name]
        Q.qlora_linear_fwd(self.w[name], X, A, B, self.r, self.alpha, Y, self.H[name], self.ws)

    def _bwd(self, name, X, dY, dX, H="saved"):
        A, B = self.ad[name]
        H = self.H[name] if H == "saved" else H
        Q.qlora_linear_bwd(self.w[name], X, dY, A, B, self.r, self.alpha, H, dX, self.dA[name],
                           self.dB[name], self.ws)

    def _check_io(self, **tensors) -> None:
        hidden = self.heads * self.d
        for name, t in tensors.items():
            if tuple(t.shape) != (self.M, hidden) or t.dtype != torch.bfloat16:
                raise ValueError(f"{name} must be bf16 [{self.M}, {hidden}], got {t.dtype} {tuple(t.shape)}")

    def _activations(self, X: torch.Tensor) -> None:
        """Everything up to h = swiglu(gate(Y1), up(Y1))."""
        a = self.act
        self._fwd("q", X, a["q"])
        self._fwd("k", X, a["k"])
        self._fwd("v", X, a["v"])
        Q.qlora_attention_fwd(a["q"], a["k"], a["v"], a["attn"], self.lse, self.batch, self.seq, self.heads, self.d,
                              self.ws)
        self._fwd("o", a["attn"], a["o_out"])
        Q.qlora_add_bf16(X, a["o_out"], a["y1"])
        self._fwd("gate", a["y1"], a["gate"])
        self._fwd("up", a["y1"], a["up"])
        Q.qlora_swiglu_fwd(a["gate"], a["up"], a["h"])

    def fwd(self, X: torch.Tensor, Y: torch.Tensor) -> None:
        self._check_io(X=X, Y=Y)
        self._activations(X)
        a = self.act
        self._fwd("down", a["h"], a["down_out"])
        Q.qlora_add_bf16(a["y1"], a["down_out"], Y)

    def bwd(self, X: torch.Tensor, dY: torch.Tensor, dX: torch.Tensor) -> None:
        """dX and self.dA / self.dB."""
        self._check_io(X=X, dY=dY, dX=dX)
        a, g = self.act, self.grad
        self._activations(X)                                     # recompute what the backward reads
        self._bwd("down", a["h"], dY, g["dh"], H=None)          # H = h A^T recomputed by the call
        Q.qlora_swiglu_bwd(a["gate"], a["up"], g["dh"], g["dgate"], g["dup"])
        self._bwd("gate", a["y1"], g["dgate"], g["dxg"])
        self._bwd("up", a["y1"], g["dup"], g["dxu"])
        Q.qlora_add_bf16_n([g["dxg"], g["dxu"], dY], g["dy1"])      # bf16(bf16(dxg + dxu) + dY)
        self._bwd("o", a["attn"], g["dy1"], g["dattn"])
        Q.qlora_attention_bwd(a["q"], a["k"], a["v"], g["dattn"], self.lse, g["dq"], g["dk"], g["dv"],
                              self.batch, self.seq, self.heads, self.d, self.ws)
        self._bwd("q", X, g["dq"], g["dxq"])
        self._bwd("k", X, g["dk"], g["dxk"])
        self._bwd("v", X, g["dv"], g["dxv"])
        Q.qlora_add_bf16_n([g["dxq"], g["dxk"], g["dxv"], g["dy1"]], dX)  # ((dxq + dxk) + dxv) + dy1
