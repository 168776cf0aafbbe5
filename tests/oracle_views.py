"""Oracle-side views of one weight for the sampled full-size parity checks.

Composes oracle functions only: the block scales of the whole tensor (which
depend on every block through the mean), and the codes / BF16 weights of any
subset of rows or of 64-column blocks (each such block lies inside one row,
so its codes depend on nothing else)."""
from __future__ import annotations

import numpy as np

from oracle import linear, nf4_dq


class OracleWeight:
    def __init__(self, W: np.ndarray, codebook: str = "nf4", scales: str = "dq"):
        self.W = np.asarray(W, np.float32)
        self.codebook = codebook
        self.n, self.k = self.W.shape
        self.kb = self.k // nf4_dq.BLOCK
        self.absmax = nf4_dq.block_absmax(self.W)
        self.offset = nf4_dq.dq_offset(self.absmax)
        self.scale_code, self.group_amax = nf4_dq.dq_encode(self.absmax, self.offset)
        self.s = nf4_dq.dq_block_scale(self.scale_code, self.group_amax, self.offset)
        if scales == "fp32":   # single-level constants: s_b = absmax_b
            self.s = self.absmax
        self.levels = nf4_dq.codebook_levels(codebook)

    def row_codes(self, rows) -> np.ndarray:
        codes, _ = nf4_dq.blockwise_quantize(self.W[rows], self.levels, nf4_dq.BLOCK)
        return codes                                   # [len(rows) * kb, 64]

    def row_packed(self, rows) -> np.ndarray:
        return nf4_dq.pack_nibbles(self.row_codes(rows)).reshape(len(rows), self.k // 2)

    def row_what_bits(self, rows) -> np.ndarray:
        rows = np.asarray(rows)
        blk = (rows[:, None] * self.kb + np.arange(self.kb)[None, :]).reshape(-1)
        return nf4_dq.dequant_blocks_bf16(self.row_codes(rows), self.s[blk], self.codebook).reshape(len(rows), self.k)

    def colblock_what_bits(self, kblocks) -> np.ndarray:
        """W_hat[:, 64*b : 64*b+64] for each block column b, concatenated."""
        parts = []
        for b in kblocks:
            sub = self.W[:, 64 * b:64 * b + 64]
            codes, _ = nf4_dq.blockwise_quantize(sub, self.levels, nf4_dq.BLOCK)
            s = self.s[np.arange(self.n) * self.kb + b]
            parts.append(nf4_dq.dequant_blocks_bf16(codes, s, self.codebook).reshape(self.n, 64))
        return np.concatenate(parts, axis=1)

    def encoding(self) -> dict:
        enc = nf4_dq.quantize_nf4_dq(self.W, self.codebook)
        return {k: enc[k] for k in ("packed", "scale_code", "group_amax", "offset")}


def bf16_f64(bits):
    return nf4_dq.bf16_bits_to_f64(bits)


def fwd(*a, **kw):
    return linear.fwd(*a, **kw)


def bwd(*a, **kw):
    return linear.bwd(*a, **kw)
