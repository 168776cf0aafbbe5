"""Seeded synthetic inputs for the NF4 QLoRA linear layer.

This module only draws random numbers and converts them to the storage
dtypes (float32 weights, bfloat16 activations / adapters, via torch's CPU
cast).  It holds none of the layer's arithmetic, and it is the one module
the product path, the tests, the benchmark and the oracle runs all share.

Workloads (LLaMA-shaped layers; out x in, i.e. W is [n, k]):
  tiny        one 256x256 layer, M = 16, r = 8,  W ~ N(0, 0.02)
  q_proj_7b   4096x4096, M = 512 (batch 1 x seq 512), r = 64, W ~ N(0, 0.02)
  mlp_7b      gate/up 11008x4096, down 4096x11008, M = 4096 (batch 8 x seq 512),
              r = 64, W ~ Student-t(df=5) * 0.02 (heavy tails)
  up_65b      22016x8192, M in {1, 4, 16}, r = 16, W ~ N(0, 0.015), forward only
  block_65b   q,k,v,o 8192x8192; gate,up 22016x8192; down 8192x22016, M = 512,
              r = 64, W ~ N(0, 0.015)
Every workload: X, dY ~ N(0, 1) -> bf16; A, B ~ U(-0.05, 0.05) -> bf16;
alpha = 16.  Each linear gets its own independent X (no activation function
between layers), so every layer is measured on its own.

Seeds: numpy PCG64 with SeedSequence([230514314, workload, layer, tensor]),
tensor = 0 W, 1 X, 2 dY, 3 A, 4 B.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SEED_ROOT = 230514314
T_W, T_X, T_DY, T_A, T_B = range(5)


@dataclass(frozen=True)
class Layer:
    name: str
    n: int  # out_features
    k: int  # in_features


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    layers: tuple
    ms: tuple
    r: int
    alpha: float = 16.0
    wdist: str = "normal"       # "normal" or "student_t5"
    wscale: float = 0.02
    backward: bool = True
    adapter_bound: float = 0.05
    notes: str = field(default="", compare=False)


WORKLOADS = {
    "tiny": Workload(0, "tiny", (Layer("w", 256, 256),), (16,), 8),
    "q_proj_7b": Workload(1, "q_proj_7b", (Layer("q_proj", 4096, 4096),), (512,), 64),
    "mlp_7b": Workload(2, "mlp_7b", (Layer("gate_proj", 11008, 4096), Layer("up_proj", 11008, 4096),
                                     Layer("down_proj", 4096, 11008)), (4096,), 64,
                       wdist="student_t5"),
    "up_65b": Workload(3, "up_65b", (Layer("up_proj", 22016, 8192),), (1, 4, 16), 16,
                       wscale=0.015, backward=False),
    "block_65b": Workload(4, "block_65b", (Layer("q_proj", 8192, 8192), Layer("k_proj", 8192, 8192),
                                           Layer("v_proj", 8192, 8192), Layer("o_proj", 8192, 8192),
                                           Layer("gate_proj", 22016, 8192), Layer("up_proj", 22016, 8192),
                                           Layer("down_proj", 8192, 22016)), (512,), 64, wscale=0.015),
}


def rng(workload: int, layer: int, tensor: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, workload, layer, tensor])))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float -> bfloat16 bit patterns through torch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def weight(w: Workload, li: int, rows: slice | None = None) -> np.ndarray:
    """float32 W [n, k] of layer ``li`` (optionally only a row range)."""
    L = w.layers[li]
    g = rng(w.index, li, T_W)
    if w.wdist == "normal":
        W = g.standard_normal((L.n, L.k), dtype=np.float32)
        W *= np.float32(w.wscale)
    elif w.wdist == "student_t5":
        W = (g.standard_t(5, size=(L.n, L.k)) * w.wscale).astype(np.float32)
    else:
        raise ValueError(w.wdist)
    return W if rows is None else W[rows]


def activation(w: Workload, li: int, m: int) -> np.ndarray:
    """X [m, k] bf16 bits, N(0,1)."""
    L = w.layers[li]
    return to_bf16_bits(rng(w.index, li, T_X).standard_normal((m, L.k), dtype=np.float32))


def grad_output(w: Workload, li: int, m: int) -> np.ndarray:
    """dY [m, n] bf16 bits, N(0,1)."""
    L = w.layers[li]
    return to_bf16_bits(rng(w.index, li, T_DY).standard_normal((m, L.n), dtype=np.float32))


def adapters(w: Workload, li: int):
    """(A [r, k], B [n, r]) bf16 bits, U(-b, b)."""
    L = w.layers[li]
    b = w.adapter_bound
    A = rng(w.index, li, T_A).uniform(-b, b, (w.r, L.k)).astype(np.float32)
    B = rng(w.index, li, T_B).uniform(-b, b, (L.n, w.r)).astype(np.float32)
    return to_bf16_bits(A), to_bf16_bits(B)


def custom_weight(n: int, k: int, seed: int, scale: float = 0.02) -> np.ndarray:
    """float32 N(0, scale) weight of any shape (edge-case tests)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, 99, seed, T_W])))
    return (g.standard_normal((n, k), dtype=np.float32) * np.float32(scale)).astype(np.float32)


def custom_bf16(shape, seed: int, tensor: int, bound: float | None = None) -> np.ndarray:
    """bf16 bits of any shape: N(0,1), or U(-bound, bound) when bound is given."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, 99, seed, tensor])))
    x = g.standard_normal(shape, dtype=np.float32) if bound is None else \
        g.uniform(-bound, bound, shape).astype(np.float32)
    return to_bf16_bits(x)
