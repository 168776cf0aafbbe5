"""ctypes binding of libqlora.so: the calls of ``include/qlora.h`` under the
same names.  Argument marshalling only -- every step of the layer runs in
the library's HIP kernels.  torch supplies device memory and the stream.

Importing this module loads ``libqlora.so`` and raises ImportError if it has
not been built (``python -m bit_nf4_quantized_qlora_amd.build``); there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

# torch first: its HIP runtime (same soname as ROCm's) is then the one the
# library binds to, so torch's streams and allocations are valid handles here.
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqlora.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run `python -m bit_nf4_quantized_qlora_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)

QLORA_OK = 0
QLORA_ERR_NULL_ARG = -1
QLORA_ERR_BAD_SHAPE = -2
QLORA_ERR_BAD_RANK = -3
QLORA_ERR_MISALIGNED = -4
QLORA_ERR_WORKSPACE = -5
QLORA_ERR_HIP = -6
QLORA_ERR_BAD_ALPHA = -7
QLORA_ERR_BAD_CODEBOOK = -8

QLORA_CODEBOOK_NF4 = 0        # NormalFloat4, the method's storage type
QLORA_CODEBOOK_FP4_E2M1 = 1   # Float4 (E2M1), the comparison type
CODEBOOKS = {"nf4": QLORA_CODEBOOK_NF4, "fp4": QLORA_CODEBOOK_FP4_E2M1}
QLORA_SCALES_DQ = 0           # double-quantized block constants (the method's)
QLORA_SCALES_FP32 = 1         # one float32 absmax per block (double quantization off)

_c_i64, _c_int, _c_float, _c_size, _vp = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p


class qlora_nf4_weight(ctypes.Structure):
    _fields_ = [("n", _c_i64), ("k", _c_i64), ("packed", _vp), ("scale_code", _vp), ("group_amax", _vp),
                ("offset", _vp), ("codebook", ctypes.c_int32), ("scales", ctypes.c_int32), ("absmax", _vp)]


_W = ctypes.POINTER(qlora_nf4_weight)
_SIGS = {
    "qlora_nf4_sizes": (_c_int, [_c_i64, _c_i64, ctypes.POINTER(_c_size), ctypes.POINTER(_c_size),
                                 ctypes.POINTER(_c_size)]),
    "qlora_quantize_workspace_bytes": (_c_size, [_c_i64, _c_i64]),
    "qlora_quantize_nf4_dq": (_c_int, [_vp, _W, _vp, _c_size, _vp]),
    "qlora_dequant_bf16": (_c_int, [_W, _vp, _vp]),
    "qlora_linear_workspace_bytes": (_c_size, [_c_i64, _c_i64, _c_i64, _c_int]),
    "qlora_linear_fwd": (_c_int, [_W, _vp, _c_i64, _vp, _vp, _c_int, _c_float, _vp, _vp, _vp, _c_size, _vp]),
    "qlora_linear_bwd": (_c_int, [_W, _vp, _vp, _c_i64, _vp, _vp, _c_int, _c_float, _vp, _vp, _vp, _vp, _vp,
                                  _c_size, _vp]),
    "qlora_nf4_codebook": (None, [ctypes.POINTER(ctypes.c_float)]),
    "qlora_nf4_thresholds": (None, [ctypes.POINTER(ctypes.c_float)]),
    "qlora_codebook": (_c_int, [_c_int, ctypes.POINTER(ctypes.c_float)]),
    "qlora_merge_workspace_bytes": (_c_size, [_c_i64, _c_i64]),
    "qlora_swiglu_fwd": (_c_int, [_vp, _vp, _vp, _c_i64, _vp]),
    "qlora_attention_workspace_bytes": (_c_size, [_c_i64, _c_i64, _c_i64, _c_i64]),
    "qlora_attention_fwd": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64, _c_i64, _vp, _c_size, _vp]),
    "qlora_attention_bwd": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64, _c_i64,
                                     _vp, _c_size, _vp]),
    "qlora_swiglu_bwd": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_i64, _vp]),
    "qlora_add_bf16": (_c_int, [_vp, _vp, _vp, _c_i64, _vp]),
    "qlora_adamw_step": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_i64, _c_float, _c_float, _c_float, _c_float, _c_float,
                                  _c_i64, _vp]),
    "qlora_merge_adapters": (_c_int, [_W, _vp, _vp, _c_int, _c_float, _vp, _W, _vp, _c_size, _vp]),
    "qlora_thresholds": (_c_int, [_c_int, ctypes.POINTER(ctypes.c_float)]),
    "qlora_strerror": (ctypes.c_char_p, [_c_int]),
    "qlora_profile_begin": (_c_int, []),
    "qlora_profile_end": (_c_int, []),
    "qlora_profile_count": (_c_int, []),
    "qlora_profile_entry": (_c_int, [_c_int, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(_c_i64),
                                     ctypes.POINTER(ctypes.c_double)]),
    "qlora_last_error": (ctypes.c_char_p, []),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype, _f.argtypes = _res, _args


class QloraError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {qlora_strerror(status)} ({status}): {qlora_last_error()}")


def _check(fn: str, status: int) -> None:
    if status != QLORA_OK:
        raise QloraError(fn, status)


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libqlora must be contiguous")
    return _vp(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return _vp(s.cuda_stream)


def _need(t, dtype, name):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


@dataclass
class NF4Weight:
    """Device buffers of one quantized weight (torch tensors) and the C view.
    Double-quantized constants use scale_code / group_amax / offset;
    single-level ones (scales == QLORA_SCALES_FP32) use absmax only."""
    n: int
    k: int
    packed: torch.Tensor                     # uint8 [n*k/2]
    scale_code: torch.Tensor | None          # uint8 [n*k/64]
    group_amax: torch.Tensor | None          # float32 [ceil(n*k/64/256)]
    offset: torch.Tensor | None              # float32 [1]
    codebook: int = QLORA_CODEBOOK_NF4
    scales: int = QLORA_SCALES_DQ
    absmax: torch.Tensor | None = None       # float32 [n*k/64]

    @staticmethod
    def empty(n: int, k: int, device="cuda", codebook: int = QLORA_CODEBOOK_NF4,
              scales: int = QLORA_SCALES_DQ) -> "NF4Weight":
        pb, sb, ng = qlora_nf4_sizes(n, k)
        packed = torch.empty(pb, dtype=torch.uint8, device=device)
        if scales == QLORA_SCALES_FP32:
            return NF4Weight(n, k, packed, None, None, None, codebook, scales,
                             torch.empty(sb, dtype=torch.float32, device=device))
        return NF4Weight(n, k, packed, torch.empty(sb, dtype=torch.uint8, device=device),
                         torch.empty(ng, dtype=torch.float32, device=device),
                         torch.empty(1, dtype=torch.float32, device=device), codebook, scales)

    def c_struct(self) -> qlora_nf4_weight:
        p = lambda t: None if t is None else t.data_ptr()
        return qlora_nf4_weight(self.n, self.k, p(self.packed), p(self.scale_code), p(self.group_amax),
                                p(self.offset), self.codebook, self.scales, p(self.absmax))


def qlora_nf4_sizes(n: int, k: int):
    a, b, c = _c_size(), _c_size(), _c_size()
    _check("qlora_nf4_sizes", _lib.qlora_nf4_sizes(n, k, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return a.value, b.value, c.value


def qlora_quantize_workspace_bytes(n: int, k: int) -> int:
    return _lib.qlora_quantize_workspace_bytes(n, k)


def qlora_quantize_nf4_dq(W: torch.Tensor, out: NF4Weight, ws: torch.Tensor, stream=None) -> None:
    _need(W, torch.float32, "W")
    st = out.c_struct()
    _check("qlora_quantize_nf4_dq",
           _lib.qlora_quantize_nf4_dq(_ptr(W), ctypes.byref(st), _ptr(ws), ws.numel() * ws.element_size(),
                                      _stream(stream)))


def qlora_dequant_bf16(w: NF4Weight, W_bf16: torch.Tensor, stream=None) -> None:
    _need(W_bf16, torch.bfloat16, "W_bf16")
    st = w.c_struct()
    _check("qlora_dequant_bf16", _lib.qlora_dequant_bf16(ctypes.byref(st), _ptr(W_bf16), _stream(stream)))


def qlora_linear_workspace_bytes(M: int, n: int, k: int, r: int) -> int:
    return _lib.qlora_linear_workspace_bytes(M, n, k, r)


def _ws_args(ws):
    if ws is None:
        return None, 0
    return _ptr(ws), ws.numel() * ws.element_size()


def qlora_linear_fwd(w: NF4Weight, X: torch.Tensor, A: torch.Tensor, B: torch.Tensor, r: int, alpha: float,
                     Y: torch.Tensor, H_out: torch.Tensor | None, ws: torch.Tensor | None, stream=None) -> None:
    for t, nm in ((X, "X"), (A, "A"), (B, "B"), (Y, "Y")):
        _need(t, torch.bfloat16, nm)
    if H_out is not None:
        _need(H_out, torch.float32, "H_out")
    st = w.c_struct()
    wp, wb = _ws_args(ws)
    _check("qlora_linear_fwd",
           _lib.qlora_linear_fwd(ctypes.byref(st), _ptr(X), X.shape[0], _ptr(A), _ptr(B), r, alpha, _ptr(Y),
                                 _ptr(H_out), wp, wb, _stream(stream)))


def qlora_linear_bwd(w: NF4Weight, X: torch.Tensor, dY: torch.Tensor, A: torch.Tensor, B: torch.Tensor, r: int,
                     alpha: float, H: torch.Tensor | None, dX: torch.Tensor | None, dA: torch.Tensor,
                     dB: torch.Tensor, ws: torch.Tensor | None, stream=None) -> None:
    for t, nm in ((X, "X"), (dY, "dY"), (A, "A"), (B, "B"), (dA, "dA"), (dB, "dB")):
        _need(t, torch.bfloat16, nm)
    if dX is not None:
        _need(dX, torch.bfloat16, "dX")
    if H is not None:
        _need(H, torch.float32, "H")
    st = w.c_struct()
    wp, wb = _ws_args(ws)
    _check("qlora_linear_bwd",
           _lib.qlora_linear_bwd(ctypes.byref(st), _ptr(X), _ptr(dY), X.shape[0], _ptr(A), _ptr(B), r, alpha,
                                 _ptr(H), _ptr(dX), _ptr(dA), _ptr(dB), wp, wb, _stream(stream)))


def qlora_swiglu_fwd(gate: torch.Tensor, up: torch.Tensor, h: torch.Tensor, stream=None) -> None:
    for t, nm in ((gate, "gate"), (up, "up"), (h, "h")):
        _need(t, torch.bfloat16, nm)
    _check("qlora_swiglu_fwd", _lib.qlora_swiglu_fwd(_ptr(gate), _ptr(up), _ptr(h), gate.numel(), _stream(stream)))


def qlora_swiglu_bwd(gate: torch.Tensor, up: torch.Tensor, dh: torch.Tensor, d_gate: torch.Tensor,
                     d_up: torch.Tensor, stream=None) -> None:
    for t, nm in ((gate, "gate"), (up, "up"), (dh, "dh"), (d_gate, "d_gate"), (d_up, "d_up")):
        _need(t, torch.bfloat16, nm)
    _check("qlora_swiglu_bwd", _lib.qlora_swiglu_bwd(_ptr(gate), _ptr(up), _ptr(dh), _ptr(d_gate), _ptr(d_up),
                                                     gate.numel(), _stream(stream)))


def qlora_add_bf16(a: torch.Tensor, b: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    for t, nm in ((a, "a"), (b, "b"), (out, "out")):
        _need(t, torch.bfloat16, nm)
    _check("qlora_add_bf16", _lib.qlora_add_bf16(_ptr(a), _ptr(b), _ptr(out), a.numel(), _stream(stream)))


def qlora_attention_workspace_bytes(batch: int, seq: int, heads: int, head_dim: int) -> int:
    return _lib.qlora_attention_workspace_bytes(batch, seq, heads, head_dim)


def qlora_attention_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
                        batch: int, seq: int, heads: int, head_dim: int, ws: torch.Tensor, stream=None) -> None:
    """q, k, v, o: bf16 [batch*seq, heads*head_dim]; lse: float32 [batch, heads, seq]."""
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _need(t, torch.bfloat16, nm)
    _need(lse, torch.float32, "lse")
    w, wb = _ws_args(ws)
    _check("qlora_attention_fwd",
           _lib.qlora_attention_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), batch, seq, heads, head_dim, w, wb,
                                    _stream(stream)))


def qlora_attention_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, d_o: torch.Tensor, lse: torch.Tensor,
                        dq: torch.Tensor, dk: torch.Tensor, dv: torch.Tensor, batch: int, seq: int,
                        heads: int, head_dim: int, ws: torch.Tensor, stream=None) -> None:
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (d_o, "d_o"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _need(t, torch.bfloat16, nm)
    _need(lse, torch.float32, "lse")
    w, wb = _ws_args(ws)
    _check("qlora_attention_bwd",
           _lib.qlora_attention_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(d_o), _ptr(lse), _ptr(dq), _ptr(dk),
                                    _ptr(dv), batch, seq, heads, head_dim, w, wb, _stream(stream)))


def qlora_adamw_step(param: torch.Tensor, param_bf16: torch.Tensor | None, grad: torch.Tensor, m, v, lr: float,
                     beta1: float, beta2: float, eps: float, weight_decay: float, step: int, stream=None) -> None:
    """m and v: device tensors, or (paged layout) integer device addresses of
    mapped host memory, as ints."""
    _need(param, torch.float32, "param")
    _need(grad, torch.bfloat16, "grad")
    if param_bf16 is not None:
        _need(param_bf16, torch.bfloat16, "param_bf16")
    mp = _vp(m) if isinstance(m, int) else _ptr(m)
    vp = _vp(v) if isinstance(v, int) else _ptr(v)
    _check("qlora_adamw_step",
           _lib.qlora_adamw_step(_ptr(param), _ptr(param_bf16), _ptr(grad), mp, vp, param.numel(), lr, beta1, beta2,
                                 eps, weight_decay, step, _stream(stream)))


def qlora_merge_workspace_bytes(n: int, k: int) -> int:
    return _lib.qlora_merge_workspace_bytes(n, k)


def qlora_merge_adapters(w: NF4Weight, A: torch.Tensor, B: torch.Tensor, r: int, alpha: float,
                         W_merged: torch.Tensor | None, out: NF4Weight | None, ws: torch.Tensor, stream=None) -> None:
    for t, nm in ((A, "A"), (B, "B")):
        _need(t, torch.bfloat16, nm)
    if W_merged is not None:
        _need(W_merged, torch.bfloat16, "W_merged")
    st = w.c_struct()
    ost = out.c_struct() if out is not None else None
    wp, wb = _ws_args(ws)
    _check("qlora_merge_adapters",
           _lib.qlora_merge_adapters(ctypes.byref(st), _ptr(A), _ptr(B), r, alpha, _ptr(W_merged),
                                     ctypes.byref(ost) if ost is not None else None, wp, wb, _stream(stream)))


def qlora_nf4_codebook():
    buf = (ctypes.c_float * 16)()
    _lib.qlora_nf4_codebook(buf)
    return list(buf)


def qlora_nf4_thresholds():
    buf = (ctypes.c_float * 15)()
    _lib.qlora_nf4_thresholds(buf)
    return list(buf)


def qlora_codebook(codebook: int):
    buf = (ctypes.c_float * 16)()
    _check("qlora_codebook", _lib.qlora_codebook(codebook, buf))
    return list(buf)


def qlora_thresholds(codebook: int):
    buf = (ctypes.c_float * 15)()
    _check("qlora_thresholds", _lib.qlora_thresholds(codebook, buf))
    return list(buf)


def qlora_strerror(status: int) -> str:
    return _lib.qlora_strerror(status).decode()


def qlora_last_error() -> str:
    return _lib.qlora_last_error().decode()


def qlora_profile_begin() -> None:
    _check("qlora_profile_begin", _lib.qlora_profile_begin())


def qlora_profile_end() -> dict:
    """Stop per-kernel event timing; {kernel name: (launches, total ms)}."""
    _check("qlora_profile_end", _lib.qlora_profile_end())
    out = {}
    for i in range(_lib.qlora_profile_count()):
        name, n, ms = ctypes.c_char_p(), _c_i64(), ctypes.c_double()
        _check("qlora_profile_entry", _lib.qlora_profile_entry(i, ctypes.byref(name), ctypes.byref(n),
                                                               ctypes.byref(ms)))
        out[name.value.decode()] = (n.value, ms.value)
    return out


def raw_library() -> ctypes.CDLL:
    """The loaded ctypes library (used by the symbol-export check)."""
    return _lib
