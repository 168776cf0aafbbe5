"""ctypes binding of libqlora.so: the calls of ``include/qlora.h`` under the
same names.  Argument marshalling only -- every step of the layer runs in
the library's HIP kernels.  torch supplies device memory and the stream.

Each wrapper checks, before the library is called, that every tensor is a
contiguous device tensor of the dtype and shape the call reads or writes
(ValueError / TypeError otherwise), so a mismatch never reaches a kernel as
an out-of-bounds pointer.  A weight in the method's storage type (NF4 codes,
double-quantized constants) goes through the plain calls with the six-field
descriptor; the comparison storage types go through the ``*_ex`` calls.

Importing this module loads ``libqlora.so`` and raises ImportError if it has
not been built (``python -m bit_nf4_quantized_qlora_amd.build``); there is no
fallback path.  ``use_tracing_library(True)`` switches every call to the
tracing build ``libqlora_prof.so`` (same kernels plus the per-kernel event
timer of the ``qlora_profile_*`` calls).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

# torch first: its HIP runtime (same soname as ROCm's) is then the one the
# library binds to, so torch's streams and allocations are valid handles here.
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqlora.so")
PROF_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqlora_prof.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run `python -m bit_nf4_quantized_qlora_amd.build`")
_product = ctypes.CDLL(LIB_PATH)
_tracing = None
_lib = _product

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
QLORA_CODEBOOK_FP4_E2M1 = 1   # Float4 (E2M1), a comparison type
QLORA_CODEBOOK_FP4_E3M0 = 2   # Float4 (E3M0), the other comparison type
CODEBOOKS = {"nf4": QLORA_CODEBOOK_NF4, "fp4": QLORA_CODEBOOK_FP4_E2M1, "fp4_e3m0": QLORA_CODEBOOK_FP4_E3M0}
QLORA_SCALES_DQ = 0           # double-quantized block constants (the method's)
QLORA_SCALES_FP32 = 1         # one float32 absmax per block (double quantization off)

_c_i64, _c_int, _c_float, _c_size, _vp = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p


QLORA_PATH_NONE, QLORA_PATH_TILE, QLORA_PATH_GEMV, QLORA_PATH_GENERAL = 0, 1, 2, 3


class qlora_nf4_weight(ctypes.Structure):
    _fields_ = [("n", _c_i64), ("k", _c_i64), ("packed", _vp), ("scale_code", _vp), ("group_amax", _vp),
                ("offset", _vp)]


class qlora_weight_ex(ctypes.Structure):
    _fields_ = [("size", _c_size), ("base", qlora_nf4_weight), ("codebook", ctypes.c_int32),
                ("scales", ctypes.c_int32), ("absmax", _vp)]


class qlora_linear_plan_info(ctypes.Structure):
    _fields_ = [("fwd_path", ctypes.c_int32), ("fwd_splits", ctypes.c_int32), ("dx_path", ctypes.c_int32),
                ("dx_splits", ctypes.c_int32)]


_W = ctypes.POINTER(qlora_nf4_weight)
_WX = ctypes.POINTER(qlora_weight_ex)
_SIGS = {
    "qlora_nf4_sizes": (_c_int, [_c_i64, _c_i64, ctypes.POINTER(_c_size), ctypes.POINTER(_c_size),
                                 ctypes.POINTER(_c_size)]),
    "qlora_quantize_workspace_bytes": (_c_size, [_c_i64, _c_i64]),
    "qlora_quantize_nf4_dq": (_c_int, [_vp, _W, _vp, _c_size, _vp]),
    "qlora_quantize_ex": (_c_int, [_vp, _WX, _vp, _c_size, _vp]),
    "qlora_dequant_bf16": (_c_int, [_W, _vp, _vp]),
    "qlora_dequant_bf16_ex": (_c_int, [_WX, _vp, _vp]),
    "qlora_linear_workspace_bytes": (_c_size, [_c_i64, _c_i64, _c_i64, _c_int]),
    "qlora_linear_fwd": (_c_int, [_W, _vp, _c_i64, _vp, _vp, _c_int, _c_float, _vp, _vp, _vp, _c_size, _vp]),
    "qlora_linear_bwd": (_c_int, [_W, _vp, _vp, _c_i64, _vp, _vp, _c_int, _c_float, _vp, _vp, _vp, _vp, _vp,
                                  _c_size, _vp]),
    "qlora_linear_fwd_ex": (_c_int, [_WX, _vp, _c_i64, _vp, _vp, _c_int, _c_float, _vp, _vp, _vp, _c_size, _vp]),
    "qlora_linear_bwd_ex": (_c_int, [_WX, _vp, _vp, _c_i64, _vp, _vp, _c_int, _c_float, _vp, _vp, _vp, _vp, _vp,
                                     _c_size, _vp]),
    "qlora_linear_fwd_noalloc": (_c_int, [_W, _vp, _c_i64, _vp, _vp, _c_int, _c_float, _vp, _vp, _vp]),
    "qlora_linear_plan": (_c_int, [_c_i64, _c_i64, _c_i64, _c_int, ctypes.c_int32,
                                   ctypes.POINTER(qlora_linear_plan_info)]),
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
    "qlora_add_bf16_n": (_c_int, [ctypes.POINTER(_vp), _c_int, _vp, _c_i64, _vp]),
    "qlora_adamw_step": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_i64, _c_float, _c_float, _c_float, _c_float, _c_float,
                                  _c_i64, _vp]),
    "qlora_merge_adapters": (_c_int, [_WX, _vp, _vp, _c_int, _c_float, _vp, _WX, _vp, _c_size, _vp]),
    "qlora_thresholds": (_c_int, [_c_int, ctypes.POINTER(ctypes.c_float)]),
    "qlora_strerror": (ctypes.c_char_p, [_c_int]),
    "qlora_last_error": (ctypes.c_char_p, []),
}
_PROF_SIGS = {
    "qlora_profile_begin": (_c_int, []),
    "qlora_profile_end": (_c_int, []),
    "qlora_profile_count": (_c_int, []),
    "qlora_profile_entry": (_c_int, [_c_int, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(_c_i64),
                                     ctypes.POINTER(ctypes.c_double)]),
    "qlora_profile_mfma_peak": (_c_int, [_c_i64, ctypes.c_int32, _vp, ctypes.POINTER(ctypes.c_double), _vp]),
    "qlora_profile_linear_fwd_bf16w": (_c_int, [_vp, _c_i64, _c_i64, _vp, _c_i64, _vp, _vp, _c_int, _c_float, _vp,
                                                _vp, _vp, _c_size, _vp]),
}


def _declare(lib, sigs):
    for name, (res, args) in sigs.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args


_declare(_product, _SIGS)


def use_tracing_library(on: bool) -> None:
    """Route every call to libqlora_prof.so (on) or back to libqlora.so."""
    global _lib, _tracing
    if on and _tracing is None:
        if not os.path.exists(PROF_LIB_PATH):
            raise ImportError(f"{PROF_LIB_PATH} is not built")
        _tracing = ctypes.CDLL(PROF_LIB_PATH)
        _declare(_tracing, _SIGS)
        _declare(_tracing, _PROF_SIGS)
    _lib = _tracing if on else _product


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


def _need(t, dtype, name, shape=None, numel=None):
    """dtype, shape (or element count) and contiguity of one tensor the
    library will read or write, checked before any call; the device is
    checked by _on_gpu once every shape has passed."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, the call needs {tuple(shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, the call needs {numel}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_gpu(**tensors):
    for name, t in tensors.items():
        if isinstance(t, torch.Tensor) and t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor, got device {t.device}")


@dataclass
class NF4Weight:
    """Device buffers of one quantized weight (torch tensors) and its C
    descriptors.  Double-quantized constants use scale_code / group_amax /
    offset; single-level ones (scales == QLORA_SCALES_FP32) use absmax only."""
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

    @property
    def is_method_type(self) -> bool:
        """NF4 codes with double-quantized constants: the plain calls' type."""
        return self.codebook == QLORA_CODEBOOK_NF4 and self.scales == QLORA_SCALES_DQ

    def buffers(self) -> dict:
        return {"packed": self.packed, "scale_code": self.scale_code, "group_amax": self.group_amax,
                "offset": self.offset, "absmax": self.absmax}

    def check_buffers(self) -> None:
        """Element counts and dtypes of the buffers the calls read (device: _on_gpu)."""
        pb, sb, ng = qlora_nf4_sizes(self.n, self.k)
        _need(self.packed, torch.uint8, "packed", numel=pb)
        if self.scales == QLORA_SCALES_FP32:
            _need(self.absmax, torch.float32, "absmax", numel=sb)
        else:
            _need(self.scale_code, torch.uint8, "scale_code", numel=sb)
            _need(self.group_amax, torch.float32, "group_amax", numel=ng)
            _need(self.offset, torch.float32, "offset", numel=1)

    def c_struct(self) -> qlora_nf4_weight:
        p = lambda t: None if t is None else t.data_ptr()
        return qlora_nf4_weight(self.n, self.k, p(self.packed), p(self.scale_code), p(self.group_amax),
                                p(self.offset))

    def c_ex(self) -> qlora_weight_ex:
        p = lambda t: None if t is None else t.data_ptr()
        return qlora_weight_ex(ctypes.sizeof(qlora_weight_ex), self.c_struct(), self.codebook, self.scales,
                               p(self.absmax))


def qlora_nf4_sizes(n: int, k: int):
    a, b, c = _c_size(), _c_size(), _c_size()
    _check("qlora_nf4_sizes", _lib.qlora_nf4_sizes(n, k, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return a.value, b.value, c.value


def qlora_quantize_workspace_bytes(n: int, k: int) -> int:
    return _lib.qlora_quantize_workspace_bytes(n, k)


def _ws_args(ws):
    if ws is None:
        return None, 0
    _need(ws, torch.uint8, "ws")
    _on_gpu(ws=ws)
    return _ptr(ws), ws.numel()


def qlora_quantize_nf4_dq(W: torch.Tensor, out: NF4Weight, ws: torch.Tensor, stream=None) -> None:
    """Quantize W [n, k] float32 into `out` (any storage type: the _ex call
    when it is not NF4 with double-quantized constants)."""
    _need(W, torch.float32, "W", shape=(out.n, out.k))
    out.check_buffers()
    _on_gpu(W=W, **out.buffers())
    wp, wb = _ws_args(ws)
    if out.is_method_type:
        st = out.c_struct()
        _check("qlora_quantize_nf4_dq", _lib.qlora_quantize_nf4_dq(_ptr(W), ctypes.byref(st), wp, wb, _stream(stream)))
    else:
        st = out.c_ex()
        _check("qlora_quantize_ex", _lib.qlora_quantize_ex(_ptr(W), ctypes.byref(st), wp, wb, _stream(stream)))


def qlora_dequant_bf16(w: NF4Weight, W_bf16: torch.Tensor, stream=None) -> None:
    _need(W_bf16, torch.bfloat16, "W_bf16", numel=w.n * w.k)
    w.check_buffers()
    _on_gpu(W_bf16=W_bf16, **w.buffers())
    if w.is_method_type:
        st = w.c_struct()
        _check("qlora_dequant_bf16", _lib.qlora_dequant_bf16(ctypes.byref(st), _ptr(W_bf16), _stream(stream)))
    else:
        st = w.c_ex()
        _check("qlora_dequant_bf16_ex", _lib.qlora_dequant_bf16_ex(ctypes.byref(st), _ptr(W_bf16), _stream(stream)))


def qlora_linear_workspace_bytes(M: int, n: int, k: int, r: int) -> int:
    return _lib.qlora_linear_workspace_bytes(M, n, k, r)


def qlora_linear_plan(M: int, n: int, k: int, r: int, scales: int = QLORA_SCALES_DQ) -> dict:
    """The kernels a call of this shape runs (host only)."""
    info = qlora_linear_plan_info()
    _check("qlora_linear_plan", _lib.qlora_linear_plan(M, n, k, r, scales, ctypes.byref(info)))
    return {"fwd_path": info.fwd_path, "fwd_splits": info.fwd_splits, "dx_path": info.dx_path,
            "dx_splits": info.dx_splits}


def qlora_linear_fwd(w: NF4Weight, X: torch.Tensor, A: torch.Tensor, B: torch.Tensor, r: int, alpha: float,
                     Y: torch.Tensor, H_out: torch.Tensor | None, ws: torch.Tensor | None, stream=None) -> None:
    if X.dim() != 2:
        raise ValueError(f"X must be [M, {w.k}], got shape {tuple(X.shape)}")
    M = X.shape[0]
    _need(X, torch.bfloat16, "X", shape=(M, w.k))
    _need(A, torch.bfloat16, "A", shape=(r, w.k))
    _need(B, torch.bfloat16, "B", shape=(w.n, r))
    _need(Y, torch.bfloat16, "Y", shape=(M, w.n))
    if H_out is not None:
        _need(H_out, torch.float32, "H_out", shape=(M, r))
    w.check_buffers()
    _on_gpu(X=X, A=A, B=B, Y=Y, H_out=H_out, **w.buffers())
    wp, wb = _ws_args(ws)
    if w.is_method_type:
        st, fn, name = w.c_struct(), _lib.qlora_linear_fwd, "qlora_linear_fwd"
    else:
        st, fn, name = w.c_ex(), _lib.qlora_linear_fwd_ex, "qlora_linear_fwd_ex"
    _check(name, fn(ctypes.byref(st), _ptr(X), M, _ptr(A), _ptr(B), r, alpha, _ptr(Y), _ptr(H_out), wp, wb,
                    _stream(stream)))


def qlora_linear_fwd_noalloc(w: NF4Weight, X: torch.Tensor, A: torch.Tensor, B: torch.Tensor, r: int, alpha: float,
                             Y: torch.Tensor, H_out: torch.Tensor | None, stream=None) -> None:
    """qlora_linear_fwd on the library's fixed device scratch (no workspace;
    NF4 weights with double-quantized constants)."""
    if not w.is_method_type:
        raise ValueError("qlora_linear_fwd_noalloc takes NF4 weights with double-quantized constants")
    if X.dim() != 2:
        raise ValueError(f"X must be [M, {w.k}], got shape {tuple(X.shape)}")
    M = X.shape[0]
    _need(X, torch.bfloat16, "X", shape=(M, w.k))
    _need(A, torch.bfloat16, "A", shape=(r, w.k))
    _need(B, torch.bfloat16, "B", shape=(w.n, r))
    _need(Y, torch.bfloat16, "Y", shape=(M, w.n))
    if H_out is not None:
        _need(H_out, torch.float32, "H_out", shape=(M, r))
    w.check_buffers()
    _on_gpu(X=X, A=A, B=B, Y=Y, H_out=H_out, **w.buffers())
    st = w.c_struct()
    _check("qlora_linear_fwd_noalloc",
           _lib.qlora_linear_fwd_noalloc(ctypes.byref(st), _ptr(X), M, _ptr(A), _ptr(B), r, alpha, _ptr(Y),
                                         _ptr(H_out), _stream(stream)))


def qlora_linear_bwd(w: NF4Weight, X: torch.Tensor, dY: torch.Tensor, A: torch.Tensor, B: torch.Tensor, r: int,
                     alpha: float, H: torch.Tensor | None, dX: torch.Tensor | None, dA: torch.Tensor,
                     dB: torch.Tensor, ws: torch.Tensor | None, stream=None) -> None:
    if X.dim() != 2:
        raise ValueError(f"X must be [M, {w.k}], got shape {tuple(X.shape)}")
    M = X.shape[0]
    _need(X, torch.bfloat16, "X", shape=(M, w.k))
    _need(dY, torch.bfloat16, "dY", shape=(M, w.n))
    _need(A, torch.bfloat16, "A", shape=(r, w.k))
    _need(B, torch.bfloat16, "B", shape=(w.n, r))
    _need(dA, torch.bfloat16, "dA", shape=(r, w.k))
    _need(dB, torch.bfloat16, "dB", shape=(w.n, r))
    if dX is not None:
        _need(dX, torch.bfloat16, "dX", shape=(M, w.k))
    if H is not None:
        _need(H, torch.float32, "H", shape=(M, r))
    w.check_buffers()
    _on_gpu(X=X, dY=dY, A=A, B=B, dA=dA, dB=dB, dX=dX, H=H, **w.buffers())
    wp, wb = _ws_args(ws)
    if w.is_method_type:
        st, fn, name = w.c_struct(), _lib.qlora_linear_bwd, "qlora_linear_bwd"
    else:
        st, fn, name = w.c_ex(), _lib.qlora_linear_bwd_ex, "qlora_linear_bwd_ex"
    _check(name, fn(ctypes.byref(st), _ptr(X), _ptr(dY), M, _ptr(A), _ptr(B), r, alpha, _ptr(H), _ptr(dX),
                    _ptr(dA), _ptr(dB), wp, wb, _stream(stream)))


def _same_numel(name0, t0, *others):
    for t, nm in others:
        _need(t, torch.bfloat16, nm, numel=t0.numel())
    _on_gpu(**{name0: t0}, **{nm: t for t, nm in others})


def qlora_swiglu_fwd(gate: torch.Tensor, up: torch.Tensor, h: torch.Tensor, stream=None) -> None:
    _need(gate, torch.bfloat16, "gate")
    _same_numel("gate", gate, (up, "up"), (h, "h"))
    _check("qlora_swiglu_fwd", _lib.qlora_swiglu_fwd(_ptr(gate), _ptr(up), _ptr(h), gate.numel(), _stream(stream)))


def qlora_swiglu_bwd(gate: torch.Tensor, up: torch.Tensor, dh: torch.Tensor, d_gate: torch.Tensor,
                     d_up: torch.Tensor, stream=None) -> None:
    _need(gate, torch.bfloat16, "gate")
    _same_numel("gate", gate, (up, "up"), (dh, "dh"), (d_gate, "d_gate"), (d_up, "d_up"))
    _check("qlora_swiglu_bwd", _lib.qlora_swiglu_bwd(_ptr(gate), _ptr(up), _ptr(dh), _ptr(d_gate), _ptr(d_up),
                                                     gate.numel(), _stream(stream)))


def qlora_add_bf16(a: torch.Tensor, b: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    _need(a, torch.bfloat16, "a")
    _same_numel("a", a, (b, "b"), (out, "out"))
    _check("qlora_add_bf16", _lib.qlora_add_bf16(_ptr(a), _ptr(b), _ptr(out), a.numel(), _stream(stream)))


def qlora_add_bf16_n(xs, out: torch.Tensor, stream=None) -> None:
    """out = the left-to-right bf16-rounded sum of the 2..4 tensors in xs."""
    for i, t in enumerate(xs):
        _need(t, torch.bfloat16, f"xs[{i}]")
    _need(out, torch.bfloat16, "out")
    _same_numel("xs[0]", xs[0], *[(t, f"xs[{i}]") for i, t in enumerate(xs) if i > 0], (out, "out"))
    ptrs = (_vp * len(xs))(*[_ptr(t) for t in xs])
    _check("qlora_add_bf16_n", _lib.qlora_add_bf16_n(ptrs, len(xs), _ptr(out), out.numel(), _stream(stream)))


def qlora_attention_workspace_bytes(batch: int, seq: int, heads: int, head_dim: int) -> int:
    return _lib.qlora_attention_workspace_bytes(batch, seq, heads, head_dim)


def qlora_attention_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
                        batch: int, seq: int, heads: int, head_dim: int, ws: torch.Tensor, stream=None) -> None:
    """q, k, v, o: bf16 [batch*seq, heads*head_dim]; lse: float32 [batch, heads, seq]."""
    shape = (batch * seq, heads * head_dim)
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _need(t, torch.bfloat16, nm, shape=shape)
    _need(lse, torch.float32, "lse", numel=batch * heads * seq)
    _on_gpu(q=q, k=k, v=v, o=o, lse=lse)
    w, wb = _ws_args(ws)
    _check("qlora_attention_fwd",
           _lib.qlora_attention_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), batch, seq, heads, head_dim, w, wb,
                                    _stream(stream)))


def qlora_attention_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, d_o: torch.Tensor, lse: torch.Tensor,
                        dq: torch.Tensor, dk: torch.Tensor, dv: torch.Tensor, batch: int, seq: int,
                        heads: int, head_dim: int, ws: torch.Tensor, stream=None) -> None:
    shape = (batch * seq, heads * head_dim)
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (d_o, "d_o"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _need(t, torch.bfloat16, nm, shape=shape)
    _need(lse, torch.float32, "lse", numel=batch * heads * seq)
    _on_gpu(q=q, k=k, v=v, d_o=d_o, lse=lse, dq=dq, dk=dk, dv=dv)
    w, wb = _ws_args(ws)
    _check("qlora_attention_bwd",
           _lib.qlora_attention_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(d_o), _ptr(lse), _ptr(dq), _ptr(dk),
                                    _ptr(dv), batch, seq, heads, head_dim, w, wb, _stream(stream)))


def qlora_adamw_step(param: torch.Tensor, param_bf16: torch.Tensor | None, grad: torch.Tensor, m, v, lr: float,
                     beta1: float, beta2: float, eps: float, weight_decay: float, step: int, stream=None) -> None:
    """m and v: device tensors, or (paged layout) integer device addresses of
    mapped host memory holding param.numel() float32 values each."""
    _need(param, torch.float32, "param")
    count = param.numel()
    _need(grad, torch.bfloat16, "grad", numel=count)
    if param_bf16 is not None:
        _need(param_bf16, torch.bfloat16, "param_bf16", numel=count)
    for t, nm in ((m, "m"), (v, "v")):
        if not isinstance(t, int):
            _need(t, torch.float32, nm, numel=count)
    _on_gpu(param=param, grad=grad, param_bf16=param_bf16, m=m, v=v)
    mp = _vp(m) if isinstance(m, int) else _ptr(m)
    vp = _vp(v) if isinstance(v, int) else _ptr(v)
    _check("qlora_adamw_step",
           _lib.qlora_adamw_step(_ptr(param), _ptr(param_bf16), _ptr(grad), mp, vp, count, lr, beta1, beta2,
                                 eps, weight_decay, step, _stream(stream)))


def qlora_merge_workspace_bytes(n: int, k: int) -> int:
    return _lib.qlora_merge_workspace_bytes(n, k)


def qlora_merge_adapters(w: NF4Weight, A: torch.Tensor, B: torch.Tensor, r: int, alpha: float,
                         W_merged: torch.Tensor | None, out: NF4Weight | None, ws: torch.Tensor, stream=None) -> None:
    _need(A, torch.bfloat16, "A", shape=(r, w.k))
    _need(B, torch.bfloat16, "B", shape=(w.n, r))
    if W_merged is not None:
        _need(W_merged, torch.bfloat16, "W_merged", numel=w.n * w.k)
    w.check_buffers()
    if out is not None:
        if (out.n, out.k) != (w.n, w.k):
            raise ValueError(f"out is [{out.n}, {out.k}], the weight is [{w.n}, {w.k}]")
        out.check_buffers()
        _on_gpu(**{"out_" + k: v for k, v in out.buffers().items()})
    _on_gpu(A=A, B=B, W_merged=W_merged, **w.buffers())
    st = w.c_ex()
    ost = out.c_ex() if out is not None else None
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
    """Start the per-kernel event timer (tracing library only)."""
    if _lib is not _tracing:
        raise RuntimeError("the event timer lives in libqlora_prof.so: call use_tracing_library(True) first")
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


def qlora_profile_linear_fwd_bf16w(W_bf16: torch.Tensor, X: torch.Tensor, A: torch.Tensor, B: torch.Tensor, r: int,
                                   alpha: float, Y: torch.Tensor, H_out: torch.Tensor | None, ws: torch.Tensor,
                                   stream=None) -> None:
    """The forward on BF16 weights [n, k] through the same tile kernel
    (tracing library: call use_tracing_library(True) first)."""
    if _lib is not _tracing:
        raise RuntimeError("qlora_profile_linear_fwd_bf16w lives in libqlora_prof.so: call use_tracing_library(True)")
    if W_bf16.dim() != 2 or X.dim() != 2:
        raise ValueError("W_bf16 and X must be 2-D")
    n, k = W_bf16.shape
    M = X.shape[0]
    _need(W_bf16, torch.bfloat16, "W_bf16", shape=(n, k))
    _need(X, torch.bfloat16, "X", shape=(M, k))
    _need(A, torch.bfloat16, "A", shape=(r, k))
    _need(B, torch.bfloat16, "B", shape=(n, r))
    _need(Y, torch.bfloat16, "Y", shape=(M, n))
    if H_out is not None:
        _need(H_out, torch.float32, "H_out", shape=(M, r))
    _on_gpu(W_bf16=W_bf16, X=X, A=A, B=B, Y=Y, H_out=H_out)
    wp, wb = _ws_args(ws)
    _check("qlora_profile_linear_fwd_bf16w",
           _lib.qlora_profile_linear_fwd_bf16w(_ptr(W_bf16), n, k, _ptr(X), M, _ptr(A), _ptr(B), r, alpha, _ptr(Y),
                                               _ptr(H_out), wp, wb, _stream(stream)))


def mfma_peak_tflops(iters: int = 20000, workgroups: int = 512, reps: int = 5) -> float:
    """The attainable BF16 MFMA rate (TFLOP/s): the tracing library's
    back-to-back v_mfma_f32_16x16x32_bf16 kernel, timed with events on the
    current stream; the fastest of `reps` launches after one warm-up."""
    use_tracing_library(True)
    try:
        out = torch.empty(workgroups * 256, dtype=torch.float32, device="cuda")
        flops = ctypes.c_double()
        st = _stream(None)
        best = float("inf")
        for i in range(reps + 1):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            _check("qlora_profile_mfma_peak", _lib.qlora_profile_mfma_peak(iters, workgroups, _ptr(out),
                                                                          ctypes.byref(flops), st))
            b.record()
            torch.cuda.synchronize()
            if i:
                best = min(best, a.elapsed_time(b))
        return flops.value / (best * 1e-3) / 1e12
    finally:
        use_tracing_library(False)


def raw_library() -> ctypes.CDLL:
    """The product library (used by the symbol-export check)."""
    return _product
