"""Host-side checks of libqlora.so (no GPU needed, no kernel launched):
every function include/qlora.h declares is exported; the library's NF4
table and decision thresholds equal the oracle's construction; argument
checks reject bad calls before anything is enqueued.
"""
import ctypes
import os
import re
from fractions import Fraction

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]
LIB = os.path.join(ROOT, "bit_nf4_quantized_qlora_amd", "libqlora.so")


def _ensure_built():
    if not os.path.exists(LIB):
        from bit_nf4_quantized_qlora_amd import build
        build.build()


@pytest.fixture(scope="module")
def q():
    _ensure_built()
    from bit_nf4_quantized_qlora_amd import qlora
    return qlora


def _declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qlora_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = _declared_functions()
    for n in ("qlora_quantize_nf4_dq", "qlora_dequant_bf16", "qlora_linear_fwd", "qlora_linear_bwd"):
        assert n in names


def test_every_declared_symbol_is_exported(q):
    lib = q.raw_library()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    # and nothing C++-mangled leaks under a qlora_ name
    out = os.popen(f"nm -D --defined-only {LIB}").read()
    exported = set(re.findall(r"\bT (qlora_\w+)", out))
    assert exported == set(_declared_functions())


def test_library_codebook_equals_oracle(q):
    from oracle import nf4_dq
    lib = np.array(q.qlora_nf4_codebook(), np.float32)
    assert np.array_equal(lib.view(np.uint32), nf4_dq.nf4_codebook().view(np.uint32))
    for name, cb in q.CODEBOOKS.items():
        lib = np.array(q.qlora_codebook(cb), np.float32)
        assert np.array_equal(lib.view(np.uint32), nf4_dq.codebook_levels(name).view(np.uint32)), name
    assert q.qlora_thresholds(q.QLORA_CODEBOOK_NF4) == q.qlora_nf4_thresholds()
    for bad in (-1, 2, 7):
        with pytest.raises(q.QloraError) as e:
            q.qlora_codebook(bad)
        assert e.value.status == q.QLORA_ERR_BAD_CODEBOOK


@pytest.mark.parametrize("name", ["nf4", "fp4"])
def test_library_thresholds_are_the_exact_midpoint_successors(q, name):
    from oracle import nf4_dq
    levels = nf4_dq.codebook_levels(name)
    t = np.array(q.qlora_thresholds(q.CODEBOOKS[name]), np.float32)
    for j in range(15):
        mid = (Fraction(float(levels[j])) + Fraction(float(levels[j + 1]))) / 2
        assert Fraction(float(t[j])) > mid
        below = np.nextafter(t[j], np.float32(-np.inf), dtype=np.float32)
        assert Fraction(float(below)) <= mid
    # the threshold count reproduces the oracle's nearest level everywhere near them
    xs = np.concatenate([t, np.nextafter(t, np.float32(-np.inf), dtype=np.float32),
                         np.random.default_rng(0).uniform(-1, 1, 20000).astype(np.float32)])
    xs = xs[np.abs(xs) <= 1]  # normalized weights; Float4's top threshold lies just above 1
    via_t = (xs[:, None] >= t[None, :]).sum(axis=1)
    assert np.array_equal(via_t, nf4_dq.nearest_level(xs, levels))


def test_sizes_and_bits(q):
    for n, k in ((256, 256), (4096, 4096), (11008, 4096), (8192, 22016), (3, 64)):
        pb, sb, ng = q.qlora_nf4_sizes(n, k)
        assert pb == n * k // 2 and sb == n * k // 64 and ng == -(-sb // 256)
        if sb % 256 == 0:
            assert 8 * (pb + sb + 4 * ng) / (n * k) == 4.126953125
    with pytest.raises(q.QloraError) as e:
        q.qlora_nf4_sizes(10, 100)
    assert e.value.status == q.QLORA_ERR_BAD_SHAPE


def test_workspace_queries(q):
    assert q.qlora_quantize_workspace_bytes(4096, 4096) >= 4096 * 4096 // 64 * 4
    assert q.qlora_quantize_workspace_bytes(4096, 100) == 0
    assert q.qlora_linear_workspace_bytes(512, 4096, 4096, 64) > 0
    assert q.qlora_linear_workspace_bytes(512, 4096, 4096, 0) == 0
    assert q.qlora_linear_workspace_bytes(512, 4096, 4096, 129) == 0
    assert q.qlora_linear_workspace_bytes(0, 4096, 4096, 64) == 0


def test_argument_errors_enqueue_nothing(q):
    lib = q.raw_library()
    W = q.qlora_nf4_weight(64, 64, 16, 16, 16, 16)          # fake but aligned, never dereferenced
    bad_k = q.qlora_nf4_weight(64, 96, 16, 16, 16, 16)
    null_buf = q.qlora_nf4_weight(64, 64, 16, None, 16, 16)
    misaligned = q.qlora_nf4_weight(64, 64, 17, 16, 16, 16)
    P = ctypes.c_void_p(16)
    assert lib.qlora_quantize_nf4_dq(None, ctypes.byref(W), P, 1 << 20, None) == q.QLORA_ERR_NULL_ARG
    assert lib.qlora_quantize_nf4_dq(P, None, P, 1 << 20, None) == q.QLORA_ERR_NULL_ARG
    assert lib.qlora_quantize_nf4_dq(P, ctypes.byref(bad_k), P, 1 << 20, None) == q.QLORA_ERR_BAD_SHAPE
    assert lib.qlora_quantize_nf4_dq(P, ctypes.byref(W), P, 8, None) == q.QLORA_ERR_WORKSPACE
    assert lib.qlora_quantize_nf4_dq(P, ctypes.byref(W), None, 1 << 20, None) == q.QLORA_ERR_WORKSPACE
    assert lib.qlora_dequant_bf16(ctypes.byref(null_buf), P, None) == q.QLORA_ERR_NULL_ARG
    assert lib.qlora_dequant_bf16(ctypes.byref(misaligned), P, None) == q.QLORA_ERR_MISALIGNED
    assert lib.qlora_dequant_bf16(ctypes.byref(W), ctypes.c_void_p(18), None) == q.QLORA_ERR_MISALIGNED
    fwd = lib.qlora_linear_fwd
    assert fwd(ctypes.byref(W), P, 16, P, P, 0, 16.0, P, None, P, 1 << 30, None) == q.QLORA_ERR_BAD_RANK
    assert fwd(ctypes.byref(W), P, 16, P, P, 129, 16.0, P, None, P, 1 << 30, None) == q.QLORA_ERR_BAD_RANK
    assert fwd(ctypes.byref(W), P, -1, P, P, 8, 16.0, P, None, P, 1 << 30, None) == q.QLORA_ERR_BAD_SHAPE
    assert fwd(ctypes.byref(W), P, 16, P, P, 8, float("nan"), P, None, P, 1 << 30, None) == q.QLORA_ERR_BAD_ALPHA
    assert fwd(ctypes.byref(W), None, 16, P, P, 8, 16.0, P, None, P, 1 << 30, None) == q.QLORA_ERR_NULL_ARG
    assert fwd(ctypes.byref(W), P, 16, P, P, 8, 16.0, P, None, P, 16, None) == q.QLORA_ERR_WORKSPACE
    assert fwd(ctypes.byref(W), P, 0, None, None, 8, 16.0, None, None, None, 0, None) == q.QLORA_OK  # M = 0
    bwd = lib.qlora_linear_bwd
    assert bwd(ctypes.byref(W), P, P, 16, P, P, 8, 16.0, None, P, None, P, P, 1 << 30, None) == q.QLORA_ERR_NULL_ARG
    assert bwd(ctypes.byref(W), P, P, 16, P, P, 8, 16.0, None, P, P, P, P, 64, None) == q.QLORA_ERR_WORKSPACE
    assert "r = 0" in (fwd(ctypes.byref(W), P, 16, P, P, 0, 16.0, P, None, P, 1 << 30, None) and q.qlora_last_error())
    bad_sc = q.qlora_nf4_weight(64, 64, 16, 16, 16, 16, 0, 2, 16)
    assert lib.qlora_dequant_bf16(ctypes.byref(bad_sc), P, None) == q.QLORA_ERR_BAD_CODEBOOK
    single_null = q.qlora_nf4_weight(64, 64, 16, None, None, None, 0, q.QLORA_SCALES_FP32, None)
    assert lib.qlora_dequant_bf16(ctypes.byref(single_null), P, None) == q.QLORA_ERR_NULL_ARG
    single = q.qlora_nf4_weight(64, 64, 16, None, None, None, 1, q.QLORA_SCALES_FP32, 16)  # DQ buffers unused
    assert fwd(ctypes.byref(single), P, 16, P, P, 8, 16.0, P, None, P, 16, None) == q.QLORA_ERR_WORKSPACE
    assert lib.qlora_swiglu_fwd(None, None, None, 0, None) == q.QLORA_OK                        # count 0
    assert lib.qlora_swiglu_fwd(P, P, None, 8, None) == q.QLORA_ERR_NULL_ARG
    assert lib.qlora_swiglu_bwd(P, P, ctypes.c_void_p(24), P, P, 8, None) == q.QLORA_ERR_MISALIGNED
    assert lib.qlora_add_bf16(P, P, P, -1, None) == q.QLORA_ERR_BAD_SHAPE
    adam = lib.qlora_adamw_step
    assert adam(P, None, P, P, P, 16, 1e-3, 0.9, 0.999, 1e-8, 0.0, 0, None) == q.QLORA_ERR_BAD_SHAPE   # step 0
    assert adam(P, None, P, P, P, 16, 1e-3, 1.0, 0.999, 1e-8, 0.0, 1, None) == q.QLORA_ERR_BAD_ALPHA   # beta1 = 1
    assert adam(P, None, P, P, P, 16, 1e-3, 0.9, 0.999, 0.0, 0.0, 1, None) == q.QLORA_ERR_BAD_ALPHA    # eps = 0
    assert adam(None, None, P, P, P, 16, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, None) == q.QLORA_ERR_NULL_ARG
    assert adam(P, None, P, ctypes.c_void_p(20), P, 16, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, None) == q.QLORA_ERR_MISALIGNED
    assert adam(None, None, None, None, None, 0, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, None) == q.QLORA_OK  # count 0
    merge = lib.qlora_merge_adapters
    small = q.qlora_nf4_weight(128, 64, 16, 16, 16, 16)
    assert merge(ctypes.byref(W), P, P, 0, 16.0, P, None, P, 1 << 30, None) == q.QLORA_ERR_BAD_RANK
    assert merge(ctypes.byref(W), P, P, 8, 16.0, P, ctypes.byref(small), P, 1 << 30, None) == q.QLORA_ERR_BAD_SHAPE
    assert merge(ctypes.byref(W), P, P, 8, 16.0, P, None, P, 64, None) == q.QLORA_ERR_WORKSPACE
    assert merge(ctypes.byref(W), None, P, 8, 16.0, P, None, P, 1 << 30, None) == q.QLORA_ERR_NULL_ARG
    assert q.qlora_merge_workspace_bytes(4096, 4096) >= 4096 * 4096 * 4 + q.qlora_quantize_workspace_bytes(4096, 4096)
    assert q.qlora_merge_workspace_bytes(4096, 100) == 0
    bad_cb = q.qlora_nf4_weight(64, 64, 16, 16, 16, 16, 3)
    assert lib.qlora_quantize_nf4_dq(P, ctypes.byref(bad_cb), P, 1 << 20, None) == q.QLORA_ERR_BAD_CODEBOOK
    assert lib.qlora_dequant_bf16(ctypes.byref(bad_cb), P, None) == q.QLORA_ERR_BAD_CODEBOOK
    assert fwd(ctypes.byref(bad_cb), P, 16, P, P, 8, 16.0, P, None, P, 1 << 30, None) == q.QLORA_ERR_BAD_CODEBOOK
    for code in range(-8, 1):
        assert q.qlora_strerror(code) != "unknown status"


def test_attention_shape_and_argument_errors(q):
    lib = q.raw_library()
    P = ctypes.c_void_p(16)
    big = 1 << 40
    assert q.qlora_attention_workspace_bytes(8, 512, 32, 128) >= 12 * 8 * 32 * 512 * 512
    assert q.qlora_attention_workspace_bytes(1, 13, 2, 64) >= 12 * 2 * 13 * 16
    for bad in ((1, 16, 2, 60), (1, 16, 2, 0), (1, 16, 0, 64), (-1, 16, 2, 64), (1, 70000, 2, 64), (1, 16, 2, 2048)):
        assert q.qlora_attention_workspace_bytes(*bad) == 0
        assert lib.qlora_attention_fwd(P, P, P, P, P, *bad, P, big, None) == q.QLORA_ERR_BAD_SHAPE
        assert lib.qlora_attention_bwd(P, P, P, P, P, P, P, P, *bad, P, big, None) == q.QLORA_ERR_BAD_SHAPE
    fwd, bwd = lib.qlora_attention_fwd, lib.qlora_attention_bwd
    assert fwd(P, P, P, P, P, 0, 16, 2, 64, None, 0, None) == q.QLORA_OK          # empty: nothing to do
    assert fwd(P, P, P, P, P, 2, 0, 2, 64, None, 0, None) == q.QLORA_OK
    assert fwd(None, P, P, P, P, 1, 16, 2, 64, P, big, None) == q.QLORA_ERR_NULL_ARG
    assert fwd(P, P, P, P, None, 1, 16, 2, 64, P, big, None) == q.QLORA_ERR_NULL_ARG
    assert fwd(P, P, ctypes.c_void_p(24), P, P, 1, 16, 2, 64, P, big, None) == q.QLORA_ERR_MISALIGNED
    assert fwd(P, P, P, P, P, 1, 16, 2, 64, P, 64, None) == q.QLORA_ERR_WORKSPACE
    assert fwd(P, P, P, P, P, 1, 16, 2, 64, None, big, None) == q.QLORA_ERR_WORKSPACE
    assert bwd(P, P, P, P, P, P, P, None, 1, 16, 2, 64, P, big, None) == q.QLORA_ERR_NULL_ARG
    assert bwd(P, P, P, P, P, P, P, P, 1, 16, 2, 64, P, 64, None) == q.QLORA_ERR_WORKSPACE
    assert "head_dim" in (fwd(P, P, P, P, P, 1, 16, 2, 60, P, big, None) and q.qlora_last_error())
