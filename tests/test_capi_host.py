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
PROF_LIB = os.path.join(ROOT, "bit_nf4_quantized_qlora_amd", "libqlora_prof.so")


def _ensure_built():
    if not (os.path.exists(LIB) and os.path.exists(PROF_LIB)):
        from bit_nf4_quantized_qlora_amd import build
        build.build()


@pytest.fixture(scope="module")
def q():
    _ensure_built()
    from bit_nf4_quantized_qlora_amd import qlora
    return qlora


def _declared_functions(headers=None):
    headers = HEADERS if headers is None else [os.path.join(ROOT, "include", h) for h in headers]
    text = "".join(open(h).read() for h in headers)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qlora_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = _declared_functions()
    for n in ("qlora_quantize_nf4_dq", "qlora_dequant_bf16", "qlora_linear_fwd", "qlora_linear_bwd"):
        assert n in names


def test_every_declared_symbol_is_exported(q):
    """libqlora.so exports exactly qlora.h; the tracing build exports that
    plus the event timer of qlora_profile.h."""
    product = set(_declared_functions(["qlora.h"]))
    timer = set(_declared_functions(["qlora_profile.h"]))
    assert product and timer and not (product & timer)
    assert set(_declared_functions()) == product | timer
    lib = q.raw_library()
    for name in product:
        assert hasattr(lib, name), name
    for path, want in ((LIB, product), (PROF_LIB, product | timer)):
        out = os.popen(f"nm -D --defined-only {path}").read()
        assert set(re.findall(r"\bT (qlora_\w+)", out)) == want, path
    # the product library keeps no event timer
    assert not hasattr(lib, "qlora_profile_begin")
    with pytest.raises(RuntimeError):
        q.qlora_profile_begin()


def test_library_codebook_equals_oracle(q):
    from oracle import nf4_dq
    lib = np.array(q.qlora_nf4_codebook(), np.float32)
    assert np.array_equal(lib.view(np.uint32), nf4_dq.nf4_codebook().view(np.uint32))
    for name, cb in q.CODEBOOKS.items():
        lib = np.array(q.qlora_codebook(cb), np.float32)
        assert np.array_equal(lib.view(np.uint32), nf4_dq.codebook_levels(name).view(np.uint32)), name
    assert q.qlora_thresholds(q.QLORA_CODEBOOK_NF4) == q.qlora_nf4_thresholds()
    for bad in (-1, 3, 7):
        with pytest.raises(q.QloraError) as e:
            q.qlora_codebook(bad)
        assert e.value.status == q.QLORA_ERR_BAD_CODEBOOK


@pytest.mark.parametrize("name", ["nf4", "fp4", "fp4_e3m0"])
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


@pytest.mark.parametrize("name", ["nf4", "fp4", "fp4_e3m0"])
def test_thresholds_fit_the_quantizer_bucket_table(q, name):
    """The quantizer finds a code from a table of 64ths of [-1, 1]: bucket
    floor(64 x) + 64 holds the count of thresholds at or below its lower edge
    and at most one threshold strictly inside.  That needs no bucket to hold
    two (thresholds more than 1/64 apart would do; E3M0's -3/128 and -1/128
    successors are a hair closer, yet fall in buckets -2 and -1) and, past
    -1, no threshold below -1 (x >= -1)."""
    t = np.array(q.qlora_thresholds(q.CODEBOOKS[name]), np.float64)
    assert np.all(np.diff(t) > 0)
    assert t[0] > -1.0
    for i in range(129):
        lo, hi = (i - 64) / 64.0, (i - 63) / 64.0
        assert np.count_nonzero((t > lo) & (t < hi)) <= 1


def test_sizes_and_bits(q):
    for n, k in ((256, 256), (4096, 4096), (11008, 4096), (8192, 22016), (3, 64)):
        pb, sb, ng = q.qlora_nf4_sizes(n, k)
        assert pb == n * k // 2 and sb == n * k // 64 and ng == -(-sb // 256)
        if sb % 256 == 0:
            assert 8 * (pb + sb + 4 * ng) / (n * k) == 4.126953125
    with pytest.raises(q.QloraError) as e:
        q.qlora_nf4_sizes(10, 100)
    assert e.value.status == q.QLORA_ERR_BAD_SHAPE


def test_workspace_and_plan_over_many_shapes(q):
    """Every size query and plan answers (host arithmetic only) over a sweep
    of shapes, degenerate ones included; split plans stay consistent."""
    ns = (1, 7, 63, 64, 65, 200, 256, 1000, 4096, 22016)
    ks = (64, 128, 192, 320, 4096, 22016)
    for n in ns:
        for k in ks:
            for m in (0, 1, 5, 16, 17, 256, 512, 4096):
                for r in (1, 64, 128):
                    nbytes = q.qlora_linear_workspace_bytes(m, n, k, r)
                    assert (nbytes == 0) == (m == 0)
                    p = q.qlora_linear_plan(m, n, k, r)
                    if m == 0:
                        assert p["fwd_path"] == q.QLORA_PATH_NONE
                        continue
                    assert p["fwd_splits"] >= 1 and p["dx_splits"] >= 1
                    assert p["fwd_splits"] <= max(1, k // 64) and p["dx_splits"] <= max(1, n // 64)
                    assert p["dx_path"] == (q.QLORA_PATH_TILE if n % 64 == 0 else q.QLORA_PATH_GENERAL)


def test_workspace_queries(q):
    assert q.qlora_quantize_workspace_bytes(4096, 4096) >= 4096 * 4096 // 64 * 4
    assert q.qlora_quantize_workspace_bytes(4096, 100) == 0
    assert q.qlora_linear_workspace_bytes(512, 4096, 4096, 64) > 0
    assert q.qlora_linear_workspace_bytes(512, 4096, 4096, 0) == 0
    assert q.qlora_linear_workspace_bytes(512, 4096, 4096, 129) == 0
    assert q.qlora_linear_workspace_bytes(0, 4096, 4096, 64) == 0


def _ex(q, base, codebook=0, scales=0, absmax=None, size=None):
    return q.qlora_weight_ex(ctypes.sizeof(q.qlora_weight_ex) if size is None else size, base, codebook, scales,
                             absmax)


def test_descriptor_layouts(q):
    """The six-field descriptor of the four calls and the extended one."""
    assert ctypes.sizeof(q.qlora_nf4_weight) == 48
    assert q.qlora_weight_ex.base.offset == 8 and ctypes.sizeof(q.qlora_weight_ex) == 72


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
    bad_sc = _ex(q, W, 0, 2, 16)
    assert lib.qlora_dequant_bf16_ex(ctypes.byref(bad_sc), P, None) == q.QLORA_ERR_BAD_CODEBOOK
    single_null = _ex(q, q.qlora_nf4_weight(64, 64, 16, None, None, None), 0, q.QLORA_SCALES_FP32, None)
    assert lib.qlora_dequant_bf16_ex(ctypes.byref(single_null), P, None) == q.QLORA_ERR_NULL_ARG
    single = _ex(q, q.qlora_nf4_weight(64, 64, 16, None, None, None), 1, q.QLORA_SCALES_FP32, 16)  # DQ bufs unused
    fwd_ex = lib.qlora_linear_fwd_ex
    assert fwd_ex(ctypes.byref(single), P, 16, P, P, 8, 16.0, P, None, P, 16, None) == q.QLORA_ERR_WORKSPACE
    short = _ex(q, W, size=ctypes.sizeof(q.qlora_weight_ex) - 8)      # an older, shorter struct
    assert lib.qlora_dequant_bf16_ex(ctypes.byref(short), P, None) == q.QLORA_ERR_BAD_CODEBOOK
    assert "size" in q.qlora_last_error()
    assert lib.qlora_dequant_bf16_ex(None, P, None) == q.QLORA_ERR_NULL_ARG
    assert lib.qlora_swiglu_fwd(None, None, None, 0, None) == q.QLORA_OK                        # count 0
    assert lib.qlora_swiglu_fwd(P, P, None, 8, None) == q.QLORA_ERR_NULL_ARG
    assert lib.qlora_swiglu_bwd(P, P, ctypes.c_void_p(24), P, P, 8, None) == q.QLORA_ERR_MISALIGNED
    assert lib.qlora_add_bf16(P, P, P, -1, None) == q.QLORA_ERR_BAD_SHAPE
    xs = (ctypes.c_void_p * 4)(P, P, P, P)
    assert lib.qlora_add_bf16_n(xs, 1, P, 8, None) == q.QLORA_ERR_BAD_SHAPE
    assert lib.qlora_add_bf16_n(xs, 5, P, 8, None) == q.QLORA_ERR_BAD_SHAPE
    assert lib.qlora_add_bf16_n(None, 3, P, 8, None) == q.QLORA_ERR_NULL_ARG
    assert lib.qlora_add_bf16_n(xs, 3, None, 8, None) == q.QLORA_ERR_NULL_ARG
    assert lib.qlora_add_bf16_n((ctypes.c_void_p * 2)(P, 24), 2, P, 8, None) == q.QLORA_ERR_MISALIGNED
    assert lib.qlora_add_bf16_n(None, 2, None, 0, None) == q.QLORA_OK                          # count 0
    adam = lib.qlora_adamw_step
    assert adam(P, None, P, P, P, 16, 1e-3, 0.9, 0.999, 1e-8, 0.0, 0, None) == q.QLORA_ERR_BAD_SHAPE   # step 0
    assert adam(P, None, P, P, P, 16, 1e-3, 1.0, 0.999, 1e-8, 0.0, 1, None) == q.QLORA_ERR_BAD_ALPHA   # beta1 = 1
    assert adam(P, None, P, P, P, 16, 1e-3, 0.9, 0.999, 0.0, 0.0, 1, None) == q.QLORA_ERR_BAD_ALPHA    # eps = 0
    assert adam(None, None, P, P, P, 16, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, None) == q.QLORA_ERR_NULL_ARG
    assert adam(P, None, P, ctypes.c_void_p(20), P, 16, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, None) == q.QLORA_ERR_MISALIGNED
    assert adam(None, None, None, None, None, 0, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, None) == q.QLORA_OK  # count 0
    merge = lib.qlora_merge_adapters
    WX = _ex(q, W)
    small = _ex(q, q.qlora_nf4_weight(128, 64, 16, 16, 16, 16))
    assert merge(ctypes.byref(WX), P, P, 0, 16.0, P, None, P, 1 << 30, None) == q.QLORA_ERR_BAD_RANK
    assert merge(ctypes.byref(WX), P, P, 8, 16.0, P, ctypes.byref(small), P, 1 << 30, None) == q.QLORA_ERR_BAD_SHAPE
    assert merge(ctypes.byref(WX), P, P, 8, 16.0, P, None, P, 64, None) == q.QLORA_ERR_WORKSPACE
    assert merge(ctypes.byref(WX), None, P, 8, 16.0, P, None, P, 1 << 30, None) == q.QLORA_ERR_NULL_ARG
    assert q.qlora_merge_workspace_bytes(4096, 4096) >= 4096 * 4096 * 4 + q.qlora_quantize_workspace_bytes(4096, 4096)
    assert q.qlora_merge_workspace_bytes(4096, 100) == 0
    bad_cb = _ex(q, W, 3)
    assert lib.qlora_quantize_ex(P, ctypes.byref(bad_cb), P, 1 << 20, None) == q.QLORA_ERR_BAD_CODEBOOK
    assert lib.qlora_dequant_bf16_ex(ctypes.byref(bad_cb), P, None) == q.QLORA_ERR_BAD_CODEBOOK
    assert fwd_ex(ctypes.byref(bad_cb), P, 16, P, P, 8, 16.0, P, None, P, 1 << 30, None) == q.QLORA_ERR_BAD_CODEBOOK
    bwd_ex = lib.qlora_linear_bwd_ex
    assert bwd_ex(ctypes.byref(bad_cb), P, P, 16, P, P, 8, 16.0, None, P, P, P, P, 1 << 30, None) == \
        q.QLORA_ERR_BAD_CODEBOOK
    # the allocation-free forward: shapes beyond its fixed scratch are rejected before any GPU use
    noalloc = lib.qlora_linear_fwd_noalloc
    big = q.qlora_nf4_weight(262144, 8192, 16, 16, 16, 16)   # a 128 MB block-scale table alone
    assert noalloc(ctypes.byref(big), P, 512, P, P, 64, 16.0, P, None, None) == q.QLORA_ERR_WORKSPACE
    assert "scratch" in q.qlora_last_error()
    assert noalloc(ctypes.byref(W), P, 16, P, P, 0, 16.0, P, None, None) == q.QLORA_ERR_BAD_RANK
    assert noalloc(None, P, 16, P, P, 8, 16.0, P, None, None) == q.QLORA_ERR_NULL_ARG
    assert noalloc(ctypes.byref(W), P, 0, None, None, 8, 16.0, None, None, None) == q.QLORA_OK   # M = 0
    # k at or above 2^22 is rejected (a 256-row activation tile would reach 2^31 bytes)
    big_k = q.qlora_nf4_weight(1, 1 << 22, 16, 16, 16, 16)
    assert fwd(ctypes.byref(big_k), P, 16, P, P, 8, 16.0, P, None, P, 1 << 40, None) == q.QLORA_ERR_BAD_SHAPE
    for code in range(-8, 1):
        assert q.qlora_strerror(code) != "unknown status"


def test_attention_shape_and_argument_errors(q):
    lib = q.raw_library()
    P = ctypes.c_void_p(16)
    big = 1 << 40
    up = lambda x: (x + 255) // 256 * 256
    # head dims 32/64/96/128: the backward's D per query
    assert q.qlora_attention_workspace_bytes(8, 512, 32, 128) == up(8 * 32 * 512 * 4)
    assert q.qlora_attention_workspace_bytes(1, 13, 2, 64) == up(2 * 13 * 4)
    assert q.qlora_attention_workspace_bytes(1, 13, 2, 96) == up(2 * 13 * 4)
    # other head dims: float32 S and dP, bf16 P and dS, rows of roundup(seq, 8)
    assert q.qlora_attention_workspace_bytes(1, 13, 2, 8) == 2 * up(2 * 13 * 16 * 4) + 2 * up(2 * 13 * 16 * 2)
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


def test_linear_plan_paths(q):
    """The kernels each shape takes; the same decision the calls make."""
    T, G, V = q.QLORA_PATH_TILE, q.QLORA_PATH_GENERAL, q.QLORA_PATH_GEMV
    p = q.qlora_linear_plan(4096, 11008, 4096, 64)            # 7B MLP: enough tiles, no splits
    assert (p["fwd_path"], p["fwd_splits"], p["dx_path"], p["dx_splits"]) == (T, 1, T, 1)
    assert q.qlora_linear_plan(4096, 4096, 11008, 64)["fwd_splits"] == 1
    p = q.qlora_linear_plan(512, 4096, 4096, 64)              # 7B q_proj at M = 512: 32 tiles, split
    assert p["fwd_path"] == T and p["fwd_splits"] > 1 and p["dx_splits"] > 1
    for n, k in ((8192, 8192), (8192, 22016)):                # 65B block at M = 512
        assert q.qlora_linear_plan(512, n, k, 64)["fwd_splits"] > 1
    assert q.qlora_linear_plan(512, 22016, 8192, 64)["dx_splits"] > 1
    for m in (1, 4, 16):                                      # small M: the GEMV forward
        assert q.qlora_linear_plan(m, 22016, 8192, 16)["fwd_path"] == V
        assert q.qlora_linear_plan(m, 22016, 8192, 16, q.QLORA_SCALES_FP32)["fwd_path"] == V
    assert q.qlora_linear_plan(37, 200, 192, 5)["dx_path"] == G          # n % 64 != 0
    assert q.qlora_linear_plan(64, 640, 512, 64)["fwd_splits"] == 1      # 8 steps: nothing to split
    # dY tiles of 256 rows x 512 n bytes must stay below 2^31: n = 2^22 takes the general kernel
    assert q.qlora_linear_plan(1, (1 << 22) - 64, 64, 1)["dx_path"] == T
    assert q.qlora_linear_plan(1, 1 << 22, 64, 1)["dx_path"] == G
    assert q.qlora_linear_plan(1, 1 << 23, 64, 1)["dx_path"] == G
    assert q.qlora_linear_plan(0, 64, 64, 1)["fwd_path"] == q.QLORA_PATH_NONE
    for bad in ((16, 64, 96, 8), (16, 64, 64, 0), (-1, 64, 64, 8)):
        with pytest.raises(q.QloraError):
            q.qlora_linear_plan(*bad)


def test_binding_rejects_bad_tensors_before_the_call(q):
    """Shape, dtype and device mismatches raise in Python before any pointer
    reaches the library (CPU tensors here: nothing is launched)."""
    import torch
    bf = lambda *s: torch.zeros(*s, dtype=torch.bfloat16)
    w = q.NF4Weight.empty(128, 256, device="cpu")
    M, r = 8, 4
    X, A, B, Y, H = bf(M, 256), bf(r, 256), bf(128, r), bf(M, 128), torch.zeros(M, r)
    ws = torch.zeros(16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="X has shape"):
        q.qlora_linear_fwd(w, bf(M, 128), A, B, r, 16.0, Y, H, ws)
    with pytest.raises(ValueError, match="A has shape"):
        q.qlora_linear_fwd(w, X, bf(r + 1, 256), B, r, 16.0, Y, H, ws)
    with pytest.raises(ValueError, match="B has shape"):
        q.qlora_linear_fwd(w, X, A, bf(256, r), r, 16.0, Y, H, ws)
    with pytest.raises(ValueError, match="Y has shape"):
        q.qlora_linear_fwd(w, X, A, B, r, 16.0, bf(M + 1, 128), H, ws)
    with pytest.raises(ValueError, match="H_out has shape"):
        q.qlora_linear_fwd(w, X, A, B, r, 16.0, Y, torch.zeros(M, r + 1), ws)
    with pytest.raises(TypeError):
        q.qlora_linear_fwd(w, X.float(), A, B, r, 16.0, Y, H, ws)
    with pytest.raises(ValueError, match="GPU tensor"):
        q.qlora_linear_fwd(w, X, A, B, r, 16.0, Y, H, ws)
    with pytest.raises(ValueError, match="dY has shape"):
        q.qlora_linear_bwd(w, X, bf(M, 127), A, B, r, 16.0, H, bf(M, 256), bf(r, 256), bf(128, r), ws)
    with pytest.raises(ValueError, match="dX has shape"):
        q.qlora_linear_bwd(w, X, Y, A, B, r, 16.0, H, bf(M, 255), bf(r, 256), bf(128, r), ws)
    with pytest.raises(ValueError, match="dB has shape"):
        q.qlora_linear_bwd(w, X, Y, A, B, r, 16.0, H, None, bf(r, 256), bf(r, 128), ws)
    with pytest.raises(ValueError, match="W has shape"):
        q.qlora_quantize_nf4_dq(torch.zeros(128, 255), w, ws)
    with pytest.raises(ValueError, match="elements"):
        q.qlora_dequant_bf16(w, bf(128, 255))
    short = q.NF4Weight(128, 256, w.packed[:-1], w.scale_code, w.group_amax, w.offset)
    with pytest.raises(ValueError, match="packed"):
        q.qlora_dequant_bf16(short, bf(128, 256))
    with pytest.raises(ValueError, match="elements"):
        q.qlora_swiglu_fwd(bf(10), bf(10), bf(9))
    with pytest.raises(ValueError, match="elements"):
        q.qlora_add_bf16(bf(10), bf(11), bf(10))
    with pytest.raises(ValueError, match="has shape"):
        q.qlora_attention_fwd(bf(32, 64), bf(32, 64), bf(32, 64), bf(32, 63), torch.zeros(2, 1, 16), 2, 16, 1, 64, ws)
    with pytest.raises(ValueError, match="lse"):
        q.qlora_attention_fwd(bf(32, 64), bf(32, 64), bf(32, 64), bf(32, 64), torch.zeros(2, 1, 15), 2, 16, 1, 64, ws)
    with pytest.raises(ValueError, match="grad"):
        q.qlora_adamw_step(torch.zeros(16), None, bf(15), torch.zeros(16), torch.zeros(16), 1e-3, 0.9, 0.999, 1e-8,
                           0.0, 1)
    with pytest.raises(ValueError, match="A has shape"):
        q.qlora_merge_adapters(w, bf(r, 128), B, r, 16.0, None, None, ws)


def test_decoder_layer_rejects_bad_shapes(q):
    import torch
    from bit_nf4_quantized_qlora_amd.layer import DecoderLayer
    hidden, inter, r, batch, seq, heads, d = 64, 128, 4, 2, 8, 2, 32
    shapes = {"q": (hidden, hidden), "k": (hidden, hidden), "v": (hidden, hidden), "o": (hidden, hidden),
              "gate": (inter, hidden), "up": (inter, hidden), "down": (hidden, inter)}
    weights = {nm: q.NF4Weight.empty(n, k, device="cpu") for nm, (n, k) in shapes.items()}
    adapters = {nm: (torch.zeros(r, k, dtype=torch.bfloat16), torch.zeros(n, r, dtype=torch.bfloat16))
                for nm, (n, k) in shapes.items()}
    lay = DecoderLayer(weights, adapters, r, 16.0, batch, seq, heads, d, device="cpu")
    M = batch * seq
    good = torch.zeros(M, hidden, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="X must be"):
        lay.fwd(torch.zeros(M + 1, hidden, dtype=torch.bfloat16), good)
    with pytest.raises(ValueError, match="dY must be"):
        lay.bwd(good, torch.zeros(M, hidden + 1, dtype=torch.bfloat16), good)
    with pytest.raises(ValueError, match="X must be"):
        lay.fwd(good.float(), good)
    with pytest.raises(ValueError, match="GPU tensor"):     # right shapes: the binding's device check
        lay.fwd(good, good.clone())
