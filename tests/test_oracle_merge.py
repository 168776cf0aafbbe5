"""Pins of the adapter-merge oracle (oracle/merge.py) against facts that do
not come from it: the layer's own forward oracle (the merged weight must
reproduce the fused forward), exact rational arithmetic on dyadic inputs,
and the B = 0 identity.  Source: "QLoRA Paper Breakdown ..." sections 4
(forward pass) and 'Limitations' (merging adapters into 16-bit weights)."""
from fractions import Fraction

import numpy as np

from oracle import linear, merge, nf4_dq

F32 = np.float32


def _bf16(x):
    return nf4_dq.bf16_rne_bits(np.asarray(x, F32))


def _round_f32(x: Fraction) -> np.float32:
    """Exact rational -> nearest float32, ties to even (no double rounding)."""
    f = F32(float(x))
    best = None
    for c in (np.nextafter(f, F32(-np.inf)), f, np.nextafter(f, F32(np.inf))):
        d = abs(Fraction(float(c)) - x)
        key = (d, int(np.asarray(c, F32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return F32(best[1])


def test_zero_b_gives_back_the_dequantized_weight():
    rng = np.random.default_rng(1)
    W = (rng.standard_normal((16, 128)) * 0.02).astype(F32)
    enc = nf4_dq.quantize_nf4_dq(W)
    wh = nf4_dq.dequant_bf16(enc["packed"], enc["scale_code"], enc["group_amax"], enc["offset"], 16, 128)
    A = _bf16(rng.uniform(-0.05, 0.05, (8, 128)))
    B = _bf16(np.zeros((16, 8)))
    out = merge.merge_and_requantize(wh, A, B, 16.0)
    assert np.array_equal(out["merged_bf16"], wh)
    assert np.array_equal(out["merged_f32"].astype(np.float64), nf4_dq.bf16_bits_to_f64(wh))


def test_dyadic_inputs_match_exact_rational_arithmetic():
    # bf16-exact dyadic A, B and a bf16 base: every float64 step is exact, so
    # the result is the exact value rounded once to float32
    rng = np.random.default_rng(2)
    n, k, r, alpha = 6, 64, 5, 10.0
    A = _bf16(rng.integers(-8, 9, (r, k)) * 2.0 ** -5)
    B = _bf16(rng.integers(-8, 9, (n, r)) * 2.0 ** -7)
    wh = _bf16(rng.standard_normal((n, k)) * 0.03)
    got = merge.merged_f32(wh, A, B, alpha)
    Af, Bf, Wf = (nf4_dq.bf16_bits_to_f64(t) for t in (A, B, wh))
    s = Fraction(float(F32(alpha) / F32(r)))
    for i in range(n):
        for c in range(k):
            t = sum(Fraction(float(Bf[i, j])) * Fraction(float(Af[j, c])) for j in range(r))
            exact = Fraction(float(Wf[i, c])) + s * t
            if exact.denominator & (exact.denominator - 1) == 0:   # dyadic: the float64 steps were exact
                assert got[i, c] == _round_f32(exact), (i, c)


def test_merged_weight_reproduces_the_fused_forward():
    # X W'^T == X W_hat^T + s X A^T B^T up to the float32 rounding of W'
    # (relative 2^-24 per element): catches a transposed product, a dropped
    # or misplaced scale, or a wrong sign
    rng = np.random.default_rng(3)
    n, k, r, M, alpha = 40, 192, 8, 12, 16.0
    W = (rng.standard_normal((n, k)) * 0.02).astype(F32)
    enc = nf4_dq.quantize_nf4_dq(W)
    wh = nf4_dq.dequant_bf16(enc["packed"], enc["scale_code"], enc["group_amax"], enc["offset"], n, k)
    A = _bf16(rng.uniform(-0.05, 0.05, (r, k)))
    B = _bf16(rng.uniform(-0.05, 0.05, (n, r)))
    X = nf4_dq.bf16_bits_to_f64(_bf16(rng.standard_normal((M, k))))
    Wm = merge.merged_f32(wh, A, B, alpha).astype(np.float64)
    Yf, _ = linear.fwd(X, nf4_dq.bf16_bits_to_f64(wh), nf4_dq.bf16_bits_to_f64(A), nf4_dq.bf16_bits_to_f64(B),
                       float(F32(alpha) / F32(r)) * r)
    Ym = X @ Wm.T
    assert np.abs(Ym - Yf).max() <= 2.0 ** -22 * (np.abs(X) @ np.abs(Wm).T).max()
    # and the adapters' contribution is not negligible in this case
    assert np.abs(Ym - X @ nf4_dq.bf16_bits_to_f64(wh).T).max() > 1e-3


def test_requantized_encoding_is_the_encoding_of_the_merged_weight():
    rng = np.random.default_rng(4)
    W = (rng.standard_normal((8, 256)) * 0.02).astype(F32)
    enc = nf4_dq.quantize_nf4_dq(W)
    wh = nf4_dq.dequant_bf16(enc["packed"], enc["scale_code"], enc["group_amax"], enc["offset"], 8, 256)
    A = _bf16(rng.uniform(-0.05, 0.05, (4, 256)))
    B = _bf16(rng.uniform(-0.05, 0.05, (8, 4)))
    out = merge.merge_and_requantize(wh, A, B, 16.0, "fp4")
    ref = nf4_dq.quantize_nf4_dq(out["merged_f32"], "fp4")
    for key in ("packed", "scale_code", "group_amax"):
        assert np.array_equal(out["encoding"][key], ref[key])
