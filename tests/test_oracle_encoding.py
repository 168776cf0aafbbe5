"""Pins of the oracle's storage encoding (quantize, double quantization,
dequantization) against what the pages and the mathematics fix.

Pins used:
  * worked examples printed on "QLoRA Explained ... Part 2/6" (NF4 lookup,
    toy three-bit block) and the bits-per-weight arithmetic printed there and
    in "QLoRA Paper Breakdown ..." section 3;
  * exact-rational brute force (fractions.Fraction) for the nearest-code
    search, the E4M3 rounding and the mean;
  * torch's CPU float8_e4m3fn / bfloat16 casts as an independent second
    implementation of the two scalar formats;
  * closed-form special cases: lossless double quantization of a single
    block, an all-zero tensor, constant block scales, the group extreme
    coding to +-1.0.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import nf4_dq

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32


def _golden():
    with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
        return json.load(f)


def _f32_next_up(x: float) -> np.float32:
    return np.nextafter(F32(x), F32(np.inf), dtype=F32)


def _f32_next_down(x: float) -> np.float32:
    return np.nextafter(F32(x), F32(-np.inf), dtype=F32)


def _smallest_f32_above(fr: Fraction) -> np.float32:
    t = F32(float(fr))
    while Fraction(float(t)) <= fr:
        t = _f32_next_up(t)
    while Fraction(float(_f32_next_down(t))) > fr:
        t = _f32_next_down(t)
    return t


def _brute_nearest(values, levels):
    lv = [Fraction(float(v)) for v in levels]
    out = []
    for x in values:
        fx = Fraction(float(x))
        d = [abs(fx - v) for v in lv]
        out.append(d.index(min(d)))          # first index on ties
    return np.array(out, dtype=np.uint8)


# ----------------------------------------------------------------- formats
def test_bf16_rne_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000).astype(F32),
        (rng.standard_normal(2000) * 1e-39).astype(F32),          # denormals
        (rng.standard_normal(2000) * 3e38).clip(-3.3e38, 3.3e38).astype(F32),
        # exact ties: low 16 bits 0x8000 with both parities of bit 16
        (rng.integers(0, 2**31, 4000, dtype=np.uint64).astype(np.uint32) & np.uint32(0x7F7F0000)
         | np.uint32(0x8000)).view(F32),
        np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf], F32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(nf4_dq.bf16_rne_bits(x), ref)


def test_e4m3_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = nf4_dq.e4m3fn_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_e4m3_known_codes():
    enc = nf4_dq.e4m3fn_encode_rne(np.array([1.0, -1.0, 0.5, 2.0 ** -9, 0.0, -0.0, -1e-30, 448.0], F32))
    assert list(enc) == [0x38, 0xB8, 0x30, 0x01, 0x00, 0x80, 0x80, 0x7E]


def test_e4m3_encode_matches_torch_and_exact_rounding():
    mags = nf4_dq.e4m3fn_decode(np.arange(0x39, dtype=np.uint8)).astype(np.float64)   # 0 .. 1.0
    mids = (mags[:-1] + mags[1:]) / 2                                                  # exact ties
    rng = np.random.default_rng(2)
    x = np.concatenate([
        rng.uniform(-1, 1, 50000), rng.uniform(-2**-6, 2**-6, 5000), mags, -mags, mids, -mids,
        np.nextafter(mids, 0), np.nextafter(mids, 2),
    ]).astype(F32)
    got = nf4_dq.e4m3fn_encode_rne(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)
    # exact-rational check on the tie set: the nearer magnitude, ties to even code
    allm = [Fraction(float(v)) for v in mags]
    for v, c in zip(x[-4 * mids.size:], got[-4 * mids.size:]):
        fv = abs(Fraction(float(v)))
        d = [abs(fv - m) for m in allm]
        best = min(d)
        cands = [i for i, di in enumerate(d) if di == best]
        want = cands[0] if len(cands) == 1 else [i for i in cands if i % 2 == 0][0]
        assert (int(c) & 0x7F) == want


# ------------------------------------------------------------ nearest code
def test_nearest_level_brute_force_tiny():
    q = nf4_dq.nf4_codebook()
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.uniform(-1, 1, 3000), q, [0.0, -0.0, 1e-45, -1e-45]]).astype(F32)
    assert np.array_equal(nf4_dq.nearest_level(x, q), _brute_nearest(x, q))


def test_nearest_level_transitions_are_the_exact_midpoints():
    """The nearest-level map is monotone in its input, so it is fixed by the
    15 points where it steps; at each exact midpoint m_j of q_j and q_{j+1}
    the tie goes to j, and the first float32 above m_j maps to j+1."""
    q = nf4_dq.nf4_codebook()
    xs, want = [], []
    for j in range(15):
        m = (Fraction(float(q[j])) + Fraction(float(q[j + 1]))) / 2
        t = _smallest_f32_above(m)
        below = _f32_next_down(t)
        xs += [t, below, _f32_next_up(t), _f32_next_down(below)]
        want += [j + 1, j, j + 1, j]
    xs = np.array(xs, F32)
    got = nf4_dq.nearest_level(xs, q)
    assert list(got) == want
    assert np.array_equal(got, _brute_nearest(xs, q))
    # six of the midpoints are float32 numbers, so exact ties do occur
    exact = [j for j in range(15)
             if Fraction(float(F32(float((Fraction(float(q[j])) + Fraction(float(q[j + 1]))) / 2))))
             == (Fraction(float(q[j])) + Fraction(float(q[j + 1]))) / 2]
    assert exact == [2, 6, 7, 9, 11, 13]


def test_worked_nf4_lookup():
    g = _golden()["nf4_lookup"]
    q = nf4_dq.nf4_codebook()
    n = F32(F32(g["value"]) / F32(g["block_scale"]))
    assert f"{float(n):.3f}" == g["normalized"]
    code = int(nf4_dq.nearest_level(np.array([n]), q)[0])
    assert f"{float(q[code]):.10f}" == g["level"]
    recon = F32(q[code] * F32(g["block_scale"]))
    assert f"{float(recon):.10f}" == g["reconstruction"]
    assert f"{float(recon) - 0.37:.10f}" == g["error"]


def test_worked_block_through_full_encoding():
    """The worked block as a one-block tensor: the double quantization is
    lossless (single block => its deviation from the mean is 0), so the scale
    is exactly 2 and the weights are the rounded products."""
    w = np.zeros((1, 64), F32)
    w[0, :4] = [-2.0, -0.4, 0.37, 2.0]
    enc = nf4_dq.quantize_nf4_dq(w)
    assert list(enc["codes"][:4]) == [0, 5, 9, 15]
    assert np.all(enc["codes"][4:] == 7)
    assert list(enc["packed"][:2]) == [0x50, 0xF9] and np.all(enc["packed"][2:] == 0x77)
    assert enc["offset"] == F32(2.0) and enc["group_amax"][0] == 0 and enc["scale_code"][0] == 0
    wh = nf4_dq.bf16_bits_to_f64(nf4_dq.dequant_bf16(enc["packed"], enc["scale_code"],
                                                     enc["group_amax"], enc["offset"], 1, 64))
    assert list(wh[0, :4]) == [-2.0, -0.369140625, 0.322265625, 2.0]
    assert np.all(wh[0, 4:] == 0)


def test_toy_three_bit_example():
    g = _golden()["toy_three_bit"]
    levels = np.array([float(v) for v in g["levels"]], F32)
    block = np.array([float(v) for v in g["block"]], F32)
    codes, absmax = nf4_dq.blockwise_quantize(block, levels, block.size)
    assert float(absmax[0]) == float(g["scale"])
    recon = levels[codes[0]].astype(np.float64) * float(absmax[0])
    assert list(recon) == [float(v) for v in g["reconstruction"]]
    err = recon - block.astype(np.float64)
    assert np.allclose(err, [float(v) for v in g["signed_errors"]], atol=1e-7)
    assert abs(np.mean(err ** 2) - float(g["mse"])) < 1e-9


# -------------------------------------------------------- double quantization
def test_mean_matches_exact_rational_mean():
    rng = np.random.default_rng(4)
    # up to 256 groups the group sums form one run; 65537 and 140000 blocks
    # take two and three runs (the last one short)
    for nb in (1, 255, 256, 257, 5000, 65537, 140000):
        a = np.abs(rng.standard_normal(nb) * 0.05).astype(F32)
        exact = sum((Fraction(float(v)) for v in a), Fraction(0)) / nb
        off = nf4_dq.dq_offset(a)
        ulp = np.spacing(F32(float(exact)))
        # float64 partial sums add at most ~nb * 2^-53 relative error
        assert abs(Fraction(float(off)) - exact) <= Fraction(float(ulp)) / 2 + exact * Fraction(nb, 2**52)


def test_mean_of_one_run_is_the_fold_over_the_group_sums():
    """The vectorized folds (padded reshapes) against plain scalar loops: up
    to MEAN_RUN groups the run level is one fold over every group sum; past
    it, the run sums of consecutive groups are folded in order."""
    rng = np.random.default_rng(8)
    for nb in (3000, 256 * nf4_dq.MEAN_RUN, 256 * nf4_dq.MEAN_RUN + 1000):
        a = np.abs(rng.standard_normal(nb) * 0.05).astype(F32).astype(np.float64)
        ng = -(-nb // 256)
        seq = 0.0
        for i in range(0, nb, 256):  # the group's own left-to-right fold
            g = 0.0
            for v in a[i:i + 256]:
                g += v
            seq += g
        runs = []
        for r0 in range(0, ng, nf4_dq.MEAN_RUN):
            acc = 0.0
            for i in range(r0 * 256, min(nb, (r0 + nf4_dq.MEAN_RUN) * 256), 256):
                g = 0.0
                for v in a[i:i + 256]:
                    g += v
                acc += g
            runs.append(acc)
        tot = 0.0
        for v in runs:
            tot += v
        off = nf4_dq.dq_offset(a.astype(F32))
        assert off == np.float32(tot / nb)
        if len(runs) == 1:
            assert off == np.float32(seq / nb)


def test_single_block_tensor_is_lossless():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((1, 64)) * 0.02).astype(F32)
    enc = nf4_dq.quantize_nf4_dq(w)
    s = nf4_dq.dq_block_scale(enc["scale_code"], enc["group_amax"], enc["offset"])
    assert s[0] == enc["absmax"][0]


def test_constant_block_scales_are_lossless():
    w = np.tile(np.linspace(-0.5, 0.5, 64, dtype=F32), (64, 8))       # every block absmax 0.5
    enc = nf4_dq.quantize_nf4_dq(w)
    s = nf4_dq.dq_block_scale(enc["scale_code"], enc["group_amax"], enc["offset"])
    assert np.all(s == F32(0.5))


def test_all_zero_tensor():
    enc = nf4_dq.quantize_nf4_dq(np.zeros((4, 128), F32))
    assert np.all(enc["codes"] == 7) and np.all(enc["packed"] == 0x77)
    assert enc["offset"] == 0 and np.all(enc["scale_code"] == 0) and np.all(enc["group_amax"] == 0)
    wh = nf4_dq.dequant_bf16(enc["packed"], enc["scale_code"], enc["group_amax"], enc["offset"], 4, 128)
    assert np.all(wh == 0)


def test_zero_weights_round_trip_to_zero():
    rng = np.random.default_rng(6)
    w = (rng.standard_normal((16, 256)) * 0.02).astype(F32)
    w[rng.random(w.shape) < 0.2] = 0.0
    w[0, 5] = -0.0
    enc = nf4_dq.quantize_nf4_dq(w)
    wh = nf4_dq.bf16_bits_to_f64(nf4_dq.dequant_bf16(enc["packed"], enc["scale_code"],
                                                     enc["group_amax"], enc["offset"], 16, 256))
    assert np.all(enc["codes"].reshape(w.shape)[w == 0] == 7)
    assert np.all(wh[w == 0] == 0)


def test_group_extreme_codes_to_plus_minus_one_and_scale_error_bound():
    rng = np.random.default_rng(7)
    n, k = 96, 512                                    # 768 blocks: 3 groups
    w = (rng.standard_normal((n, k)) * 0.02).astype(F32)
    enc = nf4_dq.quantize_nf4_dq(w)
    dev = enc["dev"].astype(np.float64)
    for g in range(3):
        sl = slice(g * 256, (g + 1) * 256)
        i = int(np.argmax(np.abs(dev[sl])))
        assert enc["scale_code"][sl][i] in (0x38, 0xB8)
        assert enc["group_amax"][g] == F32(np.abs(dev[sl]).max())
    s = nf4_dq.dq_block_scale(enc["scale_code"], enc["group_amax"], enc["offset"]).astype(np.float64)
    amax = np.repeat(enc["group_amax"].astype(np.float64), 256)
    a = enc["absmax"].astype(np.float64)
    # 3 mantissa bits: relative error <= 2^-4 in the normal range, absolute
    # 2^-10 of the group constant in the subnormal range, plus float32 roundings.
    bound = 2.0 ** -4 * np.abs(dev) + 2.0 ** -10 * amax + 4 * np.spacing(F32(a.max()))
    assert np.all(np.abs(s - a) <= bound)


def test_partial_last_group():
    rng = np.random.default_rng(8)
    w = (rng.standard_normal((5, 64 * 60)) * 0.02).astype(F32)     # 300 blocks: 256 + 44
    enc = nf4_dq.quantize_nf4_dq(w)
    assert enc["scale_code"].size == 300 and enc["group_amax"].size == 2
    dev = enc["dev"]
    assert enc["group_amax"][1] == np.abs(dev[256:]).max()


def test_reconstruction_error_is_plausible():
    # Derived sanity figure, not printed on the pages: NF4+DQ relative RMS
    # error of ~0.09 on normal weights.
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((256, 1024)) * 0.02).astype(F32)
    enc = nf4_dq.quantize_nf4_dq(w)
    wh = nf4_dq.bf16_bits_to_f64(nf4_dq.dequant_bf16(enc["packed"], enc["scale_code"],
                                                     enc["group_amax"], enc["offset"], 256, 1024))
    rel = np.sqrt(np.mean((wh - w) ** 2) / np.mean(w.astype(np.float64) ** 2))
    assert 0.08 < rel < 0.10


@pytest.mark.parametrize("codebook,half_gap", [("fp4", 6), ("fp4_e3m0", 4)])
def test_fp4_encoding_error_bound_and_shared_constants(codebook, half_gap):
    # Float4 storage keeps the same block constants (they depend on the
    # absmax values only) and bounds each error by half the widest gap of the
    # level set (E2M1: 1/3 between 2/3 and 1, so absmax/6; E3M0: 1/2 between
    # 1/2 and 1, so absmax/4), plus the block-scale error and the bf16
    # rounding of the product.
    rng = np.random.default_rng(19)
    w = (rng.standard_normal((96, 512)) * 0.02).astype(F32)
    e4, nf = nf4_dq.quantize_nf4_dq(w, codebook), nf4_dq.quantize_nf4_dq(w)
    for key in ("scale_code", "group_amax", "offset", "absmax"):
        assert np.array_equal(np.asarray(e4[key]), np.asarray(nf[key]))
    assert e4["codes"].max() <= 14
    wh = nf4_dq.bf16_bits_to_f64(nf4_dq.dequant_bf16(e4["packed"], e4["scale_code"], e4["group_amax"],
                                                     e4["offset"], 96, 512, codebook=codebook)).reshape(-1, 64)
    s = nf4_dq.dq_block_scale(e4["scale_code"], e4["group_amax"], e4["offset"]).astype(np.float64)
    a = e4["absmax"].astype(np.float64)
    bound = a / half_gap + np.abs(s - a) + 2.0 ** -8 * np.abs(s) + 1e-12
    assert np.all(np.abs(wh - w.reshape(-1, 64).astype(np.float64)) <= bound[:, None])
    # coarser than NF4 on normal weights, as the reading note's table has it
    wn = nf4_dq.bf16_bits_to_f64(nf4_dq.dequant_bf16(nf["packed"], nf["scale_code"], nf["group_amax"],
                                                     nf["offset"], 96, 512)).reshape(-1, 64)
    ref = w.reshape(-1, 64).astype(np.float64)
    assert np.mean((wh - ref) ** 2) > np.mean((wn - ref) ** 2)


@pytest.mark.parametrize("codebook", ["nf4", "fp4", "fp4_e3m0"])
def test_single_level_constants(codebook):
    # Single-level storage keeps the double-quantized layout's codes, stores
    # each block absmax as is (4 + 32/64 = 4.5 bits, the teardown's figure)
    # and so bounds each error by half the widest level gap times absmax
    # plus the bf16 rounding alone: no block-scale error.
    rng = np.random.default_rng(23)
    w = (rng.standard_normal((64, 768)) * 0.02).astype(F32)
    sl, dq = nf4_dq.quantize_single_level(w, codebook), nf4_dq.quantize_nf4_dq(w, codebook)
    assert np.array_equal(sl["packed"], dq["packed"])
    assert np.array_equal(sl["absmax"].view(np.uint32), dq["absmax"].view(np.uint32))
    bits = 8 * (sl["packed"].nbytes + sl["absmax"].nbytes) / w.size
    assert bits == 4 + 32 / 64 == float(_golden()["bits_per_weight"]["single_level_total"])
    wh = nf4_dq.bf16_bits_to_f64(nf4_dq.dequant_single_level_bf16(sl["packed"], sl["absmax"], 64, 768, codebook))
    lv = nf4_dq.codebook_levels(codebook).astype(np.float64)
    half_gap = np.diff(lv).max() / 2
    a = sl["absmax"].astype(np.float64)
    err = np.abs(wh.reshape(-1, 64) - w.reshape(-1, 64).astype(np.float64))
    assert np.all(err <= (half_gap + 2.0 ** -8) * a[:, None])
    # a block whose weights are all levels times one absmax round-trips exactly
    # up to bf16: w = q * 0.5 gives w_hat = bf16(q * 0.5)
    lvl = nf4_dq.codebook_levels(codebook)
    blk = (np.resize(lvl, 64) * np.float32(0.5)).astype(F32).reshape(1, 64)
    e1 = nf4_dq.quantize_single_level(blk, codebook)
    got = nf4_dq.dequant_single_level_bf16(e1["packed"], e1["absmax"], 1, 64, codebook)
    assert np.array_equal(got.reshape(-1), nf4_dq.bf16_rne_bits(blk.reshape(-1)))


# ------------------------------------------------------------ bit arithmetic
def test_bits_per_weight_from_buffers():
    g = _golden()["bits_per_weight"]
    for n, k in ((256, 256), (4096, 4096), (64, 16384)):
        w = np.ones((n, k), F32) if n * k > 2**20 else \
            np.random.default_rng(10).standard_normal((n, k)).astype(F32)
        if n * k > 2**20:
            sizes = nf4_dq.storage_sizes(n, k)
            bits = 8 * (sizes[0] + sizes[1] + 4 * sizes[2]) / (n * k)
        else:
            bits = nf4_dq.storage_bits_per_weight(nf4_dq.quantize_nf4_dq(w), n, k)
        assert bits == float(g["dq_total"])
    assert 32 / 64 == float(g["single_level_overhead"]) and 4 + 32 / 64 == float(g["single_level_total"])
    assert 8 / 64 + 32 / (64 * 256) == float(g["dq_overhead"])
    assert 4.5 - 4.126953125 == float(g["saving"])
    assert f"{float(g['params_65b']) * float(g['saving']) / 8 / 1e9:.3f}" == g["saving_gb_at_65b"]


def test_memory_breakdown_arithmetic():
    g = _golden()["memory_65b"]
    # 33.5 GB follows from the exact 4.126953125 bits (the "4.13" label gives 33.6)
    assert f"{65e9 * 4.126953125 / 8 / 1e9:.1f}" == g["base_weights_gb"]
    total = float(g["base_weights_gb"]) + float(g["optimizer_gb"]) + float(g["grads_activations_gb"])
    assert f"{total:.1f}" == g["total_gb"]
