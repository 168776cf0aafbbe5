"""Pins of the oracle's NF4 codebook against what the pages print.

Sources: "QLoRA Paper Breakdown ..." section 2 (the printed 16 values, the
7 negative / exact zero / 8 positive structure) and "QLoRA Explained ...
Part 2/6" (q_9 to 10 digits); "QLoRA, explained." method step 1.
"""
import os

import numpy as np
import pytest
from scipy.stats import norm

from oracle import nf4_dq

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _printed():
    with open(os.path.join(GOLDEN, "nf4_codebook_printed.txt")) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


def test_codebook_rounds_to_printed_values():
    q = nf4_dq.nf4_codebook()
    printed = _printed()
    assert len(printed) == 16
    got = [f"{float(v):.8f}" for v in q]
    # "-0.00000000" never occurs: the zero level is +0.
    assert got == printed


def test_q9_ten_digits_from_worked_lookup():
    assert f"{float(nf4_dq.nf4_codebook()[9]):.10f}" == "0.1609302014"


def test_codebook_structure():
    q = nf4_dq.nf4_codebook()
    assert q.dtype == np.float32 and q.shape == (16,)
    assert np.all(np.diff(q.astype(np.float64)) > 0)
    assert (q < 0).sum() == 7 and (q > 0).sum() == 8
    assert q[7] == 0.0 and not np.signbit(q[7])
    assert q[0] == -1.0 and q[15] == 1.0


def test_levels_are_normal_quantiles_of_an_even_probability_grid():
    # Independent route: scipy's normal quantile on a float64 probability grid
    # from delta = ((1-1/30)+(1-1/32))/2 to 1/2 (9 points positive half, 8 negative).
    delta = ((1 - 1 / 30) + (1 - 1 / 32)) / 2
    pos = norm.ppf(np.linspace(delta, 0.5, 9)[:-1])
    neg = -norm.ppf(np.linspace(delta, 0.5, 8)[:-1])
    ref = np.sort(np.concatenate([pos, [0.0], neg]))
    ref = ref / ref.max()
    q = nf4_dq.nf4_codebook().astype(np.float64)
    assert np.max(np.abs(q - ref)) < 5e-7


def test_not_the_uniform_int4_grid():
    # The levels are denser near zero than in the tails (explainer step 1 /
    # teardown sec. 1): the gaps grow monotonically away from zero on each side.
    q = nf4_dq.nf4_codebook().astype(np.float64)
    gaps = np.diff(q)
    assert np.all(np.diff(gaps[7:]) > 0)      # positive side widens outward
    assert np.all(np.diff(gaps[:7]) < 0)      # negative side widens outward


def test_q6_is_the_constructed_float_not_the_parsed_decimal():
    # Both float32 values print as -0.09105004; the construction yields the
    # first.  A table typed from the printed decimals would differ in q_6.
    q = nf4_dq.nf4_codebook()
    assert q.view(np.uint32)[6] == 0xBDBA7871
    assert np.float32(-0.09105004).view(np.uint32) == 0xBDBA7872


# --------------------------------------------------------------------------
# Float4 (E2M1): the comparison storage type of the reading note's
# 'Why NF4 rather than any 4-bit type' table.  Pins from the OCP E2M1
# format constants (largest normal 6, smallest normal 1, subnormal step 0.5,
# one mantissa bit so two values per binade) rather than from the decoder.
# --------------------------------------------------------------------------
def test_fp4_levels_from_format_constants():
    q = nf4_dq.fp4_e2m1_codebook()
    assert q.dtype == np.float32 and q.shape == (16,)
    mags = [0.5]                                   # the one subnormal step
    for e in range(0, 3):                          # binades [1, 2), [2, 4), [4, 8) up to 6
        mags += [2.0 ** e, 1.5 * 2.0 ** e]
    assert max(mags) == 6.0
    expect = sorted({-m for m in mags} | {0.0} | set(mags))
    assert len(expect) == 15
    distinct = np.array(q[:15], np.float64)
    assert np.all(np.diff(distinct) > 0)
    # each level is the float32 rounding of value / 6, the zero level is +0,
    # and the unused code 15 repeats the top level
    assert np.array_equal(q[:15], (np.array(expect, np.float32) / np.float32(6.0)).astype(np.float32))
    assert q[7] == 0 and not np.signbit(q[7])
    assert q[15] == q[14] == np.float32(1.0) and q[0] == np.float32(-1.0)


def test_fp4_decoder_covers_all_sixteen_bit_patterns():
    vals = nf4_dq.e2m1_decode(np.arange(16, dtype=np.uint8)).astype(np.float64)
    assert sorted(set(np.abs(vals))) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert np.array_equal(vals[8:], -vals[:8])      # the sign bit is the top bit


def test_fp4_nearest_level_brute_force_and_ties():
    q = nf4_dq.fp4_e2m1_codebook()
    rng = np.random.default_rng(5)
    x = rng.uniform(-1, 1, 20000).astype(np.float32)
    got = nf4_dq.nearest_level(x, q)
    d = np.abs(x.astype(np.float64)[:, None] - q.astype(np.float64)[None, :])
    assert np.array_equal(got, np.argmin(d, axis=1))
    assert got.max() <= 14                             # code 15 never produced
    # worked values: 0.3 sits nearer 1/3 than 1/4; +-1 and 0 hit their levels
    assert nf4_dq.nearest_level(np.float32([0.3, 1.0, -1.0, 0.0, 0.04]), q).tolist() == [11, 14, 0, 7, 7]
    # the float32 neighbours of the exact midpoint 7/24 between 1/4 and 1/3
    mid = np.float32(7.0 / 24.0)
    below, above = np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1))
    lo = 10 if float(mid) <= 7.0 / 24.0 else 11
    assert nf4_dq.nearest_level(np.float32([below, mid, above]), q).tolist() == [10, lo, 11]


# --------------------------------------------------------------------------
# Float4 (E3M0): the other Float4 row of the same table.  Pins from what the
# format's shape fixes (3 exponent bits and no mantissa bits: one value per
# binade, so consecutive magnitudes differ by exactly 2; seven binades plus
# zero), not from the decoder's arithmetic.
# --------------------------------------------------------------------------
def test_e3m0_levels_from_format_constants():
    q = nf4_dq.fp4_e3m0_codebook()
    assert q.dtype == np.float32 and q.shape == (16,)
    pos = np.array(q[8:15], np.float64)
    assert pos[-1] == 1.0 and np.all(pos[1:] / pos[:-1] == 2.0)   # 2^-6 .. 2^0
    assert pos[0] == 2.0 ** -6
    assert np.array_equal(q[:7], -q[8:15][::-1])                    # symmetric
    assert q[7] == 0 and not np.signbit(q[7])
    assert q[15] == q[14] == np.float32(1.0)
    assert np.all(np.diff(np.array(q[:15], np.float64)) > 0)


def test_e3m0_decoder_covers_all_sixteen_bit_patterns():
    vals = nf4_dq.e3m0_decode(np.arange(16, dtype=np.uint8)).astype(np.float64)
    assert sorted(set(np.abs(vals))) == [0.0] + [2.0 ** e for e in range(-2, 5)]
    assert np.array_equal(vals[8:], -vals[:8])      # the sign bit is the top bit
    assert vals[0] == 0 and np.all(vals[2:8] == 2 * vals[1:7])  # field 0 is zero; each exponent step doubles


def test_e3m0_nearest_level_brute_force_and_ties():
    q = nf4_dq.fp4_e3m0_codebook()
    rng = np.random.default_rng(6)
    # log-uniform magnitudes: the levels crowd towards zero
    x = (np.sign(rng.uniform(-1, 1, 20000)) * 2.0 ** rng.uniform(-9, 0, 20000)).astype(np.float32)
    got = nf4_dq.nearest_level(x, q)
    d = np.abs(x.astype(np.float64)[:, None] - q.astype(np.float64)[None, :])
    assert np.array_equal(got, np.argmin(d, axis=1))
    assert got.max() <= 14
    # every midpoint 3 * 2^-j is a float32, so exact ties occur; they go to
    # the lower index: 3/128 to 1/64 (code 8), -3/128 to -1/32 (code 5),
    # 3/4 to 1/2 (code 13), 1/128 to 0 (code 7), -1/128 to -1/64 (code 6)
    ties = np.float32([3 / 128, -3 / 128, 0.75, 1 / 128, -1 / 128])
    assert nf4_dq.nearest_level(ties, q).tolist() == [8, 5, 13, 7, 6]
    above = np.nextafter(ties, np.float32(2))
    assert nf4_dq.nearest_level(above, q).tolist() == [9, 6, 14, 8, 7]
