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
