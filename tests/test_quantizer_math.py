"""Host checks of the two shortcuts the GPU quantizer takes to reach the
oracle's codes bit for bit (no GPU; float32 arithmetic emulated exactly in
float64):

  * the quotient x = RN(w / m) as q0 = RN(w * y), y = RN(1 / m), corrected
    once with fused multiply-adds (Markstein's correction step for
    round-to-nearest): equal to the correctly rounded quotient whenever the
    quotient is a normal number, for block scales 2^-60 .. 2^60 (outside that
    range the kernel divides);
  * the code as a lookup in 64ths of [-1, 1]: count of thresholds at or below
    the bucket's lower edge, plus one comparison with the threshold inside.

Samples: random (w, m) pairs over the whole scale range and quotients placed
on every level midpoint and its float32 neighbours; every float32 within
2000 ulps of each threshold and of each bucket edge."""
import numpy as np
import pytest

from oracle import nf4_dq

F32, F64 = np.float32, np.float64


def _rn32_of_exact(s, err):
    """RN to float32 of the exact value s + err, where s = RN64(s + err)."""
    c = s.astype(F32)
    cd = c.astype(F64)
    lo = np.where(cd > s, np.nextafter(c, F32(-np.inf)), c)
    hi = np.where(cd < s, np.nextafter(c, F32(np.inf)), c)
    mid = (lo.astype(F64) + hi.astype(F64)) / 2
    at_mid = (lo != hi) & (s == mid)
    lo_even = (lo.view(np.uint32) & 1) == 0
    tie = np.where(err > 0, hi, np.where(err < 0, lo, np.where(lo_even, lo, hi)))
    return np.where(at_mid, tie, c)


def _fma32(x, y, z):
    p = x.astype(F64) * y.astype(F64)  # exact: two 24-bit significands
    zz = z.astype(F64)
    s = p + zz
    bb = s - p
    err = (p - (s - bb)) + (zz - bb)  # s + err == p + z exactly
    return _rn32_of_exact(s, err)


def _corrected_quotient(w, m):
    y = (1.0 / m.astype(F64)).astype(F32)  # RN32(1/m): double rounding is innocuous for division
    q0 = (w.astype(F64) * y.astype(F64)).astype(F32)
    r = _fma32(-q0, m, w)
    return _fma32(r, y, q0)


def _check_quotients(w, m):
    got = _corrected_quotient(w, m)
    ref = (w.astype(F64) / m.astype(F64)).astype(F32)
    bad = got.view(np.uint32) != ref.view(np.uint32)
    # a subnormal quotient may differ by an ulp; it lies far below every threshold
    assert np.all(np.abs(ref[bad].astype(F64)) < 2.0 ** -126), ref[bad][:5]


@pytest.mark.parametrize("seed", [0, 1])
def test_corrected_quotient_is_the_rounded_quotient(seed):
    rng = np.random.default_rng(seed)
    n = 1_000_000
    m = (2.0 ** rng.uniform(-60, 60, n) * rng.uniform(1, 2, n)).astype(F32)
    w = (m.astype(F64) * rng.uniform(-1, 1, n)).astype(F32)
    w = np.where(np.abs(w) > m, m, w).astype(F32)
    _check_quotients(w, m)


@pytest.mark.parametrize("codebook", ["nf4", "fp4", "fp4_e3m0"])
def test_corrected_quotient_next_to_every_midpoint(codebook):
    rng = np.random.default_rng(7)
    lv = nf4_dq.codebook_levels(codebook).astype(F64)
    targets = np.unique(np.concatenate([(lv[:-1] + lv[1:]) / 2, lv]).astype(F32))
    m = (2.0 ** rng.uniform(-60, 60, 20_000) * rng.uniform(1, 2, 20_000)).astype(F32)
    for t in targets:
        w0 = (m.astype(F64) * F64(t)).astype(F32)
        for steps in (-2, -1, 0, 1, 2):
            w = w0
            for _ in range(abs(steps)):
                w = np.nextafter(w, F32(np.inf) if steps > 0 else F32(-np.inf))
            w = np.where(np.abs(w) > m, np.sign(w) * m, w).astype(F32)
            _check_quotients(w, m)


@pytest.mark.parametrize("codebook", ["nf4", "fp4", "fp4_e3m0"])
def test_bucket_lookup_is_the_threshold_count(codebook):
    from bit_nf4_quantized_qlora_amd import qlora as q
    t = np.array(q.qlora_thresholds(q.CODEBOOKS[codebook]), F32)
    count = np.zeros(129, np.int64)
    inside = np.full(129, np.inf, F32)
    for i in range(129):
        lo, hi = (i - 64) / 64.0, (i - 63) / 64.0
        count[i] = np.count_nonzero(t.astype(F64) <= lo)
        k = np.flatnonzero((t.astype(F64) > lo) & (t.astype(F64) < hi))
        assert k.size <= 1
        if k.size:
            inside[i] = t[k[0]]
    edges = (np.arange(129) - 64) / 64.0
    centres = np.concatenate([t[np.abs(t) <= 1], edges.astype(F32)])
    offs = np.arange(-2000, 2001, dtype=np.int64)
    bits = (centres.view(np.int32).astype(np.int64)[:, None] + offs[None, :]).reshape(-1)
    x = np.concatenate([bits.astype(np.int32).view(F32),
                        np.random.default_rng(3).uniform(-1, 1, 2_000_000).astype(F32)])
    x = x[np.isfinite(x) & (np.abs(x) <= 1)]
    b = np.clip(np.floor(x.astype(F64) * 64.0).astype(np.int64) + 64, 0, 128)
    got = count[b] + (x >= inside[b])
    ref = np.searchsorted(t, x, side="right")
    assert np.array_equal(got, ref)
