"""Oracle for the NF4 + double-quantization (DQ) storage encoding.

TEST INFRASTRUCTURE ONLY: a plain, slow CPU statement of the encoding, used
by ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py``.  The product library never imports or calls it.

Every rounding point is an explicit IEEE float32 NumPy operation (NumPy never
fuses a multiply and an add), so the result is defined bit for bit.

Sources (web copies of pages about QLoRA, Dettmers et al. 2023):
  [explainer] "QLoRA, explained." -- the numbered method steps 1-4 and the
              symbol list (W^NF4, c1, c2).
  [teardown]  "QLoRA Paper Breakdown: 4-Bit NormalFloat (NF4), Double
              Quantization, and Paged Optimizers" -- section 2 (codebook),
              section 3 (blockwise quantization, Level 1 / Level 2 of double
              quantization, bit arithmetic), section 4 (dequantization helper).
  [video]     "QLoRA Explained: What Actually Trains in 4 Bits? | Part 2/6" --
              the worked NF4 lookup, the toy three-bit example and the
              bits-per-weight arithmetic.

Readings taken where the pages are silent, ambiguous or garbled (each one is
repeated at the function that applies it):
  * codebook construction: the teardown's section-2 formula evaluates the
    normal quantile at probability 0; read as equally spaced probabilities
    from an outer probability delta to 1/2 for each half (see nf4_codebook);
  * blocks are 64 consecutive elements of the row-major [n, k] tensor, groups
    are 256 consecutive blocks (the last one may be short);
  * an all-zero block normalizes to 0 (code 7);
  * nearest code: exact distances, ties go to the lower index;
  * packing: element 2i in the low nibble of byte i, element 2i+1 high;
  * the mean subtracted before the 8-bit coding is one per tensor, summed in
    float64 sequentially inside each group, then sequentially over groups,
    divided by the block count in float64 and rounded to float32;
  * the second-level constant of a group is max |absmax - mean| over it;
  * the 8-bit float is OCP E4M3FN, round to nearest, ties to even;
  * block scale s = (decode(code8) * group constant) + mean, two separately
    rounded float32 operations; weight = bf16_rne(float32(q[code] * s)).
  * the Float4 (E2M1) storage type of the teardown's data-type comparison
    (section 'Why NF4 rather than any 4-bit type' of the reading note) uses
    the same blockwise rule with the OCP E2M1 value set divided by its
    largest magnitude 6 (see fp4_e2m1_codebook); everything else, double
    quantization included, is unchanged;
  * the Float4 (E3M0) storage type of the same table likewise, with the
    values of a sign + 3-exponent-bit float with no mantissa bits divided by
    their largest magnitude (see fp4_e3m0_codebook).
"""
from __future__ import annotations

import statistics

import numpy as np

F32 = np.float32
F64 = np.float64

BLOCK = 64   # weights per first-level block  [explainer step 2; teardown sec. 3, B_1]
GROUP = 256  # block constants per second-level group  [explainer step 3; teardown sec. 3, B_2]
MEAN_RUN = 256  # group sums per run in the mean's summation order (a reading, not the pages')


# --------------------------------------------------------------------------
# NF4 codebook
# --------------------------------------------------------------------------
def _prob_grid_f32(delta: np.float32, count: int) -> list:
    """``count`` equally spaced float32 probabilities from ``delta`` to 1/2.

    The grid is evaluated from both ends (the first half as delta + i*step,
    the second half as 1/2 - (count-1-i)*step), every operation in float32,
    so that both end points are hit exactly.
    """
    step = F32((F32(0.5) - delta) / F32(count - 1))
    out = []
    for i in range(count):
        if i < count // 2:
            out.append(F32(delta + F32(F32(i) * step)))
        else:
            out.append(F32(F32(0.5) - F32(F32(count - 1 - i) * step)))
    return out


def nf4_codebook() -> np.ndarray:
    """The 16 NF4 levels q_0 < ... < q_15 as float32; the code is the index.

    [explainer step 1; teardown sec. 2 'Step-by-Step Construction of the 16
    NF4 Codebook Values']: levels are standard-normal quantiles; the negative
    half uses 2^(k-1) = 8 quantiles and the positive half 2^(k-1)+1 = 9, each
    half includes 0 and one duplicate zero is dropped, leaving 7 negative
    values, an exact 0 and 8 positive values, normalized into [-1, 1].

    Reading (the teardown's printed quantile formula puts Q at probability 0
    for i = 0, i.e. -infinity, so it cannot be literal): each half takes its
    quantiles at equally spaced probabilities running from an outer
    probability delta down to 1/2.  delta "averages two neighbouring"
    extreme probabilities, those of a 15- and a 16-interval symmetric grid:
    delta = ((1 - 1/30) + (1 - 1/32)) / 2 = 0.96770833...  The probability
    1/2 itself gives the zero (dropped once).  Numerics: delta to 7 decimals,
    the probability grid in float32 from both ends, each quantile in float64
    rounded to float32, and the final normalization by the largest value in
    float32.  Those numerics reproduce all 16 values the teardown prints to 8
    decimals and the video page's 10-digit q_9; the same construction done
    wholly in float64 misses some printed digits by ~2e-7.
    """
    nd = statistics.NormalDist()
    delta = F32(0.9677083)
    positive = [F32(nd.inv_cdf(float(p))) for p in _prob_grid_f32(delta, 9)[:-1]]
    negative = [F32(-nd.inv_cdf(float(p))) for p in _prob_grid_f32(delta, 8)[:-1]]
    levels = np.array(sorted(positive + [F32(0.0)] + negative), dtype=F32)
    return (levels / levels.max()).astype(F32)


def e2m1_decode(codes) -> np.ndarray:
    """OCP E2M1 4-bit float -> float32 (exact).

    Format (OCP microscaling FP4): 1 sign bit, 2 exponent bits with bias 1,
    1 mantissa bit; exponent field 0 is subnormal (m * 2^-1 * 2^(1-1) =
    m / 2); no infinity or NaN.  Values: +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 0x1
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    return (sign * mag).astype(F32)


def fp4_e2m1_codebook() -> np.ndarray:
    """The Float4 (E2M1) level set as 16 float32 levels, ascending.

    [reading note, 'Why NF4 rather than any 4-bit type': Float4 (E2M1) is
    one of the 4-bit storage types NF4 is compared with].  The pages name
    the format only.  Reading: the distinct values of the OCP E2M1 format
    (its +0 and -0 are one level, so there are 15), divided in float32 by
    the largest magnitude 6 so that the block absmax lands on +-1 exactly as
    for NF4; code j is the j-th level in ascending order.  Code 15 is never
    produced by the nearest-level rule (it repeats the top level 1.0, and
    ties go to the lower index); it decodes as 1.0.  The codes are indices
    into this list, not E2M1 bit patterns.
    """
    vals = np.unique(e2m1_decode(np.arange(16, dtype=np.uint8)).astype(F64))  # 15 distinct, ascending
    vals = np.where(vals == 0.0, 0.0, vals)                                    # the zero level is +0
    levels = (vals.astype(F32) / F32(6.0)).astype(F32)
    return np.concatenate([levels, levels[-1:]]).astype(F32)


def e3m0_decode(codes) -> np.ndarray:
    """E3M0 4-bit float -> float32 (exact).

    Format: 1 sign bit (bit 3), 3 exponent bits with bias 3, no mantissa
    bits.  Reading (the pages name the format only): exponent field 0 is the
    subnormal range, which with no fraction bits holds only zero; fields 1..7
    are 2^(e - 3); no field is kept for infinity or NaN, as in the OCP
    sub-byte floats.  Values: +-{0, 1/4, 1/2, 1, 2, 4, 8, 16}.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = c & 0x7
    mag = np.where(e == 0, 0.0, np.exp2(e - 3.0))
    return (sign * mag).astype(F32)


def fp4_e3m0_codebook() -> np.ndarray:
    """The Float4 (E3M0) level set as 16 float32 levels, ascending.

    [reading note, 'Why NF4 rather than any 4-bit type': Float4 (E3M0) is the
    other Float4 variant NF4 is compared with].  Built as fp4_e2m1_codebook
    is: the 15 distinct values of the format (one zero level), divided by the
    largest magnitude 16 so that the block absmax lands on +-1 (the division
    is exact: the levels are 0 and +-2^-j, j = 0..6), code j the j-th level
    in ascending order, and code 15 repeating the top level 1.0 (never
    produced by the nearest-level rule).
    """
    vals = np.unique(e3m0_decode(np.arange(16, dtype=np.uint8)).astype(F64))  # 15 distinct, ascending
    vals = np.where(vals == 0.0, 0.0, vals)                                    # the zero level is +0
    levels = (vals.astype(F32) / F32(16.0)).astype(F32)
    return np.concatenate([levels, levels[-1:]]).astype(F32)


CODEBOOKS = ("nf4", "fp4", "fp4_e3m0")


def codebook_levels(codebook: str = "nf4") -> np.ndarray:
    """The 16 float32 levels of a storage type: 'nf4' (the default, NormalFloat),
    'fp4' (Float4 E2M1) or 'fp4_e3m0' (Float4 E3M0)."""
    if codebook == "nf4":
        return nf4_codebook()
    if codebook == "fp4":
        return fp4_e2m1_codebook()
    if codebook == "fp4_e3m0":
        return fp4_e3m0_codebook()
    raise ValueError(f"unknown codebook {codebook!r}")


# --------------------------------------------------------------------------
# BF16 and E4M3FN scalar formats
# --------------------------------------------------------------------------
def bf16_rne_bits(x) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even.

    [reading note 'What the method actually is'; explainer step 4]: the
    computation type is BFloat16.  The rounding mode is not stated; reading:
    IEEE round-to-nearest-even on the upper 16 bits.  Denormals are kept.
    """
    u = np.ascontiguousarray(x, dtype=F32).view(np.uint32).astype(np.uint64)
    if np.isnan(np.asarray(x, dtype=F32)).any():
        raise ValueError("NaN has no defined bf16 code here")
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(F32).astype(F64)


def e4m3fn_decode(codes) -> np.ndarray:
    """OCP E4M3FN byte -> float32 (exact).

    Format (OCP 8-bit floating point, E4M3 'FN' variant): 1 sign bit, 4
    exponent bits with bias 7, 3 mantissa bits; exponent field 0 is
    subnormal (m * 2^-9); S.1111.111 is NaN; there is no infinity.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return (sign * mag).astype(F32)


_E4M3_MAG_CODES = np.arange(0x7F, dtype=np.uint8)            # 0x00..0x7E: finite, >= 0
_E4M3_MAG_VALUES = e4m3fn_decode(_E4M3_MAG_CODES).astype(F64)  # ascending


def e4m3fn_encode_rne(x) -> np.ndarray:
    """float32 -> OCP E4M3FN byte, round to nearest, ties to the even code.

    [explainer step 3 'quantized to 8-bit floats'; teardown sec. 3 Level 2
    quantize_fp8].  The 8-bit float format is not named on the pages;
    reading: OCP E4M3FN.  The sign is kept, so a negative value that rounds
    to zero encodes 0x80.  Only |x| <= 448 is accepted (here |x| <= 1 always).

    Brute force: the exact nearest of the 127 finite non-negative codes to
    |x|; on a tie the code whose mantissa LSB is 0.  float64 distances are
    exact here except when |x| is far below 2^-9, where code 0 wins anyway.
    """
    xf = np.asarray(x, dtype=F32).reshape(-1)
    if not np.isfinite(xf).all() or (np.abs(xf) > 448.0).any():
        raise ValueError("E4M3FN encode takes finite |x| <= 448")
    out = np.empty(xf.size, dtype=np.uint8)
    for s in range(0, xf.size, 1 << 16):
        a = np.abs(xf[s:s + (1 << 16)].astype(F64))
        d = np.abs(a[:, None] - _E4M3_MAG_VALUES[None, :])
        first = np.argmin(d, axis=1)                      # lowest code among the minima
        nxt = np.minimum(first + 1, _E4M3_MAG_VALUES.size - 1)
        tie = (d[np.arange(a.size), nxt] == d[np.arange(a.size), first]) & (nxt != first)
        pick = np.where(tie & (first % 2 == 1), nxt, first)
        out[s:s + a.size] = pick.astype(np.uint8)
    neg = np.signbit(xf)
    out = np.where(neg, out | np.uint8(0x80), out).astype(np.uint8)
    return out.reshape(np.shape(x))


# --------------------------------------------------------------------------
# Level 1: blockwise absmax + nearest level
# --------------------------------------------------------------------------
def nearest_level(normalized, levels) -> np.ndarray:
    """Index of the nearest level; ties go to the lower index.

    [explainer step 2 'stored as the 4-bit index of the nearest NF4 value';
    teardown sec. 3 Level 1 argmin_j].  The tie-break is not stated; reading:
    the lower index (first argmin).  Distances are taken in float64; for
    float32 operands in [-1, 1] they are exact unless one operand is below
    2^-29 of the other, and then the nearer level is unambiguous.
    """
    n = np.asarray(normalized, dtype=F32).reshape(-1).astype(F64)
    lv = np.asarray(levels, dtype=F32).astype(F64)
    out = np.empty(n.size, dtype=np.uint8)
    for s in range(0, n.size, 1 << 18):
        d = np.abs(n[s:s + (1 << 18), None] - lv[None, :])
        out[s:s + (1 << 18)] = np.argmin(d, axis=1)
    return out.reshape(np.shape(normalized))


def block_absmax(x, block: int = BLOCK) -> np.ndarray:
    """Per-block absolute maximum (float32, exact) of consecutive blocks of a
    flat or row-major float32 tensor [explainer step 2]."""
    xb = np.asarray(x, dtype=F32).reshape(-1, block)
    return np.abs(xb).max(axis=1).astype(F32)


def blockwise_quantize(x, levels, block: int):
    """Blockwise absmax quantization of a flat float32 vector.

    [explainer step 2; teardown sec. 3]: the vector is cut into consecutive
    blocks; each block's absolute maximum rescales it into [-1, 1]
    (normalized = float32(x / absmax), IEEE division) and each element keeps
    the index of the nearest level.  Reading for an all-zero block (absmax 0,
    not on the pages): every element normalizes to 0.

    Returns (codes [nblocks, block] uint8, absmax [nblocks] float32).
    """
    xb = np.asarray(x, dtype=F32).reshape(-1, block)
    if not np.isfinite(xb).all():
        raise ValueError("weights must be finite")
    absmax = block_absmax(xb, block)
    safe = np.where(absmax > 0, absmax, F32(1.0)).astype(F32)
    normalized = np.where(absmax[:, None] > 0, xb / safe[:, None], F32(0.0)).astype(F32)
    return nearest_level(normalized, levels), absmax


def pack_nibbles(codes) -> np.ndarray:
    """Two 4-bit codes per byte: byte i = code[2i] | code[2i+1] << 4.

    Two codes per byte is the storage; the nibble order is not on the pages
    (reading: the even element in the low nibble).
    """
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    return (c[0::2] | (c[1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(p.size * 2, dtype=np.uint8)
    out[0::2] = p & 0x0F
    out[1::2] = p >> 4
    return out


# --------------------------------------------------------------------------
# Level 2: double quantization of the block constants
# --------------------------------------------------------------------------
def _rows_padded(values, width: int, fill) -> np.ndarray:
    """values as rows of `width`, the last row padded with `fill`."""
    v = np.asarray(values).reshape(-1)
    rows = -(-v.size // width)
    out = np.full(rows * width, fill, dtype=v.dtype)
    out[:v.size] = v
    return out.reshape(rows, width)


def _groups_padded(values, fill) -> np.ndarray:
    return _rows_padded(values, GROUP, fill)


def dq_offset(absmax) -> np.float32:
    """The mean of the block absmax values, subtracted before 8-bit coding.

    [explainer step 3 'after subtracting their mean'; teardown sec. 3 Level 2
    mean(c_1)].  Reading: one mean per tensor (the video page's idealized
    4.126953125 bits/weight leaves mean offsets out, which a per-group mean
    would not allow).  The pages fix no summation order; this one is fixed so
    that the float32 result is unique, in three float64 levels, each a
    left-to-right fold: the block absmax values inside each group of 256
    blocks, then the group sums inside each run of MEAN_RUN consecutive
    groups, then the run sums; the total is divided by the block count in
    float64 and rounded to float32.  (np.add.accumulate is a left-to-right
    fold; the zero padding of a short last group or run adds +0.0, which
    leaves a non-negative sum unchanged.  A tensor of at most MEAN_RUN groups
    has one run, whose fold is the fold over all group sums.)
    """
    a = np.asarray(absmax, dtype=F32).astype(F64)
    if a.size == 0:
        raise ValueError("no blocks")
    per_group = np.add.accumulate(_groups_padded(a, 0.0), axis=1)[:, -1]
    per_run = np.add.accumulate(_rows_padded(per_group, MEAN_RUN, 0.0), axis=1)[:, -1]
    total = np.add.accumulate(per_run)[-1]
    return F32(total / F64(a.size))


def dq_encode(absmax, offset):
    """Second-level coding of the block constants.

    [explainer step 3; teardown sec. 3 Level 2]: c8_b = quantize_fp8(
    (absmax_b - mean) / c_g), one float32 constant c_g per group of 256.
    dev_b = float32(absmax_b - mean); c_g = max |dev_b| over the group
    (reading: the blockwise absmax rule of level 1 applied again, so each
    group codes into [-1, 1]); c8_b = E4M3FN(float32(dev_b / c_g)), and
    c8_b = 0x00 when c_g = 0.

    Returns (scale_code [nb] uint8, group_amax [ng] float32).
    """
    a = np.asarray(absmax, dtype=F32).reshape(-1)
    dev = (a - F32(offset)).astype(F32)
    g = _groups_padded(dev, F32(0.0))
    amax = np.abs(g).max(axis=1).astype(F32)
    per_block_amax = np.repeat(amax, GROUP)[:a.size]
    safe = np.where(per_block_amax > 0, per_block_amax, F32(1.0)).astype(F32)
    ratio = (dev / safe).astype(F32)
    code = e4m3fn_encode_rne(ratio)
    code = np.where(per_block_amax > 0, code, np.uint8(0)).astype(np.uint8)
    return code, amax


def dq_block_scale(scale_code, group_amax, offset) -> np.ndarray:
    """s_b = float32(float32(decode(c8_b) * c_g) + mean).

    [teardown sec. 4 'Dequantization Helper': dequant(c_1^(FP8), c_2^(FP32))].
    The operation order is not stated; reading: multiply, then add the mean,
    each rounded to float32 (no fused multiply-add).
    """
    c = np.asarray(scale_code, dtype=np.uint8).reshape(-1)
    amax = np.repeat(np.asarray(group_amax, dtype=F32), GROUP)[:c.size]
    return ((e4m3fn_decode(c) * amax).astype(F32) + F32(offset)).astype(F32)


# --------------------------------------------------------------------------
# Whole-tensor quantize / dequantize
# --------------------------------------------------------------------------
def storage_sizes(n: int, k: int):
    """(packed bytes, scale-code bytes, group constants) for an [n, k] weight."""
    nb = n * k // BLOCK
    return n * k // 2, nb, -(-nb // GROUP)


def quantize_nf4_dq(W, codebook: str = "nf4") -> dict:
    """NF4 + DQ encoding of a float32 weight W [n, k] (row-major, k % 64 == 0);
    ``codebook='fp4'`` stores Float4 (E2M1) codes instead of NF4.

    [explainer steps 1-3; teardown sec. 3].  Returns a dict with the stored
    buffers ``packed``, ``scale_code``, ``group_amax``, ``offset`` and the
    intermediates ``codes`` [n*k], ``absmax`` [nb], ``dev`` [nb].
    """
    W = np.asarray(W, dtype=F32)
    if W.ndim != 2 or W.shape[1] % BLOCK or W.size == 0:
        raise ValueError("W must be [n, k] with n >= 1, k >= 64 and k % 64 == 0")
    codes, absmax = blockwise_quantize(W.reshape(-1), codebook_levels(codebook), BLOCK)
    offset = dq_offset(absmax)
    scale_code, group_amax = dq_encode(absmax, offset)
    return {
        "packed": pack_nibbles(codes),
        "scale_code": scale_code,
        "group_amax": group_amax,
        "offset": offset,
        "codes": codes.reshape(-1),
        "absmax": absmax,
        "dev": (absmax - offset).astype(F32),
    }


def quantize_single_level(W, codebook: str = "nf4") -> dict:
    """Single-level blockwise quantization: the codes of quantize_nf4_dq and
    one float32 constant per block, the block absmax itself, with no second
    level.

    [teardown sec. 3 'The Hidden Memory Overhead of Block Scales': one
    float32 scale per 64 weights, 4 + 32/64 = 4.5 bits per parameter, the
    layout double quantization improves on].  Returns ``packed``, ``absmax``
    [nb] float32 and ``codes`` [n*k].
    """
    W = np.asarray(W, dtype=F32)
    if W.ndim != 2 or W.shape[1] % BLOCK or W.size == 0:
        raise ValueError("W must be [n, k] with n >= 1, k >= 64 and k % 64 == 0")
    codes, absmax = blockwise_quantize(W.reshape(-1), codebook_levels(codebook), BLOCK)
    return {"packed": pack_nibbles(codes), "absmax": absmax, "codes": codes.reshape(-1)}


def dequant_single_level_bf16(packed, absmax, n: int, k: int, codebook: str = "nf4") -> np.ndarray:
    """W_hat [n, k] bfloat16 bits for single-level constants: s_b = absmax_b,
    w_hat = bf16_rne(float32(q[code] * absmax_b)) [teardown sec. 4 with the
    float32 constant used as stored]."""
    codes = unpack_nibbles(packed)
    if codes.size != n * k:
        raise ValueError("packed size does not match n*k")
    return dequant_blocks_bf16(codes.reshape(-1, BLOCK), np.asarray(absmax, F32), codebook).reshape(n, k)


def dequant_bf16(packed, scale_code, group_amax, offset, n: int, k: int, codebook: str = "nf4") -> np.ndarray:
    """W_hat [n, k] as bfloat16 bit patterns (uint16).

    [explainer step 4; teardown sec. 4 'Dequantization Helper':
    NF4_CODEBOOK[W_NF4] * dequant(c_1^(FP8), c_2^(FP32))]:
    w_hat = bf16_rne(float32(q[code] * s_b)).
    """
    codes = unpack_nibbles(packed)
    if codes.size != n * k:
        raise ValueError("packed size does not match n*k")
    s = dq_block_scale(scale_code, group_amax, offset)
    return dequant_blocks_bf16(codes.reshape(-1, BLOCK), s, codebook).reshape(n, k)


def dequant_blocks_bf16(codes, scales, codebook: str = "nf4") -> np.ndarray:
    """w_hat = bf16_rne(float32(q[code] * s_b)) for blocks of codes
    [nblk, 64] with their block scales s_b [nblk] (any subset of blocks)."""
    q = codebook_levels(codebook)[np.asarray(codes, dtype=np.uint8)].reshape(-1, BLOCK)
    prod = (q * np.asarray(scales, dtype=F32)[:, None]).astype(F32)
    return bf16_rne_bits(prod)


def storage_bits_per_weight(enc: dict, n: int, k: int) -> float:
    """Stored bits per weight from the actual buffers, excluding the one
    float32 mean per tensor, as the video page's idealized arithmetic does:
    4 (code) + 8/64 (8-bit constant) + 32/(64*256) (group constant)."""
    bits = 8 * (enc["packed"].nbytes + enc["scale_code"].nbytes + enc["group_amax"].nbytes)
    return bits / (n * k)
