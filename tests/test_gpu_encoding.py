"""GPU parity of qlora_quantize_nf4_dq and qlora_dequant_bf16 against the
oracle: bit-exact codes, packed bytes, 8-bit scale codes, group constants,
mean offset and BF16 weights."""
import numpy as np
import pytest
import torch

from bit_nf4_quantized_qlora_amd import inputs as I
from gpu_helpers import assert_encoding_equal, encoding_to_host, gpu_quantize, host_bf16, note
from oracle import nf4_dq
from oracle_views import OracleWeight

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    from bit_nf4_quantized_qlora_amd import qlora
    return qlora


def _gpu_dequant(q, w):
    out = torch.empty(w.n, w.k, dtype=torch.bfloat16, device="cuda")
    q.qlora_dequant_bf16(w, out)
    torch.cuda.synchronize()
    return host_bf16(out)


def _full_check(q, W, ctx, codebook="nf4"):
    note(f"[encoding] {ctx} shape={W.shape} codebook={codebook}")
    n, k = W.shape
    w = gpu_quantize(q, W, codebook)
    got = encoding_to_host(w)
    ref = nf4_dq.quantize_nf4_dq(W, codebook)
    assert_encoding_equal(got, ref, ctx)
    wh = _gpu_dequant(q, w)
    ref_wh = nf4_dq.dequant_bf16(ref["packed"], ref["scale_code"], ref["group_amax"], ref["offset"], n, k, codebook)
    bad = np.flatnonzero(wh.reshape(-1) != ref_wh.reshape(-1))
    assert bad.size == 0, f"{ctx} dequant: {bad.size} differ, first {bad[:5]}"


def test_tiny_workload(q):
    w = I.WORKLOADS["tiny"]
    _full_check(q, I.weight(w, 0), "tiny")


@pytest.mark.parametrize("codebook", ["nf4", "fp4", "fp4_e3m0"])
def test_decision_thresholds_and_special_values(q, codebook):
    """Blocks whose absmax is exactly 1 carry the 15 thresholds, their float32
    neighbours, every level, signed zeros and subnormals; other blocks scale
    the same pattern, hold a single nonzero, or are all zero."""
    t = np.array(q.qlora_thresholds(q.CODEBOOKS[codebook]), np.float32)
    t = t[t <= 1]  # Float4's top threshold lies above every normalized weight
    lv = nf4_dq.codebook_levels(codebook)
    down = np.nextafter(t, np.float32(-np.inf), dtype=np.float32)
    vals = np.concatenate([t, down, lv, np.array([0.0, -0.0, 1e-45, -1e-45, 1e-38, -3e-39], np.float32)])
    rows = []
    for start in range(0, vals.size, 63):
        blk = np.zeros(64, np.float32)
        chunk = vals[start:start + 63]
        blk[0] = 1.0
        blk[1:1 + chunk.size] = chunk
        rows.append(blk)
    base = np.stack(rows)
    scaled = np.concatenate([base * np.float32(s) for s in (1.0, 0.02, 3.0e-3, 7.5e1, 1e-30)])
    single = np.zeros((4, 64), np.float32)
    single[0, 17] = -0.01
    single[1, 63] = 2.5
    single[2, 0] = 1e-40
    W = np.concatenate([scaled, single, np.zeros((3, 64), np.float32)]).astype(np.float32)
    _full_check(q, W, "thresholds", codebook)


@pytest.mark.parametrize("codebook", ["nf4", "fp4", "fp4_e3m0"])
@pytest.mark.parametrize("shape,seed", [((5, 3840), 34), ((300, 640), 35), ((1024, 4096), 36)])
def test_single_level_encoding(q, shape, seed, codebook):
    """Single-level constants (one float32 absmax per block): packed bytes and
    absmax bit-exact, and the BF16 dequantization with s_b = absmax_b."""
    W = I.custom_weight(*shape, seed=seed)
    note(f"[encoding] single-level {shape} codebook={codebook}")
    n, k = W.shape
    w = gpu_quantize(q, W, codebook, "fp32")
    torch.cuda.synchronize()
    ref = nf4_dq.quantize_single_level(W, codebook)
    assert np.array_equal(w.packed.cpu().numpy(), ref["packed"]), "packed"
    assert np.array_equal(w.absmax.cpu().numpy().view(np.uint32), ref["absmax"].view(np.uint32)), "absmax"
    wh = _gpu_dequant(q, w)
    ref_wh = nf4_dq.dequant_single_level_bf16(ref["packed"], ref["absmax"], n, k, codebook)
    bad = np.flatnonzero(wh.reshape(-1) != ref_wh.reshape(-1))
    assert bad.size == 0, f"single-level dequant: {bad.size} differ, first {bad[:5]}"


@pytest.mark.parametrize("codebook", ["fp4", "fp4_e3m0"])
@pytest.mark.parametrize("shape,seed", [((5, 3840), 31), ((300, 640), 32), ((1024, 4096), 33)])
def test_fp4_encoding(q, shape, seed, codebook):
    """Float4 (E2M1, E3M0) storage: the same bit-exact bar on ragged and full groups."""
    _full_check(q, I.custom_weight(*shape, seed=seed), f"{codebook}{shape}", codebook)


@pytest.mark.parametrize("shape,seed", [((1, 64), 1), ((5, 3840), 2), ((7, 64 * 37), 3), ((64, 4096), 4),
                                        ((300, 640), 5)])
def test_ragged_groups(q, shape, seed):
    _full_check(q, I.custom_weight(*shape, seed=seed), f"ragged{shape}")


def test_degenerate_tensors(q):
    _full_check(q, np.zeros((16, 512), np.float32), "all-zero")
    _full_check(q, np.tile(np.linspace(-0.5, 0.5, 64, dtype=np.float32), (32, 4)), "constant-absmax")
    g = np.random.default_rng(12)
    heavy = (g.standard_t(2, size=(128, 1024)) * 0.02).astype(np.float32)
    _full_check(q, heavy, "student-t(2)")
    _full_check(q, (I.custom_weight(64, 256, seed=6) * np.float32(1e30)).astype(np.float32), "huge")
    _full_check(q, (I.custom_weight(64, 256, seed=7) * np.float32(1e-36)).astype(np.float32), "denormal-range")


def test_q_proj_full_tensor(q):
    w = I.WORKLOADS["q_proj_7b"]
    _full_check(q, I.weight(w, 0), "q_proj_7b")


@pytest.mark.parametrize("k", [32768, 33280])
def test_mean_offset_past_one_staging_pass(q, k):
    """A weight of 4,194,304 blocks (k = 32768: 16,384 groups, 64 runs of
    group sums, the most one staging pass holds, so the mean and the scale
    encoding share one launch) or 4,259,840 blocks (k = 33280: 16,640
    groups, 65 runs: the mean's run folds take two passes through LDS, in a
    launch of their own).  One nonzero per block makes every absmax a known
    draw, so the oracle's offset, scale codes and group constants come from
    those values alone; the packed codes of every block's first byte are
    checked too (the nonzero codes to the top or bottom level, the rest to
    zero)."""
    n = 8192  # k / 64 blocks per row
    nb = n * k // 64
    note(f"[encoding] mean over {nb} blocks, {-(-nb // 256)} groups")
    rng = np.random.default_rng(21)
    a = (2.0 ** rng.uniform(-9, 2, nb)).astype(np.float32)
    sign = np.where(rng.random(nb) < 0.5, -1.0, 1.0).astype(np.float32)
    W = np.zeros((nb, 64), np.float32)
    W[:, 0] = a * sign
    W = W.reshape(n, k)
    w = gpu_quantize(q, W)
    del W
    got = encoding_to_host(w)
    off = nf4_dq.dq_offset(a)
    assert np.float32(got["offset"]).view(np.uint32) == np.float32(off).view(np.uint32), "offset"
    code, amax = nf4_dq.dq_encode(a, off)
    assert np.array_equal(got["scale_code"], code), "scale_code"
    assert np.array_equal(got["group_amax"].view(np.uint32), amax.view(np.uint32)), "group_amax"
    first = got["packed"].reshape(nb, 32)[:, 0]
    assert np.array_equal(first, np.where(sign > 0, 0x7F, 0x70).astype(np.uint8)), "first byte of each block"
    assert np.all(got["packed"].reshape(nb, 32)[:, 1:] == 0x77), "the zero weights"


@pytest.mark.parametrize("wname,li", [("up_65b", 0)] + [("block_65b", i) for i in range(7)])
def test_full_size_sampled(q, wname, li):
    """Full-size 65B layers (the 7B MLP layers are compared whole in the
    linear tests): every scale code, group constant and the offset compared
    whole; packed bytes and BF16 weights on a random row of every 256-row
    group plus both ends."""
    wl = I.WORKLOADS[wname]
    W = I.weight(wl, li)
    note(f"[encoding] {wname}[{li}] {W.shape} sampled per 256-row group")
    n, k = W.shape
    ow = OracleWeight(W)
    w = gpu_quantize(q, W)
    got = encoding_to_host(w)
    assert np.array_equal(got["scale_code"], ow.scale_code), "scale_code"
    assert np.array_equal(got["group_amax"].view(np.uint32), ow.group_amax.view(np.uint32)), "group_amax"
    assert np.float32(got["offset"]).view(np.uint32) == np.float32(ow.offset).view(np.uint32), "offset"
    g = np.random.default_rng(li)
    rows = np.unique(np.concatenate([[0, n - 1]] + [g.integers(r0, min(r0 + 256, n), 1) for r0 in range(0, n, 256)]))
    gp = got["packed"].reshape(n, k // 2)[rows]
    assert np.array_equal(gp, ow.row_packed(rows)), "packed rows"
    wh = _gpu_dequant(q, w)[rows]
    assert np.array_equal(wh, ow.row_what_bits(rows)), "dequant rows"
