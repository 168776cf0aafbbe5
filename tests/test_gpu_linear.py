"""GPU parity of qlora_linear_fwd / qlora_linear_bwd against the fp64
oracle on the same dequantized weights: relative Frobenius error <= 5e-3
and max |diff| <= 2e-2 * max |ref| for Y, H, dX, dA and dB."""
import numpy as np
import pytest
import torch

from bit_nf4_quantized_qlora_amd import inputs as I
from gpu_helpers import Linear, assert_close, assert_encoding_equal, encoding_to_host, gpu_quantize, host_bf16, note
from oracle import nf4_dq
from oracle_views import OracleWeight, bf16_f64, bwd, fwd

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    from bit_nf4_quantized_qlora_amd import qlora
    return qlora


def _run_full(q, W, X, A, B, dY, r, alpha, ctx, h_none=False, want_dx=True, codebook="nf4", scales="dq"):
    """Full comparison of every output (small shapes)."""
    note(f"[linear] {ctx} W={W.shape} M={X.shape[0]} r={r} alpha={alpha} codebook={codebook} scales={scales}")
    ow = OracleWeight(W, codebook, scales)
    What = bf16_f64(ow.row_what_bits(np.arange(W.shape[0])))
    Xf, Af, Bf, dYf = bf16_f64(X), bf16_f64(A), bf16_f64(B), bf16_f64(dY)
    Yr, Hr = fwd(Xf, What, Af, Bf, alpha)
    dXr, dAr, dBr, _ = bwd(Xf, dYf, What, Af, Bf, alpha)
    lin = Linear(q, gpu_quantize(q, W, codebook, scales), X, A, B, r, alpha)
    Y, H = lin.fwd()
    dX, dA, dB = lin.bwd(dY, H=None if h_none else H, want_dx=want_dx)
    torch.cuda.synchronize()
    if X.shape[0]:
        assert_close(bf16_f64(host_bf16(Y)), Yr, f"{ctx} Y")
        assert_close(H.cpu().numpy(), Hr, f"{ctx} H")
        if want_dx:
            assert_close(bf16_f64(host_bf16(dX)), dXr, f"{ctx} dX")
    assert_close(bf16_f64(host_bf16(dA)), dAr, f"{ctx} dA")
    assert_close(bf16_f64(host_bf16(dB)), dBr, f"{ctx} dB")


def _workload_inputs(wl, li, m):
    W = I.weight(wl, li)
    A, B = I.adapters(wl, li)
    return W, I.activation(wl, li, m), A, B, I.grad_output(wl, li, m)


def test_tiny_workload(q):
    wl = I.WORKLOADS["tiny"]
    W, X, A, B, dY = _workload_inputs(wl, 0, wl.ms[0])
    _run_full(q, W, X, A, B, dY, wl.r, wl.alpha, "tiny")


def test_q_proj_full(q):
    wl = I.WORKLOADS["q_proj_7b"]
    W, X, A, B, dY = _workload_inputs(wl, 0, wl.ms[0])
    _run_full(q, W, X, A, B, dY, wl.r, wl.alpha, "q_proj_7b")


@pytest.mark.parametrize("n,k,m,r,alpha,seed", [
    (200, 192, 37, 5, -3.5, 1),     # ragged n (not a multiple of 8), ragged M, odd rank, negative alpha
    (1, 64, 1, 1, 16.0, 2),         # one row, one block
    (300, 640, 130, 100, 32.0, 3),  # rank 100, partial tiles on every axis
    (96, 256, 65, 128, 16.0, 4),    # maximum rank
    (256, 1024, 300, 16, 0.0, 5),   # alpha = 0: adapters contribute nothing to Y
    (640, 512, 200, 80, 16.0, 6),   # rank 80 (padded to 96), n % 64 == 0: the backward tile kernel
    (1088, 320, 96, 64, 8.0, 7),    # k % 256 != 0 (5 blocks per row), 17 backward row blocks
    (512, 768, 520, 48, 16.0, 8),   # three m tiles, rank 48 (padded to 64)
])
def test_edge_shapes(q, n, k, m, r, alpha, seed):
    W = I.custom_weight(n, k, seed)
    X = I.custom_bf16((m, k), seed, 1)
    dY = I.custom_bf16((m, n), seed, 2)
    A = I.custom_bf16((r, k), seed, 3, bound=0.05)
    B = I.custom_bf16((n, r), seed, 4, bound=0.05)
    _run_full(q, W, X, A, B, dY, r, alpha, f"edge n{n} k{k} m{m} r{r}")


# Shapes whose tile launches split the contraction (few tiles, long
# contraction), each with what it exercises; test_split_shapes_take_the_split_path
# checks the plan so the cases cannot silently stop covering it.
SPLIT_CASES = [
    (640, 4096, 300, 64, 16.0, 61),    # fwd 8 splits x 8 steps, two m tiles (ragged); dX 2 splits, the last 2 steps
    (1000, 2560, 77, 16, 16.0, 62),    # ragged n (1000) and M: fwd 5 splits; dX on the general kernel
    (300, 3200, 50, 8, -2.0, 63),      # 50 steps: last fwd split of 2 steps inside a partial super-step
    (1088, 320, 96, 64, 8.0, 64),      # dX: 17 row steps as splits of 8, 8 and 1 (a partial super-step)
    (2048, 4096, 512, 64, 16.0, 65),   # M = 512 on both passes with rank 64 (the q_proj regime, smaller n)
    (512, 8192, 33, 128, 16.0, 66),    # maximum rank on split 0, 128 steps
]


@pytest.mark.parametrize("n,k,m,r,alpha,seed", SPLIT_CASES)
def test_split_contraction(q, n, k, m, r, alpha, seed):
    """Tile launches with a split contraction: every output compared."""
    W = I.custom_weight(n, k, seed)
    X = I.custom_bf16((m, k), seed, 1)
    dY = I.custom_bf16((m, n), seed, 2)
    A = I.custom_bf16((r, k), seed, 3, bound=0.05)
    B = I.custom_bf16((n, r), seed, 4, bound=0.05)
    _run_full(q, W, X, A, B, dY, r, alpha, f"split n{n} k{k} m{m} r{r} plan {q.qlora_linear_plan(m, n, k, r)}")


def test_split_shapes_take_the_split_path(q):
    plans = [q.qlora_linear_plan(m, n, k, r) for n, k, m, r, _, _ in SPLIT_CASES]
    assert all(p["fwd_path"] == q.QLORA_PATH_TILE for p in plans)
    assert sum(p["fwd_splits"] > 1 for p in plans) >= 5
    assert sum(p["dx_path"] == q.QLORA_PATH_TILE and p["dx_splits"] > 1 for p in plans) >= 3
    assert plans[3]["dx_splits"] == 3 and plans[0]["fwd_splits"] == 8


@pytest.mark.parametrize("n,k,m,r,alpha,seed", [
    (300, 768, 5, 100, 32.0, 11),    # two ragged row groups, one 4-block unit per workgroup, rank 100
    (1000, 4096, 3, 16, 16.0, 12),   # 256 workgroups, ragged last group
    (4000, 2560, 7, 8, -2.0, 13),    # odd M, groups split across workgroups
    (2048, 8192, 16, 64, 16.0, 14),  # M = 16, 16 blocks per workgroup
    (64, 256, 2, 1, 16.0, 15),       # one partial row group, one unit, rank 1
    (300, 640, 4, 8, 16.0, 16),      # k % 256 != 0: the tile kernels serve M <= 16 too
])
def test_small_m_shapes(q, n, k, m, r, alpha, seed):
    """M <= 16 takes the GEMV forward when k % 256 == 0; every output is compared."""
    W = I.custom_weight(n, k, seed)
    X = I.custom_bf16((m, k), seed, 1)
    dY = I.custom_bf16((m, n), seed, 2)
    A = I.custom_bf16((r, k), seed, 3, bound=0.05)
    B = I.custom_bf16((n, r), seed, 4, bound=0.05)
    _run_full(q, W, X, A, B, dY, r, alpha, f"small-M n{n} k{k} m{m} r{r}")


@pytest.mark.parametrize("codebook", ["fp4", "fp4_e3m0"])
@pytest.mark.parametrize("n,k,m,r,alpha,seed", [
    (640, 512, 300, 64, 16.0, 41),   # tile kernels, backward tile (n % 64 == 0), two m tiles
    (200, 192, 37, 5, -3.5, 42),     # ragged everything, fallback backward
    (1000, 4096, 3, 16, 16.0, 43),   # small-M GEMV forward
])
def test_fp4_linear(q, n, k, m, r, alpha, seed, codebook):
    """Float4 (E2M1, E3M0) weights through every forward / backward path."""
    W = I.custom_weight(n, k, seed)
    X = I.custom_bf16((m, k), seed, 1)
    dY = I.custom_bf16((m, n), seed, 2)
    A = I.custom_bf16((r, k), seed, 3, bound=0.05)
    B = I.custom_bf16((n, r), seed, 4, bound=0.05)
    _run_full(q, W, X, A, B, dY, r, alpha, f"{codebook} n{n} k{k} m{m} r{r}", codebook=codebook)


@pytest.mark.parametrize("n,k,m,r,alpha,seed,codebook", [
    (640, 512, 300, 64, 16.0, 51, "nf4"),   # tile kernels both ways
    (200, 192, 37, 5, -3.5, 52, "fp4"),     # ragged everything, fallback backward
    (1000, 4096, 3, 16, 16.0, 53, "nf4"),   # M <= 16: the GEMV with float32 block constants
    (640, 512, 300, 64, 16.0, 54, "fp4_e3m0"),
    (300, 1024, 16, 8, 2.0, 55, "fp4"),     # the GEMV at M = 16, rows past a row group, Float4
    (4352, 4096, 1, 64, 16.0, 56, "nf4"),   # the GEMV at M = 1: 272 four-block units on 256 workgroups, so ranges straddle row groups
])
def test_single_level_linear(q, n, k, m, r, alpha, seed, codebook):
    """Single-level float32 block constants through forward and backward
    (M <= 16 with k % 256 == 0: the small-M GEMV forward)."""
    if m <= 16 and k % 256 == 0:
        assert q.qlora_linear_plan(m, n, k, r, q.QLORA_SCALES_FP32)["fwd_path"] == q.QLORA_PATH_GEMV
    W = I.custom_weight(n, k, seed)
    X = I.custom_bf16((m, k), seed, 1)
    dY = I.custom_bf16((m, n), seed, 2)
    A = I.custom_bf16((r, k), seed, 3, bound=0.05)
    B = I.custom_bf16((n, r), seed, 4, bound=0.05)
    _run_full(q, W, X, A, B, dY, r, alpha, f"single-level n{n} k{k} m{m} r{r}", codebook=codebook, scales="fp32")


def test_bwd_recomputes_h_and_skips_dx(q):
    W = I.custom_weight(192, 320, 8)
    X, dY = I.custom_bf16((70, 320), 8, 1), I.custom_bf16((70, 192), 8, 2)
    A, B = I.custom_bf16((8, 320), 8, 3, bound=0.05), I.custom_bf16((192, 8), 8, 4, bound=0.05)
    _run_full(q, W, X, A, B, dY, 8, 16.0, "H=None", h_none=True)
    _run_full(q, W, X, A, B, dY, 8, 16.0, "dX=None", want_dx=False)


def test_zero_weight_and_empty_batch(q):
    W = np.zeros((128, 256), np.float32)
    X, dY = I.custom_bf16((40, 256), 9, 1), I.custom_bf16((40, 128), 9, 2)
    A, B = I.custom_bf16((16, 256), 9, 3, bound=0.05), I.custom_bf16((128, 16), 9, 4, bound=0.05)
    _run_full(q, W, X, A, B, dY, 16, 16.0, "zero W")
    # M = 0: forward is a no-op; the adapter gradients are zero
    lin = Linear(q, gpu_quantize(q, I.custom_weight(128, 256, 10)), X[:0], A, B, 16, 16.0)
    lin.fwd()
    _, dA, dB = lin.bwd(dY[:0], want_dx=False)
    torch.cuda.synchronize()
    assert torch.all(dA.float() == 0) and torch.all(dB.float() == 0)


def test_repeat_calls_and_shared_workspace(q):
    """Calls are deterministic (every reduction has a fixed order): the same
    inputs give identical bits on a second call, also after another problem
    ran through the same workspace; the smaller problem, run after the larger
    one left its partial sums behind, still matches the oracle."""
    cases = [(640, 512, 300, 64, 16.0, 21), (200, 192, 37, 8, -2.0, 22)]
    lins, data = [], []
    for n, k, m, r, alpha, seed in cases:
        W = I.custom_weight(n, k, seed)
        X = I.custom_bf16((m, k), seed, 1)
        dY = I.custom_bf16((m, n), seed, 2)
        A = I.custom_bf16((r, k), seed, 3, bound=0.05)
        B = I.custom_bf16((n, r), seed, 4, bound=0.05)
        lins.append(Linear(q, gpu_quantize(q, W), X, A, B, r, alpha))
        data.append((W, X, A, B, dY, alpha))
    ws = torch.empty(max(int(l.ws.numel()) for l in lins), dtype=torch.uint8, device="cuda")
    for l in lins:
        l.ws = ws

    def run(i):
        Y, H = lins[i].fwd()
        dX, dA, dB = lins[i].bwd(data[i][4], H=H)
        torch.cuda.synchronize()
        return [t.clone() for t in (Y, H, dX, dA, dB)]

    first = [run(0), run(1)]
    again = [run(1), run(0)][::-1]
    for i in range(2):
        for name, a, b in zip(("Y", "H", "dX", "dA", "dB"), first[i], again[i]):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), \
                f"case {i} {name} differs between calls"
    W, X, A, B, dY, alpha = data[1]
    What = bf16_f64(OracleWeight(W).row_what_bits(np.arange(W.shape[0])))
    Xf, Af, Bf, dYf = bf16_f64(X), bf16_f64(A), bf16_f64(B), bf16_f64(dY)
    Yr, Hr = fwd(Xf, What, Af, Bf, alpha)
    dXr, dAr, dBr, _ = bwd(Xf, dYf, What, Af, Bf, alpha)
    Y, H, dX, dA, dB = again[1]
    for name, got, ref in (("Y", bf16_f64(host_bf16(Y)), Yr), ("H", H.cpu().numpy(), Hr),
                           ("dX", bf16_f64(host_bf16(dX)), dXr), ("dA", bf16_f64(host_bf16(dA)), dAr),
                           ("dB", bf16_f64(host_bf16(dB)), dBr)):
        assert_close(got, ref, f"shared workspace {name}")


def _per_tile(extent: int, rng, per: int = 1, tile: int = 256) -> np.ndarray:
    """Sample indices along one output axis: `per` random ones inside every
    256-wide tile (the tile kernels' and the GEMV's row groups) plus both
    ends, so every output tile of a launch is compared somewhere."""
    picks = [0, extent - 1]
    for t0 in range(0, extent, tile):
        hi = min(t0 + tile, extent)
        picks += list(rng.choice(np.arange(t0, hi), min(per, hi - t0), replace=False))
    return np.unique(np.asarray(picks, np.int64))


def _per_tile_blocks(k: int, rng) -> list:
    """One random 64-column block inside every 256-column tile of k, plus the
    first and last block."""
    nb = k // 64
    picks = {0, nb - 1}
    for t0 in range(0, nb, 4):
        picks.add(int(rng.integers(t0, min(t0 + 4, nb))))
    return sorted(picks)


def _sampled(q, wname, li, m=None, backward=True, codebook="nf4", scales="dq"):
    """Full-size layer on samples that touch every 256 x 256 output tile of
    every launch: Y on rows of every m tile x columns of every n tile, H on
    those rows; dX and dA on one 64-column block of every k tile over all M;
    dB on the sampled rows of every n tile.  codebook / scales pick the
    storage type (the oracle's weights follow it)."""
    wl = I.WORKLOADS[wname]
    m = m or wl.ms[0]
    W, X, A, B, dY = _workload_inputs(wl, li, m)
    n, k = W.shape
    plan = q.qlora_linear_plan(m, n, k, wl.r, q.QLORA_SCALES_FP32 if scales == "fp32" else q.QLORA_SCALES_DQ)
    note(f"[linear] {wname}[{li}] W={W.shape} M={m} {codebook}/{scales} sampled per tile, plan {plan}")
    lin = Linear(q, gpu_quantize(q, W, codebook, scales), X, A, B, wl.r, wl.alpha)
    Y, H = lin.fwd()
    if backward:
        dX, dA, dB = lin.bwd(dY, H=H)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1000 + li)
    ns = _per_tile(n, rng)
    ms = _per_tile(m, rng, per=4)
    kbs = _per_tile_blocks(k, rng)
    kcols = np.concatenate([np.arange(64 * b, 64 * b + 64) for b in kbs])
    ow = OracleWeight(W, codebook, scales)
    Xf, Af, Bf, dYf = bf16_f64(X), bf16_f64(A), bf16_f64(B), bf16_f64(dY)
    Yr, Hr = fwd(Xf[ms], bf16_f64(ow.row_what_bits(ns)), Af, Bf[ns], wl.alpha)
    assert_close(bf16_f64(host_bf16(Y))[np.ix_(ms, ns)], Yr, f"{wname}[{li}] Y")
    assert_close(H.cpu().numpy()[ms], Hr, f"{wname}[{li}] H")
    if not backward:
        return
    Hfull = Xf @ Af.T
    Wc = bf16_f64(ow.colblock_what_bits(kbs))
    dXr, dAr, _, _ = bwd(Xf[:, kcols], dYf, Wc, Af[:, kcols], Bf, wl.alpha, H=Hfull)
    assert_close(bf16_f64(host_bf16(dX))[:, kcols], dXr, f"{wname}[{li}] dX")
    assert_close(bf16_f64(host_bf16(dA))[:, kcols], dAr, f"{wname}[{li}] dA")
    _, _, dBr, _ = bwd(Xf, dYf[:, ns], bf16_f64(ow.row_what_bits(ns)), Af, Bf[ns], wl.alpha, H=Hfull)
    assert_close(bf16_f64(host_bf16(dB))[ns], dBr, f"{wname}[{li}] dB")


@pytest.mark.parametrize("codebook,scales", [("fp4", "dq"), ("fp4_e3m0", "dq"), ("nf4", "fp32")])
def test_storage_types_full_size_sampled(q, codebook, scales):
    """The comparison storage types at the 7B gate layer's full shape
    (M = 4096: 688 forward tiles in three rounds, 256 input-gradient tiles),
    every output tile of both launches compared on samples."""
    _sampled(q, "mlp_7b", 0, codebook=codebook, scales=scales)


def _full_size(q, wname, li):
    """Full-size layer compared whole: the encoding and the BF16 weights bit
    for bit, and every element of Y, H, dX, dA and dB against the fp64
    oracle on the oracle's own BF16 weights."""
    wl = I.WORKLOADS[wname]
    m = wl.ms[0]
    W, X, A, B, dY = _workload_inputs(wl, li, m)
    n, k = W.shape
    note(f"[linear] {wname}[{li}] W={W.shape} M={m} full, plan {q.qlora_linear_plan(m, n, k, wl.r)}")
    ref = nf4_dq.quantize_nf4_dq(W)
    w = gpu_quantize(q, W)
    assert_encoding_equal(encoding_to_host(w), ref, f"{wname}[{li}]")
    ref_wh = nf4_dq.dequant_bf16(ref["packed"], ref["scale_code"], ref["group_amax"], ref["offset"], n, k)
    Wh = torch.empty(n, k, dtype=torch.bfloat16, device="cuda")
    q.qlora_dequant_bf16(w, Wh)
    torch.cuda.synchronize()
    bad = np.flatnonzero(host_bf16(Wh).reshape(-1) != ref_wh.reshape(-1))
    assert bad.size == 0, f"{wname}[{li}] dequant: {bad.size} differ, first {bad[:5]}"
    del Wh
    lin = Linear(q, w, X, A, B, wl.r, wl.alpha)
    Y, H = lin.fwd()
    dX, dA, dB = lin.bwd(dY, H=H)
    torch.cuda.synchronize()
    What = bf16_f64(ref_wh)
    del ref, ref_wh
    Xf, Af, Bf, dYf = bf16_f64(X), bf16_f64(A), bf16_f64(B), bf16_f64(dY)
    Yr, Hr = fwd(Xf, What, Af, Bf, wl.alpha)
    assert_close(bf16_f64(host_bf16(Y)), Yr, f"{wname}[{li}] Y")
    assert_close(H.cpu().numpy(), Hr, f"{wname}[{li}] H")
    del Yr, Y
    dXr, dAr, dBr, _ = bwd(Xf, dYf, What, Af, Bf, wl.alpha, H=Hr)
    assert_close(bf16_f64(host_bf16(dX)), dXr, f"{wname}[{li}] dX")
    assert_close(bf16_f64(host_bf16(dA)), dAr, f"{wname}[{li}] dA")
    assert_close(bf16_f64(host_bf16(dB)), dBr, f"{wname}[{li}] dB")


@pytest.mark.parametrize("li", [0, 1, 2])
def test_mlp_7b_full(q, li):
    _full_size(q, "mlp_7b", li)


@pytest.mark.parametrize("m", [1, 4, 16])
def test_up_65b_small_m(q, m):
    _sampled(q, "up_65b", 0, m=m, backward=False)


@pytest.mark.parametrize("m,codebook", [(1, "nf4"), (16, "fp4_e3m0")])
def test_up_65b_small_m_single_level(q, m, codebook):
    """The small-M GEMV on single-level constants at the 65B up_proj shape
    (2,752 four-block units over 256 workgroups: ranges straddle row
    groups), sampled in every 256-row group."""
    assert q.qlora_linear_plan(m, 22016, 8192, 16, q.QLORA_SCALES_FP32)["fwd_path"] == q.QLORA_PATH_GEMV
    _sampled(q, "up_65b", 0, m=m, backward=False, codebook=codebook, scales="fp32")


@pytest.mark.parametrize("li", range(7))
def test_block_65b(q, li):
    _sampled(q, "block_65b", li)


@pytest.mark.parametrize("n,k,m,r,alpha,seed", [
    (640, 512, 300, 64, 16.0, 81),     # two m tiles, one 8-step round
    (200, 192, 37, 5, -3.5, 82),       # ragged n, k, M and rank, negative alpha
    (1088, 320, 96, 128, 16.0, 83),    # ragged row tile, maximum rank (two LoRA chunks)
    (11008, 4096, 4096, 64, 16.0, 84),  # the 7B gate/up shape (688 tiles)
    (4096, 11008, 4096, 64, 16.0, 85),  # the 7B down shape (172 steps)
])
def test_bf16_weight_forward_is_the_nf4_forward(q, n, k, m, r, alpha, seed):
    """The tile kernel on pre-expanded BF16 weights (the 16-bit baseline of
    the tracing library), given the dequantized W_hat, reproduces the NF4
    forward bit for bit: the expansion hands the MFMAs exactly these
    operands.  The small case is also checked against the fp64 oracle."""
    assert q.qlora_linear_plan(m, n, k, r)["fwd_splits"] == 1
    W = I.custom_weight(n, k, seed)
    X = I.custom_bf16((m, k), seed, 1)
    A = I.custom_bf16((r, k), seed, 3, bound=0.05)
    B = I.custom_bf16((n, r), seed, 4, bound=0.05)
    note(f"[bf16-weight fwd] n={n} k={k} M={m} r={r}")
    lin = Linear(q, gpu_quantize(q, W), X, A, B, r, alpha)
    Y, H = lin.fwd()
    Wh = torch.empty(n, k, dtype=torch.bfloat16, device="cuda")
    q.qlora_dequant_bf16(lin.w, Wh)
    Y16 = torch.empty_like(Y)
    H16 = torch.empty_like(H)
    q.use_tracing_library(True)
    try:
        q.qlora_profile_linear_fwd_bf16w(Wh, lin.X, lin.A, lin.B, r, alpha, Y16, H16, lin.ws)
        torch.cuda.synchronize()
    finally:
        q.use_tracing_library(False)
    assert torch.equal(Y16.view(torch.int16), Y.view(torch.int16)), "Y differs from the NF4 forward"
    assert torch.equal(H16.view(torch.int32), H.view(torch.int32)), "H differs from the NF4 forward"
    if n * k <= 1 << 20:
        What = bf16_f64(host_bf16(Wh))
        Yr, Hr = fwd(bf16_f64(X), What, bf16_f64(A), bf16_f64(B), alpha)
        assert_close(bf16_f64(host_bf16(Y16)), Yr, "bf16-weight Y")
