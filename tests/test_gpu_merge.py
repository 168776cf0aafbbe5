"""GPU parity of qlora_merge_adapters against the oracle (oracle/merge.py):
the merged float32 weight, its bf16 copy and its re-encoding, bit for bit."""
import numpy as np
import pytest
import torch

from bit_nf4_quantized_qlora_amd import inputs as I
from gpu_helpers import dev_bf16, encoding_to_host, gpu_quantize, host_bf16, note
from oracle import merge, nf4_dq
from oracle_views import OracleWeight

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    from bit_nf4_quantized_qlora_amd import qlora
    return qlora


def _oracle_what(W, codebook, scales):
    n, k = W.shape
    if scales == "fp32":
        e = nf4_dq.quantize_single_level(W, codebook)
        return nf4_dq.dequant_single_level_bf16(e["packed"], e["absmax"], n, k, codebook)
    e = nf4_dq.quantize_nf4_dq(W, codebook)
    return nf4_dq.dequant_bf16(e["packed"], e["scale_code"], e["group_amax"], e["offset"], n, k, codebook)


@pytest.mark.parametrize("n,k,r,alpha,seed,src,dst", [
    (64, 256, 8, 16.0, 61, ("nf4", "dq"), ("nf4", "dq")),
    (300, 640, 100, 32.0, 62, ("nf4", "dq"), ("fp4", "dq")),       # ragged rows, rank 100, Float4 out
    (1024, 4096, 64, 16.0, 63, ("fp4", "fp32"), ("nf4", "fp32")),  # single-level in and out
    (5, 3840, 1, -2.0, 64, ("nf4", "dq"), None),                   # rank 1, merged bf16 only
    (67, 512, 16, 16.0, 65, ("nf4", "dq"), ("nf4", "dq")),         # rows not a multiple of a thread's 4, B read 8 at a time
    (66, 1024, 12, 24.0, 66, ("fp4", "dq"), ("nf4", "dq")),        # the same with a rank not a multiple of 8
    (128, 768, 32, 16.0, 67, ("fp4_e3m0", "dq"), ("fp4_e3m0", "fp32")),  # Float4 (E3M0) in and out
])
def test_merge_adapters(q, n, k, r, alpha, seed, src, dst):
    note(f"[merge] n={n} k={k} r={r} src={src} dst={dst}")
    W = I.custom_weight(n, k, seed)
    A = I.custom_bf16((r, k), seed, 3, bound=0.05)
    B = I.custom_bf16((n, r), seed, 4, bound=0.05)
    w = gpu_quantize(q, W, *src)
    Wb = torch.empty(n, k, dtype=torch.bfloat16, device="cuda")
    out = None
    if dst is not None:
        out = q.NF4Weight.empty(n, k, codebook=q.CODEBOOKS[dst[0]],
                                scales=q.QLORA_SCALES_FP32 if dst[1] == "fp32" else q.QLORA_SCALES_DQ)
    ws = torch.empty(q.qlora_merge_workspace_bytes(n, k), dtype=torch.uint8, device="cuda")
    q.qlora_merge_adapters(w, dev_bf16(A), dev_bf16(B), r, alpha, Wb, out, ws)
    torch.cuda.synchronize()
    ref = merge.merged_f32(_oracle_what(W, *src), A, B, alpha)
    got = ws[: n * k * 4].view(torch.float32).cpu().numpy().reshape(n, k)
    bad = np.flatnonzero(got.view(np.uint32) != ref.view(np.uint32))
    assert bad.size == 0, f"merged float32: {bad.size} differ, first {bad[:5]}"
    assert np.array_equal(host_bf16(Wb), nf4_dq.bf16_rne_bits(ref)), "merged bf16"
    if dst is None:
        return
    if dst[1] == "fp32":
        e = nf4_dq.quantize_single_level(ref, dst[0])
        assert np.array_equal(out.packed.cpu().numpy(), e["packed"]), "re-encoded packed"
        assert np.array_equal(out.absmax.cpu().numpy().view(np.uint32), e["absmax"].view(np.uint32)), "absmax"
    else:
        e = nf4_dq.quantize_nf4_dq(ref, dst[0])
        h = encoding_to_host(out)
        for key in ("packed", "scale_code"):
            assert np.array_equal(h[key], e[key]), f"re-encoded {key}"
        assert np.array_equal(h["group_amax"].view(np.uint32), e["group_amax"].view(np.uint32)), "group_amax"
        assert np.float32(h["offset"]).view(np.uint32) == np.float32(e["offset"]).view(np.uint32), "offset"


def test_merge_full_size_sampled(q):
    """The 7B gate layer (11008 x 4096, r = 64): W' and its bf16 copy bit for
    bit on a random row of every 256-row group and both ends, against the
    oracle's merge of those rows (each row of W' depends only on its own row
    of W_hat and of B)."""
    wl = I.WORKLOADS["mlp_7b"]
    W = I.weight(wl, 0)
    n, k = W.shape
    note(f"[merge] full size {n}x{k} r={wl.r}, sampled rows")
    Ab, Bb = I.adapters(wl, 0)
    w = gpu_quantize(q, W)
    Wb = torch.empty(n, k, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(q.qlora_merge_workspace_bytes(n, k), dtype=torch.uint8, device="cuda")
    q.qlora_merge_adapters(w, dev_bf16(Ab), dev_bf16(Bb), wl.r, wl.alpha, Wb, None, ws)
    torch.cuda.synchronize()
    g = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, n - 1]] + [g.integers(r0, min(r0 + 256, n), 1) for r0 in range(0, n, 256)]))
    ow = OracleWeight(W)
    ref = merge.merged_f32(ow.row_what_bits(rows), Ab, Bb[rows], wl.alpha)
    got = ws[: n * k * 4].view(torch.float32).view(n, k)[torch.as_tensor(rows, device="cuda")].cpu().numpy()
    bad = np.flatnonzero(got.view(np.uint32) != ref.view(np.uint32))
    assert bad.size == 0, f"merged float32 rows: {bad.size} differ, first {bad[:5]}"
    assert np.array_equal(host_bf16(Wb)[rows], nf4_dq.bf16_rne_bits(ref)), "merged bf16 rows"
