"""qlora_linear_fwd_noalloc -- the forward on the library's fixed device
scratch, for callers that cannot allocate -- against qlora_linear_fwd with a
caller workspace: on each path two calls in a row, the second on a smaller
input (so it runs over what the first left in the scratch); each output bit
for bit equal to the workspace call's and within the stated tolerance of the
fp64 oracle (relative Frobenius <= 5e-3, max |diff| <= 2e-2 max |ref|)."""
import numpy as np
import pytest
import torch

from bit_nf4_quantized_qlora_amd import inputs as I
from gpu_helpers import Linear, assert_close, bf16_f64, dev_bf16, gpu_quantize, host_bf16, note
from oracle_views import OracleWeight, fwd

pytestmark = pytest.mark.gpu

# (n, k, M, r, alpha, seed); the first of each pair is the larger problem
SEQUENCES = {
    "tile": [(4096, 4096, 512, 64, 16.0, 71),   # the 7B q_proj shape: contraction split 8 ways (~69 MB of scratch)
             (640, 512, 37, 8, -2.0, 72)],      # tile path, one split, ragged M
    "gemv": [(4096, 8192, 16, 16, 16.0, 73),    # small-M GEMV, M = 16
             (300, 768, 5, 100, 32.0, 74)],     # GEMV, two ragged row groups, rank 100
}


@pytest.fixture(scope="module")
def q():
    from bit_nf4_quantized_qlora_amd import qlora
    return qlora


@pytest.mark.parametrize("path", sorted(SEQUENCES))
def test_noalloc_matches_workspace_call(q, path):
    cases = []
    for n, k, m, r, alpha, seed in SEQUENCES[path]:
        W = I.custom_weight(n, k, seed)
        X = I.custom_bf16((m, k), seed, 1)
        A = I.custom_bf16((r, k), seed, 3, bound=0.05)
        B = I.custom_bf16((n, r), seed, 4, bound=0.05)
        lin = Linear(q, gpu_quantize(q, W), X, A, B, r, alpha)
        plan = q.qlora_linear_plan(m, n, k, r)
        note(f"[noalloc] {path}: n={n} k={k} M={m} r={r} plan {plan}")
        Y_ref, H_ref = lin.fwd()                       # the workspace entry point
        cases.append((lin, W, X, A, B, alpha, Y_ref, H_ref))
    if path == "tile":
        assert q.qlora_linear_plan(*[SEQUENCES[path][0][i] for i in (2, 0, 1, 3)])["fwd_splits"] > 1
    else:
        assert all(q.qlora_linear_plan(m, n, k, r)["fwd_path"] == q.QLORA_PATH_GEMV
                   for n, k, m, r, _, _ in SEQUENCES[path])
    torch.cuda.synchronize()
    outs = []
    for lin, *_ in cases:                              # two calls in a row, larger first
        Y = torch.empty(lin.M, lin.w.n, dtype=torch.bfloat16, device="cuda")
        H = torch.empty(lin.M, lin.r, dtype=torch.float32, device="cuda")
        q.qlora_linear_fwd_noalloc(lin.w, lin.X, lin.A, lin.B, lin.r, lin.alpha, Y, H)
        outs.append((Y, H))
    torch.cuda.synchronize()
    for (lin, W, X, A, B, alpha, Y_ref, H_ref), (Y, H) in zip(cases, outs):
        ctx = f"{path} n={lin.w.n} M={lin.M}"
        assert torch.equal(Y.view(torch.int16), Y_ref.view(torch.int16)), f"{ctx}: Y differs from the workspace call"
        assert torch.equal(H.view(torch.int32), H_ref.view(torch.int32)), f"{ctx}: H differs from the workspace call"
        What = bf16_f64(OracleWeight(W).row_what_bits(np.arange(W.shape[0])))
        Yr, Hr = fwd(bf16_f64(X), What, bf16_f64(A), bf16_f64(B), alpha)
        assert_close(bf16_f64(host_bf16(Y)), Yr, f"{ctx} Y")
        assert_close(H.cpu().numpy(), Hr, f"{ctx} H")
