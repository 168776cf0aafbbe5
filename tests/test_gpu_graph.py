"""The library's calls captured in a HIP graph (torch.cuda.graph records the
kernels the calls launch on the current stream) and replayed: the linear
layer's forward and backward on the tile path with a split contraction (the
7B q_proj at M = 512) and on the small-M GEMV path, the allocation-free
forward, and the causal attention core's forward and backward.

Every replay follows eager work that reuses the same workspace (another
shape's forward and backward) and the overwriting of every output with NaN,
and must equal the eager result bit for bit, three replays in a row.  The
calls allocate nothing and record no memset, so a graph holds only their
kernels; a call the capture could not record would raise here."""
import numpy as np
import pytest
import torch

from bit_nf4_quantized_qlora_amd import inputs as I
from gpu_helpers import dev_bf16, gpu_quantize, note

pytestmark = pytest.mark.gpu

# (n, k, M, r, alpha, seed)
LINEAR_CASES = [(4096, 4096, 512, 64, 16.0, 81),   # tile path, contraction split 8 ways each pass
                (2048, 1024, 8, 16, 16.0, 82)]     # small-M GEMV forward (k % 256 == 0, M <= 16)


@pytest.fixture(scope="module")
def q():
    from bit_nf4_quantized_qlora_amd import qlora
    return qlora


def _linear(q, n, k, m, r, seed):
    w = gpu_quantize(q, I.custom_weight(n, k, seed))
    t = {"X": dev_bf16(I.custom_bf16((m, k), seed, 1)), "dY": dev_bf16(I.custom_bf16((m, n), seed, 2)),
         "A": dev_bf16(I.custom_bf16((r, k), seed, 3, bound=0.05)),
         "B": dev_bf16(I.custom_bf16((n, r), seed, 4, bound=0.05))}
    bf = lambda *s: torch.empty(*s, dtype=torch.bfloat16, device="cuda")
    out = {"Y": bf(m, n), "Y_na": bf(m, n), "H": torch.empty(m, r, dtype=torch.float32, device="cuda"),
           "H_na": torch.empty(m, r, dtype=torch.float32, device="cuda"), "dX": bf(m, k), "dA": bf(r, k),
           "dB": bf(n, r)}
    return w, t, out


def _replay_and_compare(g, outs: dict, ref: dict, eager_between, what: str) -> None:
    for rep in range(3):
        eager_between()
        for v in outs.values():
            v.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key, v in outs.items():
            assert torch.equal(v.view(torch.int32) if v.dtype == torch.float32 else v.view(torch.int16),
                               ref[key].view(torch.int32) if v.dtype == torch.float32 else ref[key].view(torch.int16)), \
                f"{what}: replay {rep} {key} differs from the eager call"


def _capture(calls):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one run off the capture, as torch asks before capturing
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("n,k,m,r,alpha,seed", LINEAR_CASES)
def test_linear_calls_replay_bit_identical(q, n, k, m, r, alpha, seed):
    note(f"[graph] linear n={n} k={k} M={m} r={r}")
    w, t, out = _linear(q, n, k, m, r, seed)
    w2, t2, out2 = _linear(q, 640, 512, 37, 8, seed + 100)   # the eager work between replays
    ws = torch.empty(max(q.qlora_linear_workspace_bytes(m, n, k, r), q.qlora_linear_workspace_bytes(37, 640, 512, 8)),
                     dtype=torch.uint8, device="cuda")

    def calls():
        q.qlora_linear_fwd(w, t["X"], t["A"], t["B"], r, alpha, out["Y"], out["H"], ws)
        q.qlora_linear_fwd_noalloc(w, t["X"], t["A"], t["B"], r, alpha, out["Y_na"], out["H_na"])
        q.qlora_linear_bwd(w, t["X"], t["dY"], t["A"], t["B"], r, alpha, out["H"], out["dX"], out["dA"], out["dB"],
                           ws)

    def other():
        q.qlora_linear_fwd(w2, t2["X"], t2["A"], t2["B"], 8, -2.0, out2["Y"], out2["H"], ws)
        q.qlora_linear_fwd_noalloc(w2, t2["X"], t2["A"], t2["B"], 8, -2.0, out2["Y_na"], out2["H_na"])
        q.qlora_linear_bwd(w2, t2["X"], t2["dY"], t2["A"], t2["B"], 8, -2.0, out2["H"], out2["dX"], out2["dA"],
                           out2["dB"], ws)

    calls()
    torch.cuda.synchronize()
    ref = {key: v.clone() for key, v in out.items()}
    assert torch.equal(ref["Y"].view(torch.int16), ref["Y_na"].view(torch.int16))
    g = _capture(calls)
    _replay_and_compare(g, out, ref, other, f"linear {n}x{k} M={m}")


def test_attention_calls_replay_bit_identical(q):
    batch, seq, heads, d = 2, 200, 4, 128
    note(f"[graph] attention batch={batch} seq={seq} heads={heads} d={d}")
    rng = np.random.default_rng(83)
    shape = (batch * seq, heads * d)
    bits = lambda: I.to_bf16_bits(rng.standard_normal(shape).astype(np.float32))
    Q, K, V, dO = (dev_bf16(bits()) for _ in range(4))
    bf = lambda: torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    out = {"O": bf(), "lse": torch.empty(batch, heads, seq, dtype=torch.float32, device="cuda"),
           "dQ": bf(), "dK": bf(), "dV": bf()}
    ws = torch.empty(max(q.qlora_attention_workspace_bytes(batch, seq, heads, d),
                         q.qlora_attention_workspace_bytes(1, 77, 2, 64)), dtype=torch.uint8, device="cuda")
    small = [dev_bf16(I.to_bf16_bits(rng.standard_normal((77, 128)).astype(np.float32))) for _ in range(4)]
    small_out = [torch.empty(77, 128, dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    small_lse = torch.empty(1, 2, 77, dtype=torch.float32, device="cuda")

    def calls():
        q.qlora_attention_fwd(Q, K, V, out["O"], out["lse"], batch, seq, heads, d, ws)
        q.qlora_attention_bwd(Q, K, V, dO, out["lse"], out["dQ"], out["dK"], out["dV"], batch, seq, heads, d, ws)

    def other():
        a, b, c, e = small
        q.qlora_attention_fwd(a, b, c, small_out[0], small_lse, 1, 77, 2, 64, ws)
        q.qlora_attention_bwd(a, b, c, e, small_lse, small_out[1], small_out[2], small_out[3], 1, 77, 2, 64, ws)

    calls()
    torch.cuda.synchronize()
    ref = {key: v.clone() for key, v in out.items()}
    g = _capture(calls)
    _replay_and_compare(g, out, ref, other, "attention")
