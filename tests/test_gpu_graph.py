"""The library's calls captured in a HIP graph (torch.cuda.graph records the
kernels the calls launch on the current stream) and replayed: the linear
layer's forward and backward on the tile path with a split contraction (the
7B q_proj at M = 512) and on the small-M GEMV path, the allocation-free
forward, the causal attention core's forward and backward, the quantizer
(both storage types), dequantization, the adapter merge with re-encoding,
the SwiGLU and add kernels, and the AdamW step.

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


def _bits_of(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def test_setup_and_elementwise_calls_replay_bit_identical(q):
    """Quantize (NF4 + double quantization over four runs of group sums, and
    Float4 with float32 block constants), dequantize, merge with re-encoding,
    and the SwiGLU / add kernels, captured once and replayed: every output
    equals the eager call's bit for bit, three replays in a row, with eager
    calls on other inputs sharing the workspaces in between."""
    n, k, r = 2048, 8192, 16   # 262144 blocks: 1024 groups, four runs of the mean's fold
    note(f"[graph] setup calls n={n} k={k} r={r}")
    g = np.random.default_rng(84)
    dev_f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    W = dev_f32(I.custom_weight(n, k, 84))
    W2 = dev_f32(I.custom_weight(n, k, 85))
    A = dev_bf16(I.custom_bf16((r, k), 84, 3, bound=0.05))
    B = dev_bf16(I.custom_bf16((n, r), 84, 4, bound=0.05))
    m = 1 << 20
    gate, up, dh, x2 = (dev_bf16(I.to_bf16_bits(g.standard_normal(m).astype(np.float32))) for _ in range(4))
    qws = torch.empty(q.qlora_quantize_workspace_bytes(n, k), dtype=torch.uint8, device="cuda")
    mws = torch.empty(q.qlora_merge_workspace_bytes(n, k), dtype=torch.uint8, device="cuda")
    w_nf4 = q.NF4Weight.empty(n, k)
    w_fp4 = q.NF4Weight.empty(n, k, codebook=q.CODEBOOKS["fp4"], scales=q.QLORA_SCALES_FP32)
    w_re = q.NF4Weight.empty(n, k)
    bf = lambda *s: torch.empty(*s, dtype=torch.bfloat16, device="cuda")
    out = {"what": bf(n, k), "merged": bf(n, k), "h": bf(m), "dg": bf(m), "du": bf(m), "sum": bf(m)}
    for name, w in (("nf4", w_nf4), ("fp4", w_fp4), ("re", w_re)):
        for key, t in w.buffers().items():
            if t is not None:
                out[f"{name}.{key}"] = t
    o_what, o_h = bf(n, k), bf(m)
    w_other = q.NF4Weight.empty(n, k)

    def calls():
        q.qlora_quantize_nf4_dq(W, w_nf4, qws)
        q.qlora_quantize_nf4_dq(W, w_fp4, qws)
        q.qlora_dequant_bf16(w_nf4, out["what"])
        q.qlora_merge_adapters(w_nf4, A, B, r, 16.0, out["merged"], w_re, mws)
        q.qlora_swiglu_fwd(gate, up, out["h"])
        q.qlora_swiglu_bwd(gate, up, dh, out["dg"], out["du"])
        q.qlora_add_bf16(out["h"], x2, out["sum"])

    def other():
        q.qlora_quantize_nf4_dq(W2, w_other, qws)
        q.qlora_dequant_bf16(w_other, o_what)
        q.qlora_merge_adapters(w_other, A, B, r, -4.0, o_what, None, mws)
        q.qlora_swiglu_fwd(up, gate, o_h)

    calls()
    torch.cuda.synchronize()
    ref = {key: v.clone() for key, v in out.items()}
    g_ = _capture(calls)
    for rep in range(3):
        other()
        for v in out.values():
            v.view(torch.uint8).fill_(0xFF)
        torch.cuda.synchronize()
        g_.replay()
        torch.cuda.synchronize()
        for key, v in out.items():
            assert torch.equal(_bits_of(v), _bits_of(ref[key])), f"replay {rep}: {key} differs from the eager call"


def test_adamw_step_replays_bit_identical(q):
    """One AdamW step captured and replayed from the same starting state
    (parameters and moments restored by eager copies before each replay):
    every replay's parameters, bf16 copy and moments equal the eager step's."""
    count = 3 * (1 << 18) + 77
    note(f"[graph] adamw count={count}")
    g = np.random.default_rng(86)
    f32 = lambda a: torch.from_numpy(a.astype(np.float32)).cuda()
    p0, m0 = f32(g.standard_normal(count) * 0.02), f32(g.standard_normal(count) * 1e-3)
    v0 = f32(np.abs(g.standard_normal(count)) * 1e-6)
    grad = dev_bf16(I.to_bf16_bits((g.standard_normal(count) * 1e-2).astype(np.float32)))
    p, m, v = p0.clone(), m0.clone(), v0.clone()
    pb = torch.empty(count, dtype=torch.bfloat16, device="cuda")
    args = (1e-3, 0.9, 0.999, 1e-8, 0.01, 7)

    def step():
        q.qlora_adamw_step(p, pb, grad, m, v, *args)

    def restore():
        p.copy_(p0)
        m.copy_(m0)
        v.copy_(v0)

    step()
    torch.cuda.synchronize()
    ref = {"p": p.clone(), "pb": pb.clone(), "m": m.clone(), "v": v.clone()}
    restore()
    torch.cuda.synchronize()
    g_ = _capture(step)   # the capture's warm-up step advances the state: restore again below
    for rep in range(3):
        restore()
        pb.fill_(float("nan"))
        torch.cuda.synchronize()
        g_.replay()
        torch.cuda.synchronize()
        for key, t in (("p", p), ("pb", pb), ("m", m), ("v", v)):
            assert torch.equal(_bits_of(t), _bits_of(ref[key])), f"replay {rep}: {key} differs from the eager step"
