"""GPU parity of the MLP-block pieces (qlora_swiglu_fwd / _bwd,
qlora_add_bf16) and of a whole block composed from library calls, against
the float64 oracle (oracle/mlp.py, oracle/linear.py).

Elementwise tolerance: the GPU computes in float32 and rounds once to bf16,
so an output is within half a bf16 ulp of the exact value plus the float32
error before rounding: |got - ref| <= 2^-8 |ref| + 2^-20 (|dh u| (1 + |g|))
(the last term covers dg near silu's stationary point, where the float32
factor 1 + g (1 - sigma) cancels).  The block is compared with the layers'
own tolerance (relative Frobenius 5e-3, max 2e-2 of the largest value),
the oracle taking the bf16 roundings at the same tensors as the library's
composition (gate/up outputs, h, dh, d_gate, d_up)."""
import numpy as np
import pytest
import torch

from bit_nf4_quantized_qlora_amd import inputs as I
from gpu_helpers import Linear, assert_close, dev_bf16, gpu_quantize, host_bf16, note
from oracle import linear, mlp, nf4_dq
from oracle_views import OracleWeight

pytestmark = pytest.mark.gpu
f64 = nf4_dq.bf16_bits_to_f64
rb = lambda x: nf4_dq.bf16_rne_bits(np.asarray(x, np.float32))


@pytest.fixture(scope="module")
def q():
    from bit_nf4_quantized_qlora_amd import qlora
    return qlora


def _inputs(count, seed):
    rng = np.random.default_rng(seed)
    g = rng.standard_normal(count) * 4
    g[:8] = [0.0, -0.0, 30.0, -30.0, -1.2784645, 1e-30, -90.0, 90.0]   # zero, saturation, silu' = 0
    return rb(g), rb(rng.standard_normal(count)), rb(rng.standard_normal(count))


@pytest.mark.parametrize("count,seed", [(9, 1), (1000003, 2)])
def test_swiglu_elementwise(q, count, seed):
    note(f"[mlp] swiglu count={count}")
    g, u, dh = _inputs(count, seed)
    G, U, DH = dev_bf16(g), dev_bf16(u), dev_bf16(dh)
    h = torch.empty_like(G)
    dg, du = torch.empty_like(G), torch.empty_like(G)
    s = torch.empty_like(G)
    q.qlora_swiglu_fwd(G, U, h)
    q.qlora_swiglu_bwd(G, U, DH, dg, du)
    q.qlora_add_bf16(U, DH, s)
    torch.cuda.synchronize()
    gf, uf, dhf = f64(g), f64(u), f64(dh)
    rh = mlp.swiglu_fwd(gf, uf)
    rdg, rdu = mlp.swiglu_bwd(gf, uf, dhf)
    slack = 2.0 ** -20 * np.abs(dhf * uf) * (1 + np.abs(gf)) + 1e-38
    for name, got, ref, extra in (("h", h, rh, 1e-38), ("du", du, rdu, 1e-38), ("dg", dg, rdg, slack)):
        err = np.abs(f64(host_bf16(got)) - ref)
        bad = np.flatnonzero(err > 2.0 ** -8 * np.abs(ref) + extra)
        assert bad.size == 0, f"{name}: {bad.size} outside, first {bad[:5]}"
    want = rb(uf.astype(np.float32) + dhf.astype(np.float32))
    assert np.array_equal(host_bf16(s), want), "add"


@pytest.mark.parametrize("count,seed", [(9, 3), (1000003, 4)])
def test_add_chain_equals_chained_adds(q, count, seed):
    """qlora_add_bf16_n over 2, 3 and 4 summands: bit for bit the chained
    qlora_add_bf16 calls and the float32 sums rounded to bf16 after each
    addition (left to right); also with the output aliasing the first or
    the last summand.  The values mix magnitudes so the intermediate roundings show."""
    note(f"[mlp] add chain count={count}")
    rng = np.random.default_rng(seed)
    xs = [rb(rng.standard_normal(count) * 10.0 ** rng.integers(-3, 4, count)) for _ in range(4)]
    X = [dev_bf16(x) for x in xs]
    for n in (2, 3, 4):
        out = torch.empty_like(X[0])
        q.qlora_add_bf16_n(X[:n], out)
        chained = X[0].clone()
        for j in range(1, n):
            q.qlora_add_bf16(chained, X[j], chained)
        alias = X[0].clone()
        q.qlora_add_bf16_n([alias] + X[1:n], alias)
        alias_last = X[n - 1].clone()
        q.qlora_add_bf16_n(X[:n - 1] + [alias_last], alias_last)
        torch.cuda.synchronize()
        want = xs[0]                                   # bf16 bit patterns throughout
        for j in range(1, n):
            want = rb(f64(want).astype(np.float32) + f64(xs[j]).astype(np.float32))
        got = host_bf16(out)
        assert np.array_equal(got, host_bf16(chained)), f"n={n}: chained calls"
        assert np.array_equal(got, host_bf16(alias)), f"n={n}: output aliasing the first summand"
        assert np.array_equal(got, host_bf16(alias_last)), f"n={n}: output aliasing the last summand"
        assert np.array_equal(got, want), f"n={n}: reference"


def test_mlp_block_composed(q):
    """A small LLaMA-style block: gate, up (n = 320), SwiGLU, down (k = 192),
    M = 70, rank 8, every projection with its own adapters; backward with
    the gate/up outputs recomputed from X."""
    M, k, n, r, alpha = 70, 192, 320, 8, 16.0
    note(f"[mlp] block M={M} k={k} n={n} r={r}")
    Wg, Wu, Wd = I.custom_weight(n, k, 71), I.custom_weight(n, k, 72), I.custom_weight(k, n, 73)
    ad = lambda shape, s, t: I.custom_bf16(shape, s, t, bound=0.05)
    Ag, Bg, Au, Bu, Ad, Bd = ad((r, k), 74, 1), ad((n, r), 74, 2), ad((r, k), 74, 3), ad((n, r), 74, 4), \
        ad((r, n), 74, 5), ad((k, r), 74, 6)
    X, dY = I.custom_bf16((M, k), 75, 1), I.custom_bf16((M, k), 75, 2)
    # library composition
    lg, lu = Linear(q, gpu_quantize(q, Wg), X, Ag, Bg, r, alpha), Linear(q, gpu_quantize(q, Wu), X, Au, Bu, r, alpha)
    Yg, Hg = lg.fwd()
    Yu, Hu = lu.fwd()
    h = torch.empty_like(Yg)
    q.qlora_swiglu_fwd(Yg, Yu, h)
    torch.cuda.synchronize()
    ld = Linear(q, gpu_quantize(q, Wd), host_bf16(h), Ad, Bd, r, alpha)
    Y, Hd = ld.fwd()
    dh, dAd, dBd = ld.bwd(dY, H=Hd)
    Yg2, _ = lg.fwd()                      # recomputed (checkpointing)
    Yu2, _ = lu.fwd()
    dg, du = torch.empty_like(Yg2), torch.empty_like(Yg2)
    q.qlora_swiglu_bwd(Yg2, Yu2, dh, dg, du)
    torch.cuda.synchronize()
    dXg, dAg, dBg = lg.bwd(host_bf16(dg), H=Hg)
    dXu, dAu, dBu = lu.bwd(host_bf16(du), H=Hu)
    dX = torch.empty_like(dXg)
    q.qlora_add_bf16(dXg, dXu, dX)
    torch.cuda.synchronize()
    # oracle, bf16 roundings at the same tensors
    Wgh, Wuh, Wdh = (f64(OracleWeight(W).row_what_bits(np.arange(W.shape[0]))) for W in (Wg, Wu, Wd))
    Xf, dYf = f64(X), f64(dY)
    Agf, Bgf, Auf, Buf, Adf, Bdf = (f64(t) for t in (Ag, Bg, Au, Bu, Ad, Bd))
    rYg = f64(rb(linear.fwd(Xf, Wgh, Agf, Bgf, alpha)[0]))
    rYu = f64(rb(linear.fwd(Xf, Wuh, Auf, Buf, alpha)[0]))
    rh = f64(rb(mlp.swiglu_fwd(rYg, rYu)))
    rY, _ = linear.fwd(rh, Wdh, Adf, Bdf, alpha)
    rdh, rdAd, rdBd, _ = linear.bwd(rh, dYf, Wdh, Adf, Bdf, alpha)
    rdg, rdu = (f64(rb(t)) for t in mlp.swiglu_bwd(rYg, rYu, f64(rb(rdh))))
    rdXg, rdAg, rdBg, _ = linear.bwd(Xf, rdg, Wgh, Agf, Bgf, alpha)
    rdXu, rdAu, rdBu, _ = linear.bwd(Xf, rdu, Wuh, Auf, Buf, alpha)
    for name, got, ref in (("Y", Y, rY), ("dh", dh, rdh), ("dX", dX, rdXg + rdXu), ("dA_gate", dAg, rdAg),
                           ("dB_gate", dBg, rdBg), ("dA_up", dAu, rdAu), ("dB_up", dBu, rdBu),
                           ("dA_down", dAd, rdAd), ("dB_down", dBd, rdBd)):
        assert_close(f64(host_bf16(got)), ref, f"block {name}")
    assert torch.equal(Yg2.view(torch.int16), Yg.view(torch.int16))   # recompute is bit-identical
