"""GPU parity of the causal attention core (qlora_attention_fwd / _bwd)
against the float64 oracle (oracle/attention.py), on the same bf16 inputs.

Bar: the fwd/bwd tolerance of the layers (relative Frobenius error <= 5e-3,
max |diff| <= 2e-2 of the largest reference value) for O, dQ, dK and dV;
lse within 1e-5 relative + 1e-5 absolute (float32 sums of exponentials,
no bf16 rounding on the way).  The GPU rounds P and dS to bf16 before the
products that take them (2^-9 relative per element, independent in sign),
which the Frobenius bar holds with room.  Shapes span several 64-wide
tiles, ragged sequence tails, one-token sequences, rows longer than one
512-column chunk of the row kernels (seq 600, 700), sequences of several
128-row workgroup tiles with a ragged last one (seq 1000) or one row past
a tile (seq 65), head dims 8, 48 and 160 (the materialised path), 32, 64, 96
and 128 (the fused kernels), the LLaMA-7B layer's 32 heads of 128 on 512-token
sequences, and peaked attention (Q scaled by 8 or 20)."""
import numpy as np
import pytest
import torch

from gpu_helpers import assert_close, dev_bf16, host_bf16, note
from oracle import attention as at
from oracle import nf4_dq

pytestmark = pytest.mark.gpu
f64 = nf4_dq.bf16_bits_to_f64


@pytest.fixture(scope="module")
def q():
    from bit_nf4_quantized_qlora_amd import qlora
    return qlora


def _bits(rng, shape, scale=1.0):
    return nf4_dq.bf16_rne_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def _run(q, batch, seq, heads, d, seed, qscale=1.0):
    rng = np.random.default_rng(seed)
    shape = (batch * seq, heads * d)
    Qb, Kb, Vb, dOb = (_bits(rng, shape, scale) for scale in (qscale, 1.0, 1.0, 1.0))
    Q, K, V, dO = (dev_bf16(t) for t in (Qb, Kb, Vb, dOb))
    O = torch.empty_like(Q)
    lse = torch.empty(batch, heads, seq, dtype=torch.float32, device="cuda")
    dQ, dK, dV = (torch.full_like(Q, float("nan")) for _ in range(3))
    ws = torch.empty(max(q.qlora_attention_workspace_bytes(batch, seq, heads, d), 16), dtype=torch.uint8,
                     device="cuda")
    q.qlora_attention_fwd(Q, K, V, O, lse, batch, seq, heads, d, ws)
    q.qlora_attention_bwd(Q, K, V, dO, lse, dQ, dK, dV, batch, seq, heads, d, ws)
    torch.cuda.synchronize()
    return (Qb, Kb, Vb, dOb), (host_bf16(O), lse.cpu().numpy(), host_bf16(dQ), host_bf16(dK), host_bf16(dV))


@pytest.mark.parametrize("batch,seq,heads,d", [(2, 77, 3, 64), (1, 130, 2, 128), (3, 1, 2, 64), (2, 200, 1, 8),
                                               (1, 512, 4, 128), (1, 700, 2, 64), (1, 600, 1, 8), (2, 200, 3, 32),
                                               (1, 1000, 1, 128), (2, 65, 1, 128), (1, 300, 3, 96), (2, 100, 2, 96),
                                               (2, 150, 2, 48), (1, 130, 1, 160)])
def test_attention_matches_oracle(q, batch, seq, heads, d):
    note(f"[attention] batch={batch} seq={seq} heads={heads} d={d}")
    (Qb, Kb, Vb, dOb), (O, lse, dQ, dK, dV) = _run(q, batch, seq, heads, d, seed=seq + 7 * heads + d)
    Qf, Kf, Vf, dOf = (f64(t) for t in (Qb, Kb, Vb, dOb))
    rO, rlse = at.fwd(Qf, Kf, Vf, batch, seq, heads, d)
    np.testing.assert_allclose(lse, rlse, rtol=1e-5, atol=1e-5)
    assert_close(f64(O), rO, "O")
    rdQ, rdK, rdV = at.bwd(Qf, Kf, Vf, dOf, batch, seq, heads, d)
    for name, got, ref in (("dQ", dQ, rdQ), ("dK", dK, rdK), ("dV", dV, rdV)):
        if seq == 1 and name in ("dQ", "dK"):
            # exactly 0 in exact arithmetic; dP - D cancels only to float32 rounding here
            assert np.abs(f64(got)).max() <= 1e-4, f"{name} must vanish for one-token sequences"
            continue
        assert_close(f64(got), ref, name)


@pytest.mark.parametrize("batch,seq,heads,d,qscale", [(1, 300, 2, 128, 8.0), (2, 130, 2, 64, 20.0),
                                                      (1, 200, 1, 96, 8.0), (1, 150, 1, 32, 20.0),
                                                      (1, 100, 2, 8, 20.0), (1, 90, 2, 48, 20.0)])
def test_attention_peaked_matches_oracle(q, batch, seq, heads, d, qscale):
    """Peaked attention: Q scaled so the logits spread over tens of units and
    most rows put nearly all their weight on one or two keys.  The running
    maximum then jumps by large amounts inside a row (the online rescale),
    most exponentials underflow to zero, and dP - D cancels to a few leading
    bits, the case where a D taken from the bf16-rounded O went wrong."""
    note(f"[attention] peaked batch={batch} seq={seq} heads={heads} d={d} qscale={qscale}")
    (Qb, Kb, Vb, dOb), (O, lse, dQ, dK, dV) = _run(q, batch, seq, heads, d, seed=5 * seq + d, qscale=qscale)
    Qf, Kf, Vf, dOf = (f64(t) for t in (Qb, Kb, Vb, dOb))
    rO, rlse = at.fwd(Qf, Kf, Vf, batch, seq, heads, d)
    np.testing.assert_allclose(lse, rlse, rtol=1e-5, atol=1e-5)
    assert_close(f64(O), rO, "O")
    rdQ, rdK, rdV = at.bwd(Qf, Kf, Vf, dOf, batch, seq, heads, d)
    for name, got, ref in (("dQ", dQ, rdQ), ("dK", dK, rdK), ("dV", dV, rdV)):
        assert_close(f64(got), ref, name)


def test_attention_llama7b_layer_sampled(q):
    """The 7B layer's shape (8 sequences of 512, 32 heads of 128), as the
    layer bench runs it; the oracle checks two sampled (sequence, head) pairs."""
    batch, seq, heads, d = 8, 512, 32, 128
    note(f"[attention] llama7b batch={batch} seq={seq} heads={heads} d={d}")
    (Qb, Kb, Vb, dOb), (O, lse, dQ, dK, dV) = _run(q, batch, seq, heads, d, seed=11)
    for b, h in ((0, 0), (7, 31), (3, 17)):
        rows = slice(b * seq, (b + 1) * seq)
        cols = slice(h * d, (h + 1) * d)
        pick = lambda t: f64(t[rows, cols])
        rO, rlse = at.fwd(pick(Qb), pick(Kb), pick(Vb), 1, seq, 1, d)
        np.testing.assert_allclose(lse[b, h], rlse[0, 0], rtol=1e-5, atol=1e-5)
        assert_close(pick(O), rO, f"O[{b},{h}]")
        rdQ, rdK, rdV = at.bwd(pick(Qb), pick(Kb), pick(Vb), pick(dOb), 1, seq, 1, d)
        for name, got, ref in (("dQ", dQ, rdQ), ("dK", dK, rdK), ("dV", dV, rdV)):
            assert_close(pick(got), ref, f"{name}[{b},{h}]")


def test_attention_repeat_is_bitwise_deterministic(q):
    note("[attention] determinism")
    _, a = _run(q, 2, 96, 2, 64, seed=3)
    _, b = _run(q, 2, 96, 2, 64, seed=3)
    for x, y in zip(a, b):
        assert np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8))
