"""GPU AdamW step (qlora_adamw_step) against the float64 oracle
(oracle/adamw.py), with the moments in device memory and in pinned host
memory mapped for the device (the paged layout).  Tolerance derived from
float32 arithmetic: about eight roundings of 2^-24 per updated value, so
|got - ref| <= 2e-6 * (sum of the magnitudes of the terms) + 1e-30, plus,
for the parameter, the moment's own error carried through the step."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_helpers import dev_bf16, host_bf16, note
from oracle import adamw, nf4_dq

pytestmark = pytest.mark.gpu
HP = dict(lr=2e-4, b1=float(np.float32(0.9)), b2=float(np.float32(0.999)), eps=1e-8, wd=0.01)


@pytest.fixture(scope="module")
def q():
    from bit_nf4_quantized_qlora_amd import qlora
    return qlora


def _check_step(p, g, m, v, t, gp, gm, gv, gp16):
    rp, rm, rv = adamw.adamw_step(p, g, m, v, t, **HP)
    f = lambda x: np.asarray(x, np.float64)
    b1, b2, lr, wd = HP["b1"], HP["b2"], HP["lr"], HP["wd"]
    tol_m = 2e-6 * (np.abs(b1 * f(m)) + np.abs((1 - b1) * f(g))) + 1e-30
    tol_v = 2e-6 * (np.abs(b2 * f(v)) + np.abs((1 - b2) * f(g) ** 2)) + 1e-30
    upd = np.abs(f(p) * (1 - lr * wd) - rp)
    # the moment m_t may cancel (b1 m and (1 - b1) g of opposite signs): its
    # absolute error, scaled by the step, adds to the parameter's
    scale = (lr / (1 - b1 ** t)) / (np.sqrt(rv) / np.sqrt(1 - b2 ** t) + HP["eps"])
    tol_p = 2e-6 * (np.abs(f(p)) + upd) + scale * tol_m + 1e-30
    assert np.all(np.abs(f(gm) - rm) <= tol_m), "m"
    assert np.all(np.abs(f(gv) - rv) <= tol_v), "v"
    assert np.all(np.abs(f(gp) - rp) <= tol_p), "param"
    assert np.array_equal(gp16, nf4_dq.bf16_rne_bits(np.asarray(gp, np.float32))), "bf16 copy"


def _run(q, count, seed, m_dev, v_dev, m_host=None, v_host=None, steps=3):
    rng = np.random.default_rng(seed)
    p = (rng.standard_normal(count) * 0.05).astype(np.float32)
    P = torch.from_numpy(p.copy()).cuda()
    P16 = torch.empty(count, dtype=torch.bfloat16, device="cuda")
    m = np.zeros(count, np.float32)
    v = np.zeros(count, np.float32)
    for t in range(1, steps + 1):
        g = nf4_dq.bf16_rne_bits((rng.standard_normal(count) * 10.0 ** rng.uniform(-4, -1)).astype(np.float32))
        G = dev_bf16(g)
        q.qlora_adamw_step(P, P16, G, m_dev, v_dev, HP["lr"], HP["b1"], HP["b2"], HP["eps"], HP["wd"], t)
        torch.cuda.synchronize()
        gm = (m_host if m_host is not None else m_dev).cpu().numpy().copy()
        gv = (v_host if v_host is not None else v_dev).cpu().numpy().copy()
        gp = P.cpu().numpy().copy()
        _check_step(p, nf4_dq.bf16_bits_to_f64(g), m, v, t, gp, gm, gv, host_bf16(P16))
        p, m, v = gp, gm, gv


@pytest.mark.parametrize("count,seed", [(1, 1), (1000003, 2), (64 * 15104, 3)])
def test_adamw_device_state(q, count, seed):
    note(f"[adamw] device state count={count}")
    m = torch.zeros(count, dtype=torch.float32, device="cuda")
    v = torch.zeros(count, dtype=torch.float32, device="cuda")
    _run(q, count, seed, m, v)


def _device_pointer(host_tensor):
    """Device address of pinned host memory, or None when the runtime does not
    map it (then the paged case is skipped rather than risked)."""
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        return None
    dptr = ctypes.c_void_p()
    rc = hip.hipHostGetDevicePointer(ctypes.byref(dptr), ctypes.c_void_p(host_tensor.data_ptr()), 0)
    return dptr.value if rc == 0 and dptr.value else None


def test_adamw_paged_host_state(q):
    count = 100003
    note(f"[adamw] pinned host state count={count}")
    mh = torch.zeros(count, dtype=torch.float32).pin_memory()
    vh = torch.zeros(count, dtype=torch.float32).pin_memory()
    md, vd = _device_pointer(mh), _device_pointer(vh)
    if md is None or vd is None:
        pytest.skip("pinned host memory is not mapped for the device here")
    _run(q, count, 4, md, vd, m_host=mh, v_host=vh)
