"""GPU parity for one GLA decode step (include/gla_decode.h) against the CPU
oracle, through the C ABI.

Bounds, from the fp32 operations the kernel performs per state element
(exp from the device library, within 1 ulp; one product e*S; one FMA adding
k*v) and per output (an fp32 sum over dk in a fixed order, one product by
scale, one rounding to 16 bits):
  |S_gpu - S_new| <= 4 * 2^-24 * (|e S| + |k v|)
  |o_gpu - o|     <= ulp + |scale| * sum_i |q_i| errS_ij + 2^-24 (dk + 8) oabs + 2^-24 |o|
Integer inputs with gk = 0 (e = 1 exactly) and scale = 1 are exact: bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import memory_bound_dense_amd as mbd
import oracle
from gemv_inputs import BF16, F16, gla_inputs, torch_dtype, values_to_bits
from parity import to_bits, to_device, ulp

pytestmark = pytest.mark.gpu
U = 2.0 ** -24


@pytest.fixture(scope="module")
def gla():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    g = mbd.Gemv()
    yield mbd.GlaDecode(g)
    g.close()


def _dev(q, k, v, gk, S, dtype):
    return (to_device(q, dtype), to_device(k, dtype), to_device(v, dtype), to_device(gk, dtype),
            torch.from_numpy(np.ascontiguousarray(S)).cuda())


def run(gla, q, k, v, gk, S, scale, dtype, in_place=False):
    qd, kd, vd, gd, Sd = _dev(q, k, v, gk, S, dtype)
    bh, dv = v.shape
    So = Sd if in_place else torch.full_like(Sd, float("nan"))
    o = torch.full((bh, dv), float("nan"), dtype=torch_dtype(dtype), device="cuda")
    gla(qd, kd, vd, gd, Sd, So, o, scale)
    torch.cuda.synchronize()
    return So.cpu().numpy(), to_bits(o)


def check(dtype, q, k, v, gk, S, scale, Sg, og):
    Sn, o, s64, o64, oabs = oracle.gla_decode(dtype, q, k, v, gk, S, scale)
    e = np.exp(oracle.decode(dtype, gk).astype(np.float64))[:, :, None]
    kv = np.abs(oracle.decode(dtype, k)[:, :, None] * oracle.decode(dtype, v)[:, None, :])
    errS = 4 * U * (np.abs(e * S.astype(np.float64)) + kv) + 2.0 ** -140
    dS = np.abs(Sg.astype(np.float64) - s64)
    assert np.all(dS <= errS), float((dS / errS).max())
    qa = np.abs(oracle.decode(dtype, q))
    dk = q.shape[1]
    prop = abs(float(np.float32(scale))) * np.einsum("hi,hij->hj", qa, errS)
    gv, rv = oracle.decode(dtype, og), oracle.decode(dtype, o)
    bound = ulp(dtype, np.maximum(np.abs(gv), np.abs(rv))) + prop + U * (dk + 8) * oabs \
        + U * np.abs(o64)
    d = np.abs(gv - rv)
    assert np.all(d <= bound), float((d / bound).max())


SHAPES = [(32, 128, 128, BF16), (32, 128, 128, F16), (3, 100, 36, BF16), (5, 1, 4, F16),
          (2, 513, 132, BF16), (7, 64, 512, F16), (300, 32, 64, BF16)]


@pytest.mark.parametrize("bh,dk,dv,dtype", SHAPES,
                         ids=["%dx%dx%d_%s" % (b, k, v, "f16" if d == F16 else "bf16")
                              for b, k, v, d in SHAPES])
def test_gla_decode_matches_oracle(gla, bh, dk, dv, dtype):
    q, k, v, gk, S = gla_inputs(bh, dk, dv, dtype, seed=bh + dk + dv)
    scale = 1.0 / math.sqrt(dk)
    for in_place in (False, True):
        Sg, og = run(gla, q, k, v, gk, S, scale, dtype, in_place)
        check(dtype, q, k, v, gk, S, scale, Sg, og)


@pytest.mark.parametrize("dtype", [F16, BF16], ids=["f16", "bf16"])
def test_gla_integer_inputs_bit_exact(gla, dtype):
    rng = np.random.default_rng(11)
    bh, dk, dv = 9, 200, 68
    qi, ki = rng.integers(-3, 4, size=(bh, dk)), rng.integers(-3, 4, size=(bh, dk))
    vi = rng.integers(-3, 4, size=(bh, dv))
    Si = rng.integers(-50, 51, size=(bh, dk, dv)).astype(np.float32)
    q, k, v = (values_to_bits(x.astype(np.float32), dtype) for x in (qi, ki, vi))
    gk = np.zeros((bh, dk), np.uint16)
    Sn, o, _, _, _ = oracle.gla_decode(dtype, q, k, v, gk, Si, 1.0)
    for in_place in (False, True):
        Sg, og = run(gla, q, k, v, gk, Si, 1.0, dtype, in_place)
        assert np.array_equal(Sg, Sn)
        assert np.array_equal(og, o)


def test_gla_edges(gla):
    dtype = BF16
    # dk == 0: o is the empty sum, the (empty) state untouched
    q = np.zeros((4, 0), np.uint16)
    v = values_to_bits(np.ones((4, 8), np.float32), dtype)
    o = torch.full((4, 8), 7.0, dtype=torch.bfloat16, device="cuda")
    e = torch.empty((4, 0), dtype=torch.bfloat16, device="cuda")
    S = torch.empty((4, 0, 8), dtype=torch.float32, device="cuda")
    gla(e, e, to_device(v, dtype), e, S, S, o, 1.0)
    torch.cuda.synchronize()
    assert torch.all(o == 0)
    # k = 0 and gk = -inf: the state is cleared, o = 0
    q, k, v, gk, S = gla_inputs(6, 40, 16, dtype, seed=3)
    k[:] = 0
    gk[:] = values_to_bits(np.array([-np.inf]), dtype)[0]
    Sg, og = run(gla, q, k, v, gk, S, 0.5, dtype)
    assert np.all(Sg == 0) and np.all(oracle.decode(dtype, og) == 0)


@pytest.mark.parametrize("bh", [4, 512], ids=["unstaged", "staged"])
def test_gla_empty_rows_null_inputs(gla, bh):
    """dk == 0 with every input but o a null pointer (the header allows it):
    o is the empty sum.  4 heads of 128 columns launch fewer workgroups than
    there are CUs (the form that loads row scalars with the state rows),
    512 heads more (the form that stages them in LDS); neither may touch q, k,
    gk, v or the state."""
    dv = 128
    for dtype in (F16, BF16):
        o = torch.full((bh, dv), 7.0, dtype=torch_dtype(dtype), device="cuda")
        s = mbd.gla_decode_step(gla.g.h, None, None, None, None, None, None, o.data_ptr(),
                                bh, 0, dv, 0.5, dtype, None)
        assert s == mbd.GEMV_OK
        torch.cuda.synchronize()
        assert torch.all(o == 0)


def test_gla_batched_every_head(gla):
    """The batched shape (64 x 32 heads of 128 x 128), in place as a decode
    loop would run it: every head against the oracle."""
    bh, dk, dv = 64 * 32, 128, 128
    dtype = BF16
    q, k, v, gk, S = gla_inputs(bh, dk, dv, dtype, seed=0)
    scale = 1.0 / math.sqrt(dk)
    Sg, og = run(gla, q, k, v, gk, S, scale, dtype, in_place=True)
    check(dtype, q, k, v, gk, S, scale, Sg, og)


def test_gla_rejects_bad_calls(gla):
    q, k, v, gk, S = gla_inputs(2, 8, 8, BF16, seed=1)
    qd, kd, vd, gd, Sd = _dev(q, k, v, gk, S, BF16)
    o = torch.full((2, 8), 3.0, dtype=torch.bfloat16, device="cuda")
    h = gla.g.h
    # o inside the state
    s = mbd.gla_decode_step(h, qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), gd.data_ptr(),
                            Sd.data_ptr(), Sd.data_ptr(), Sd.data_ptr() + 64, 2, 8, 8, 1.0, 1, None)
    assert s == mbd._lib.GEMV_ERR_ALIASING
    # misaligned state
    s = mbd.gla_decode_step(h, qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), gd.data_ptr(),
                            Sd.data_ptr() + 4, Sd.data_ptr() + 4, o.data_ptr(), 1, 8, 8, 1.0, 1, None)
    assert s == mbd._lib.GEMV_ERR_MISALIGNED
    torch.cuda.synchronize()
    assert torch.all(o == 3.0)
    assert np.array_equal(Sd.cpu().numpy(), S)
