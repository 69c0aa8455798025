"""Pins for the GLA decode oracle (no GPU): one step of
S_new = diag(exp(gk)) S + outer(k, v), o = scale * q^T S_new
(TileLang Case Studies, Case D "Background")."""
import math
import os

import numpy as np
import pytest

import oracle
import refround
from gemv_inputs import BF16, F16, gla_inputs, values_to_bits

DTYPES = [F16, BF16]
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "gla_hand_cases.txt")


def _dec(dtype, x):
    return oracle.decode(dtype, x)


@pytest.mark.parametrize("dtype", DTYPES)
def test_zero_state_gives_outer_product(dtype):
    q, k, v, gk, S = gla_inputs(3, 37, 50, dtype, seed=1)
    S[:] = 0.0
    Sn, o, s64, _, _ = oracle.gla_decode(dtype, q, k, v, gk, S, 0.25)
    for h in range(3):
        outer = np.outer(_dec(dtype, k[h]), _dec(dtype, v[h]))   # products are exact in float32
        assert np.array_equal(Sn[h], outer.astype(np.float32))


@pytest.mark.parametrize("dtype", DTYPES)
def test_full_decay_forgets_the_state(dtype):
    """gk = -inf: exp(gk) = 0, S_new = outer(k, v) whatever S held."""
    q, k, v, gk, S = gla_inputs(2, 16, 24, dtype, seed=2)
    gk[:] = values_to_bits(np.array([-np.inf]), dtype)[0]
    Sn, _, _, _, _ = oracle.gla_decode(dtype, q, k, v, gk, S, 1.0)
    for h in range(2):
        assert np.array_equal(Sn[h], np.outer(_dec(dtype, k[h]), _dec(dtype, v[h])).astype(np.float32))


@pytest.mark.parametrize("dtype", DTYPES)
def test_no_decay_no_input_keeps_state(dtype):
    q, k, v, gk, S = gla_inputs(2, 20, 30, dtype, seed=3)
    gk[:] = 0
    k[:] = 0
    Sn, _, _, _, _ = oracle.gla_decode(dtype, q, k, v, gk, S, 1.0)
    assert np.array_equal(Sn, S)


@pytest.mark.parametrize("dtype", DTYPES)
def test_one_hot_query_reads_a_row(dtype):
    """q one-hot at i: o = scale * S_new[i, :] (rounded to the dtype)."""
    q, k, v, gk, S = gla_inputs(1, 12, 40, dtype, seed=4)
    for i in (0, 5, 11):
        qq = np.zeros_like(q)
        qq[0, i] = values_to_bits(np.array([1.0]), dtype)[0]
        Sn, o, s64, _, _ = oracle.gla_decode(dtype, qq, k, v, gk, S, 0.5)
        want = [refround.round_bits(dtype, 0.5 * float(x)) for x in s64[0, i]]
        assert list(o[0]) == want


def test_decay_uses_the_natural_exponential():
    """exp(-1) = 1/e: S = 1, k = 0, gk = -1 gives S_new = 1/e in float32."""
    one = values_to_bits(np.array([1.0]), F16)[0]
    q = np.full((1, 1), one, np.uint16)
    k = np.zeros((1, 1), np.uint16)
    v = np.full((1, 1), one, np.uint16)
    gk = values_to_bits(np.array([[-1.0]]), F16)
    S = np.ones((1, 1, 1), np.float32)
    Sn, _, s64, _, _ = oracle.gla_decode(F16, q, k, v, gk, S, 1.0)
    inv_e = 0.36787944117144233        # 1/e = sum_n (-1)^n / n!
    assert abs(s64[0, 0, 0] - inv_e) <= 2e-16
    assert Sn[0, 0, 0] == np.float32(inv_e)


@pytest.mark.parametrize("dtype", DTYPES)
def test_integer_inputs_exact(dtype):
    """Integer q, k, v, S with gk = 0: S_new = S + outer(k, v) and
    o = q @ S_new exactly (integer arithmetic), rounded once."""
    rng = np.random.default_rng(9)
    bh, dk, dv = 2, 30, 17
    qi = rng.integers(-3, 4, size=(bh, dk))
    ki = rng.integers(-3, 4, size=(bh, dk))
    vi = rng.integers(-3, 4, size=(bh, dv))
    Si = rng.integers(-20, 21, size=(bh, dk, dv))
    q, k, v = (values_to_bits(x.astype(np.float32), dtype) for x in (qi, ki, vi))
    gk = np.zeros((bh, dk), np.uint16)
    Sn, o, _, o64, _ = oracle.gla_decode(dtype, q, k, v, gk, Si.astype(np.float32), 1.0)
    want_S = Si + ki[:, :, None] * vi[:, None, :]
    assert np.array_equal(Sn, want_S.astype(np.float32))
    want_o = np.einsum("hi,hij->hj", qi, want_S)
    assert np.array_equal(o64, want_o.astype(np.float64))
    assert np.array_equal(o, np.array([[refround.round_bits(dtype, float(x)) for x in row]
                                       for row in want_o], dtype=np.uint16))


@pytest.mark.parametrize("dtype", DTYPES)
def test_absolute_sum_of_the_output(dtype):
    """oabs (it scales the GPU tolerance of o) is |scale| * sum_i |q_i S_new[i][j]|
    with S_new = S + outer(k, v) at gk = 0: integer inputs of both signs and a
    negative power-of-two scale make it an exact integer computation.  A
    missing |scale|, a signed sum, or the old state in place of S_new each
    give a different value here."""
    rng = np.random.default_rng(17)
    bh, dk, dv = 3, 41, 12
    qi = rng.integers(-3, 4, size=(bh, dk))
    ki = rng.integers(-3, 4, size=(bh, dk))
    vi = rng.integers(-3, 4, size=(bh, dv))
    Si = rng.integers(-20, 21, size=(bh, dk, dv))
    q, k, v = (values_to_bits(x.astype(np.float32), dtype) for x in (qi, ki, vi))
    gk = np.zeros((bh, dk), np.uint16)
    scale = -0.25
    _, _, _, o64, oabs = oracle.gla_decode(dtype, q, k, v, gk, Si.astype(np.float32), scale)
    Snew = Si + ki[:, :, None] * vi[:, None, :]
    want = np.abs(qi[:, :, None] * Snew).sum(axis=1)          # exact integers
    assert np.array_equal(oabs, 0.25 * want.astype(np.float64))
    assert np.array_equal(o64, scale * np.einsum("hi,hij->hj", qi, Snew).astype(np.float64))
    # the pin tells these readings apart on this input
    assert not np.array_equal(want, np.abs(np.einsum("hi,hij->hj", qi, Snew)))
    assert not np.array_equal(want, np.abs(qi[:, :, None] * Si).sum(axis=1))


@pytest.mark.parametrize("dtype", DTYPES)
def test_linear_in_q(dtype):
    q, k, v, gk, S = gla_inputs(2, 64, 32, dtype, seed=5)
    _, _, _, o1, a1 = oracle.gla_decode(dtype, q, k, v, gk, S, 1.0)
    q2 = values_to_bits(2.0 * _dec(dtype, q), dtype)       # doubling is exact
    _, _, _, o2, _ = oracle.gla_decode(dtype, q2, k, v, gk, S, 1.0)
    assert np.all(np.abs(o2 - 2 * o1) <= 64 * 2.0 ** -52 * 2 * a1)
    assert np.abs(o1).max() > 0.01


def _parse(path):
    cases, cur = [], None
    for raw in open(path):
        line = raw.split("#", 1)[0].strip()
        if not line:
            continue
        tok = line.split()
        if tok[0] == "case":
            cur = {"name": tok[1], "dtype": F16 if tok[2] == "f16" else BF16,
                   "dk": int(tok[3]), "dv": int(tok[4])}
        elif tok[0] == "end":
            cases.append(cur)
        else:
            cur[tok[0]] = [float(t) for t in tok[1:]]
    return cases


CASES = _parse(GOLDEN)


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_hand_cases(case):
    dt, dk, dv = case["dtype"], case["dk"], case["dv"]
    bits = lambda key, shape: values_to_bits(np.array(case[key]).reshape(shape), dt)
    S = np.array(case["S"], dtype=np.float32).reshape(1, dk, dv)
    Sn, o, _, _, _ = oracle.gla_decode(dt, bits("q", (1, dk)), bits("k", (1, dk)),
                                       bits("v", (1, dv)), bits("gk", (1, dk)), S,
                                       case["scale"][0])
    assert list(Sn.ravel()) == case["Snew"]
    assert list(oracle.decode(dt, o.ravel())) == case["o"]


def test_inputs_recipe():
    q, k, v, gk, S = gla_inputs(4, 128, 128, BF16, seed=0)
    g = oracle.decode(BF16, gk)
    assert g.max() <= 0.0 and g.min() > -20            # log decays
    assert S.dtype == np.float32 and S.shape == (4, 128, 128)
    q2, _, _, _, S2 = gla_inputs(4, 128, 128, BF16, seed=0)
    assert np.array_equal(q, q2) and np.array_equal(S, S2)
