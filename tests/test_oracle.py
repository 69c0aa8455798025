"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself: Python's IEEE binary16
codec, brute-force rounding, closed forms (identity, permutation, one-hot
columns), exact integer arithmetic, exact rational sums, invariants and the
hand-worked cases in tests/golden/.  The definition pinned is the GEMV of
TileLang Case Studies, Case B "Background": c = B @ a, B (n, k) row-major,
a (k,), c (n,) in the input dtype.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import refround
from gemv_inputs import BF16, F16, integer_inputs, random_inputs, values_to_bits

DTYPES = [F16, BF16]
ALL_BITS = np.arange(65536, dtype=np.uint16)
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "gemv_hand_cases.txt")


# ---- P1: exact decode of every pattern ------------------------------------

@pytest.mark.parametrize("dtype", DTYPES)
def test_decode_all_patterns(dtype):
    got = oracle.decode(dtype, ALL_BITS)
    exp = np.array([refround.value(dtype, b) for b in range(65536)])
    nan = np.isnan(exp)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], exp[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(exp[~nan]))


# ---- P2: round-to-nearest-even encode ---------------------------------------

def _encode_cases(dtype):
    vals = oracle.decode(dtype, ALL_BITS)
    fin = vals[np.isfinite(vals)]
    pos = np.unique(fin[fin > 0])
    mids = (pos[:-1] + pos[1:]) / 2            # exact midpoints (ties)
    up = np.nextafter(fin, np.inf)
    dn = np.nextafter(fin, -np.inf)
    rng = np.random.default_rng(1)
    rnd = np.ldexp(rng.uniform(-2, 2, 20000), rng.integers(-140 if dtype else -30,
                                                            130 if dtype else 18, 20000))
    top = pos[-1]
    edge = np.array([top, top * (1 + 2.0 ** -60), 0.0, -0.0, np.inf, -np.inf,
                     2 * top, -2 * top])
    return np.concatenate([fin, mids, -mids, up, dn, rnd, edge])


@pytest.mark.parametrize("dtype", DTYPES)
def test_encode_rne(dtype):
    xs = _encode_cases(dtype)
    got = oracle.encode(dtype, xs)
    exp = np.array([refround.round_bits(dtype, float(x)) for x in xs], dtype=np.uint16)
    bad = np.nonzero(got != exp)[0]
    assert bad.size == 0, [(float(xs[i]), hex(got[i]), hex(exp[i])) for i in bad[:10]]


@pytest.mark.parametrize("dtype", DTYPES)
def test_encode_nan_and_overflow(dtype):
    got = oracle.encode(dtype, np.array([np.nan, 1e300, -1e300]))
    if dtype == F16:
        assert list(got) == [0x7E00, 0x7C00, 0xFC00]
        # 65504 is the largest finite; 65520 is the tie with the next binade
        assert list(oracle.encode(F16, np.array([65519.999, 65520.0]))) == [0x7BFF, 0x7C00]
    else:
        assert list(got) == [0x7FC0, 0x7F80, 0xFF80]


# ---- P3-P7: closed forms --------------------------------------------------

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n", [1, 40, 129])
def test_identity(dtype, n):
    _, a = random_inputs(1, n, dtype, seed=3)
    B = values_to_bits(np.eye(n), dtype)
    c, _, _ = oracle.gemv(dtype, B, a)
    assert np.array_equal(c, a)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n,k", [(37, 53), (64, 1031), (5, 7)])
def test_permutation_rows(dtype, n, k):
    rng = np.random.default_rng(n * 1000 + k)
    cols = rng.choice(k, size=n, replace=n > k)
    cols[0], cols[-1] = 0, k - 1
    Bv = np.zeros((n, k))
    Bv[np.arange(n), cols] = 1.0
    _, a = random_inputs(1, k, dtype, seed=5)
    c, _, _ = oracle.gemv(dtype, values_to_bits(Bv, dtype), a)
    assert np.array_equal(c, a[cols])


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n,k", [(19, 71), (8, 1031), (3, 4096)])
def test_column_extraction(dtype, n, k):
    B, _ = random_inputs(n, k, dtype, seed=7)
    rng = np.random.default_rng(k)
    cols = sorted(set(list(range(8)) + list(range(k - 8, k)) + list(rng.integers(0, k, 8))))
    for j in cols:
        av = np.zeros(k)
        av[j] = 1.0
        c, _, _ = oracle.gemv(dtype, B, values_to_bits(av, dtype))
        assert np.array_equal(c, B[:, j]), j


def _exact_int_matvec(Bi, ai):
    return Bi.astype(np.int64) @ ai.astype(np.int64)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n,k", [(33, 100), (7, 3000)])
def test_all_ones_a_integer_B(dtype, n, k):
    g = np.random.default_rng(11)
    Bi = g.integers(-3, 4, size=(n, k))
    c, s, _ = oracle.gemv(dtype, values_to_bits(Bi, dtype), values_to_bits(np.ones(k), dtype))
    sums = Bi.sum(axis=1)
    assert np.array_equal(s, sums.astype(np.float64))
    exp = np.array([refround.round_bits(dtype, float(v)) for v in sums], dtype=np.uint16)
    assert np.array_equal(c, exp)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n,k", [(256, 512), (50, 7169), (4, 65536)])
def test_integer_inputs_exact(dtype, n, k):
    B, a = integer_inputs(n, k, dtype, seed=13)
    Bi = oracle.decode(dtype, B).astype(np.int64)
    ai = oracle.decode(dtype, a).astype(np.int64)
    # the inputs really are the integers -2..2
    assert Bi.min() >= -2 and Bi.max() <= 2 and ai.min() >= -2 and ai.max() <= 2
    exact = _exact_int_matvec(Bi, ai)
    c, s, ab = oracle.gemv(dtype, B, a)
    assert np.array_equal(s, exact.astype(np.float64))
    assert np.array_equal(ab, np.abs(Bi * ai[None, :]).sum(axis=1).astype(np.float64))
    exp = np.array([refround.round_bits(dtype, float(v)) for v in exact], dtype=np.uint16)
    assert np.array_equal(c, exp)


# ---- P8: linearity in a (on the unrounded sum) ------------------------------

@pytest.mark.parametrize("dtype", DTYPES)
def test_linearity_in_a(dtype):
    n, k = 16, 2000
    B, _ = random_inputs(n, k, dtype, seed=17)
    g = np.random.default_rng(2)
    a1 = g.integers(-8, 9, size=k).astype(np.float64)
    a2 = g.integers(-8, 9, size=k).astype(np.float64)
    for alpha, beta in [(1.0, 1.0), (2.0, -1.0), (0.5, 0.25), (-4.0, 0.0)]:
        comb = alpha * a1 + beta * a2          # small dyadic values: exact in both dtypes
        _, s1, ab1 = oracle.gemv(dtype, B, values_to_bits(a1, dtype))
        _, s2, ab2 = oracle.gemv(dtype, B, values_to_bits(a2, dtype))
        _, s12, ab12 = oracle.gemv(dtype, B, values_to_bits(comb, dtype))
        bound = 4 * k * 2.0 ** -53 * (abs(alpha) * ab1 + abs(beta) * ab2 + ab12)
        assert np.all(np.abs(s12 - (alpha * s1 + beta * s2)) <= bound)
    # and not trivially: the sums are not all zero
    assert np.abs(s1).max() > 0.1


# ---- P9: hand-worked cases --------------------------------------------------

def _parse_golden(path):
    cases, cur = [], None
    for raw in open(path):
        line = raw.split("#", 1)[0].strip()
        if not line:
            continue
        tok = line.split()
        if tok[0] == "case":
            cur = {"name": tok[1], "dtype": F16 if tok[2] == "f16" else BF16,
                   "n": int(tok[3]), "k": int(tok[4]), "B": []}
        elif tok[0] == "a":
            cur["a"] = [float(t) for t in tok[1:]]
        elif tok[0] == "c":
            cur["c"] = [float(t) for t in tok[1:]]
        elif tok[0] == "end":
            cases.append(cur)
            cur = None
        else:
            cur["B"].append([float(t) for t in tok])
    return cases


GOLDEN_CASES = _parse_golden(GOLDEN)


@pytest.mark.parametrize("case", GOLDEN_CASES, ids=[c["name"] for c in GOLDEN_CASES])
def test_hand_cases(case):
    dtype = case["dtype"]
    B = np.array(case["B"])
    a = np.array(case["a"])
    assert B.shape == (case["n"], case["k"]) and a.shape == (case["k"],)
    Bb, ab = values_to_bits(B, dtype), values_to_bits(a, dtype)
    # the inputs are exactly representable (the cast changed nothing)
    assert np.array_equal(oracle.decode(dtype, Bb), B)
    assert np.array_equal(oracle.decode(dtype, ab), a)
    c, _, _ = oracle.gemv(dtype, Bb, ab)
    got = oracle.decode(dtype, c)
    assert np.array_equal(got, np.array(case["c"])), (got, case["c"])


# ---- P10: special values ------------------------------------------------------

@pytest.mark.parametrize("dtype", DTYPES)
def test_special_values(dtype):
    inf, nan = np.inf, np.nan
    B = np.array([[1.0, 2.0, 3.0],
                  [nan, 0.0, 0.0],
                  [inf, 1.0, 0.0],
                  [inf, -inf, 0.0],
                  [0.0, 1.0, 1.0],
                  [-inf, 0.0, 5.0]])
    a = np.array([1.0, 1.0, 1.0])
    c, _, _ = oracle.gemv(dtype, values_to_bits(B, dtype), values_to_bits(a, dtype))
    v = oracle.decode(dtype, c)
    assert v[0] == 6.0
    assert math.isnan(v[1])                       # NaN propagates
    assert v[2] == inf                            # inf + finite
    assert math.isnan(v[3])                       # inf - inf
    assert v[4] == 2.0
    assert v[5] == -inf
    # inf * 0 is NaN
    a0 = np.array([0.0, 1.0, 1.0])
    c, _, _ = oracle.gemv(dtype, values_to_bits(B[[2]], dtype), values_to_bits(a0, dtype))
    assert math.isnan(oracle.decode(dtype, c)[0])
    # NaN in a reaches every row
    an = np.array([1.0, nan, 1.0])
    c, _, _ = oracle.gemv(dtype, values_to_bits(B[[0, 4]], dtype), values_to_bits(an, dtype))
    assert np.all(np.isnan(oracle.decode(dtype, c)))
    # canonical quiet NaN output
    assert c[0] == (0x7E00 if dtype == F16 else 0x7FC0)


@pytest.mark.parametrize("dtype", DTYPES)
def test_empty_shapes(dtype):
    c, s, ab = oracle.gemv(dtype, np.zeros((5, 0), np.uint16), np.zeros(0, np.uint16))
    assert list(c) == [0] * 5 and list(s) == [0.0] * 5 and list(ab) == [0.0] * 5
    c, _, _ = oracle.gemv(dtype, np.zeros((0, 9), np.uint16), np.zeros(9, np.uint16))
    assert c.shape == (0,)


# ---- P14: the fp64 sum against the exact rational sum ----------------------

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("k", [1, 7, 64])
def test_against_exact_rational_sum(dtype, k):
    n = 24
    B, a = random_inputs(n, k, dtype, seed=19 + k)
    Bf = [[Fraction(refround.value(dtype, b)) for b in row] for row in B]
    af = [Fraction(refround.value(dtype, x)) for x in a]
    c, s, ab = oracle.gemv(dtype, B, a)
    for i in range(n):
        exact = sum(Bf[i][j] * af[j] for j in range(k))
        bound = Fraction(max(k - 1, 0)) * Fraction(2) ** -53 * Fraction(ab[i])
        assert abs(Fraction(s[i]) - exact) <= bound
        assert c[i] == refround.round_fraction_bits(dtype, exact) or bound > 0 and \
            refround.round_fraction_bits(dtype, exact - bound) != \
            refround.round_fraction_bits(dtype, exact + bound)


def test_oracle_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.gemv(F16, np.zeros((3, 4), np.uint16), np.zeros(5, np.uint16))


def test_inputs_are_seeded():
    B1, a1 = random_inputs(8, 100, F16, seed=0)
    B2, a2 = random_inputs(8, 100, F16, seed=0)
    B3, _ = random_inputs(8, 100, F16, seed=1)
    assert np.array_equal(B1, B2) and np.array_equal(a1, a2)
    assert not np.array_equal(B1, B3)
    # N(0,1)/sqrt(k) rows: the row norm is near 1
    v = oracle.decode(F16, B1)
    assert 0.5 < float(np.sqrt((v ** 2).sum(axis=1)).mean()) < 1.5


# ---- epilogue: c = round(alpha * (B @ a) + bias) --------------------------------

@pytest.mark.parametrize("dtype", DTYPES)
def test_epilogue_identity_settings_match_plain(dtype):
    """alpha = 1 and no bias is the plain product, bit for bit."""
    B, a = random_inputs(40, 1031, dtype, seed=31)
    c0, s0, _ = oracle.gemv(dtype, B, a)
    c1, y1, _ = oracle.gemv_epilogue(dtype, B, a, 1.0, None)
    assert np.array_equal(c0, c1) and np.array_equal(s0, y1)


@pytest.mark.parametrize("dtype", DTYPES)
def test_epilogue_integer_exact(dtype):
    """Integer B, a, bias and a power-of-two alpha: the result is the exact
    integer expression, rounded once (checked with Python integers)."""
    n, k = 50, 700
    B, a = integer_inputs(n, k, dtype, seed=33)
    g = np.random.default_rng(3)
    bias_v = g.integers(-40, 41, size=n).astype(np.float64)
    bias = values_to_bits(bias_v, dtype)
    Bi = oracle.decode(dtype, B).astype(np.int64)
    ai = oracle.decode(dtype, a).astype(np.int64)
    exact = Bi @ ai
    for alpha in (1.0, 2.0, -0.5, 0.25):
        c, y, _ = oracle.gemv_epilogue(dtype, B, a, alpha, bias)
        want = [alpha * float(e) + float(b) for e, b in zip(exact, bias_v)]
        assert np.array_equal(y, np.array(want))
        assert np.array_equal(c, np.array([refround.round_bits(dtype, w) for w in want],
                                          dtype=np.uint16))


def test_epilogue_hand_case():
    """By hand (fp16): B = [[1, 2], [3, 4]], a = [1, 1], alpha = 0.5,
    bias = [10, -1]: c = [0.5*3 + 10, 0.5*7 - 1] = [11.5, 2.5]."""
    B = values_to_bits(np.array([[1.0, 2.0], [3.0, 4.0]]), F16)
    a = values_to_bits(np.array([1.0, 1.0]), F16)
    bias = values_to_bits(np.array([10.0, -1.0]), F16)
    c, _, _ = oracle.gemv_epilogue(F16, B, a, 0.5, bias)
    assert list(oracle.decode(F16, c)) == [11.5, 2.5]


def test_epilogue_alpha_is_float32():
    """alpha is taken at float32 precision: 0.1 becomes 0.100000001490116..."""
    B = values_to_bits(np.array([[1.0]]), F16)
    a = values_to_bits(np.array([1024.0]), F16)
    _, y, _ = oracle.gemv_epilogue(F16, B, a, 0.1, None)
    assert y[0] == float(np.float32(0.1)) * 1024.0
