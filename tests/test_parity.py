"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle
on the same seeded input bits.

* small and ragged shapes (several tiles, k tails, misaligned rows, row
  tails), every compiled variant, full oracle;
* integer inputs: every variant bit-exact (the fp32 sum is exact);
* closed forms on the GPU: identity, permutation, one-hot columns;
* every workload shape at full size, every row, in the automatic
  configuration the benchmark times and in every variant;
* determinism, misaligned base pointers, special values, empty and tiny
  sizes, rejected calls that must not touch c.
"""
import numpy as np
import pytest
import torch

import memory_bound_dense_amd as mbd
import oracle
from gemv_inputs import (ALL_WORKLOADS, BF16, EXTRA_WORKLOADS, F16, integer_inputs, random_inputs,
                         torch_dtype, values_to_bits)
from parity import compare, to_bits, to_device

pytestmark = pytest.mark.gpu

NV = mbd.gemv_num_variants()
VARIANTS = list(range(NV))
# The automatic plan through gemv_run_ws with a workspace (-1, the plan the
# benchmark times) and through gemv_run, which has no scratch (-2).
AUTO = [-1, -2]


def _extra_adds(g, n, k, dtype, use_ws=True):
    """fp32 additions after the per-lane sums, beyond the wave tree: the
    in-workgroup slices plus the cross-workgroup k-groups of the plan in use."""
    v, _, q = g.query_config(n, k, dtype, with_workspace=use_ws)
    return mbd.gemv_variant_info(v)[1].splits + (q if q > 1 else 0)


@pytest.fixture(scope="module")
def g():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    h = mbd.Gemv(workspace=True)
    yield h
    h.close()


LAST_EXTRA = [0]


def fits(g, v, n, k, dtype):
    """Whether variant v can run (n, k): a forced variant whose LDS or
    scratch needs exceed what there is is rejected with GEMV_ERR_UNSUPPORTED
    (or GEMV_ERR_TOO_LARGE: more k-split partials than the scratch holds)."""
    if v < 0 or n == 0:
        return True
    g.force_config(v)
    try:
        g.query_config(n, k, dtype)
        return True
    except mbd.GemvError as e:
        assert e.status in (mbd._lib.GEMV_ERR_UNSUPPORTED, mbd._lib.GEMV_ERR_TOO_LARGE), e
        return False
    finally:
        g.force_config(-1)


def staged_rejects(v, Bd):
    """The pipelined-B variants take 16-byte aligned rows only (and say so
    with GEMV_ERR_UNSUPPORTED)."""
    k = Bd.shape[1]
    return v >= 0 and mbd.gemv_variant_info(v)[1].stages > 0 and k > 0 and \
        (k % 8 != 0 or Bd.data_ptr() % 16 != 0)


def run(g, Bd, ad, variant=-1, grid=0, kgroups=0):
    """c = B @ a with a forced configuration (-1: the automatic plan with the
    workspace, -2: without); None if the variant cannot run this shape."""
    use_ws = variant != -2
    variant = max(variant, -1)
    n, k = Bd.shape
    dtype = mbd.GEMV_F16 if Bd.dtype == torch.float16 else mbd.GEMV_BF16
    if not fits(g, variant, n, k, dtype):
        return None
    c = torch.full((n,), float("nan"), dtype=Bd.dtype, device=Bd.device)
    g.force_config(variant, grid, kgroups)
    try:
        if n > 0:
            LAST_EXTRA[0] = _extra_adds(g, n, k, dtype, use_ws)
        if staged_rejects(variant, Bd):
            with pytest.raises(mbd.GemvError) as ei:
                g(Bd, ad, c)
            assert ei.value.status == mbd._lib.GEMV_ERR_UNSUPPORTED
            torch.cuda.synchronize()
            assert torch.all(torch.isnan(c))     # nothing was launched
            return None
        g(Bd, ad, c, use_workspace=use_ws)
    finally:
        g.force_config(-1)
    torch.cuda.synchronize()
    return to_bits(c)


def _check(dtype, got, ref, ab, k, v, what):
    ok_g, ok_s, rg, rs, first = compare(dtype, got, ref, ab, k, LAST_EXTRA[0])
    assert ok_g, "%s variant %d: outside the grading tolerance (%s)" % (what, v, first)
    assert ok_s, "%s variant %d: outside the strict fp32 bound (max ratio %.3g, %s)" % (
        what, v, rs, first)


SMALL = [(256, 512, F16, "uniform"), (256, 512, BF16, "uniform"),
         (100, 1000, F16, "normal"), (129, 1537, BF16, "normal"),
         (37, 7169, F16, "normal"), (37, 7169, BF16, "normal"),
         (1000, 7000, BF16, "normal"), (300, 4096, F16, "normal"),
         (64, 65536, BF16, "normal"), (3, 513, F16, "normal"), (1, 8, BF16, "normal"),
         (7, 1, F16, "normal"), (5, 511, BF16, "normal")]


@pytest.mark.parametrize("n,k,dtype,dist", SMALL,
                         ids=["%dx%d_%s" % (n, k, "f16" if d == F16 else "bf16")
                              for n, k, d, _ in SMALL])
def test_small_shapes_every_variant(g, n, k, dtype, dist):
    B, a = random_inputs(n, k, dtype, dist, seed=0)
    ref, _, ab = oracle.gemv(dtype, B, a)
    Bd, ad = to_device(B, dtype), to_device(a, dtype)
    for v in AUTO + VARIANTS:
        got = run(g, Bd, ad, v)
        if got is None:
            continue
        _check(dtype, got, ref, ab, k, v, "%dx%d" % (n, k))


INT_SHAPES = [(256, 512), (50, 7169), (1000, 7000), (64, 65536), (33, 100), (5, 8), (129, 1031)]


@pytest.mark.parametrize("dtype", [F16, BF16], ids=["f16", "bf16"])
@pytest.mark.parametrize("n,k", INT_SHAPES, ids=["%dx%d" % s for s in INT_SHAPES])
def test_integer_inputs_bit_exact_every_variant(g, n, k, dtype):
    B, a = integer_inputs(n, k, dtype, seed=13)
    ref, _, _ = oracle.gemv(dtype, B, a)
    Bd, ad = to_device(B, dtype), to_device(a, dtype)
    for v in AUTO + VARIANTS:
        got = run(g, Bd, ad, v)
        if got is None:
            continue
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, "variant %d rows %s: gpu %s ref %s" % (
            v, bad[:5], got[bad[:5]], ref[bad[:5]])


@pytest.mark.parametrize("dtype", [F16, BF16], ids=["f16", "bf16"])
def test_identity_and_permutation(g, dtype):
    for n, k in [(520, 520), (37, 7169), (200, 1031)]:
        rng = np.random.default_rng(n + k)
        cols = rng.choice(k, size=n, replace=n > k)
        cols[0], cols[-1] = 0, k - 1
        Bv = np.zeros((n, k), dtype=np.float32)
        Bv[np.arange(n), cols] = 1.0
        _, a = random_inputs(1, k, dtype, seed=5)
        Bd, ad = to_device(values_to_bits(Bv, dtype), dtype), to_device(a, dtype)
        for v in AUTO + VARIANTS:
            got = run(g, Bd, ad, v)
            assert got is None or np.array_equal(got, a[cols]), (n, k, v)


@pytest.mark.parametrize("dtype", [F16, BF16], ids=["f16", "bf16"])
def test_column_extraction(g, dtype):
    for n, k in [(19, 71), (130, 1031), (9, 7169), (4, 65536)]:
        B, _ = random_inputs(n, k, dtype, seed=7)
        Bd = to_device(B, dtype)
        rng = np.random.default_rng(k)
        cols = sorted(set(list(range(9)) + list(range(max(0, k - 9), k))
                          + [int(x) for x in rng.integers(0, k, 6)]
                          + [j for j in (511, 512, 513) if j < k]))
        for j in cols:
            av = np.zeros(k, dtype=np.float32)
            av[j] = 1.0
            ad = to_device(values_to_bits(av, dtype), dtype)
            for v in [-1, 0, 3, 6, NV - 1]:
                got = run(g, Bd, ad, v)
                assert got is None or np.array_equal(got, B[:, j]), (n, k, j, v)


@pytest.mark.parametrize("wl", ALL_WORKLOADS + EXTRA_WORKLOADS,
                         ids=[w[0] for w in ALL_WORKLOADS + EXTRA_WORKLOADS])
def test_workload_full_size(g, wl):
    """Every workload at its full size, in every variant and both automatic
    plans, against the oracle on every row (c starts as NaN, so a row that
    no workgroup writes fails)."""
    name, n, k, dtype, dist = wl
    B, a = random_inputs(n, k, dtype, dist, seed=0)
    ref, _, ab = oracle.gemv(dtype, B, a)
    Bd, ad = to_device(B, dtype), to_device(a, dtype)
    del B
    print("full-size %s: oracle done, %d variants" % (name, NV), flush=True)
    for v in AUTO + VARIANTS:
        got = run(g, Bd, ad, v)
        if got is None:
            continue
        _check(dtype, got, ref, ab, k, v, name)


# One shape per branch of the automatic plan for aligned rows, with the plan
# shape (rows, unroll, waves, splits, a_mode) that branch picks.
RULE_BRANCH_SHAPES = [
    (4096, 1280, F16, (2, 4, 4, 1, 1)),      # short rows: 3 steps
    (12288, 512, BF16, (4, 2, 4, 1, 1)),     # one step from 12288 rows
    (2048, 6104, BF16, (1, 4, 2, 1, 1)),     # 12 steps on 2048..6143 rows
    (8192, 5000, BF16, (3, 2, 8, 8, 1)),     # short rows off 128-byte lines
    (8192, 7000, F16, (3, 2, 8, 8, 1)),      # rows off lines, 13..16 steps
    (6144, 9000, BF16, (3, 3, 8, 8, 1)),     # rows off lines, 17..31 steps
    (2048, 16936, BF16, (2, 2, 8, 8, 3)),    # long rows off lines: the shifted window
    (4096, 11008, F16, (2, 3, 8, 8, 1)),     # the two-row table
    (2048, 28672, BF16, (2, 8, 8, 8, 1)),    # the table, 56 steps
    (1024, 20480, BF16, (2, 3, 16, 16, 1)),  # the table, 40 steps: sixteen slices
    (1024, 33792, F16, (2, 5, 8, 8, 1)),     # 65..80 steps
    (4096, 51200, BF16, (3, 3, 8, 8, 1)),    # more than 96 steps from 4096 rows
    (32768, 2048, BF16, (1, 4, 4, 1, 1)),    # one row of four slots, five workgroups per CU
    (16384, 5120, F16, (2, 3, 4, 4, 1)),     # two rows x four slices, five workgroups per CU
    (448, 1216, F16, (1, 4, 2, 1, 1)),       # 3..4 steps below 1024 rows: four slots, two waves
    (408, 3200, BF16, (1, 2, 4, 4, 1)),      # 5..8 steps up to 512 rows: four slices of two slots
]


@pytest.mark.parametrize("n,k,dtype,want", RULE_BRANCH_SHAPES,
                         ids=["%dx%d_%s" % (n, k, "f16" if d == F16 else "bf16")
                              for n, k, d, _ in RULE_BRANCH_SHAPES])
def test_auto_plan_rule_branches(g, n, k, dtype, want):
    """Each branch of the automatic plan on a shape that takes it: every row
    against the oracle, integer inputs bit-exact, and the automatic launch
    (whose workgroups per CU may be capped by padding their LDS) bit for bit
    the same as the same variant and grid forced without the cap."""
    v, grid, q = g.query_config(n, k, dtype)
    i = mbd.gemv_variant_info(v)[1]
    assert (i.rows, i.unroll, i.waves, i.splits, i.a_mode) == want, (n, k, v)
    B, a = random_inputs(n, k, dtype, "normal", seed=51)
    ref, _, ab = oracle.gemv(dtype, B, a)
    Bd, ad = to_device(B, dtype), to_device(a, dtype)
    del B
    got = run(g, Bd, ad)
    _check(dtype, got, ref, ab, k, v, "%dx%d auto" % (n, k))
    forced = run(g, Bd, ad, v, grid, q)
    assert np.array_equal(got, forced), (n, k, v)
    Bi, ai = integer_inputs(n, k, dtype, seed=52)
    refi, _, _ = oracle.gemv(dtype, Bi, ai)
    assert np.array_equal(run(g, to_device(Bi, dtype), to_device(ai, dtype)), refi), (n, k, v)


def test_deterministic(g):
    for n, k, dtype in [(7168, 16384, BF16), (64, 65536, BF16), (1000, 7000, F16)]:
        B, a = random_inputs(n, k, dtype, seed=1)
        Bd, ad = to_device(B, dtype), to_device(a, dtype)
        for v in [-1, 3, NV - 1]:
            first = run(g, Bd, ad, v)
            if first is None:
                continue
            for _ in range(20):
                assert np.array_equal(run(g, Bd, ad, v), first), (n, k, v)


@pytest.mark.parametrize("dtype", [F16, BF16], ids=["f16", "bf16"])
def test_misaligned_base_pointers(g, dtype):
    n, k = 77, 1000
    B, a = random_inputs(n, k, dtype, seed=3)
    ref, _, ab = oracle.gemv(dtype, B, a)
    # shift each buffer by one element so that no base is 16-byte aligned
    Bbig = to_device(np.concatenate([np.zeros(1, np.uint16), B.ravel()]), dtype)
    abig = to_device(np.concatenate([np.zeros(3, np.uint16), a]), dtype)
    Bd = Bbig[1:].view(n, k)
    ad = abig[3:]
    assert Bd.data_ptr() % 16 != 0 and ad.data_ptr() % 16 != 0
    for v in AUTO + VARIANTS:
        if not fits(g, v, n, k, dtype):
            continue
        if staged_rejects(v, Bd):
            assert run(g, Bd, ad, v) is None
            continue
        cbig = torch.full((n + 5,), 7.0, dtype=torch_dtype(dtype), device="cuda")
        c = cbig[5:]
        g.force_config(max(v, -1))
        LAST_EXTRA[0] = _extra_adds(g, n, k, dtype, v != -2)
        g(Bd, ad, c, use_workspace=v != -2)
        g.force_config(-1)
        torch.cuda.synchronize()
        _check(dtype, to_bits(c), ref, ab, k, v, "misaligned")
        assert torch.all(cbig[:5] == 7.0)


@pytest.mark.parametrize("dtype", [F16, BF16], ids=["f16", "bf16"])
def test_special_values(g, dtype):
    inf, nan = np.inf, np.nan
    k = 1100
    rng = np.random.default_rng(0)
    Bv = rng.integers(-3, 4, size=(8, k)).astype(np.float32)
    Bv[1, 700] = nan
    Bv[2, 5] = inf
    Bv[3, 5], Bv[3, 1099] = inf, -inf
    Bv[4, 1099] = -inf
    av = rng.integers(-2, 3, size=k).astype(np.float32)
    av[5] = av[700] = av[1099] = 1.0
    av[600] = 0.0
    Bv[5, 600] = inf            # inf * 0 -> NaN
    Bv[6, :] = 0.0
    Bb, ab = values_to_bits(Bv, dtype), values_to_bits(av, dtype)
    ref, _, _ = oracle.gemv(dtype, Bb, ab)
    Bd, ad = to_device(Bb, dtype), to_device(ab, dtype)
    r = oracle.decode(dtype, ref)
    for v in AUTO + VARIANTS:
        gb = run(g, Bd, ad, v)
        if gb is None:
            continue
        got = oracle.decode(dtype, gb)
        assert np.array_equal(np.isnan(got), np.isnan(r)), (v, got, r)
        fin = ~np.isnan(r)
        assert np.array_equal(got[fin], r[fin]), (v, got, r)


def _golden_cases():
    """The hand-worked cases of tests/golden/gemv_hand_cases.txt (parsed as
    the oracle's own pins parse them)."""
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "gemv_hand_cases.txt")
    cases, cur = [], None
    for raw in open(path):
        line = raw.split("#", 1)[0].strip()
        if not line:
            continue
        tok = line.split()
        if tok[0] == "case":
            cur = {"name": tok[1], "dtype": F16 if tok[2] == "f16" else BF16, "B": []}
        elif tok[0] in ("a", "c"):
            cur[tok[0]] = [float(t) for t in tok[1:]]
        elif tok[0] == "end":
            cases.append(cur)
        else:
            cur["B"].append([float(t) for t in tok])
    return cases


def _scaled_integers(n, k, dtype, eb, ea, seed, lo=-2, hi=2):
    """B = Bi * 2^eb, a = ai * 2^ea with small integers Bi, ai: every value,
    product and partial sum is exact in fp32, so any summation order gives
    the exact sum and the GPU must match the oracle bit for bit."""
    rng = np.random.default_rng(seed)
    Bv = rng.integers(lo, hi + 1, size=(n, k)).astype(np.float64) * 2.0 ** eb
    av = rng.integers(lo, hi + 1, size=k).astype(np.float64) * 2.0 ** ea
    return Bv, av


def _edge_cases():
    """(name, dtype, B values, a values): hand cases and the edges of the
    dtypes that no random input reaches."""
    out = [("hand_" + c["name"], c["dtype"], np.array(c["B"]), np.array(c["a"]))
           for c in _golden_cases()]
    for n, k in ((37, 1031), (5, 65), (3, 4100)):
        # bf16: products in [2^-133, 2^-131], fp32 subnormals, summed to
        # subnormal and small normal bf16 outputs
        out.append(("bf16_subnormal_products_%dx%d" % (n, k), BF16)
                   + _scaled_integers(n, k, BF16, -64, -69, seed=n + k))
        # bf16 subnormal inputs (B = i * 2^-133), normal products
        out.append(("bf16_subnormal_inputs_%dx%d" % (n, k), BF16)
                   + _scaled_integers(n, k, BF16, -133, 100, seed=n + k + 1))
        # fp16: products of normals on a 2^-25 grid, subnormal outputs
        out.append(("f16_subnormal_outputs_%dx%d" % (n, k), F16)
                   + _scaled_integers(n, k, F16, -12, -13, seed=n + k + 2, lo=-1, hi=1))
        # fp16 subnormal inputs (B = i * 2^-24)
        out.append(("f16_subnormal_inputs_%dx%d" % (n, k), F16)
                   + _scaled_integers(n, k, F16, -24, 10, seed=n + k + 3))
    # bf16 overflow at the tie: (2 - 2^-7) 2^127 (the largest bf16) plus half
    # its spacing rounds to even, i.e. to inf; a quarter of the spacing
    # rounds back to the largest value.  The fp32 sums stay finite.  The
    # rows are long, with the two terms far apart, so the sum crosses the
    # main loop and a k-split.
    k = 3000
    Bv = np.zeros((4, k))
    big = (2.0 - 2.0 ** -7) * 2.0 ** 127
    Bv[0, 3], Bv[0, 2900] = big, 2.0 ** 119
    Bv[1, 3], Bv[1, 2900] = big, 2.0 ** 118
    Bv[2, 3], Bv[2, 2900] = -big, -(2.0 ** 119)
    Bv[3, 0] = 1.0
    out.append(("bf16_overflow_tie", BF16, Bv, np.ones(k)))
    # fp16: a finite fp32 sum past the largest fp16 (1100 * 64 = 70400 -> inf),
    # and 65504 + 16 = 65520 spread over a long row (the tie -> inf)
    k = 1100
    Bv = np.zeros((3, k))
    Bv[0, :] = 64.0
    Bv[1, 0], Bv[1, 1099] = 65504.0, 16.0
    Bv[2, 0], Bv[2, 1099] = 65504.0, 8.0
    out.append(("f16_finite_sum_overflow", F16, Bv, np.ones(k)))
    return out


EDGE = _edge_cases()


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_edge_values_bit_exact_every_variant(g, case):
    """Subnormal inputs and outputs (no flush to zero in the fp32 FMAs or in
    the conversions), the overflow ties and finite sums past the largest
    16-bit value, and the hand-worked cases: every sum is exact in fp32, so
    every variant must give the oracle's bits."""
    name, dtype, Bv, av = case
    Bb, ab = values_to_bits(Bv, dtype), values_to_bits(av, dtype)
    assert np.array_equal(oracle.decode(dtype, Bb), Bv), "inputs must be representable"
    assert np.array_equal(oracle.decode(dtype, ab), av)
    ref, _, _ = oracle.gemv(dtype, Bb, ab)
    Bd, ad = to_device(Bb, dtype), to_device(ab, dtype)
    ran = 0
    for v in AUTO + VARIANTS:
        got = run(g, Bd, ad, v)
        if got is None:
            continue
        ran += 1
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, "%s variant %d rows %s: gpu %s ref %s" % (
            name, v, bad[:5], oracle.decode(dtype, got[bad[:5]]), oracle.decode(dtype, ref[bad[:5]]))
    assert ran >= len(VARIANTS) // 2


def test_empty_and_tiny(g):
    dev = "cuda"
    for dtype in (F16, BF16):
        td = torch_dtype(dtype)
        # n == 0: a no-op that succeeds
        B = torch.empty((0, 16), dtype=td, device=dev)
        a = torch.ones(16, dtype=td, device=dev)
        c = torch.empty(0, dtype=td, device=dev)
        g(B, a, c)
        # k == 0: the empty sum
        B = torch.empty((5, 0), dtype=td, device=dev)
        a = torch.empty(0, dtype=td, device=dev)
        c = torch.full((5,), 3.0, dtype=td, device=dev)
        for v in AUTO + VARIANTS:
            if not fits(g, v, 5, 0, dtype):
                continue
            c.fill_(3.0)
            g.force_config(max(v, -1))
            g(B, a, c, use_workspace=v != -2)
            g.force_config(-1)
            torch.cuda.synchronize()
            assert torch.all(c == 0), v
        # every small k, for row-tail and k-tail coverage
        for k in list(range(1, 18)) + [63, 64, 65, 520]:
            Bb, ab = integer_inputs(3, k, dtype, seed=k)
            ref, _, _ = oracle.gemv(dtype, Bb, ab)
            got = run(g, to_device(Bb, dtype), to_device(ab, dtype))
            assert np.array_equal(got, ref), k


def test_rejected_calls_leave_c_untouched(g):
    n, k = 64, 256
    B = torch.ones((n, k), dtype=torch.float16, device="cuda")
    a = torch.ones(k, dtype=torch.float16, device="cuda")
    # c overlapping B
    s = mbd.gemv_run(g.h, B.data_ptr(), a.data_ptr(), B.data_ptr() + 64, n, k, 0,
                     torch.cuda.current_stream().cuda_stream)
    assert s == mbd._lib.GEMV_ERR_ALIASING
    torch.cuda.synchronize()
    assert torch.all(B == 1)
    # bad dtype and misaligned c
    c = torch.full((n + 1,), 5.0, dtype=torch.float16, device="cuda")
    assert mbd.gemv_run(g.h, B.data_ptr(), a.data_ptr(), c.data_ptr(), n, k, 7, None) == \
        mbd._lib.GEMV_ERR_UNSUPPORTED_DTYPE
    assert mbd.gemv_run(g.h, B.data_ptr(), a.data_ptr(), c.data_ptr() + 1, n, k, 0, None) == \
        mbd._lib.GEMV_ERR_MISALIGNED
    torch.cuda.synchronize()
    assert torch.all(c == 5.0)


def test_query_config_matches_a_variant(g):
    for n, k, dtype in [(18432, 7168, F16), (7168, 16384, BF16), (64, 65536, BF16)]:
        v, grid, q = g.query_config(n, k, dtype)
        assert 0 <= v < NV and grid >= 1 and q >= 1


XWG = [v for v in VARIANTS if mbd.gemv_variant_info(v)[1].cross_wg]
XWG_SHAPES = [(64, 65536, BF16), (7, 20000, F16), (300, 4096, BF16), (1, 513, F16),
              (33, 1031, BF16), (1000, 7000, BF16), (5, 0, F16)]


@pytest.mark.parametrize("n,k,dtype", XWG_SHAPES,
                         ids=["%dx%d_%s" % (n, k, "f16" if d == F16 else "bf16")
                              for n, k, d in XWG_SHAPES])
def test_cross_workgroup_split(g, n, k, dtype):
    """k shared by several workgroups: every k-group count, including more
    slices than there are steps (empty slices), calls repeated back to back
    (the arrival counters must return to zero), random and integer inputs."""
    B, a = random_inputs(n, k, dtype, "normal", seed=21)
    ref, _, ab = oracle.gemv(dtype, B, a)
    Bi, ai = integer_inputs(n, k, dtype, seed=22)
    refi, _, _ = oracle.gemv(dtype, Bi, ai)
    Bd, ad = to_device(B, dtype), to_device(a, dtype)
    Bid, aid = to_device(Bi, dtype), to_device(ai, dtype)
    assert XWG
    for v in XWG:
        for q in (1, 2, 3, 8, 33, 64):
            for grid in (0, 1, 3):
                if n * -(-q // 32) * 32 > (1 << 18):   # the partials' share of the workspace
                    continue
                for _ in range(2):
                    got = run(g, Bd, ad, v, grid, q)
                    if got is None:
                        break
                    _check(dtype, got, ref, ab, k, v, "%dx%d q=%d grid=%d" % (n, k, q, grid))
                    goti = run(g, Bid, aid, v, grid, q)
                    assert np.array_equal(goti, refi), (v, q, grid)


AUTO_XWG_SHAPES = [(96, 131072, BF16), (100, 65544, F16), (129, 262152, BF16), (200, 262144, F16),
                   (16, 262144, BF16), (48, 131075, F16), (3, 1048576, BF16), (194, 131073, F16),
                   (40, 262147, F16), (8, 131072, BF16), (72, 131072, F16)]


@pytest.mark.parametrize("n,k,dtype", AUTO_XWG_SHAPES,
                         ids=["%dx%d_%s" % (n, k, "f16" if d == F16 else "bf16")
                              for n, k, d in AUTO_XWG_SHAPES])
def test_auto_plan_cross_workgroup_rows(g, n, k, dtype):
    """The automatic plan's cross-workgroup split over its whole range (up
    to 256 rows, 8 to 64 k-groups, one row per 8-wave workgroup or four per
    4-wave workgroup, rows with and without a partial step): every row
    against the oracle, three calls back to back (the counters return to
    zero between calls), and integer inputs bit-exact."""
    v, grid, q = g.query_config(n, k, dtype)
    assert mbd.gemv_variant_info(v)[1].cross_wg and 2 <= q <= 64, (n, k, v, q)
    B, a = random_inputs(n, k, dtype, "normal", seed=31)
    ref, _, ab = oracle.gemv(dtype, B, a)
    Bd, ad = to_device(B, dtype), to_device(a, dtype)
    for _ in range(3):
        got = run(g, Bd, ad)
        _check(dtype, got, ref, ab, k, v, "%dx%d auto q=%d" % (n, k, q))
    Bi, ai = integer_inputs(n, k, dtype, seed=32)
    refi, _, _ = oracle.gemv(dtype, Bi, ai)
    goti = run(g, to_device(Bi, dtype), to_device(ai, dtype))
    assert np.array_equal(goti, refi)


@pytest.mark.parametrize("n,k,dtype", [(64, 65536, BF16), (7, 100003, F16), (33, 70000, BF16)],
                         ids=["64x65536_bf16", "7x100003_f16", "33x70000_bf16"])
def test_ticketed_and_counted_combines_agree_bitwise(g, n, k, dtype):
    """With one row per workgroup (and at most 512 workgroups) the split
    combines by tickets, with fewer row ranges by counting arrivals; both sum
    a row's k-group partials in the same fixed lane order, so for the same
    variant and k-groups c must have the same bits, on random data."""
    B, a = random_inputs(n, k, dtype, "normal", seed=41)
    Bd, ad = to_device(B, dtype), to_device(a, dtype)
    xwg1 = [v for v in XWG if mbd.gemv_variant_info(v)[1].waves == mbd.gemv_variant_info(v)[1].splits
            and mbd.gemv_variant_info(v)[1].rows == 1]
    assert xwg1
    for v in xwg1:
        for q in (2, 5, 8):
            if n * q > 512:
                continue
            ticketed = run(g, Bd, ad, v, 0, q)        # grid n: one row per workgroup
            counted = run(g, Bd, ad, v, 3, q)         # three row ranges
            assert ticketed is not None and counted is not None
            assert np.array_equal(ticketed, counted), (v, q)


def test_cross_workgroup_config_rules(g):
    nonx = [v for v in VARIANTS if not mbd.gemv_variant_info(v)[1].cross_wg][0]
    with pytest.raises(mbd.GemvError):
        g.force_config(nonx, 0, 4)          # k-groups only exist for cross_wg variants
    g.force_config(-1)
    # too many partials for the workspace: rejected, c untouched
    v = XWG[0]
    n, k = 40000, 4096
    B = torch.zeros((n, k), dtype=torch.float16, device="cuda")
    a = torch.zeros(k, dtype=torch.float16, device="cuda")
    c = torch.full((n,), 5.0, dtype=torch.float16, device="cuda")
    g.force_config(v, 0, 64)
    with pytest.raises(mbd.GemvError) as e:
        g(B, a, c)
    assert e.value.status == mbd._lib.GEMV_ERR_TOO_LARGE
    g.force_config(-1)
    # a row's partials take whole 128-byte lines: 2 k-groups take 32 slots a
    # row, so 8192 rows fit the 2^18 partials and 8193 do not
    g.force_config(v, 0, 2)
    assert g.query_config(8192, 4096, mbd.GEMV_F16)[2] == 2
    with pytest.raises(mbd.GemvError) as e:
        g.query_config(8193, 4096, mbd.GEMV_F16)
    assert e.value.status == mbd._lib.GEMV_ERR_TOO_LARGE
    g.force_config(-1)
    torch.cuda.synchronize()
    assert torch.all(c == 5.0)
    # a cross-workgroup variant needs the caller's scratch: not from gemv_run
    n, k = 64, 4096
    B, a, c = B[:n, :k].contiguous(), a[:k].contiguous(), c[:n].contiguous()
    g.force_config(v, 0, 4)
    try:
        with pytest.raises(mbd.GemvError) as e:
            g(B, a, c, use_workspace=False)
        assert e.value.status == mbd._lib.GEMV_ERR_UNSUPPORTED
    finally:
        g.force_config(-1)
    # workspace checks: too small, misaligned, overlapping c or B
    sp = torch.cuda.current_stream().cuda_stream
    ws, nb = g.ws.data_ptr(), g.ws.numel()
    big = torch.zeros(nb + 4096, dtype=torch.uint8, device="cuda")
    for wptr, wbytes, want in [(ws, nb - 1, mbd._lib.GEMV_ERR_INVALID_ARG),
                               (big.data_ptr() + 8, nb, mbd._lib.GEMV_ERR_MISALIGNED),
                               (c.data_ptr() - 1024, nb, mbd._lib.GEMV_ERR_ALIASING),
                               (B.data_ptr() + 4096, nb, mbd._lib.GEMV_ERR_ALIASING)]:
        s = mbd.gemv_run_ws(g.h, B.data_ptr(), a.data_ptr(), c.data_ptr(), n, k, mbd.GEMV_F16,
                            wptr, wbytes, stream=sp)
        assert s == want, (wptr - ws, wbytes, s)
    torch.cuda.synchronize()
    assert torch.all(c == 5.0)


def test_query_config_many_shapes(g):
    """Every automatic plan names a compiled variant that fits."""
    for n in (1, 7, 64, 255, 256, 1000, 4096, 7168, 18432, 100000):
        for k in (0, 1, 511, 512, 4096, 7169, 16384, 65536, 200000):
            for dtype in (F16, BF16):
                v, grid, q = g.query_config(n, k, dtype)
                assert 0 <= v < NV and grid >= 1 and q >= 1, (n, k, dtype)


def test_query_config_matches_the_host_plan(g):
    """The handle's plan is the host-only rule of gemv_plan_config (the
    device's per-workgroup LDS limit is 160 KiB)."""
    for n in (1, 64, 127, 128, 1000, 2048, 4096, 18432, 18433):
        for k in (1, 512, 7168, 7169, 12289, 16383, 65536):
            for dtype in (F16, BF16):
                for ws in (0, 1):
                    v, grid, q = g.query_config(n, k, dtype, with_workspace=ws)
                    s, cfg = mbd.gemv_plan_config(n, k, dtype, 1, 160 * 1024, ws)
                    assert s == mbd.GEMV_OK
                    assert (v, grid, q) == (cfg.variant, cfg.grid, cfg.kgroups), (n, k, dtype, ws)


# the kernels for rows off 16-byte boundaries: a staged twice in LDS (a_mode 2)
# or read at each row's shift through the caches (a_mode 3)
REALIGN = [v for v in VARIANTS if mbd.gemv_variant_info(v)[1].a_mode in (2, 3)]


@pytest.mark.parametrize("dtype", [F16, BF16], ids=["f16", "bf16"])
def test_realigned_rows_do_not_leak(g, dtype):
    """Rows whose starts fall inside 16-byte granules: alternate all-NaN rows
    with clean rows, for every row offset (odd k), base pointers shifted by
    0..7 elements, and every grid; a clean row must never pick up its
    neighbours' elements from a shared granule."""
    assert REALIGN
    for k in (13, 7169, 515, 1):
        n = 24
        B, a = random_inputs(n, k, dtype, seed=k)
        B = B.copy()
        nan = values_to_bits(np.array([np.nan]), dtype)[0]
        B[0::2, :] = nan
        ref, _, ab = oracle.gemv(dtype, B, a)
        for shift in range(8):
            Bbig = to_device(np.concatenate([np.zeros(shift, np.uint16), B.ravel(),
                                             np.full(9, nan, np.uint16)]), dtype)
            Bd = Bbig[shift:shift + n * k].view(n, k)
            ad = to_device(a, dtype)
            for v in [-1] + REALIGN:
                for grid in (0, 1, 5):
                    got = run(g, Bd, ad, v, grid)
                    if got is None:
                        continue
                    r, gg = oracle.decode(dtype, ref), oracle.decode(dtype, got)
                    assert np.array_equal(np.isnan(gg), np.isnan(r)), (k, shift, v, grid)
                    _check(dtype, got, ref, ab, k, v, "realign k=%d shift=%d" % (k, shift))


def test_auto_plan_realigns_misaligned_rows(g):
    """Misaligned rows on the device handle: from 768 rows the shifted-window
    kernel (a_mode 3), mostly in its two-slot forms, by the rows' granule
    steps and count; rows of at most 2 steps from 8192 rows two rows per trip
    of the realigning kernel (a_mode 2), and 5 steps from 12288 rows one; 5
    steps below 1024 rows and fewer than 768 rows the plan of aligned rows."""
    for n, k, want in [(18433, 7169, (3, 2, 4, 4)), (3072, 7169, (3, 2, 8, 8)),
                       (1000, 16383, (3, 2, 8, 8)), (3072, 12289, (3, 2, 8, 8)),
                       (4096, 12289, (3, 2, 8, 8)), (6144, 20993, (3, 2, 8, 8)),
                       (6144, 4097, (3, 2, 4, 4)), (9000, 4097, (3, 2, 4, 4)),
                       (16384, 1025, (3, 2, 4, 1)), (8192, 1025, (3, 2, 4, 1)),
                       (8192, 961, (2, 2, 8, 1)), (4040, 641, (3, 1, 4, 1)),
                       (12288, 2049, (2, 1, 8, 1)), (768, 2049, (1, 1, 2, 1)),
                       (100, 1000, (1, 1, 4, 1))]:
        v, grid, q = g.query_config(n, k, BF16)
        info = mbd.gemv_variant_info(v)[1]
        assert (info.a_mode, info.rows, info.waves, info.splits) == want, (n, k, v)


LONG_MIS = [(4096, 12289, BF16, 3), (4096, 16001, F16, 1), (1000, 16383, BF16, 5),
            (6144, 4097, BF16, 2), (6400, 2049, F16, 7), (3072, 1025, F16, 0),
            (8192, 4097, BF16, 3), (6144, 20003, BF16, 1), (16385, 1025, F16, 5),
            (9000, 4097, BF16, 2), (8200, 2559, F16, 4), (1536, 9217, BF16, 6),
            (800, 5121, F16, 1), (2000, 2049, BF16, 7), (3072, 12289, F16, 2),
            (6144, 20993, BF16, 3), (12288, 2049, F16, 6), (8192, 24577, BF16, 5),
            (900, 65537, F16, 4), (2048, 1025, BF16, 3), (4096, 32769, F16, 2),
            (8192, 961, BF16, 3), (30001, 719, F16, 5), (4040, 641, BF16, 1),
            (768, 9, F16, 2), (65536, 9, BF16, 1), (8193, 1545, F16, 6),
            (6145, 1545, BF16, 7), (137, 11919, F16, 3), (237, 79545, BF16, 1)]


@pytest.mark.parametrize("n,k,dtype,shift", LONG_MIS,
                         ids=["%dx%d_%s" % (n, k, "f16" if d == F16 else "bf16")
                              for n, k, d, _ in LONG_MIS])
def test_auto_plan_long_misaligned_rows(g, n, k, dtype, shift):
    """Each tier of the automatic plan for misaligned rows against the full
    oracle, with B's base pointer off 16-byte alignment as well."""
    B, a = random_inputs(n, k, dtype, seed=n + k)
    ref, _, ab = oracle.gemv(dtype, B, a)
    Bbig = to_device(np.concatenate([np.zeros(shift, np.uint16), B.ravel()]), dtype)
    Bd = Bbig[shift:].view(n, k)
    got = run(g, Bd, to_device(a, dtype))
    _check(dtype, got, ref, ab, k, -1, "auto %dx%d shift %d" % (n, k, shift))


def run_ex(g, Bd, ad, alpha, bias, variant=-1, c=None):
    n, k = Bd.shape
    dtype = mbd.GEMV_F16 if Bd.dtype == torch.float16 else mbd.GEMV_BF16
    if not fits(g, variant, n, k, dtype):
        return None
    if staged_rejects(variant, Bd):
        assert run(g, Bd, ad, variant) is None
        return None
    if c is None:
        c = torch.full((n,), float("nan"), dtype=Bd.dtype, device=Bd.device)
    use_ws = variant != -2
    g.force_config(max(variant, -1))
    try:
        if n > 0:
            LAST_EXTRA[0] = _extra_adds(g, n, k, dtype, use_ws)
        g(Bd, ad, c, alpha=alpha, bias=bias, use_workspace=use_ws)
    finally:
        g.force_config(-1)
    torch.cuda.synchronize()
    return to_bits(c)


EPI_SHAPES = [(300, 4096, F16), (129, 1537, BF16), (64, 65536, BF16), (37, 7169, F16)]


@pytest.mark.parametrize("n,k,dtype", EPI_SHAPES,
                         ids=["%dx%d_%s" % (n, k, "f16" if d == F16 else "bf16")
                              for n, k, d in EPI_SHAPES])
def test_epilogue_every_variant(g, n, k, dtype):
    """c = alpha * (B @ a) + bias against the oracle: every variant, with and
    without bias; the bound adds |alpha| to the fp32 sum term and one fp32
    rounding of the FMA."""
    B, a = random_inputs(n, k, dtype, seed=41)
    Bd, ad = to_device(B, dtype), to_device(a, dtype)
    rng = np.random.default_rng(5)
    bias_bits = values_to_bits(rng.normal(size=n).astype(np.float32), dtype)
    biasd = to_device(bias_bits, dtype)
    for alpha in (1.0, -0.5, 0.1):
        for with_bias in (False, True):
            ref, y, ab = oracle.gemv_epilogue(dtype, B, a, alpha, bias_bits if with_bias else None)
            a32 = abs(float(np.float32(alpha)))
            for v in AUTO + VARIANTS:
                got = run_ex(g, Bd, ad, alpha, biasd if with_bias else None, v)
                if got is None:
                    continue
                gv, rv = oracle.decode(dtype, got), oracle.decode(dtype, ref)
                from parity import ulp
                u = ulp(dtype, np.maximum(np.abs(gv), np.abs(rv)))
                strict = u + 2.0 ** -24 * ((np.ceil(k / 64) + 8 + LAST_EXTRA[0]) * a32 * ab
                                           + np.abs(y))
                grade = 4e-3 * a32 * ab + ulp(dtype, rv)
                d = np.abs(gv - rv)
                assert np.all(d <= grade), (alpha, with_bias, v)
                assert np.all(d <= strict), (alpha, with_bias, v, float((d / strict).max()))


@pytest.mark.parametrize("dtype", [F16, BF16], ids=["f16", "bf16"])
def test_epilogue_integer_exact_and_in_place(g, dtype):
    """Integer B, a, bias and a power-of-two alpha: every variant bit-exact;
    bias == c accumulates in place."""
    n, k = 200, 3000
    B, a = integer_inputs(n, k, dtype, seed=43)
    rng = np.random.default_rng(7)
    bias_bits = values_to_bits(rng.integers(-30, 31, size=n).astype(np.float32), dtype)
    Bd, ad = to_device(B, dtype), to_device(a, dtype)
    for alpha in (2.0, -0.25):
        ref, _, _ = oracle.gemv_epilogue(dtype, B, a, alpha, bias_bits)
        for v in AUTO + VARIANTS:
            biasd = to_device(bias_bits, dtype)
            got = run_ex(g, Bd, ad, alpha, biasd, v)
            if got is None:
                continue
            assert np.array_equal(got, ref), (alpha, v)
            # in place: c starts as the bias
            c = to_device(bias_bits, dtype)
            got = run_ex(g, Bd, ad, alpha, c, v, c=c)
            assert np.array_equal(got, ref), ("in place", alpha, v)


def test_random_shapes(g):
    """Seeded random (n, k, dtype), base pointers shifted by 0..7 elements,
    the automatic plan and three random variants (random grid) per shape,
    one with the epilogue: against the full oracle."""
    rng = np.random.default_rng(123)
    for case in range(40):
        n = int(np.exp(rng.uniform(0, np.log(4000))))
        k = int(np.exp(rng.uniform(0, np.log(30000))))
        if n * k > 12_000_000:
            k = max(1, 12_000_000 // n)
        dtype = F16 if rng.random() < 0.5 else BF16
        shift = int(rng.integers(0, 8))
        B, a = random_inputs(n, k, dtype, seed=1000 + case)
        ref, _, ab = oracle.gemv(dtype, B, a)
        Bbig = to_device(np.concatenate([np.zeros(shift, np.uint16), B.ravel()]), dtype)
        Bd = Bbig[shift:].view(n, k)
        ad = to_device(a, dtype)
        picks = [-1] + [int(x) for x in rng.choice(VARIANTS, size=3, replace=False)]
        for v in picks:
            grid = 0 if v < 0 else int(rng.choice([0, 1, 7, 300]))
            got = run(g, Bd, ad, v, grid)
            if got is None:
                continue
            _check(dtype, got, ref, ab, k, v, "random case %d (%d x %d, shift %d, grid %d)"
                   % (case, n, k, shift, grid))
        alpha = float(rng.choice([0.5, -1.0, 3.0]))
        bias = values_to_bits(rng.normal(size=n).astype(np.float32), dtype)
        ref_e, y, ab_e = oracle.gemv_epilogue(dtype, B, a, alpha, bias)
        got = run_ex(g, Bd, ad, alpha, to_device(bias, dtype))
        gv, rv = oracle.decode(dtype, got), oracle.decode(dtype, ref_e)
        from parity import ulp
        bound = 4e-3 * abs(alpha) * ab_e + ulp(dtype, rv)
        assert np.all(np.abs(gv - rv) <= bound), ("epilogue", case, n, k)


STAGED = [v for v in VARIANTS if mbd.gemv_variant_info(v)[1].stages > 0]


@pytest.mark.parametrize("dtype", [F16, BF16], ids=["f16", "bf16"])
def test_staged_pipeline(g, dtype):
    """The pipelined-B variants: many row trips per wave (small grids), item
    counts that are not multiples of the depth, groups past the last full
    step, k below one step, partial last steps, and the 64-row store
    batches; integer inputs make every order exact, so the result must equal
    the oracle bit for bit, and c's neighbours stay untouched."""
    assert STAGED
    for n, k in [(1000, 7168), (300, 512), (129, 1536), (77, 4104), (65, 256), (333, 2560),
                 (5, 8)]:
        B, a = integer_inputs(n, k, dtype, seed=n + k)
        ref = oracle.gemv(dtype, B, a)[0]
        Bd, ad = to_device(B, dtype), to_device(a, dtype)
        for v in STAGED:
            for grid in (0, 1, 3, 17):
                cbig = torch.full((n + 130,), 5.0, dtype=torch_dtype(dtype), device="cuda")
                c = cbig[65:65 + n]
                g.force_config(v, grid)
                try:
                    g(Bd, ad, c)
                finally:
                    g.force_config(-1)
                torch.cuda.synchronize()
                got = to_bits(c)
                bad = np.nonzero(got != ref)[0]
                assert bad.size == 0, (n, k, v, grid, bad[:5])
                assert torch.all(cbig[:65] == 5.0) and torch.all(cbig[65 + n:] == 5.0), (n, k, v)
