"""GPU: gemv_run_noalloc, the entry point for callers that cannot allocate
(it runs gemv_run_ws on the library's static per-GPU scratch), against
gemv_run_ws with a caller workspace, through the C ABI.

Both launch the same plan with the same kernels, so c must have the same
bits; each result is also checked against the oracle.  Two calls in a row
on the same scratch, the second on a smaller input (the scratch keeps the
first call's contents, and the counters must be back at zero), for plans
that split k across workgroups (different k-group counts use different
counter banks) and for plans that use no scratch at all; an oversized
forced split is refused with GEMV_ERR_TOO_LARGE and c stays untouched.
"""
import numpy as np
import pytest
import torch

import memory_bound_dense_amd as mbd
import oracle
from gemv_inputs import BF16, F16, random_inputs, values_to_bits
from parity import compare, to_bits, to_device, ulp

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    h = mbd.Gemv(workspace=True)
    yield h
    h.close()


def _dt(Bd):
    return mbd.GEMV_F16 if Bd.dtype == torch.float16 else mbd.GEMV_BF16


def _pair(g, Bd, ad, alpha=None, bias=None):
    """c from gemv_run_noalloc and from gemv_run_ws (caller workspace), on the
    current stream; both start as NaN so an unwritten row shows."""
    n, k = Bd.shape
    sp = torch.cuda.current_stream().cuda_stream
    bp = None if bias is None else bias.data_ptr()
    c0 = torch.full((n,), float("nan"), dtype=Bd.dtype, device="cuda")
    c1 = torch.full((n,), float("nan"), dtype=Bd.dtype, device="cuda")
    s = mbd.gemv_run_noalloc(g.h, Bd.data_ptr(), ad.data_ptr(), c0.data_ptr(), n, k, _dt(Bd),
                             alpha, bp, sp)
    assert s == mbd.GEMV_OK, mbd.gemv_status_string(s)
    s = mbd.gemv_run_ws(g.h, Bd.data_ptr(), ad.data_ptr(), c1.data_ptr(), n, k, _dt(Bd),
                        g.ws.data_ptr(), g.ws.numel(), alpha, bp, sp)
    assert s == mbd.GEMV_OK, mbd.gemv_status_string(s)
    torch.cuda.synchronize()
    return to_bits(c0), to_bits(c1)


def _check(g, n, k, dtype, seed, alpha=None, with_bias=False):
    B, a = random_inputs(n, k, dtype, seed=seed)
    Bd, ad = to_device(B, dtype), to_device(a, dtype)
    bias_bits = None
    if with_bias:
        rng = np.random.default_rng(seed)
        bias_bits = values_to_bits(rng.normal(size=n).astype(np.float32), dtype)
    bias = None if bias_bits is None else to_device(bias_bits, dtype)
    got, ref_ws = _pair(g, Bd, ad, alpha, bias)
    assert np.array_equal(got, ref_ws), (n, k, dtype, np.nonzero(got != ref_ws)[0][:5])
    v, _, q = g.query_config(n, k, dtype)
    extra = mbd.gemv_variant_info(v)[1].splits + (q if q > 1 else 0)
    if alpha is None and bias is None:
        ref, _, ab = oracle.gemv(dtype, B, a)
        ok_g, ok_s, _, rs, first = compare(dtype, got, ref, ab, k, extra)
        assert ok_g and ok_s, (n, k, rs, first)
    else:
        ref, y, ab = oracle.gemv_epilogue(dtype, B, a, 1.0 if alpha is None else alpha, bias_bits)
        gv, rv = oracle.decode(dtype, got), oracle.decode(dtype, ref)
        # the grading tolerance with alpha applied to the sum's term
        bound = 4e-3 * abs(1.0 if alpha is None else alpha) * ab + ulp(dtype, rv)
        assert np.all(np.abs(gv - rv) <= bound), (n, k, float((np.abs(gv - rv) / bound).max()))
    return q


@pytest.mark.parametrize("first,second", [
    ((64, 65536, BF16), (8, 65536, BF16)),       # k split across 4 workgroups, then 4 again
    ((32, 131072, F16), (1, 65536, BF16)),       # 8 k-groups, then 8 (one row: doubled)
    ((64, 65536, BF16), (600, 5000, BF16)),      # a split, then a plan with no scratch
    ((18432, 7168, F16), (7, 65536, F16)),       # no scratch, then a split of one row range
])
def test_noalloc_matches_workspace_entry(g, first, second):
    """Two calls in a row on the static scratch, the second smaller."""
    q1 = _check(g, *first, seed=1)
    q2 = _check(g, *second, seed=2)
    assert first[0] * first[1] > second[0] * second[1]
    assert max(q1, q2) > 1          # at least one call used the scratch's split


def test_noalloc_epilogue_and_repeats(g):
    """The fused epilogue on the split plan, and the same call repeated: the
    counters must be back at zero after each call."""
    for _ in range(3):
        assert _check(g, 64, 65536, BF16, seed=5, alpha=0.5, with_bias=True) > 1
        assert _check(g, 16, 65536, F16, seed=6) > 1


def test_noalloc_forced_splits_and_limit(g):
    """Forced k-group counts (each its own counter bank), then one whose
    partials exceed the scratch: GEMV_ERR_TOO_LARGE, c untouched."""
    xwg = [v for v in range(mbd.gemv_num_variants()) if mbd.gemv_variant_info(v)[1].cross_wg]
    n, k, dtype = 33, 20000, BF16
    B, a = random_inputs(n, k, dtype, seed=9)
    Bd, ad = to_device(B, dtype), to_device(a, dtype)
    ref, _, ab = oracle.gemv(dtype, B, a)
    try:
        for q in (2, 3, 16, 64):
            g.force_config(xwg[0], 0, q)
            got, ref_ws = _pair(g, Bd, ad)
            assert np.array_equal(got, ref_ws), q
            ok_g, ok_s, _, rs, first = compare(dtype, got, ref, ab, k, 8 + q)
            assert ok_g and ok_s, (q, rs, first)
        # 64 k-groups x 8192 rows = 2^19 partials > 2^18
        n2, k2 = 8192, 1024
        B2 = torch.zeros((n2, k2), dtype=torch.float16, device="cuda")
        a2 = torch.zeros(k2, dtype=torch.float16, device="cuda")
        c2 = torch.full((n2,), 5.0, dtype=torch.float16, device="cuda")
        g.force_config(xwg[0], 0, 64)
        s = mbd.gemv_run_noalloc(g.h, B2.data_ptr(), a2.data_ptr(), c2.data_ptr(), n2, k2,
                                 mbd.GEMV_F16, stream=torch.cuda.current_stream().cuda_stream)
        assert s == mbd._lib.GEMV_ERR_TOO_LARGE
    finally:
        g.force_config(-1)
    torch.cuda.synchronize()
    assert torch.all(c2 == 5.0)
