"""GPU: the largest sizes the boundary accepts, through the C ABI.

* k = GEMV_MAX_K (2^27, 16-byte aligned rows) and k = GEMV_MAX_K - 1 (every
  row misaligned) on a few rows, against the oracle: the longest buffer
  descriptors and step offsets any kernel builds, on the cross-workgroup
  split the plan takes for so few rows;
* n = GEMV_MAX_N (2^30) rows of k = 8 with a one-hot a: c must equal the
  picked column of B exactly (a closed form that holds at any size), on the
  largest grid the host launches (work-items along x capped at 2^31) with
  each wave walking many rows;
* one GLA step whose grid would exceed that cap is refused with
  GEMV_ERR_TOO_LARGE before any launch.
"""

import pytest
import torch

import memory_bound_dense_amd as mbd
from memory_bound_dense_amd import _lib
import oracle
from gemv_inputs import BF16, F16, random_inputs, torch_dtype
from parity import compare, to_bits, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    h = mbd.Gemv()
    yield h
    h.close()


def _extra_adds(g, n, k, dtype):
    v, _, q = g.query_config(n, k, dtype)
    return mbd.gemv_variant_info(v)[1].splits + (q if q > 1 else 0)


@pytest.mark.parametrize("n,k,dtype", [(2, _lib.GEMV_MAX_K, BF16), (3, _lib.GEMV_MAX_K - 1, F16)],
                         ids=["2xMAXK_bf16", "3x(MAXK-1)_f16"])
def test_longest_rows(g, n, k, dtype):
    print("max-k case n=%d k=%d dtype=%d plan %s" % (n, k, dtype, g.query_config(n, k, dtype)),
          flush=True)
    B, a = random_inputs(n, k, dtype, seed=5)
    ref, _, ab = oracle.gemv(dtype, B, a)
    Bd, ad = to_device(B, dtype), to_device(a, dtype)
    del B
    c = torch.full((n,), float("nan"), dtype=torch_dtype(dtype), device="cuda")
    g(Bd, ad, c)
    torch.cuda.synchronize()
    ok_g, ok_s, rg, rs, first = compare(dtype, to_bits(c), ref, ab, k, _extra_adds(g, n, k, dtype))
    assert ok_g, ("grading tolerance", rg, first)
    assert ok_s, ("strict fp32 bound", rs, first)


def test_most_rows_column_extraction(g):
    n, k, dtype, col = _lib.GEMV_MAX_N, 8, F16, 3
    print("max-n case n=%d k=%d plan %s" % (n, k, g.query_config(n, k, dtype)), flush=True)
    td = torch_dtype(dtype)
    B = torch.zeros((n, k), dtype=td, device="cuda")
    # column `col` holds integers in [-1023, 1023] (exact in fp16), varying
    # along the rows; filled in slices to bound the temporary
    step = 1 << 26
    for r0 in range(0, n, step):
        idx = torch.arange(r0, min(n, r0 + step), device="cuda", dtype=torch.int64)
        B[r0:r0 + idx.numel(), col] = ((idx * 7919) % 2047 - 1023).to(td)
        del idx
    a = torch.zeros(k, dtype=td, device="cuda")
    a[col] = 1.0
    c = torch.full((n,), float("nan"), dtype=td, device="cuda")
    g(B, a, c)
    torch.cuda.synchronize()
    bad = int((c != B[:, col]).sum().item())
    assert bad == 0, "%d of %d rows differ from the picked column" % (bad, n)
    del B, c
    torch.cuda.empty_cache()


def test_gla_grid_beyond_the_dispatch_cap_is_refused(g):
    # 2^23 + 1 heads of (1 x 4): one column block each, one workgroup per
    # head, so the grid's work-items along x exceed 2^31; nothing launches
    bh, dk, dv = (1 << 23) + 1, 1, 4
    gla = mbd.GlaDecode(g)
    q = torch.zeros((bh, dk), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((bh, dv), dtype=torch.bfloat16, device="cuda")
    S = torch.zeros((bh, dk, dv), dtype=torch.float32, device="cuda")
    o = torch.full((bh, dv), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mbd.GemvError) as e:
        gla(q, q, v, q, S, S, o, 1.0)
    assert e.value.status == _lib.GEMV_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert bool(torch.all(o == 7.0))
