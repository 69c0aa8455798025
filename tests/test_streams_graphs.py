"""GPU: gemv_run under HIP graph capture and from several streams.

* capture: calls enqueued while torch captures a HIP graph (one shape on
  each path: rows, in-workgroup split, cross-workgroup split, realigned
  rows) replay correctly, every replay checked against the eager result,
  with eager work and synchronisations between replays;
* streams: ONE handle driving two streams (default priority) at once, with
  host delays in between -- gemv_run with no scratch, and gemv_run_ws with
  one workspace per stream -- gives bitwise the same c as a quiet run.
"""
import random
import time

import numpy as np
import pytest
import torch

import memory_bound_dense_amd as mbd
from gemv_inputs import BF16, F16, random_inputs
from parity import to_bits, to_device

pytestmark = pytest.mark.gpu

SHAPES = [(18432, 7168, F16), (7168, 16384, BF16), (64, 65536, BF16), (1000, 7001, BF16),
          (256, 512, F16)]


def _inputs():
    out = []
    for i, (n, k, dtype) in enumerate(SHAPES):
        B, a = random_inputs(n, k, dtype, seed=100 + i)
        out.append((to_device(B, dtype), to_device(a, dtype)))
    return out


def test_graph_capture_replays():
    g = mbd.Gemv(workspace=True)
    ins = _inputs()
    eager = []
    for Bd, ad in ins:
        c = torch.empty(Bd.shape[0], dtype=Bd.dtype, device="cuda")
        g(Bd, ad, c)
        eager.append(c)
    torch.cuda.synchronize()
    ref = [to_bits(c) for c in eager]
    outs = [torch.zeros(Bd.shape[0], dtype=Bd.dtype, device="cuda") for Bd, _ in ins]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for (Bd, ad), c in zip(ins, outs):
                g(Bd, ad, c)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(5):
        for c in outs:
            c.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()     # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, c in enumerate(outs):
            assert np.array_equal(to_bits(c), ref[i]), (rep, SHAPES[i])
        # an eager call between replays must not disturb the next replay
        Bd, ad = ins[2]
        g(Bd, ad, eager[2])
        torch.cuda.synchronize()
        del junk
    g.close()


def test_two_streams_one_handle_repeatable():
    """The handle is read-only after gemv_create, so one handle may serve two
    streams at once.  Every shape (the 64 x 65536 one included, whose
    scratch-free plan splits k inside a workgroup) runs on both streams,
    interleaved in random order with random host delays: through gemv_run,
    and through gemv_run_ws with a workspace per stream (the 64 x 65536 plan
    then splits k across workgroups on both streams at once).  Every result
    must have the bits of a quiet run of the same entry point."""
    ins = _inputs()
    g = mbd.Gemv()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    ws = [torch.zeros(mbd._lib.GEMV_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
          for _ in range(2)]
    sp = (s1.cuda_stream, s2.cuda_stream)
    torch.cuda.synchronize()          # inputs and zeroed workspaces ready for both streams
    dt = lambda Bd: mbd.GEMV_F16 if Bd.dtype == torch.float16 else mbd.GEMV_BF16

    def call(Bd, ad, c, which, use_ws):
        n, k = Bd.shape
        if use_ws:
            st = mbd.gemv_run_ws(g.h, Bd.data_ptr(), ad.data_ptr(), c.data_ptr(), n, k, dt(Bd),
                                 ws[which].data_ptr(), ws[which].numel(), stream=sp[which])
        else:
            st = mbd.gemv_run(g.h, Bd.data_ptr(), ad.data_ptr(), c.data_ptr(), n, k, dt(Bd),
                              sp[which])
        assert st == mbd.GEMV_OK

    assert g.query_config(64, 65536, mbd.GEMV_BF16, with_workspace=1)[2] > 1
    assert g.query_config(64, 65536, mbd.GEMV_BF16, with_workspace=0)[2] == 1
    rng = random.Random(0)
    for use_ws in (False, True):
        ref = []
        for Bd, ad in ins:
            c = torch.empty(Bd.shape[0], dtype=Bd.dtype, device="cuda")
            call(Bd, ad, c, 0, use_ws)
            torch.cuda.synchronize()
            ref.append(to_bits(c))
        outs = [[torch.empty(Bd.shape[0], dtype=Bd.dtype, device="cuda") for Bd, _ in ins]
                for _ in range(2)]
        for it in range(40):
            order = list(range(len(ins)))
            rng.shuffle(order)
            for i in order:
                Bd, ad = ins[i]
                call(Bd, ad, outs[0][i], 0, use_ws)
                if rng.random() < 0.3:
                    time.sleep(rng.random() * 1e-4)
                call(Bd, ad, outs[1][i], 1, use_ws)
            torch.cuda.synchronize()
            for i in range(len(ins)):
                for w in range(2):
                    assert np.array_equal(to_bits(outs[w][i]), ref[i]), (use_ws, it, w, SHAPES[i])
    g.close()


def test_stress_split_and_lds_variants_repeatable():
    """Variants with synchronisation inside (LDS staging, in-workgroup splits,
    cross-workgroup splits, realigned rows, B pipelined through LDS with
    explicit waits): 150 back-to-back runs each with
    random host delays and eager work between them must all give the bits
    of the first run."""
    g = mbd.Gemv(workspace=True)
    rng = random.Random(7)
    picks = []
    for v in range(mbd.gemv_num_variants()):
        info = mbd.gemv_variant_info(v)[1]
        if info.layout == 0 and (info.a_mode != 1 or info.splits > 1 or info.cross_wg or info.b_lds):
            picks.append(v)
    shapes = [(64, 65536, BF16), (1000, 7001, F16), (300, 4096, BF16)]
    for i, (n, k, dtype) in enumerate(shapes):
        B, a = random_inputs(n, k, dtype, seed=200 + i)
        Bd, ad = to_device(B, dtype), to_device(a, dtype)
        for v in rng.sample(picks, 6):
            g.force_config(v)
            try:
                g.query_config(n, k, dtype)
            except mbd.GemvError:
                g.force_config(-1)
                continue
            c = torch.empty(n, dtype=Bd.dtype, device="cuda")
            g(Bd, ad, c)
            torch.cuda.synchronize()
            first = to_bits(c)
            for it in range(150):
                if rng.random() < 0.2:
                    time.sleep(rng.random() * 2e-4)
                if rng.random() < 0.2:
                    torch.randn(1 << 16, device="cuda").sum()
                c.fill_(float("nan"))
                g(Bd, ad, c)
                if rng.random() < 0.5:
                    torch.cuda.synchronize()
                    assert np.array_equal(to_bits(c), first), (n, k, v, it)
            torch.cuda.synchronize()
            assert np.array_equal(to_bits(c), first), (n, k, v)
            g.force_config(-1)
    g.close()


@pytest.mark.parametrize("grid", [0, 3], ids=["ticketed", "counted"])
def test_racing_calls_leave_the_workspace_usable(grid):
    """Calls that overlap on one workspace race: their c is undefined (and
    may be NaN where a ticketed combiner found a partial missing and gave up
    after its bounded polls).  Once they have completed, the workspace must
    serve the next call exactly: 64 x 65536 bf16 split across 8 workgroups
    per row, the ticketed combine (one row per workgroup, the automatic
    plan's grid) and the counted one (a grid of 3 row ranges), raced from
    two streams on one workspace with different inputs, then run quietly
    and compared bit for bit with the same call on a fresh workspace."""
    n, k, dtype = 64, 65536, BF16
    g = mbd.Gemv(workspace=True)
    v, _, q = g.query_config(n, k, dtype)
    assert mbd.gemv_variant_info(v)[1].cross_wg and q > 1
    (B1, a1), (B2, a2) = [random_inputs(n, k, dtype, seed=300 + i) for i in range(2)]
    B1d, a1d, B2d, a2d = (to_device(x, dtype) for x in (B1, a1, B2, a2))
    fresh = torch.zeros(mbd._lib.GEMV_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    c1 = torch.empty(n, dtype=B1d.dtype, device="cuda")
    c2 = torch.empty(n, dtype=B1d.dtype, device="cuda")
    ref = torch.empty(n, dtype=B1d.dtype, device="cuda")

    def call(Bd, ad, c, ws, stream):
        st = mbd.gemv_run_ws(g.h, Bd.data_ptr(), ad.data_ptr(), c.data_ptr(), n, k, mbd.GEMV_BF16,
                             ws.data_ptr(), ws.numel(), stream=stream)
        assert st == mbd.GEMV_OK

    g.force_config(v, grid, q)
    try:
        torch.cuda.synchronize()
        call(B1d, a1d, ref, fresh, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        want = to_bits(ref)
        for _ in range(4):
            call(B1d, a1d, c1, g.ws, s1.cuda_stream)
            call(B2d, a2d, c2, g.ws, s2.cuda_stream)
        torch.cuda.synchronize()
        for _ in range(2):
            c1.fill_(float("nan"))
            call(B1d, a1d, c1, g.ws, torch.cuda.current_stream().cuda_stream)
            torch.cuda.synchronize()
            assert np.array_equal(to_bits(c1), want)
    finally:
        g.force_config(-1)
    g.close()
