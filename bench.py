#!/usr/bin/env python3
"""Benchmark of the dense GEMV c = B @ a on one MI355X.

One step = one gemv_run_ws over one (B, a) pair (gemv_run with caller scratch,
so that every shape gets its fastest plan; for all but a few long rows it is
the same launch gemv_run makes).  The default workload is
n=18432, k=7168, fp16 with B ~ N(0,1)/sqrt(k), a ~ N(0,1), seed 0.  Inputs are
resident in HBM before timing starts; successive steps rotate over copies of
(B, a, c) that together exceed 1 GiB, so neither the L2 nor the 256 MiB
Infinity Cache can serve B from one step to the next.

Timing (TileLang Case Studies, Case C: a fixed configuration, no tuning
inside the measured region):
  * the timed region: W warmup steps, then a synchronise, K steps, a
    synchronise, all on one stream; ms_per_step = wall time / K and
    value = algorithmic bytes per step / ms_per_step;
  * a HIP event pair on the launch stream brackets the same K launches; the
    launches run back to back with no idle gap between kernels (a graph
    replay, or host launches that enqueue far faster than a kernel runs),
    so the event time / K is the kernel's average duration:
    roofline.achieved = algorithmic bytes per launch / that average.  (An
    event pair around every single launch would add the event packets' own
    cost to each duration.)
Algorithmic bytes per step = 2 * (n*k + k + n): B, a and c once each.

On MI355X the first ~20 ms of sustained load after the GPU has been idle
run 1-5% slower while the memory clocks come up (a kernel trace of the
headline shows 38.5-39.6 us per launch there, then 37.5-37.6 us), so the
timed region is preceded by at least 50 ms of the same launches, untimed
(graph replays, or host launches with --stream), whatever K is.  K defaults
to 2000 (75 ms of timed work for the headline).

The K timed steps are replayed from one HIP graph, captured once before the
timed region (as a decode loop replays its graph); --stream launches each
step from the host instead.  Either way every step is one full launch on the
stream, in order.  --epilogue runs gemv_run_ex with c = 0.5 * (B @ a) + bias
(bias counts 2n more bytes).

Prints ONE JSON line on stdout; human-readable detail goes to stderr.
"""
import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "achieved HBM GB/s (% of MI355X peak) and µs/call, n=18432 k=7168 fp16"


def metric_of(n, k, dtype_name):
    """The metric line of a GEMV workload (the default workload's is METRIC)."""
    return "achieved HBM GB/s (%% of MI355X peak) and µs/call, n=%d k=%d %s" % (
        n, k, {"f16": "fp16", "bf16": "bf16"}.get(dtype_name, dtype_name))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(sources=None):
    from memory_bound_dense_amd.profile_counters import kernel_source_hash as ksh
    return ksh(sources)


def read_traffic(workload, n_launch_bytes, plan, sources=None):
    """HBM traffic per launch from the committed counter summary, if it was
    taken on the current kernel source (`sources`: the GEMV's by default)
    and the same plan; else None."""
    path = os.path.join(ROOT, "profiles", "%s.counters.txt" % workload)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            kv[key.strip()] = val.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash(sources) or kv.get("plan") != plan:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or the platform's."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(B_bits, a_bits, dtype, n, k, target_s=10.0):
    """The oracle, as it is, timed on the host: whole calls on the same
    inputs, repeated until about `target_s` seconds have passed (or, if one
    call would take longer than that, one call on the first rows)."""
    import numpy as np
    import oracle
    probe = min(n, 64)
    t0 = time.perf_counter()
    oracle.gemv(dtype, B_bits[:probe], a_bits)
    est_call = (time.perf_counter() - t0) / probe * n
    if est_call > target_s:
        rows = int(max(1, n * target_s / est_call))
        Bs = np.ascontiguousarray(B_bits[:rows])
        t0 = time.perf_counter()
        oracle.gemv(dtype, Bs, a_bits)
        dt = time.perf_counter() - t0
        calls, what = 1, "one call on the first %d of %d rows" % (rows, n)
    else:
        rows, calls, dt = n, 0, 0.0
        t0 = time.perf_counter()
        while dt < target_s:
            oracle.gemv(dtype, B_bits, a_bits)
            calls += 1
            dt = time.perf_counter() - t0
        what = "%d whole calls" % calls
    nbytes = 2 * (rows * k + k + rows) * calls
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "%s (n=%d, k=%d), %.1f s on 1 thread" % (what, n, k, dt),
            "host_cores": os.cpu_count(), "host_cpu": cpu_model(),
            "us_per_call": round(dt / calls * 1e6 * n / rows, 1)}


def time_launches(launch, steps, nbuf, stream, dev, graph):
    """Average device time (us) of `steps` calls of launch(i, stream_handle)
    over `nbuf` rotating input copies, back to back on `stream` after a
    sustained untimed run (graph replays, or host launches), bracketed by
    one event pair."""
    import torch
    lau = Launcher(launch, steps, nbuf, stream, dev, graph)
    sustain(lau.run)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    lau.run()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / steps


def stream_probe(nbytes, steps, dev, graph=True):
    """A plain streaming read of the same number of bytes (rounded down to
    whole KiB), timed like the GEMV (the same launch mode), best of a few
    launch shapes: the practical read ceiling."""
    import torch
    from memory_bound_dense_amd import probe
    nbytes = nbytes // probe.READ_BLOCK * probe.READ_BLOCK
    nbuf = rotation(nbytes)
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(nbuf)]
    out = torch.empty(1 << 24, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    best = None
    for unroll in (4, 8, 16):
        for grid in (0, 1024, 2048, 4096):
            def launch(i, sp, grid=grid, unroll=unroll):
                probe.stream_read(bufs[i % nbuf].data_ptr(), nbytes, out.data_ptr(), out.numel(),
                                  grid, unroll, True, sp)
            for i in range(10):
                launch(i, stream.cuda_stream)
            us = time_launches(launch, steps, nbuf, stream, dev, graph)
            if best is None or us < best[0]:
                best = (us, grid, unroll)
    del bufs
    return {"bytes": nbytes, "us": round(best[0], 3), "gbs": round(nbytes / best[0] / 1e3, 1),
            "grid": best[1], "unroll": best[2]}


def access_probe(vinfo, Bs, n, k, grid, kgroups, ws_ptr, steps, dev, graph=True):
    """The GEMV launch itself with its arithmetic taken out (the same B
    loads, grid, k-slices and reductions; a never read), on the same rotated
    copies of B: what the plan's access pattern costs alone.  None when the
    probe library has no build of this plan shape."""
    import torch
    from memory_bound_dense_amd import probe
    if not probe.gemv_probe_has(vinfo) or k % 8 != 0:
        return None
    nbuf = len(Bs)
    outs = [torch.empty(n, dtype=torch.float16, device=dev) for _ in range(nbuf)]
    stream = torch.cuda.current_stream(dev)

    def launch(i, sp):
        probe.gemv_probe(vinfo, Bs[i % nbuf].data_ptr(), n, k, outs[i % nbuf].data_ptr(),
                         ws_ptr if vinfo.cross_wg else None, grid, kgroups, sp)
    for i in range(10):
        launch(i, stream.cuda_stream)
    us = time_launches(launch, steps, nbuf, stream, dev, graph)
    return {"bytes_of_B": 2 * n * k, "us": round(us, 3), "gbs": round(2 * n * k / us / 1e3, 1)}


# Untimed sustained load before a timed region: on MI355X the memory clocks
# need ~20 ms of sustained traffic to come up after the GPU has been idle.
SUSTAIN_S = 0.05


def sustain(run_once, min_s=SUSTAIN_S, max_runs=10000):
    """Run `run_once` (enqueue work on the GPU) back to back, untimed, until
    the GPU has been busy for at least min_s seconds (and at least once)."""
    import torch
    t0 = time.perf_counter()
    for _ in range(max_runs):
        run_once()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= min_s:
            break


# Copies of an input kept in rotation: together > 1 GiB, so neither the L2
# nor the 256 MiB Infinity Cache holds a copy from one use to the next.
MAX_COPIES = 4096


def rotation(nbytes):
    return int(min(MAX_COPIES, max(2, math.ceil((1 << 30) / max(nbytes, 1)))))


class Launcher:
    """K launches of step(i, stream_handle) per run(); launch i uses input
    copy i % nbuf and the index keeps counting across runs, so consecutive
    launches never reuse a copy before nbuf others.  Graph mode: the launches
    are captured once (every path of gemv_run and gla_decode_step is
    capture-safe: no allocation, no memset, no synchronisation) as windows of
    K that together cover every copy, replayed round robin; host_us is the
    host cost of one replay per launch.  Stream mode: host launches."""

    def __init__(self, step, steps, nbuf, stream, dev, graph):
        import torch
        self.step, self.steps, self.stream, self.graph = step, steps, stream, graph
        self.next = 0
        self.graphs = []
        self.host_us = None
        if graph:
            # (at most 256 windows: a very short K covers fewer copies)
            windows = 1 if steps >= nbuf else min(256, -(-nbuf // steps))
            side = torch.cuda.Stream(dev)
            try:
                for w in range(windows):
                    gph = torch.cuda.CUDAGraph()
                    side.wait_stream(stream)
                    with torch.cuda.stream(side):
                        with torch.cuda.graph(gph, stream=side):
                            for j in range(steps):
                                step(w * steps + j, side.cuda_stream)
                    stream.wait_stream(side)
                    self.graphs.append(gph)
            except RuntimeError as e:
                # a capture the runtime refuses: time host launches instead
                # (the JSON line then says "launch": "stream")
                log("[bench] HIP graph capture failed (%s); using host launches" % e)
                torch.cuda.synchronize()
                self.graphs, self.graph = [], False
                return
            torch.cuda.synchronize()
            t = time.perf_counter()
            self.run()
            self.host_us = (time.perf_counter() - t) / steps * 1e6
            torch.cuda.synchronize()

    def run(self):
        """Enqueue the next K launches on the stream."""
        if self.graph:
            self.graphs[self.next % len(self.graphs)].replay()
            self.next += 1
        else:
            for _ in range(self.steps):
                self.step(self.next, self.stream.cuda_stream)
                self.next += 1


def gla_bench(args):
    """One GLA decode step per step (include/gla_decode.h), the state updated
    in place as a decode loop does; copies of the state rotate over > 1 GiB."""
    import numpy as np
    import torch
    import memory_bound_dense_amd as mbd
    from gemv_inputs import (DTYPE_NAMES, GLA_BATCHED, GLA_DECODE, gla_inputs, gla_step_bytes,
                             torch_dtype)
    from memory_bound_dense_amd.profile_counters import GLA_PLAN, GLA_SOURCES
    wl = {w[0]: w for w in (GLA_DECODE, GLA_BATCHED)}.get(args.workload, GLA_DECODE)
    name, bh, dk, dv, dtype = wl
    dev = torch.device("cuda", 0)
    td = torch_dtype(dtype)
    q, k, v, gk, S = gla_inputs(bh, dk, dv, dtype, seed=0)
    t = lambda x: torch.from_numpy(x.view(np.int16)).to(dev).view(td)
    qd, kd, vd, gd = t(q), t(k), t(v), t(gk)
    S0 = torch.from_numpy(S).to(dev)
    state_bytes = 4 * bh * dk * dv
    nbuf = rotation(state_bytes)
    Ss = [S0] + [S0.clone() for _ in range(nbuf - 1)]
    os_ = [torch.empty((bh, dv), dtype=td, device=dev) for _ in range(nbuf)]
    step_bytes = gla_step_bytes(bh, dk, dv)
    g = mbd.Gemv()
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    scale = 1.0 / math.sqrt(dk)
    P = [(Ss[i].data_ptr(), os_[i].data_ptr()) for i in range(nbuf)]

    def step(i, sp=sp):
        s_, o_ = P[i % nbuf]
        rc = mbd.gla_decode_step(g.h, qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), gd.data_ptr(),
                                 s_, s_, o_, bh, dk, dv, scale, dtype, sp)
        if rc != 0:
            raise mbd.GemvError(rc, "gla_decode_step")

    for i in range(args.warmup):
        step(i)
    lau = Launcher(step, args.steps, nbuf, stream, dev, not args.stream)
    sustain(lau.run)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    lau.run()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_us = ev0.elapsed_time(ev1) * 1e3 / args.steps
    value = step_bytes / (wall / args.steps) / 1e9
    log("[bench] %s: wall %.2f us/step, kernel avg %.2f us -> %.1f GB/s" % (
        name, wall / args.steps * 1e6, avg_us, step_bytes / avg_us / 1e3))
    # the practical ceiling for this traffic mix: a plain copy of the state
    ceiling = None
    if not args.no_probe:
        from memory_bound_dense_amd import probe
        nbytes = state_bytes // probe.CHUNK * probe.CHUNK
        if nbytes:
            dst = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(nbuf)]
            best = None
            for grid in (0, 512, 2048):
                def launch(i, sp, grid=grid):
                    probe.stream_copy(Ss[i % nbuf].data_ptr(), dst[i % nbuf].data_ptr(), nbytes, grid,
                                      True, sp)
                for i in range(5):
                    launch(i, sp)
                us = time_launches(launch, args.steps, nbuf, stream, dev, not args.stream)
                best = us if best is None else min(best, us)
            ceiling = {"bytes_moved": 2 * nbytes, "us": round(best, 3),
                       "gbs": round(2 * nbytes / best / 1e3, 1)}
            log("[bench] streaming copy of the state: %.2f us -> %.1f GB/s" % (best, ceiling["gbs"]))
            del dst
    out = {"metric": "GLA decode step: achieved HBM GB/s and us/call", "value": round(value, 2),
           "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(wall / args.steps * 1e3, 5), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": DTYPE_NAMES[dtype],
           "data": "synthetic",
           "config": {"workload": name, "bh": bh, "dk": dk, "dv": dv, "in_place": True,
                      "rotating_buffers": nbuf, "launch": "graph" if lau.graph else "stream"},
           "us_per_call": round(wall / args.steps * 1e6, 3), "kernel_us_avg": round(avg_us, 3),
           "roofline": {"bound": "hbm", "achieved": round(step_bytes / avg_us / 1e3, 2),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(step_bytes / avg_us / 1e3 / HBM_PEAK_GBS, 4),
                        "traffic": read_traffic(name, step_bytes, GLA_PLAN, GLA_SOURCES)}}
    if ceiling:
        out["stream_copy_probe"] = ceiling
    g.close()
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=25)
    ap.add_argument("--workload", default="gemv_18432x7168_f16",
                    help="workload name (gemv_inputs.ALL_WORKLOADS / EXTRA_WORKLOADS)")
    ap.add_argument("--shape", default="", help="ad-hoc shape 'n,k,f16|bf16' instead of --workload")
    ap.add_argument("--variant", type=int, default=-1, help="force a kernel variant (-1 = auto)")
    ap.add_argument("--grid", type=int, default=0, help="force the workgroup count (0 = auto)")
    ap.add_argument("--kgroups", type=int, default=0,
                    help="force the k-groups of a cross-workgroup variant (0 = auto)")
    ap.add_argument("--rotate-bytes", type=float, default=float(1 << 30))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--op", choices=("gemv", "gla"), default="gemv",
                    help="gemv (default, the headline) or gla: one GLA decode step")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the streaming-read probe (the practical read ceiling)")
    ap.add_argument("--stream", action="store_true",
                    help="launch each step from the host onto the stream instead of replaying "
                         "one HIP graph that holds the K launches (the default)")
    ap.add_argument("--epilogue", action="store_true",
                    help="run gemv_run_ex with c = 0.5 * (B @ a) + bias (bias: one more n-vector)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py: measures one GPU (the kernel on one GPU's share of the rows); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: one process, one GPU; WORLD_SIZE > 1 is not supported", file=sys.stderr)
        sys.exit(2)

    if args.op == "gla":
        if args.workload == "gemv_18432x7168_f16":
            args.workload = "gla_decode_b1h32_128x128_bf16"
        return gla_bench(args)

    import numpy as np
    import torch
    import memory_bound_dense_amd as mbd
    from gemv_inputs import (ALL_WORKLOADS, DTYPE_NAMES, EXTRA_WORKLOADS, algorithmic_bytes,
                             find_workload, random_inputs, shape_workload, torch_dtype)

    wl = shape_workload(args.shape) if args.shape else find_workload(args.workload)
    if wl is None:
        print("unknown workload %r; known: %s" % (
            args.workload, [w[0] for w in ALL_WORKLOADS + EXTRA_WORKLOADS]), file=sys.stderr)
        sys.exit(2)
    name, n, k, dtype, dist = wl
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    td = torch_dtype(dtype)

    log("[bench] workload %s n=%d k=%d %s %s; generating inputs" % (name, n, k,
                                                                    DTYPE_NAMES[dtype], dist))
    B_bits, a_bits = random_inputs(n, k, dtype, dist, seed=0)
    B0 = torch.from_numpy(B_bits.view(np.int16)).to(dev).view(td)
    a0 = torch.from_numpy(a_bits.view(np.int16)).to(dev).view(td)
    step_bytes = algorithmic_bytes(n, k)
    nbuf = int(min(MAX_COPIES, max(2, math.ceil(args.rotate_bytes / (2.0 * n * k)))))
    Bs = [B0] + [B0.clone() for _ in range(nbuf - 1)]
    As = [a0] + [a0.clone() for _ in range(nbuf - 1)]
    Cs = [torch.empty(n, dtype=td, device=dev) for _ in range(nbuf)]
    torch.cuda.synchronize()

    g = mbd.Gemv(workspace=True)
    if args.variant >= 0:
        g.force_config(args.variant, args.grid, args.kgroups)
    variant, grid, kgroups = g.query_config(n, k, dtype)
    _, vinfo = mbd.gemv_variant_info(variant)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    h, ws, wsb = g.h, g.ws.data_ptr(), g.ws.numel()
    ptrs = [(Bs[i].data_ptr(), As[i].data_ptr(), Cs[i].data_ptr()) for i in range(nbuf)]
    log("[bench] variant %d (rows %d unroll %d waves %d splits %d a_mode %d b_policy %d "
        "cross_wg %d), grid %d x %d, %d rotating buffers of %.1f MB" % (
            variant, vinfo.rows, vinfo.unroll, vinfo.waves, vinfo.splits, vinfo.a_mode,
            vinfo.b_policy, vinfo.cross_wg, grid, kgroups, nbuf, 2.0 * n * k / 1e6))

    if args.epilogue:
        # c = 0.5 * (B @ a) + bias, bias one more n-vector per rotation slot
        biases = [torch.randn(n, device=dev).to(td) for _ in range(nbuf)]
        bptr = [x.data_ptr() for x in biases]
        step_bytes += 2 * n

    def step(i, sp=sp):
        b, a, c = ptrs[i % nbuf]
        if args.epilogue:
            s = mbd.gemv_run_ws(h, b, a, c, n, k, dtype, ws, wsb, 0.5, bptr[i % nbuf], sp)
        else:
            s = mbd.gemv_run_ws(h, b, a, c, n, k, dtype, ws, wsb, stream=sp)
        if s != 0:
            raise mbd.GemvError(s, "gemv_run_ws")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log("[bench] warmup done (%d steps); timing %d steps" % (args.warmup, args.steps))

    # host cost of one gemv_run_ws (validation, plan lookup, launch; ctypes
    # included), measured on launches that queue behind a busy GPU
    torch.cuda.synchronize()
    host = 0.0
    for i in range(args.steps):
        t = time.perf_counter()
        step(i)
        host += time.perf_counter() - t
    torch.cuda.synchronize()
    host_us = host / args.steps * 1e6

    lau = Launcher(step, args.steps, nbuf, stream, dev, not args.stream)
    replay_host_us = lau.host_us
    if lau.graphs:
        log("[bench] captured %d launches into %d HIP graph(s)" % (args.steps, len(lau.graphs)))
    sustain(lau.run)

    # timed region: whole-job throughput, with one event pair on the stream
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    lau.run()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3
    value = step_bytes / (wall / args.steps) / 1e9
    avg_us = ev0.elapsed_time(ev1) * 1e3 / args.steps
    achieved = step_bytes / (avg_us * 1e-6) / 1e9
    log("[bench] wall %.2f us/step -> %.1f GB/s; kernel avg %.2f us (HIP events over the timed "
        "region) -> %.1f GB/s = %.1f%% of %.0f GB/s" % (
            ms_per_step * 1e3, value, avg_us, achieved, 100 * achieved / HBM_PEAK_GBS,
            HBM_PEAK_GBS))

    ceiling = access = None
    if not args.no_probe:
        ceiling = stream_probe(2 * n * k, args.steps, dev, not args.stream)
        log("[bench] streaming-read probe over the same bytes: %.2f us -> %.1f GB/s (grid %d, "
            "unroll %d)" % (ceiling["us"], ceiling["gbs"], ceiling["grid"], ceiling["unroll"]))
        access = access_probe(vinfo, Bs, n, k, grid, kgroups, ws, args.steps, dev, not args.stream)
        if access:
            log("[bench] the same launch without its arithmetic: %.2f us -> %.1f GB/s of B" % (
                access["us"], access["gbs"]))
    from memory_bound_dense_amd.profile_counters import plan_signature
    # the counter summaries are taken on plain launches (no epilogue)
    traffic = None if args.epilogue else read_traffic(name, step_bytes,
                                                      plan_signature(variant, grid, kgroups))
    out = {
        "metric": metric_of(n, k, DTYPE_NAMES[dtype]),
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAMES[dtype],
        "data": "synthetic",
        "config": {"workload": name, "n": n, "k": k, "distribution": dist, "seed": 0,
                   "variant": variant, "grid": grid, "kgroups": kgroups,
                   "rows_per_wave": vinfo.rows,
                   "unroll": vinfo.unroll, "waves_per_wg": vinfo.waves, "splits": vinfo.splits,
                   "a_mode": {0: "lds", 1: "cached", 2: "lds_shifted", 3: "shifted_window"}[vinfo.a_mode],
                   "layout": ["lanes_along_k", "row_per_lane"][vinfo.layout],
                   "rotating_buffers": nbuf, "launch": "graph" if lau.graph else "stream",
                   "entry": "gemv_run_ws",
                   "epilogue": "alpha_bias" if args.epilogue else "none"},
        "us_per_call": round(ms_per_step * 1e3, 3),
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "kernel_us_avg": round(avg_us, 3),
        "host_us_per_call": round(host_us, 3),
        "graph_replay_host_us_per_step": None if replay_host_us is None else round(replay_host_us, 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
    }
    # bytes moved per output row: the algorithmic 2k + 2 (+ a's share, 2k / n)
    # against the counted HBM bytes, when a counter summary applies
    out["bytes_per_output"] = {"algorithmic": round(step_bytes / n, 2),
                               "counted": None if traffic is None else round(traffic / n, 2)}
    if ceiling:
        out["stream_read_probe"] = ceiling
    if access:
        out["access_pattern_probe"] = access
    # the pages' figure for the uncoalesced kernel before their fix (TileLang
    # Case Studies, Case B, on H200): context for the coalescing, not a target
    out["context"] = {"pages_uncoalesced_gbs_h200": 110, "pages_coalesced_tbs_h200": [3.65, 3.85]}
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        out["cpu_baseline"] = cpu_baseline(B_bits, a_bits, dtype, n, k)
    g.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
