"""Profiling helper: programs to run under rocprofv3, and summarisers that turn
rocprofv3's CSV output into the short text summaries kept under profiles/.

Programs (run as the profiled program, after ``rocprofv3 ... --``):

  python3 -m memory_bound_dense_amd.profile_counters gemv --workload NAME --launches N
      N launches of the GEMV in its automatic configuration (or the one given
      by --variant/--grid), rotating over copies of the inputs that exceed
      1 GiB (as bench.py does).
  python3 -m memory_bound_dense_amd.profile_counters gla --workload NAME --launches N
      N in-place GLA decode steps of a workload, rotating over > 1 GiB of
      state copies.
  python3 -m memory_bound_dense_amd.profile_counters copy --bytes X --launches N
      N device-to-device copies of X bytes (a plain copy kernel of known
      traffic: X bytes read and X bytes written), to calibrate the counters.

Summarisers (run anywhere, on the CSV files rocprofv3 wrote):

  ... summarize-trace --stats DIR/.._kernel_stats.csv --trace DIR/.._kernel_trace.csv
                      --command "..." [--kind gla] [--bench-json FILE] --out profiles/NAME.txt
  ... summarize-counters --workload NAME --fetch CSV --write CSV --copy-fetch CSV [CSV ...]
                      --copy-write CSV [CSV ...] --copy-bytes X [X ...] --commands "..."
                      --out profiles/...

FETCH_SIZE and WRITE_SIZE are in KiB per dispatch.  The copy kernel's reading
fixes a scale factor per counter (known bytes / counted bytes) that is applied
to the GEMV kernel's reading; copies of several sizes give one factor each,
and their mean is applied.
"""
import argparse
import csv
import hashlib
import math
import os
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
# the GEMV device code and the flags it is compiled with; which kernel a
# workload runs (the plan) is recorded and checked separately
KERNEL_SOURCES = [os.path.join(PKG, "csrc", f) for f in ("gemv_kernel.h", "gemv_shift.h",
                                                          "gemv_staged.h")] + \
    [os.path.join(PKG, "build.py")]
# the GLA step: its device code (which uses gemv_kernel.h's helpers), the host
# code that picks its launch, and the build flags
GLA_SOURCES = [os.path.join(PKG, "csrc", f) for f in ("gla_kernel.h", "gla.hip", "gemv_kernel.h")] + \
    [os.path.join(PKG, "build.py")]
GEMV_KERNEL = "gemv_"              # every GEMV kernel (row, realigning, row-per-lane)
GLA_KERNEL = "gla_decode_kernel"
# the GLA step's launch is picked on the host from the shape; the summary's
# hash covers that host code, so its plan line is this fixed text
GLA_PLAN = "the launch gla_decode_step picks (its host code is hashed above)"
COPY_KERNEL = "copyBuffer"


def _strip_comments(text):
    """C/C++ source without comments and with whitespace collapsed."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(sources=None):
    """Hash of the GEMV device code and its build flags (or of `sources`),
    blind to comments and whitespace: a summary taken on other code is not
    reused."""
    h = hashlib.sha256()
    for p in (KERNEL_SOURCES if sources is None else sources):
        with open(p) as f:
            h.update(_strip_comments(f.read()).encode())
    return h.hexdigest()[:16]


def plan_signature(variant, grid, kgroups):
    """The kernel a launch runs, by shape rather than by table index."""
    sys.path.insert(0, ROOT)
    import memory_bound_dense_amd as mbd
    i = mbd.gemv_variant_info(variant)[1]
    return "R%d U%d W%d S%d a%d p%d x%d l%d st%d lds%d grid %d kgroups %d" % (
        i.rows, i.unroll, i.waves, i.splits, i.a_mode, i.b_policy, i.cross_wg, i.layout, i.stages,
        i.b_lds, grid, kgroups)


def workload_plan_signature(n, k, dtype):
    """The automatic plan of a workload (host rule, 16-byte aligned B, with
    caller scratch: the plan gemv_run_ws launches and the benchmark times)."""
    sys.path.insert(0, ROOT)
    import memory_bound_dense_amd as mbd
    s, cfg = mbd.gemv_plan_config(n, k, dtype, 1, 160 * 1024, 1)
    if s != mbd.GEMV_OK:
        raise RuntimeError(mbd.gemv_status_string(s))
    return plan_signature(cfg.variant, cfg.grid, cfg.kgroups)


# ---- programs ----------------------------------------------------------------

def run_gemv(workload, launches, variant=-1, grid=0):
    sys.path.insert(0, ROOT)
    import numpy as np
    import torch
    import memory_bound_dense_amd as mbd
    from gemv_inputs import find_workload, random_inputs, torch_dtype
    name, n, k, dtype, dist = find_workload(workload)
    dev = torch.device("cuda", 0)
    td = torch_dtype(dtype)
    B_bits, a_bits = random_inputs(n, k, dtype, dist, seed=0)
    B0 = torch.from_numpy(B_bits.view(np.int16)).to(dev).view(td)
    a0 = torch.from_numpy(a_bits.view(np.int16)).to(dev).view(td)
    nbuf = int(min(4096, max(2, math.ceil((1 << 30) / (2.0 * n * k)))))
    Bs = [B0] + [B0.clone() for _ in range(nbuf - 1)]
    As = [a0] + [a0.clone() for _ in range(nbuf - 1)]
    Cs = [torch.empty(n, dtype=td, device=dev) for _ in range(nbuf)]
    torch.cuda.synchronize()
    g = mbd.Gemv(workspace=True)
    if variant >= 0:
        g.force_config(variant, grid)
    v, grid, kgroups = g.query_config(n, k, dtype)
    for i in range(launches):
        g(Bs[i % nbuf], As[i % nbuf], Cs[i % nbuf])
    torch.cuda.synchronize()
    g.close()
    print("gemv %s: %d launches, variant %d grid %d x %d" % (name, launches, v, grid, kgroups),
          flush=True)


def run_gla(workload, launches):
    """`launches` GLA decode steps of a workload, the state updated in place,
    rotating over copies of the state that exceed 1 GiB (as bench.py does)."""
    sys.path.insert(0, ROOT)
    import numpy as np
    import torch
    import memory_bound_dense_amd as mbd
    from gemv_inputs import find_gla_workload, gla_inputs, torch_dtype
    name, bh, dk, dv, dtype = find_gla_workload(workload)
    dev = torch.device("cuda", 0)
    td = torch_dtype(dtype)
    q, k, v, gk, S = gla_inputs(bh, dk, dv, dtype, seed=0)
    t = lambda x: torch.from_numpy(x.view(np.int16)).to(dev).view(td)
    qd, kd, vd, gd = t(q), t(k), t(v), t(gk)
    S0 = torch.from_numpy(S).to(dev)
    nbuf = int(min(4096, max(2, math.ceil((1 << 30) / (4.0 * bh * dk * dv)))))
    Ss = [S0] + [S0.clone() for _ in range(nbuf - 1)]
    os_ = [torch.empty((bh, dv), dtype=td, device=dev) for _ in range(nbuf)]
    torch.cuda.synchronize()
    g = mbd.Gemv()
    sp = torch.cuda.current_stream(dev).cuda_stream
    for i in range(launches):
        p = Ss[i % nbuf].data_ptr()
        rc = mbd.gla_decode_step(g.h, qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), gd.data_ptr(),
                                 p, p, os_[i % nbuf].data_ptr(), bh, dk, dv,
                                 1.0 / math.sqrt(dk), dtype, sp)
        if rc != 0:
            raise mbd.GemvError(rc, "gla_decode_step")
    torch.cuda.synchronize()
    g.close()
    print("gla %s: %d launches" % (name, launches), flush=True)


def run_copy(nbytes, launches):
    import torch
    dev = torch.device("cuda", 0)
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    for _ in range(launches):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("copy: %d launches of %d bytes" % (launches, nbytes), flush=True)


# ---- summarisers ---------------------------------------------------------------

def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _col(row, *names):
    for n in names:
        if n in row:
            return row[n]
    raise KeyError("none of %s in %s" % (names, list(row)))


def counter_per_dispatch(path, kernel_substr, counter):
    vals = []
    for r in _rows(path):
        if kernel_substr in _col(r, "Kernel_Name", "Kernel-Name") and \
                _col(r, "Counter_Name", "Counter-Name") == counter:
            vals.append(float(_col(r, "Counter_Value", "Counter-Value")))
    if not vals:
        raise ValueError("no %s rows for a kernel matching %r in %s" % (counter, kernel_substr, path))
    return vals


def _bench_line(path):
    """The JSON line bench.py printed (the last line of `path` that parses)."""
    import json
    line = None
    for raw in open(path):
        raw = raw.strip()
        if raw.startswith("{"):
            try:
                line = json.loads(raw)
            except ValueError:
                pass
    if line is None:
        raise ValueError("no JSON line in %s" % path)
    return line


def summarize_trace(stats_csv, trace_csv, command, out, last=0, kind="gemv", bench_json=""):
    sources = GLA_SOURCES if kind == "gla" else None
    lines = ["# rocprofv3 kernel trace summary", "command: %s" % command,
             "kernel_source_sha256_16: %s" % kernel_source_hash(sources)]
    if bench_json:
        b = _bench_line(bench_json)
        cfg = b.get("config", {})
        lines.append("bench line of the same run: workload %s, kernel_us_avg %s us (HIP events "
                     "over the timed region), value %s %s, launch %s%s" % (
                         cfg.get("workload"), b.get("kernel_us_avg"), b.get("value"), b.get("unit"),
                         cfg.get("launch"),
                         "" if kind == "gla" else ", plan variant %s grid %s kgroups %s" % (
                             cfg.get("variant"), cfg.get("grid"), cfg.get("kgroups"))))
    lines.append("")
    stats = _rows(stats_csv)
    keys = list(stats[0].keys()) if stats else []
    lines.append("kernel_stats.csv (all kernels):")
    lines.append("  " + " | ".join(keys))
    for r in stats:
        lines.append("  " + " | ".join(r[k] for k in keys))
    if trace_csv:
        durs = {}
        rows = sorted(_rows(trace_csv), key=lambda r: int(_col(r, "Start_Timestamp",
                                                                "Start-Timestamp")))
        for r in rows:
            nm = _col(r, "Kernel_Name", "Kernel-Name")
            d = (int(_col(r, "End_Timestamp", "End-Timestamp")) -
                 int(_col(r, "Start_Timestamp", "Start-Timestamp"))) / 1000.0
            durs.setdefault(nm, []).append(d)
        lines.append("")
        lines.append("per-kernel durations from kernel_trace.csv (us):")
        for nm, d in durs.items():
            lines.append("  %s: dispatches %d avg %.3f median %.3f min %.3f max %.3f" % (
                nm, len(d), statistics.fmean(d), statistics.median(d), min(d), max(d)))
        if last:
            # the timed region: a kernel's last `last` dispatches, in start order
            lines.append("")
            lines.append("the last %d dispatches of each kernel with at least that many "
                         "(the timed region), us:" % last)
            for nm, d in durs.items():
                if len(d) >= last:
                    t = sorted(d[-last:])
                    med = statistics.median(t)
                    sd = statistics.pstdev(t)
                    lines.append("  %s: avg %.3f median %.3f min %.3f max %.3f p10 %.3f p90 %.3f "
                                 "sd/median %.4f%s" % (
                                     nm, statistics.fmean(t), med, t[0], t[-1],
                                     t[int(0.1 * (len(t) - 1))], t[int(0.9 * (len(t) - 1))],
                                     sd / med, "  (> 0.10: contaminated)" if sd / med > 0.10 else ""))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_counters(workload, fetch, write, copy_fetch, copy_write, copy_bytes, commands, out):
    sys.path.insert(0, ROOT)
    from gemv_inputs import algorithmic_bytes, find_gla_workload, find_workload, gla_step_bytes
    gla = find_gla_workload(workload)
    if gla is not None:
        name, bh, dk, dv, dtype = gla
        n = bh * dv                     # outputs: o; bytes per output below are per o element
        alg = gla_step_bytes(bh, dk, dv)
        kernel, sources = GLA_KERNEL, GLA_SOURCES
        what = "%s (bh=%d dk=%d dv=%d)" % (name, bh, dk, dv)
        plan = GLA_PLAN
    else:
        name, n, k, dtype, dist = find_workload(workload)
        alg = algorithmic_bytes(n, k)
        kernel, sources = GEMV_KERNEL, None
        what = "%s (n=%d k=%d)" % (name, n, k)
        plan = workload_plan_signature(n, k, dtype)
    f_g = statistics.median(counter_per_dispatch(fetch, kernel, "FETCH_SIZE")) * 1024
    w_g = statistics.median(counter_per_dispatch(write, kernel, "WRITE_SIZE")) * 1024
    # one scale per counter from each copy calibration (copies of different
    # sizes); the mean is applied, the spread says how far it can be trusted
    if not (len(copy_fetch) == len(copy_write) == len(copy_bytes)):
        raise ValueError("one fetch and one write CSV per copy size")
    cal = []
    for cf, cw, cb in zip(copy_fetch, copy_write, copy_bytes):
        f_c = statistics.median(counter_per_dispatch(cf, COPY_KERNEL, "FETCH_SIZE")) * 1024
        w_c = statistics.median(counter_per_dispatch(cw, COPY_KERNEL, "WRITE_SIZE")) * 1024
        cal.append((cb, f_c, w_c, cb / f_c, cb / w_c))
    sf = statistics.fmean(c[3] for c in cal)
    sw = statistics.fmean(c[4] for c in cal)
    traffic = f_g * sf + w_g * sw
    lines = [
        "# HBM traffic of the %s kernel from rocprofv3 counters (median per dispatch)" % (
            "GLA decode" if gla is not None else "GEMV"),
        "workload: %s" % what,
        "commands:",
    ] + ["  " + c for c in commands] + [
        "kernel_source_sha256_16: %s" % kernel_source_hash(sources),
        "plan: %s" % plan,
    ] + ["copy_calibration: %d bytes read and written: fetch counted %.0f (scale %.5f), "
         "write counted %.0f (scale %.5f)" % (cb, f_c, a, w_c, b) for cb, f_c, w_c, a, b in cal] + [
        "fetch_scale: %.5f (spread %.5f over %d copy sizes)" % (
            sf, max(c[3] for c in cal) - min(c[3] for c in cal), len(cal)),
        "write_scale: %.5f (spread %.5f over %d copy sizes)" % (
            sw, max(c[4] for c in cal) - min(c[4] for c in cal), len(cal)),
        "gemv_fetch_counted_bytes: %.0f" % f_g,
        "gemv_write_counted_bytes: %.0f" % w_g,
        "algorithmic_bytes_per_launch: %d" % alg,
        "hbm_bytes_per_launch: %.0f" % traffic,
        "traffic_over_algorithmic: %.4f" % (traffic / alg),
        "hbm_bytes_per_output: %.1f" % (traffic / n),
        "algorithmic_bytes_per_output: %.1f" % (alg / n),
    ]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    p = sub.add_parser("gemv")
    p.add_argument("--workload", default="gemv_18432x7168_f16")
    p.add_argument("--launches", type=int, default=20)
    p.add_argument("--variant", type=int, default=-1, help="force this variant (-1: automatic)")
    p.add_argument("--grid", type=int, default=0, help="grid of a forced variant (0: full)")
    p = sub.add_parser("gla")
    p.add_argument("--workload", default="gla_decode_b64h32_128x128_bf16")
    p.add_argument("--launches", type=int, default=20)
    p = sub.add_parser("copy")
    p.add_argument("--bytes", type=int, default=256 << 20)
    p.add_argument("--launches", type=int, default=10)
    p = sub.add_parser("summarize-trace")
    p.add_argument("--stats", required=True)
    p.add_argument("--trace", default="")
    p.add_argument("--command", required=True)
    p.add_argument("--out", required=True)
    p.add_argument("--last", type=int, default=0,
                   help="also summarise each kernel's last N dispatches (the timed region)")
    p.add_argument("--kind", choices=("gemv", "gla"), default="gemv",
                   help="whose device code the summary's source hash covers")
    p.add_argument("--bench-json", default="",
                   help="bench.py's output of the profiled run: its line is quoted")
    p = sub.add_parser("summarize-counters")
    p.add_argument("--workload", required=True)
    p.add_argument("--fetch", required=True)
    p.add_argument("--write", required=True)
    p.add_argument("--copy-fetch", nargs="+", required=True, help="one CSV per copy size")
    p.add_argument("--copy-write", nargs="+", required=True, help="one CSV per copy size")
    p.add_argument("--copy-bytes", type=int, nargs="+", required=True)
    p.add_argument("--commands", nargs="+", required=True)
    p.add_argument("--out", required=True)
    a = ap.parse_args()
    if a.cmd == "gemv":
        run_gemv(a.workload, a.launches, a.variant, a.grid)
    elif a.cmd == "gla":
        run_gla(a.workload, a.launches)
    elif a.cmd == "copy":
        run_copy(a.bytes, a.launches)
    elif a.cmd == "summarize-trace":
        summarize_trace(a.stats, a.trace, a.command, a.out, a.last, a.kind, a.bench_json)
    else:
        summarize_counters(a.workload, a.fetch, a.write, a.copy_fetch, a.copy_write, a.copy_bytes,
                           a.commands, a.out)


if __name__ == "__main__":
    main()
