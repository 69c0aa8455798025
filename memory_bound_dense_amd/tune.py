"""Offline tuner: time every compiled variant (x grid x k-groups) on one shape
and rank them against the automatic plan.

    python -m memory_bound_dense_amd.tune --shape 18432,7168,f16
    python -m memory_bound_dense_amd.tune --workload gemv_7168x16384_bf16 --grids 0,512,1024

Method (page "Optimizing TileLang Programs", the change-one-thing method and
its before/after template; TileLang Case Studies, Case C: fixed
configurations, never tuning inside a profiled run): every candidate is a
forced configuration; each is timed as K back-to-back launches rotating over
> 1 GiB of input copies, with one HIP event pair; the candidates are measured
in interleaved rounds (so a drifting clock or a neighbour's load hits them
alike) and ranked by their median round.  --out appends one JSON line per
candidate, so a sweep can be resumed and compared later.

The inputs are random (their values do not change the timing); correctness
is the test suite's business.
"""
import argparse
import json
import math
import os
import statistics
import sys


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--shape", default="", help="'n,k,f16|bf16'")
    ap.add_argument("--workload", default="gemv_18432x7168_f16")
    ap.add_argument("--variants", default="", help="comma list (default: all that fit)")
    ap.add_argument("--grids", default="0,512,768,1024,1536,2048")
    ap.add_argument("--kgroups", default="2,4,8", help="k-groups tried on cross-workgroup variants")
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--rounds", type=int, default=3)
    ap.add_argument("--top", type=int, default=15)
    ap.add_argument("--include-ablation", action="store_true",
                    help="also time the uncoalesced layout (slow)")
    ap.add_argument("--out", default="", help="append JSON lines here")
    ap.add_argument("--xcd", action="store_true",
                    help="also time every candidate with its row ranges numbered XCD by XCD")
    ap.add_argument("--graph", action="store_true",
                    help="time each candidate's launches as one HIP graph replay (as bench.py "
                         "does by default) instead of host launches")
    args = ap.parse_args()

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import torch
    import memory_bound_dense_amd as mbd
    from gemv_inputs import algorithmic_bytes, find_workload, shape_workload, torch_dtype

    wl = shape_workload(args.shape) if args.shape else find_workload(args.workload)
    if wl is None:
        sys.exit("unknown workload %r" % args.workload)
    name, n, k, dtype, _ = wl
    dev = torch.device("cuda", 0)
    td = torch_dtype(dtype)
    B0 = (torch.randn(n, k, device=dev) / math.sqrt(max(k, 1))).to(td)
    a0 = torch.randn(k, device=dev).to(td)
    nbuf = int(min(4096, max(2, math.ceil((1 << 30) / max(2.0 * n * k, 1.0)))))
    Bs = [B0] + [B0.clone() for _ in range(nbuf - 1)]
    As = [a0.clone() for _ in range(nbuf)]
    Cs = [torch.empty(n, dtype=td, device=dev) for _ in range(nbuf)]
    P = [(Bs[i].data_ptr(), As[i].data_ptr(), Cs[i].data_ptr()) for i in range(nbuf)]
    # with caller scratch, so that the cross-workgroup variants run too (the
    # automatic plan is then gemv_run_ws's, as the benchmark times it)
    g = mbd.Gemv(workspace=True)
    ws, wsb = g.ws.data_ptr(), g.ws.numel()
    auto = g.query_config(n, k, dtype)
    nv = mbd.gemv_num_variants()
    variants = [int(x) for x in args.variants.split(",")] if args.variants else list(range(nv))
    grids = [int(x) for x in args.grids.split(",")]
    kgs = [int(x) for x in args.kgroups.split(",")]

    cands = []                         # (variant, grid asked, kgroups asked, resolved config, flags)
    for v in variants:
        info = mbd.gemv_variant_info(v)[1]
        if info.layout == 1 and not args.include_ablation:
            continue
        seen = set()
        for gr in grids:
            for kq in (kgs if info.cross_wg else [0]):
                try:
                    g.force_config(v, gr, kq)
                    cfg = g.query_config(n, k, dtype)
                except mbd.GemvError:
                    continue
                if cfg not in seen:
                    seen.add(cfg)
                    for fl in ((0, 1) if args.xcd else (0,)):
                        cands.append((v, gr, kq, cfg, fl))
    g.force_config(-1)
    if auto not in [c[3] for c in cands if c[4] == 0]:
        cands.append((-1, 0, 0, auto, 0))
    print("[tune] %s: %d candidates, %d rounds of %d launches, %d rotating buffers" % (
        name, len(cands), args.rounds, args.steps, nbuf), file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    times = {i: [] for i in range(len(cands))}
    graphs = {}
    if args.graph:
        # one graph per candidate, captured once (the forced configuration is
        # baked into the captured launches)
        side = torch.cuda.Stream(dev)
        for i, (v, gr, kq, cfg, fl) in enumerate(cands):
            g.force_config(v, gr, kq, fl)
            gph = torch.cuda.CUDAGraph()
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                with torch.cuda.graph(gph, stream=side):
                    for j in range(args.steps):
                        mbd.gemv_run_ws(g.h, *P[j % nbuf], n, k, dtype, ws, wsb, stream=side.cuda_stream)
            stream.wait_stream(side)
            graphs[i] = gph
        torch.cuda.synchronize()
    for rnd in range(args.rounds):
        for i, (v, gr, kq, cfg, fl) in enumerate(cands):
            g.force_config(v, gr, kq, fl)
            for j in range(5):
                mbd.gemv_run_ws(g.h, *P[j % nbuf], n, k, dtype, ws, wsb, stream=sp)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            if args.graph:
                graphs[i].replay()
            else:
                for j in range(args.steps):
                    mbd.gemv_run_ws(g.h, *P[j % nbuf], n, k, dtype, ws, wsb, stream=sp)
            e1.record(stream)
            torch.cuda.synchronize()
            times[i].append(e0.elapsed_time(e1) * 1e3 / args.steps)
        print("[tune] round %d done" % (rnd + 1), file=sys.stderr, flush=True)
    g.force_config(-1)

    nbytes = algorithmic_bytes(n, k)
    rows = []
    for i, (v, gr, kq, cfg, fl) in enumerate(cands):
        med = statistics.median(times[i])
        info = mbd.gemv_variant_info(cfg[0])[1]
        rows.append({"workload": name, "n": n, "k": k, "variant": cfg[0], "grid": cfg[1],
                     "kgroups": cfg[2], "rows": info.rows, "unroll": info.unroll,
                     "waves": info.waves, "splits": info.splits, "a_mode": info.a_mode,
                     "b_policy": info.b_policy, "cross_wg": info.cross_wg, "layout": info.layout,
                     "stages": info.stages, "b_lds": info.b_lds,
                     "us_median": round(med, 3), "us_min": round(min(times[i]), 3),
                     "gbs": round(nbytes / med / 1e3, 1), "xcd": fl, "auto": cfg == auto and fl == 0})
    rows.sort(key=lambda r: r["us_median"])
    best = rows[0]["us_median"]
    print("%4s %4s %6s %3s | %2s %2s %2s %2s %2s %2s %2s %2s %2s %2s | %9s %8s %7s" % (
        "rank", "var", "grid", "kg", "R", "U", "W", "S", "am", "pl", "x", "P", "L", "X", "us", "GB/s",
        "vs best"))
    for r_i, r in enumerate(rows):
        if r_i < args.top or r["auto"]:
            print("%4d %4d %6d %3d | %2d %2d %2d %2d %2d %2d %2d %2d %2d %2d | %9.3f %8.1f %6.1f%%%s" % (
                r_i + 1, r["variant"], r["grid"], r["kgroups"], r["rows"], r["unroll"], r["waves"],
                r["splits"], r["a_mode"], r["b_policy"], r["cross_wg"], r["stages"], r["b_lds"],
                r["xcd"], r["us_median"], r["gbs"],
                100 * (r["us_median"] / best - 1), "  <- automatic plan" if r["auto"] else ""))
    if args.out:
        with open(args.out, "a") as f:
            for r in rows:
                f.write(json.dumps(r) + "\n")
    g.close()


if __name__ == "__main__":
    main()
