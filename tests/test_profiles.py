"""Host logic behind the committed profiles and the bench's `traffic` field
(no GPU): the source hash that ties a counter summary to the kernel code,
the rule that reuses a summary only for the same code and plan, and the
arithmetic that turns rocprofv3 counter and trace CSVs into the figures the
summaries give."""
import csv
import glob
import json
import os
import re

import pytest

import bench
from gemv_inputs import algorithmic_bytes, find_gla_workload, find_workload, gla_step_bytes
from memory_bound_dense_amd import profile_counters as pc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _kv(path):
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#") and not line.startswith(" "):
            key, val = line.split(":", 1)
            kv[key.strip()] = val.strip()
    return kv


def _calibrations(path):
    """(bytes, fetch counted, fetch scale, write counted, write scale) per
    copy_calibration line of a counter summary."""
    pat = re.compile(r"copy_calibration: (\d+) bytes read and written: fetch counted ([\d.]+) "
                     r"\(scale ([\d.]+)\), write counted ([\d.]+) \(scale ([\d.]+)\)")
    out = []
    for line in open(path):
        m = pat.match(line.strip())
        if m:
            out.append(tuple(float(x) for x in m.groups()))
    return out


def test_source_hash_ignores_comments_and_whitespace(tmp_path):
    a, b, c = tmp_path / "a.h", tmp_path / "b.h", tmp_path / "c.h"
    a.write_text("int f(int x) {\n  return x + 1;  // one more\n}\n")
    b.write_text("/* header */ int f(int x)\n{ return x + 1; }\n")
    c.write_text("int f(int x) { return x + 2; }\n")
    h = lambda p: pc.kernel_source_hash([str(p)])
    assert h(a) == h(b)
    assert h(a) != h(c)
    # the order of the sources is part of the hash
    assert pc.kernel_source_hash([str(a), str(c)]) != pc.kernel_source_hash([str(c), str(a)])


@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(ROOT, "profiles", "*.counters.txt"))),
                         ids=lambda p: os.path.basename(p))
def test_counter_summaries_add_up(path):
    """Each committed counter summary: traffic = fetch x its copy scale +
    write x its copy scale, over the workload's algorithmic bytes."""
    kv = _kv(path)
    name = os.path.basename(path)[:-len(".counters.txt")]
    gla = find_gla_workload(name)
    if gla is not None:
        _, bh, dk, dv, _ = gla
        alg = gla_step_bytes(bh, dk, dv)
    else:
        _, n, k, _, _ = find_workload(name)
        alg = algorithmic_bytes(n, k)
    assert int(kv["algorithmic_bytes_per_launch"]) == alg
    sf, sw = float(kv["fetch_scale"].split()[0]), float(kv["write_scale"].split()[0])
    cal = _calibrations(path)
    # at least two copy sizes; each line's scale is its bytes over its count,
    # and the applied scale is their mean
    assert len(cal) >= 2 and len({c[0] for c in cal}) == len(cal)
    for cb, f_c, a, w_c, b in cal:
        assert abs(a - cb / f_c) < 1e-4 * a and abs(b - cb / w_c) < 1e-4 * b
    assert abs(sf - sum(c[2] for c in cal) / len(cal)) < 1e-4 * sf
    assert abs(sw - sum(c[4] for c in cal) / len(cal)) < 1e-4 * sw
    traffic = float(kv["gemv_fetch_counted_bytes"]) * sf + float(kv["gemv_write_counted_bytes"]) * sw
    assert abs(traffic - float(kv["hbm_bytes_per_launch"])) <= 1e-4 * traffic
    assert abs(float(kv["traffic_over_algorithmic"]) - traffic / alg) < 1e-4
    # no kernel here reads less than the bytes it must read once
    assert traffic / alg > 0.99


def test_read_traffic_requires_the_same_code_and_plan(tmp_path):
    name, n, k, dtype, _ = find_workload("gemv_18432x7168_f16")
    path = os.path.join(ROOT, "profiles", "%s.counters.txt" % name)
    kv = _kv(path)
    plan = pc.workload_plan_signature(n, k, dtype)
    fresh = kv["kernel_source_sha256_16"] == pc.kernel_source_hash() and kv["plan"] == plan
    got = bench.read_traffic(name, algorithmic_bytes(n, k), plan)
    assert got == (float(kv["hbm_bytes_per_launch"]) if fresh else None)
    # another plan, or other code, and the summary is not reused
    assert bench.read_traffic(name, algorithmic_bytes(n, k), plan + " (other)") is None
    other = tmp_path / "other.h"
    other.write_text("int g() { return 0; }\n")
    assert bench.read_traffic(name, algorithmic_bytes(n, k), kv["plan"], sources=[str(other)]) is None
    # no summary for a workload: None
    assert bench.read_traffic("no_such_workload", 1, plan) is None


def _write_csv(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_counter_summary_arithmetic(tmp_path):
    """Synthetic counter CSVs: medians per dispatch of the matching kernel
    only, KiB to bytes, each counter scaled by what it reads for a copy of
    known size."""
    name, n, k, dtype, _ = find_workload("tiny_256x512_f16")
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    gk = "void mbd::gemv_kernel<0, 1, 2, 4, 1, 1, 2, false>(...)"
    other = "void at::native::fill(...)"
    f = tmp_path / "f.csv"
    w = tmp_path / "w.csv"
    cf = tmp_path / "cf.csv"
    cw = tmp_path / "cw.csv"
    # fetch: 100, 130 (median of three), 101 KiB; a foreign kernel's row ignored
    _write_csv(f, hdr, [[1, gk, "FETCH_SIZE", 100], [2, other, "FETCH_SIZE", 9999],
                        [3, gk, "FETCH_SIZE", 130], [4, gk, "FETCH_SIZE", 101]])
    _write_csv(w, hdr, [[1, gk, "WRITE_SIZE", 1], [2, gk, "WRITE_SIZE", 1]])
    _write_csv(cf, hdr, [[1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 512]])    # half of 1 MiB
    _write_csv(cw, hdr, [[1, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 1024]])   # all of it
    # a second copy of 4 MiB: fetch counts 2000 KiB (scale 2.048), write all
    cf2, cw2 = tmp_path / "cf2.csv", tmp_path / "cw2.csv"
    _write_csv(cf2, hdr, [[1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 2000]])
    _write_csv(cw2, hdr, [[1, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 4096]])
    out = tmp_path / "s.txt"
    pc.summarize_counters(name, str(f), str(w), [str(cf), str(cf2)], [str(cw), str(cw2)],
                          [1 << 20, 4 << 20], ["cmd"], str(out))
    kv = _kv(out)
    sf = (2.0 + 4096 / 2000) / 2
    assert float(kv["fetch_scale"].split()[0]) == pytest.approx(sf, abs=1e-5)
    assert "spread 0.04800 over 2 copy sizes" in kv["fetch_scale"]
    assert float(kv["write_scale"].split()[0]) == pytest.approx(1.0)
    assert len(_calibrations(out)) == 2
    assert float(kv["gemv_fetch_counted_bytes"]) == 101 * 1024
    assert float(kv["hbm_bytes_per_launch"]) == pytest.approx(101 * 1024 * sf + 1 * 1024, rel=1e-6)
    # one write CSV short of the fetch CSVs: an error
    with pytest.raises(ValueError):
        pc.summarize_counters(name, str(f), str(w), [str(cf), str(cf2)], [str(cw)],
                              [1 << 20, 4 << 20], ["cmd"], str(out))
    assert int(kv["algorithmic_bytes_per_launch"]) == algorithmic_bytes(n, k)
    assert kv["plan"] == pc.workload_plan_signature(n, k, dtype)
    assert kv["kernel_source_sha256_16"] == pc.kernel_source_hash()
    # a counter file without the kernel is an error, not a zero
    with pytest.raises(ValueError):
        pc.counter_per_dispatch(str(f), "no_such_kernel", "FETCH_SIZE")


def test_trace_summary_of_the_last_dispatches(tmp_path):
    """Durations from start/end timestamps (ns -> us), in start order; the
    timed region is each kernel's last N dispatches."""
    stats = tmp_path / "stats.csv"
    trace = tmp_path / "trace.csv"
    _write_csv(stats, ["Name", "Calls"], [["k", 12]])
    # 2 slow warm-up dispatches, then 10 of 1..10 us; rows written out of order
    rows, t = [], 0
    for i, d in enumerate([50, 40] + list(range(1, 11))):
        rows.append([i, "k", t, t + d * 1000])
        t += 100000
    rows.reverse()
    _write_csv(trace, ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    out = tmp_path / "t.txt"
    pc.summarize_trace(str(stats), str(trace), "cmd", str(out), last=10)
    text = out.read_text()
    assert "k: dispatches 12 avg %.3f" % ((50 + 40 + 55) / 12) in text
    # last 10: 1..10 us -> avg 5.5, median 5.5, p10 = t[0] = 1, p90 = t[8] = 9
    assert "k: avg 5.500 median 5.500 min 1.000 max 10.000 p10 1.000 p90 9.000" in text
    assert "contaminated" in text        # sd/median of 1..10 is far above 0.10


def test_trace_summary_hash_and_bench_line(tmp_path):
    """A GLA trace summary hashes the GLA step's sources, a GEMV one the
    GEMV's; the bench line of the profiled run is quoted."""
    stats = tmp_path / "stats.csv"
    _write_csv(stats, ["Name", "Calls"], [["k", 1]])
    bj = tmp_path / "bench.out"
    line = {"value": 7000.0, "unit": "GB/s", "kernel_us_avg": 37.5,
            "config": {"workload": "w", "launch": "graph", "variant": 3, "grid": 9, "kgroups": 1}}
    bj.write_text("[bench] noise\n" + json.dumps(line) + "\n")
    for kind, sources in (("gemv", None), ("gla", pc.GLA_SOURCES)):
        out = tmp_path / ("%s.txt" % kind)
        pc.summarize_trace(str(stats), "", "cmd", str(out), kind=kind, bench_json=str(bj))
        kv = _kv(out)
        assert kv["kernel_source_sha256_16"] == pc.kernel_source_hash(sources)
        assert "kernel_us_avg 37.5 us" in out.read_text()
    assert pc.kernel_source_hash(pc.GLA_SOURCES) != pc.kernel_source_hash()


@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(ROOT, "profiles", "*.trace.txt"))),
                         ids=lambda p: os.path.basename(p))
def test_trace_summaries_name_their_code(path):
    """Each committed trace summary gives its command and the hash of the
    device code it ran (the GLA step's sources for a GLA summary)."""
    kv = _kv(path)
    assert kv["command"]
    gla = os.path.basename(path).startswith("gla_")
    want = pc.kernel_source_hash(pc.GLA_SOURCES if gla else None)
    assert len(kv["kernel_source_sha256_16"]) == 16
    if kv["kernel_source_sha256_16"] != want:
        pytest.skip("summary taken on other device code: %s" % os.path.basename(path))
