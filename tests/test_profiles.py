"""Host logic behind the committed profiles and the bench's `traffic` field
(no GPU): the source hash that ties a counter summary to the kernel code,
the rule that reuses a summary only for the same code and plan, and the
arithmetic that turns rocprofv3 counter and trace CSVs into the figures the
summaries give."""
import csv
import glob
import os

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
    cb = float(kv["copy_kernel_bytes"])
    sf, sw = float(kv["fetch_scale"]), float(kv["write_scale"])
    assert abs(sf - cb / float(kv["copy_fetch_counted_bytes"])) < 1e-4 * sf
    assert abs(sw - cb / float(kv["copy_write_counted_bytes"])) < 1e-4 * sw
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
    copy_bytes = 1 << 20
    _write_csv(cf, hdr, [[1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 512]])    # half of 1 MiB
    _write_csv(cw, hdr, [[1, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 1024]])   # all of it
    out = tmp_path / "s.txt"
    pc.summarize_counters(name, str(f), str(w), str(cf), str(cw), copy_bytes, ["cmd"], str(out))
    kv = _kv(out)
    assert float(kv["fetch_scale"]) == pytest.approx(2.0)
    assert float(kv["write_scale"]) == pytest.approx(1.0)
    assert float(kv["gemv_fetch_counted_bytes"]) == 101 * 1024
    assert float(kv["hbm_bytes_per_launch"]) == pytest.approx(101 * 1024 * 2.0 + 1 * 1024)
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
