"""bench.py's output contract: one JSON line with the metric, the roofline
object and the oracle's CPU baseline; one GPU only."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, timeout=300):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + list(args),
                          cwd=ROOT, capture_output=True, text=True, timeout=timeout)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _line(r):
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


@pytest.mark.gpu
def test_json_line_graph_with_cpu_baseline():
    out = _line(_bench("--workload", "tiny_256x512_f16", "--steps", "20", "--warmup", "5",
                       "--no-probe"))
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in out, key
    assert out["n_gpus"] == 1 and out["steps"] == 20 and out["warmup"] == 5
    assert out["unit"] == "GB/s" and out["value"] > 0 and out["dtype"] == "f16"
    assert out["config"]["workload"] == "tiny_256x512_f16" and out["config"]["launch"] == "graph"
    assert out["metric"].endswith("n=256 k=512 fp16")
    rf = out["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert 0 < rf["frac"] < 1.2 and abs(rf["achieved"] / rf["peak"] - rf["frac"]) < 1e-3
    cb = out["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0 and cb["sample"]
    # 2k + 2 bytes per row, plus a's 2k bytes shared over the n rows
    assert out["bytes_per_output"]["algorithmic"] == round(2 * (256 * 512 + 512 + 256) / 256, 2)


@pytest.mark.gpu
def test_json_line_stream_and_epilogue():
    out = _line(_bench("--workload", "square_1024x1024_f16", "--steps", "20", "--warmup", "5",
                       "--no-probe", "--no-cpu-baseline", "--stream", "--epilogue"))
    assert out["config"]["launch"] == "stream" and out["config"]["epilogue"] == "alpha_bias"
    assert out["roofline"]["traffic"] is None and "cpu_baseline" not in out
    assert out["value"] > 0


@pytest.mark.gpu
def test_json_line_gla():
    out = _line(_bench("--op", "gla", "--steps", "20", "--warmup", "5", "--no-probe"))
    assert out["config"]["workload"] == "gla_decode_b1h32_128x128_bf16"
    assert out["config"]["launch"] == "graph" and out["roofline"]["frac"] > 0


def test_metric_names_the_workload():
    import bench
    # the default workload's metric line is the headline's
    assert bench.metric_of(18432, 7168, "f16") == bench.METRIC
    assert bench.metric_of(7168, 16384, "bf16").endswith("n=7168 k=16384 bf16")


def test_rotation_exceeds_the_infinity_cache():
    import bench
    for nbytes in (263680, 2 << 20, 8 << 20, 264292352, 940 << 20):
        m = bench.rotation(nbytes)
        assert m >= 2 and m <= bench.MAX_COPIES
        assert m * nbytes >= (1 << 30), (nbytes, m)         # >= 1 GiB between two uses of a copy
    assert bench.rotation(1) == bench.MAX_COPIES


def test_host_launches_keep_rotating_across_runs():
    import bench

    class FakeStream:
        cuda_stream = None

    seen = []
    lau = bench.Launcher(lambda i, sp: seen.append(i), 3, 5, FakeStream(), None, graph=False)
    for _ in range(4):
        lau.run()
    # the launch index keeps counting, so copies are used round robin: copy i % 5
    assert seen == list(range(12))
    assert [i % 5 for i in seen[:10]] == [0, 1, 2, 3, 4, 0, 1, 2, 3, 4]
