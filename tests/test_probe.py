"""GPU: the measurement aids of libmbd_probe.so (include/stream_probe.h).

* the streaming read covers every byte exactly once, whatever the grid and
  unroll: the sum of its per-wave words equals the sum, over every 16-byte
  vector of the buffer, of the xor of its four words (mod 2^32);
* the GEMV kernel without its arithmetic runs the plan shapes it has, with
  and without a cross-workgroup split, writes its n outputs and nothing
  past them;
* the bench line carries both probes.
"""
import numpy as np
import pytest
import torch

import memory_bound_dense_amd as mbd
from memory_bound_dense_amd import probe

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [1024, 5 * 1024, 1 << 20, 37 * 1024 + 8 * 1024 * 1024])
def test_stream_read_covers_every_byte_once(nbytes):
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    want = int(np.bitwise_xor.reduce(words.reshape(-1, 4), axis=1).astype(np.uint64).sum()) % 2 ** 32
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    out = torch.zeros(1 << 20, dtype=torch.int32, device="cuda")
    for unroll in (2, 4, 8, 16):
        for grid in (0, 1, 3, 1000):
            out.zero_()
            g = probe.stream_read(buf.data_ptr(), nbytes, out.data_ptr(), out.numel(), grid,
                                  unroll, True, torch.cuda.current_stream().cuda_stream)
            torch.cuda.synchronize()
            got = int(out[:4 * g].cpu().numpy().view(np.uint32).astype(np.uint64).sum()) % 2 ** 32
            assert got == want, (nbytes, unroll, grid)
            assert not torch.any(out[4 * g:] != 0)


def test_gemv_probe_runs_the_plan_shapes():
    g = mbd.Gemv(workspace=True)
    for n, k, dtype in [(18432, 7168, mbd.GEMV_F16), (64, 65536, mbd.GEMV_BF16),
                        (1000, 7000, mbd.GEMV_BF16), (4096, 4096, mbd.GEMV_F16),
                        (256, 512, mbd.GEMV_F16), (4096, 11008, mbd.GEMV_BF16),
                        (8192, 7000, mbd.GEMV_BF16), (4096, 9216, mbd.GEMV_BF16)]:
        v, grid, kgroups = g.query_config(n, k, dtype)
        info = mbd.gemv_variant_info(v)[1]
        assert probe.gemv_probe_has(info), (n, k, v)
        B = torch.randn(n, k, device="cuda").half()
        outbig = torch.full((n + 64,), 3.0, dtype=torch.float16, device="cuda")
        for _ in range(2):
            probe.gemv_probe(info, B.data_ptr(), n, k, outbig.data_ptr(), g.ws.data_ptr(), grid,
                             kgroups, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert torch.all(outbig[n:] == 3.0), (n, k)
        assert not torch.all(outbig[:n] == 3.0), (n, k)
    # shapes it has no build of, and bad arguments, are refused
    with pytest.raises(RuntimeError):
        info = mbd.gemv_variant_info(0)[1]
        probe.gemv_probe(info, 0, 4, 512, 0, None, 1, 1)
    g.close()


def test_bench_line_carries_both_probes():
    import json
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--workload",
                        "ragged_1000x7000_bf16", "--steps", "20", "--warmup", "5",
                        "--no-cpu-baseline"], cwd=root, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    out = json.loads(r.stdout.strip().splitlines()[-1])
    sp, ap = out["stream_read_probe"], out["access_pattern_probe"]
    assert sp["us"] > 0 and sp["gbs"] > 0 and sp["unroll"] in (4, 8, 16)
    assert ap["us"] > 0 and ap["bytes_of_B"] == 2 * 1000 * 7000
    assert out["context"]["pages_uncoalesced_gbs_h200"] == 110
