"""The automatic plan without a GPU (gemv_plan_config: the rule gemv_run
applies, worked out on the host).

* the plan of every configured workload, as measured best on MI355X with the
  tuner (a change to the rule shows up here first);
* the tiers for rows off 16-byte boundaries and for few rows;
* properties over a wide sweep of shapes: a valid, compiled, non-ablation
  variant whose LDS fits, and bad arguments rejected with the documented
  status.
"""
import itertools

import pytest

import memory_bound_dense_amd as mbd
from memory_bound_dense_amd import _lib
from gemv_inputs import ALL_WORKLOADS, BF16, EXTRA_WORKLOADS, F16

MAX_LDS = 160 * 1024          # bytes of LDS per workgroup on MI355X


def plan(n, k, dtype, aligned=True, ws=True):
    """The plan of gemv_run_ws with a workspace (ws=True, what the benchmark
    times) or of gemv_run / gemv_run_ex (ws=False)."""
    s, cfg = mbd.gemv_plan_config(n, k, dtype, 1 if aligned else 0, MAX_LDS, 1 if ws else 0)
    assert s == mbd.GEMV_OK, (n, k, dtype, aligned, mbd.gemv_status_string(s))
    info = mbd.gemv_variant_info(cfg.variant)[1]
    return cfg, info


def shape_of(info):
    return (info.rows, info.unroll, info.waves, info.splits, info.a_mode, info.cross_wg)


# (rows, unroll, waves, splits, a_mode, cross_wg) per configured workload;
# a_mode 0 = a staged in LDS, 1 = a through the caches, 2 = the realigning
# kernel's shifted LDS copies, 3 = the shifted-window kernel (line-aligned
# granules of B, a read through the caches at each row's shift)
WORKLOAD_PLANS = {
    "tiny_256x512_f16": (1, 2, 4, 1, 1, 0),
    "gemv_18432x7168_f16": (2, 4, 4, 4, 1, 0),
    "gemv_7168x16384_bf16": (2, 3, 16, 16, 1, 0),
    "sweep_4096x4096_f16": (1, 8, 4, 1, 1, 0),
    "sweep_4096x4096_bf16": (1, 8, 4, 1, 1, 0),
    "sweep_11008x4096_f16": (1, 8, 4, 1, 1, 0),
    "sweep_11008x4096_bf16": (1, 8, 4, 1, 1, 0),
    "sweep_4096x11008_f16": (2, 3, 8, 8, 1, 0),
    "sweep_4096x11008_bf16": (2, 3, 8, 8, 1, 0),
    "sweep_14336x4096_f16": (1, 8, 4, 1, 1, 0),
    "sweep_14336x4096_bf16": (1, 8, 4, 1, 1, 0),
    "sweep_4096x14336_f16": (2, 8, 4, 4, 1, 0),
    "sweep_4096x14336_bf16": (2, 8, 4, 4, 1, 0),
    "ragged_64x65536_bf16": (1, 2, 8, 8, 1, 1),
    "ragged_1000x7000_bf16": (2, 2, 8, 8, 1, 0),
    "ragged_18433x7169_bf16": (2, 4, 4, 4, 3, 0),
    "large_28672x8192_f16": (2, 3, 8, 8, 1, 0),
    "large_28672x8192_bf16": (2, 3, 8, 8, 1, 0),
    "large_57344x7168_f16": (2, 4, 4, 4, 1, 0),
    "large_57344x7168_bf16": (2, 4, 4, 4, 1, 0),
    "square_1024x1024_f16": (1, 2, 4, 1, 1, 0),
}


@pytest.mark.parametrize("wl", ALL_WORKLOADS + EXTRA_WORKLOADS, ids=lambda w: w[0])
def test_plan_of_every_workload(wl):
    name, n, k, dtype, _ = wl
    cfg, info = plan(n, k, dtype)
    assert shape_of(info) == WORKLOAD_PLANS[name], (name, shape_of(info))
    assert cfg.grid >= 1 and cfg.kgroups >= 1


def test_plan_grids_of_the_production_shapes():
    # one trip per workgroup: 2 rows (one row group of 4 k-slices) per
    # workgroup for the headline, 2 rows (8 k-slices) for (7168, 16384)
    assert plan(18432, 7168, F16)[0].grid == 9216
    assert plan(7168, 16384, BF16)[0].grid == 3584
    # (4096, 14336): two rows x four slices of eight-slot batches, one row
    # group per workgroup
    assert plan(4096, 14336, F16)[0].grid == 2048
    assert plan(4096, 14336, BF16)[0].grid == 2048
    # the shifted-window kernel pairs rows 64 apart: 64 pairs per 128 rows (the
    # last block of 128 partly empty), one pair per workgroup of 4 or 8
    # k-slices, on the full grid
    assert plan(18433, 7169, BF16)[0].grid == 9280
    assert plan(18432, 7169, BF16)[0].grid == 9216
    assert plan(12288, 7169, BF16)[0].grid == 6144
    assert plan(3072, 7169, BF16)[0].grid == 1536
    assert plan(7000, 7169, BF16)[0].grid == 3520
    assert plan(7169, 14337, BF16)[0].grid == 3648
    assert plan(18433, 4097, BF16)[0].grid == 9280
    # rows of at most 3 steps from 12288 rows: 4 pairs per 4-wave workgroup
    assert plan(16384, 1025, BF16)[0].grid == 2048
    # the realigning kernel keeps its persistent 1024 for 4..5 steps from
    # 12288 rows; one row per wave with a in LDS at most 1536 workgroups for
    # rows of at most 3 steps
    assert plan(12288, 2049, BF16)[0].grid == 1024
    # 64 rows: k shared by 8 workgroups per row
    assert plan(64, 65536, BF16)[0].kgroups == 8


def _nst(k):
    """Granule steps of a misaligned row: its k elements from a 16-byte
    boundary up to 63 elements before its start, in steps of 512."""
    return (k + 63 + 511) // 512


@pytest.mark.parametrize("n,k,want", [
    # from 768 misaligned rows: the shifted-window kernel (a_mode 3), by
    # granule steps nst = ceil((k + 63) / 512) and row count
    # from 6144 rows: two rows x four slices of two-slot batches up to 31 steps
    (8192, 8191, (2, 2, 4, 4, 3, 0)),      # 17
    (32768, 6143, (2, 2, 4, 4, 3, 0)),     # 13
    (8192, 7169, (2, 2, 4, 4, 3, 0)),      # 15
    (16384, 6147, (2, 2, 4, 4, 3, 0)),
    (32768, 8121, (2, 2, 4, 4, 3, 0)),
    (32768, 8185, (2, 2, 4, 4, 3, 0)),
    (7169, 14337, (2, 2, 4, 4, 3, 0)),     # 29
    (8192, 9217, (2, 2, 4, 4, 3, 0)),
    (8192, 12289, (2, 2, 4, 4, 3, 0)),     # 25
    (6144, 4097, (2, 2, 4, 4, 3, 0)),      # 9
    (8193, 2051, (2, 2, 4, 4, 3, 0)),      # 5
    (12288, 4097, (2, 2, 4, 4, 3, 0)),
    (14336, 2559, (2, 2, 4, 4, 3, 0)),     # 6 from 12288 rows
    # ... but four-slot batches at 14..15 steps from 12288 rows
    (18432, 7169, (2, 4, 4, 4, 3, 0)),
    (12288, 7169, (2, 4, 4, 4, 3, 0)),
    # 32..64 steps: eight slices of two-slot batches; beyond: four-slot
    (7169, 16383, (2, 2, 8, 8, 3, 0)),     # 33
    (8192, 16383, (2, 2, 8, 8, 3, 0)),
    (8192, 20481, (2, 2, 8, 8, 3, 0)),     # 41
    (8192, 24577, (2, 2, 8, 8, 3, 0)),     # 49
    (8192, 32705, (2, 2, 8, 8, 3, 0)),     # 64
    (8192, 32769, (2, 4, 8, 8, 3, 0)),     # 65
    # 1024..6143 rows: four slices up to 9 steps, eight for 10..64 (and
    # beyond below 3072 rows)
    (4096, 2051, (2, 2, 4, 4, 3, 0)),      # 5
    (4095, 2049, (2, 2, 4, 4, 3, 0)),
    (4096, 2561, (2, 2, 4, 4, 3, 0)),
    (1500, 4097, (2, 2, 4, 4, 3, 0)),      # 9
    (3072, 7169, (2, 2, 8, 8, 3, 0)),      # 15
    (2048, 5121, (2, 2, 8, 8, 3, 0)),      # 11
    (2560, 6143, (2, 2, 8, 8, 3, 0)),
    (2048, 7169, (2, 2, 8, 8, 3, 0)),
    (1024, 16897, (2, 2, 8, 8, 3, 0)),     # 34
    (3072, 12289, (2, 2, 8, 8, 3, 0)),
    (2048, 32769, (2, 2, 8, 8, 3, 0)),     # 65 below 3072 rows
    (2048, 65537, (2, 2, 8, 8, 3, 0)),
    (4096, 24577, (2, 2, 8, 8, 3, 0)),     # 49
    (4096, 32769, (2, 4, 8, 8, 3, 0)),     # 65 from 3072 rows
    # below 1024 rows: eight slices for 6..48 steps, one row beyond
    (1000, 7169, (2, 2, 8, 8, 3, 0)),
    (768, 4097, (2, 2, 8, 8, 3, 0)),
    (1000, 16897, (2, 2, 8, 8, 3, 0)),
    (800, 16385, (2, 2, 8, 8, 3, 0)),
    (900, 65537, (1, 4, 8, 8, 3, 0)),
    # at most 4 steps: 1..2 from 8192 rows two rows per trip of the
    # realigning kernel (a_mode 2) in eight-wave workgroups ...
    (8192, 961, (2, 2, 8, 1, 2, 0)),       # 2
    (30000, 719, (2, 2, 8, 1, 2, 0)),
    (65536, 9, (2, 2, 8, 1, 2, 0)),        # 1
    # ... 3, and 4 from 8192 rows, two rows per four-wave workgroup ...
    (16384, 1025, (2, 4, 4, 1, 3, 0)),     # 3
    (8192, 1025, (2, 4, 4, 1, 3, 0)),
    (3072, 1025, (2, 4, 4, 1, 3, 0)),
    (2048, 1025, (2, 4, 4, 1, 3, 0)),
    (768, 1473, (2, 4, 4, 1, 3, 0)),
    (65536, 1535, (2, 4, 4, 1, 3, 0)),     # 4
    (8193, 1545, (2, 4, 4, 1, 3, 0)),
    # ... the rest one row per four-wave workgroup
    (8191, 961, (1, 2, 4, 1, 3, 0)),       # 2
    (4040, 641, (1, 2, 4, 1, 3, 0)),
    (768, 9, (1, 2, 4, 1, 3, 0)),          # 1
    (6145, 1545, (1, 2, 4, 1, 3, 0)),      # 4
    (4096, 1545, (1, 2, 4, 1, 3, 0)),
    # 5 steps from 12288 rows: the realigning kernel, one row per trip ...
    (12288, 2049, (1, 2, 8, 1, 2, 0)),
    (16384, 2177, (1, 2, 8, 1, 2, 0)),
    # ... below 1024 rows one row per two-wave workgroup ...
    (768, 2049, (1, 4, 2, 1, 1, 0)),
    # ... and below 768 rows the plan of aligned rows
    (512, 5121, (1, 4, 4, 4, 1, 0)),
    (700, 16385, (1, 2, 4, 4, 1, 0)),      # (the small-row plan of aligned rows)
])
def test_plan_misaligned_tiers(n, k, want):
    for dtype in (F16, BF16):
        assert shape_of(plan(n, k, dtype)[1]) == want, (n, k, dtype)
    # a B pointer off 16-byte alignment makes every row misaligned, whatever k
    if k % 8 == 1:
        assert _nst(k - 1) == _nst(k)
        assert shape_of(plan(n, k - 1, F16, aligned=False)[1]) == want, (n, k)


def _takes_shifted_window(n, nst):
    """Whether tier 0 takes n misaligned rows of nst granule steps."""
    if n < 768:
        return False
    if nst <= 2:
        return n < 8192         # from 8192 rows the realigning kernel
    if nst == 5:
        return 1024 <= n < 12288
    return True


def test_plan_shifted_window_only_for_misaligned_rows():
    """The shifted-window kernel serves misaligned rows from 768 of them
    (tier 0), and 16-byte aligned rows only where they start off 128-byte
    lines, from 2048 rows of at least 32 steps."""
    ns = [767, 768, 1023, 1024, 2047, 2048, 4095, 4096, 6143, 6144, 8191, 8192, 12287, 12288,
          65536]
    ks = [9, 511, 1025, 1535, 1537, 2049, 2559, 2561, 4097, 4607, 4609, 8705, 8767, 20415,
          20481, 65537]
    for n, k in itertools.product(ns, ks):
        info = plan(n, k, BF16)[1]
        assert (info.a_mode == 3) == _takes_shifted_window(n, _nst(k)), (n, k, shape_of(info))
        ka = k - k % 8                  # aligned rows of about the same length
        off_lines_long = ka % 64 != 0 and n >= 2048 and (ka + 511) // 512 >= 32
        assert (plan(n, ka, BF16)[1].a_mode == 3) == off_lines_long, (n, ka)
        kl = k - k % 64                 # rows on 128-byte lines: never
        if kl > 0:
            assert plan(n, kl, BF16)[1].a_mode != 3, (n, kl)


@pytest.mark.parametrize("n,k,want", [
    (18432, 7168, (2, 4, 4, 4, 1, 0)),     # the headline: two rows, four slices, 4 waves
    (3072, 65536, (2, 4, 1, 1, 1, 0)),     # >= 96 steps, n >= 1536: no split
    (1536, 49152, (2, 4, 1, 1, 1, 0)),
    (1024, 65536, (2, 4, 8, 8, 1, 0)),     # fewer rows: still split
    (768, 8192, (1, 4, 4, 4, 1, 0)),       # <= 768 rows of 9..16 steps: 4 slices, 4 waves
    (256, 5120, (1, 4, 4, 4, 1, 0)),
    (800, 8192, (1, 4, 8, 4, 1, 0)),       # more rows: the general split
    (1000, 8192, (2, 3, 8, 8, 1, 0)),      # n >= 896, k >= 6144: two rows per wave
    (768, 4096, (1, 8, 4, 1, 1, 0)),       # <= 8 steps: one wave per row
    (1024, 1024, (1, 2, 4, 1, 1, 0)),      # 1-2 steps: two load slots
    (256, 512, (1, 2, 4, 1, 1, 0)),
    (3000, 1000, (2, 2, 4, 1, 1, 0)),      # >= 2048 rows: the short-row rule
    (3000, 1536, (2, 4, 4, 1, 1, 0)),      # 3 steps
    (512, 4096, (1, 2, 4, 4, 1, 0)),       # <= 512 rows of 5..8 steps: 4 slices of two-slot batches
    (256, 2049, (1, 2, 4, 4, 1, 0)),       # (4 full steps and a partial one)
    (640, 4096, (1, 8, 4, 1, 1, 0)),
    (448, 1216, (1, 4, 2, 1, 1, 0)),       # 3..4 steps below 1024 rows: four slots, two waves
    (900, 2048, (1, 4, 2, 1, 1, 0)),
    (64, 1537, (1, 4, 2, 1, 1, 0)),
])
def test_plan_aligned_rules(n, k, want):
    assert shape_of(plan(n, k, F16)[1]) == want, (n, k)


def test_plan_long_misaligned_rows_below_320():
    """Misaligned rows of at least 24 granule steps on 96..319 rows: one row
    over eight slices of the shifted-window kernel; fewer rows, or shorter
    ones, the plans of aligned rows with unaligned loads."""
    for n, k in [(96, 11777), (137, 11919), (237, 79545), (319, 20001)]:
        for dtype in (F16, BF16):
            assert shape_of(plan(n, k, dtype)[1]) == (1, 4, 8, 8, 3, 0), (n, k)
    for n, k in [(95, 11777), (320, 20001), (200, 11201), (96, 11713)]:
        assert plan(n, k, BF16)[1].a_mode != 3, (n, k)


@pytest.mark.parametrize("n,k,want", [
    (4096, 4096, (1, 8, 4, 1, 1, 0)),      # bf16, <= 8 steps: one batch of 8 as for fp16
    (2048, 4096, (1, 8, 4, 1, 1, 0)),
    (1000, 4096, (1, 8, 4, 1, 1, 0)),
])
def test_plan_bf16_short_rows(n, k, want):
    assert shape_of(plan(n, k, BF16)[1]) == want, (n, k)


@pytest.mark.parametrize("n,k,dtype,want", [
    (7168, 16384, F16, (2, 3, 16, 16, 1, 0)),   # 32 steps: sixteen slices of three-slot batches
    (1024, 16384, F16, (2, 3, 16, 16, 1, 0)),
    (28672, 16384, F16, (2, 3, 16, 16, 1, 0)),
    (7168, 16384, BF16, (2, 3, 16, 16, 1, 0)),
    (7168, 18432, F16, (2, 3, 16, 16, 1, 0)),   # 36 steps
])
def test_plan_rows_of_32_steps(n, k, dtype, want):
    assert shape_of(plan(n, k, dtype)[1]) == want, (n, k, dtype)


@pytest.mark.parametrize("n,k,dtype,want", [
    # 12 or 18..24 whole steps on 1536..2560 rows: one row per two-wave workgroup
    (1536, 9216, F16, (1, 4, 2, 1, 1, 0)),
    (2048, 12288, BF16, (1, 4, 2, 1, 1, 0)),
    (2560, 10240, BF16, (1, 4, 2, 1, 1, 0)),
    (2048, 6144, F16, (1, 4, 2, 1, 1, 0)),
    # a partial last step, other step counts, or outside those bounds: the
    # two-row table
    (2048, 11008, BF16, (2, 3, 8, 8, 1, 0)),
    (2048, 6656, BF16, (2, 4, 4, 4, 1, 0)),
    (2048, 14336, BF16, (2, 8, 4, 4, 1, 0)),
    (4096, 12288, F16, (2, 3, 8, 8, 1, 0)),
    (6144, 10240, F16, (2, 5, 4, 4, 1, 0)),
    (1024, 12288, BF16, (2, 3, 8, 8, 1, 0)),
    (3072, 9216, F16, (2, 5, 4, 4, 1, 0)),
])
def test_plan_whole_step_rows_unsplit(n, k, dtype, want):
    assert shape_of(plan(n, k, dtype)[1]) == want, (n, k, dtype)


@pytest.mark.parametrize("k,dtype,want", [
    # two rows per wave on >= 896 rows of 12..64 steps (a partial step
    # counts): (rows, batch, waves, slices) from the measured table
    (6144, BF16, (2, 3, 4, 4)),      # 12 steps: four slices, batches of three
    (6656, BF16, (2, 4, 4, 4)),      # 13
    (7680, F16, (2, 2, 8, 8)),       # 15: eight slices of two
    (8192, BF16, (2, 3, 8, 8)),      # 16: eight slices, batches of three
    (8256, F16, (2, 5, 4, 4)),       # 17..20: four slices, batches of five
    (10240, BF16, (2, 5, 4, 4)),
    (10304, BF16, (2, 3, 8, 8)),     # 21..26: eight slices, batches of three
    (13312, F16, (2, 3, 8, 8)),
    (13376, BF16, (2, 8, 4, 4)),     # 27..29: four slices, eight-slot batches
    (14848, F16, (2, 8, 4, 4)),
    (15360, BF16, (2, 4, 8, 8)),     # 30: eight slices of four
    (15872, BF16, (2, 2, 4, 4)),     # 31: four slices, two-slot batches
    (16384, BF16, (2, 3, 16, 16)),   # 32..52: sixteen slices of three-slot batches
    (16384, F16, (2, 3, 16, 16)),
    (17472, BF16, (2, 3, 16, 16)),
    (21568, F16, (2, 3, 16, 16)),
    (24640, BF16, (2, 3, 16, 16)),
    (26624, F16, (2, 3, 16, 16)),    # 52
    (26688, BF16, (2, 8, 8, 8)),     # 53..64: eight slices of seven or eight
    (32768, F16, (2, 8, 8, 8)),
    (32832, F16, (2, 5, 8, 8)),      # 65..80: five-slot batches
    (40960, BF16, (2, 5, 8, 8)),
    (41024, BF16, (2, 3, 8, 8)),     # 81..96: three-slot batches
    (47104, F16, (2, 3, 8, 8)),
])
def test_plan_two_row_table(k, dtype, want):
    assert k % 64 == 0                    # rows on 128-byte lines (others: below)
    for n in (896, 1000, 3072, 4096, 8192, 18432):
        if k <= 6144 and 2048 <= n < 6144:
            continue                      # the short-row rule (below)
        assert shape_of(plan(n, k, dtype)[1]) == want + (1, 0), (n, k, dtype)


def test_plan_two_row_table_14_steps():
    # 14 steps: four slices of four from 4096 rows, eight slices of two below
    for k in (7168, 7040):
        for dtype in (F16, BF16):
            for n in (896, 1000, 2048, 4095):
                assert shape_of(plan(n, k, dtype)[1]) == (2, 2, 8, 8, 1, 0), (n, k, dtype)
            for n in (4096, 18432, 57344):
                assert shape_of(plan(n, k, dtype)[1]) == (2, 4, 4, 4, 1, 0), (n, k, dtype)


@pytest.mark.parametrize("n,k,dtype,want", [
    # fewer than 896 rows of at least 20 steps: balance the workgroups over
    # the CUs.  320..512 rows: two rows per wave in eight slices, with the
    # batch-filling bands of the two-row plans (at most 256 workgroups)
    (320, 20480, BF16, (2, 2, 8, 8, 1, 0)),      # 40 steps: two-slot batches
    (512, 12288, F16, (2, 4, 8, 8, 1, 0)),       # 24: four-slot
    (448, 28672, BF16, (2, 8, 8, 8, 1, 0)),      # 56: eight-slot
    (512, 14336, BF16, (2, 8, 4, 4, 1, 0)),      # 28: eight-slot, four slices
    (384, 49152, F16, (2, 4, 8, 8, 1, 0)),       # 96: the general split
    (512, 16384, F16, (2, 4, 8, 8, 1, 0)),       # fp16 32 steps: not the 8 x 4 plan here
    # 513..831 rows: one row, four slices of two-slot batches
    (576, 12288, BF16, (1, 2, 4, 4, 1, 0)),
    (704, 40960, F16, (1, 2, 4, 4, 1, 0)),
    (831, 10240, F16, (1, 2, 4, 4, 1, 0)),
    # 832..895 rows: the same with two rows per wave
    (832, 20480, BF16, (2, 2, 4, 4, 1, 0)),
    (895, 12288, F16, (2, 2, 4, 4, 1, 0)),
    # outside: 896 rows and more take the two-row bands, fewer than 320 rows
    # or rows of fewer than 20 steps the one-row rule
    (896, 20480, BF16, (2, 3, 16, 16, 1, 0)),
    (256, 20480, BF16, (1, 4, 16, 16, 1, 0)),
    (512, 8192, BF16, (1, 4, 4, 4, 1, 0)),
    (700, 9216, F16, (1, 4, 8, 8, 1, 0)),
])
def test_plan_fewer_rows_balance(n, k, dtype, want):
    assert shape_of(plan(n, k, dtype)[1]) == want, (n, k, dtype)
    cfg = plan(n, k, dtype)[0]
    rows_per_block = want[0] * want[2] // want[3]
    assert cfg.grid == (n + rows_per_block - 1) // rows_per_block


@pytest.mark.parametrize("n,k,want", [
    (1280, 65536, (1, 4, 2, 1, 1, 0)),      # >= 128 steps on 1280..2048 rows: one row per wave
    (2048, 65536, (1, 4, 2, 1, 1, 0)),
    (1500, 131072, (1, 4, 2, 1, 1, 0)),
    (2049, 65536, (2, 4, 1, 1, 1, 0)),      # more rows: two rows per one-wave workgroup
    (1536, 49152, (2, 4, 1, 1, 1, 0)),      # 96 steps: the same
    (1279, 65536, (2, 4, 8, 8, 1, 0)),      # fewer rows: the split
])
def test_plan_very_long_rows(n, k, want):
    for dtype in (F16, BF16):
        assert shape_of(plan(n, k, dtype)[1]) == want, (n, k, dtype)


@pytest.mark.parametrize("n,k,xwg", [
    (32, 131072, True), (64, 65536, True), (1, 65536, True), (7, 65536, True), (8, 65536, True),
    (65, 65536, True), (127, 65536, True), (128, 65536, True), (192, 65536, True),
    (193, 65536, False), (256, 131071, False),   # more rows of fewer steps: the in-workgroup split
    (193, 131072, True), (256, 131072, True), (256, 262144, True), (257, 262144, False),
    (64, 65535, False), (64, 32768, False),     # shorter rows: the in-workgroup split
    (128, 32768, False), (200, 16384, False),
    (64, 511, False), (64, 16383, False),
])
def test_plan_cross_workgroup_only_for_few_rows(n, k, xwg):
    cfg, info = plan(n, k, BF16)
    assert bool(info.cross_wg) == xwg, (n, k, shape_of(info))
    assert (cfg.kgroups > 1) == xwg
    if xwg:
        nfull = k // 512
        q = cfg.kgroups
        assert 2 <= q <= 64
        if n <= 64 and n * min(64, nfull // 8) <= 512:
            # one row per 4-wave workgroup, two steps per wave, at most 512
            # workgroups (the ticketed combine's grid)
            assert shape_of(info) == (1, 2, 4, 4, 1, 1)
            assert q == min(64, nfull // 8) and cfg.grid == n
        elif n <= 64:
            # one row per 8-wave workgroup, about 512 workgroups
            assert q == max(2, min(64, nfull // 16, 512 // n)) and cfg.grid == n
            assert shape_of(info) == (1, 4 if nfull // (q * 8) >= 4 else 2, 8, 8, 1, 1)
        else:
            # four rows per 4-wave workgroup, each wave one row's share
            assert shape_of(info) == (1, 4, 4, 1, 1, 1)
            assert q == (max(2, min(64, nfull // 8, 2048 // n)) if n <= 96 else min(64, nfull // 8))
            assert cfg.grid == (n + 3) // 4


@pytest.mark.parametrize("n,k,q", [
    (64, 65536, 8),      # 64 x 16 four-wave workgroups would be 1024: 8 eight-wave ones a row
    (1, 65536, 16),      # 128 steps, two a wave over four waves: 16 workgroups
    (32, 65536, 16),     # 512 four-wave workgroups
    (33, 65536, 8),      # 528 would exceed 512: 8-wave workgroups, 512 // 33 = 15 > 128 / 16
    (48, 262144, 10),    # 512 // 48 = 10 eight-wave workgroups a row
    (16, 262144, 32),    # 16 x 64 = 1024: 8-wave, min(512 / 16, 32) = 32
    (8, 1048576, 64),    # 8 x 64 = 512 four-wave workgroups
    (80, 131072, 25),    # four rows a workgroup: 2048 // 80 = 25 (20 x 25 = 500 workgroups)
    (97, 65536, 16),     # from 97 rows, steps / 8
    (256, 262144, 64),
])
def test_plan_cross_workgroup_q(n, k, q):
    cfg, info = plan(n, k, BF16)
    assert info.cross_wg and cfg.kgroups == q, (n, k, cfg.kgroups)


def test_plan_without_workspace_never_splits_across_workgroups():
    """gemv_run and gemv_run_ex bring no scratch: their plan is the
    workspace plan wherever that is not a cross-workgroup split, and the
    in-workgroup split where it is (below 128 rows one row per 8-wave
    workgroup, eight k-slices)."""
    ns = [1, 7, 8, 32, 63, 64, 65, 127, 128, 1000, 18432]
    ks = [0, 511, 16384, 32768, 65535, 65536, 131072, 200000]
    for n, k, dtype in itertools.product(ns, ks, (F16, BF16)):
        cfg0, info0 = plan(n, k, dtype, ws=False)
        cfg1, info1 = plan(n, k, dtype, ws=True)
        assert not info0.cross_wg and cfg0.kgroups == 1
        if info1.cross_wg and n < 128:
            assert shape_of(info0) == (1, 4, 8, 8, 1, 0) and cfg0.grid == n, (n, k)
        elif info1.cross_wg:
            assert info0.splits > 1, (n, k, shape_of(info0))
        else:
            assert (cfg0.variant, cfg0.grid, cfg0.kgroups) == \
                (cfg1.variant, cfg1.grid, cfg1.kgroups), (n, k, dtype)


@pytest.mark.parametrize("n,k", [(127, 65528), (96, 60000), (64, 32768), (32, 16384), (1, 16384), (95, 65535)])
def test_plan_few_rows_split_in_workgroup(n, k):
    # fewer than 128 rows of >= 32 steps, not split across workgroups: one
    # row per 8-wave workgroup, eight k-slices
    cfg, info = plan(n, k, BF16)
    assert shape_of(info) == (1, 4, 8, 8, 1, 0) and cfg.kgroups == 1 and cfg.grid == n


def test_plan_properties_over_a_sweep():
    ns = [1, 7, 63, 64, 127, 128, 255, 256, 1000, 1023, 1024, 2047, 2048, 4095, 4096, 7168, 18433,
          100000]
    ks = [0, 1, 7, 8, 9, 511, 512, 513, 4096, 5000, 6143, 6144, 7000, 7169, 9217, 12289, 16383,
          16384, 16936, 65536, 65537, 65544, 200000]
    for n, k, dtype, aligned in itertools.product(ns, ks, (F16, BF16), (True, False)):
        cfg, info = plan(n, k, dtype, aligned)
        assert 0 <= cfg.variant < mbd.gemv_num_variants()
        assert cfg.grid >= 1 and cfg.kgroups >= 1
        assert info.layout == 0 and info.stages == 0, "an ablation variant was chosen"
        misaligned = k > 0 and (k % 8 != 0 or not aligned)
        off_lines_long = k % 64 != 0 and n >= 2048 and (k + 511) // 512 >= 32
        if info.a_mode == 2:
            assert misaligned
        if info.a_mode == 3:
            assert misaligned or off_lines_long, (n, k, aligned)
        if info.rows == 3:
            # three rows per wave: rows off 128-byte lines, or very long rows
            assert k % 64 != 0 or k > 96 * 512, (n, k)
        if info.cross_wg:
            assert n <= 192 or (n <= 256 and k >= 256 * 512)
        if info.a_mode == 3 and info.rows == 2:
            # pairs of rows 64 apart: 64 pairs per block of 128 rows
            items, per_block = 64 * ((n + 127) // 128), info.waves // info.splits
        else:
            items, per_block = n, info.rows * info.waves // info.splits
        assert cfg.grid <= (items + per_block - 1) // per_block


@pytest.mark.parametrize("args,expect", [
    ((0, 8, 0, 1, MAX_LDS), _lib.GEMV_ERR_INVALID_ARG),
    ((-1, 8, 0, 1, MAX_LDS), _lib.GEMV_ERR_INVALID_ARG),
    ((4, -1, 0, 1, MAX_LDS), _lib.GEMV_ERR_INVALID_ARG),
    ((4, 8, 2, 1, MAX_LDS), _lib.GEMV_ERR_UNSUPPORTED_DTYPE),
    ((4, 8, 0, 1, 0), _lib.GEMV_ERR_INVALID_ARG),
    ((2 ** 30 + 1, 8, 0, 1, MAX_LDS), _lib.GEMV_ERR_INVALID_ARG),
    ((4, 2 ** 27 + 1, 0, 1, MAX_LDS), _lib.GEMV_ERR_INVALID_ARG),
    ((4, 0, 0, 1, MAX_LDS), _lib.GEMV_OK),
])
def test_plan_rejects_bad_arguments(args, expect):
    assert mbd.gemv_plan_config(*args)[0] == expect


def test_plan_null_output():
    lib = _lib.load()
    assert lib.gemv_plan_config(4, 8, 0, 1, MAX_LDS, 0, None) == _lib.GEMV_ERR_INVALID_ARG
    assert lib.gemv_plan_config(4, 8, 0, 1, MAX_LDS, 1, None) == _lib.GEMV_ERR_INVALID_ARG


@pytest.mark.parametrize("k,want", [
    # short rows (<= 12 steps) on >= 2048 rows: a batch no larger than needed
    (256, (2, 2, 4, 1)), (512, (2, 2, 4, 1)),           # 1 step (below 16384 rows)
    (1024, (2, 2, 4, 1)), (984, (2, 2, 4, 1)),          # 2
    (1280, (2, 4, 4, 1)), (1536, (2, 4, 4, 1)),         # 3
    (2048, (1, 4, 4, 1)), (2008, (1, 4, 4, 1)),         # 4
    (2560, (2, 2, 4, 4)), (3072, (2, 2, 4, 4)),         # 5..6: four slices of two
    (3584, (1, 8, 4, 1)), (4096, (1, 8, 4, 1)),         # 7..8: one row, eight slots
    (4608, (2, 3, 4, 4)), (5120, (2, 3, 4, 4)),         # 9..10: four slices of three
])
def test_plan_short_rows(k, want):
    for n in (2048, 3000, 8192, 12287):
        for dtype in (F16, BF16):
            assert shape_of(plan(n, k, dtype)[1]) == want + (1, 0), (n, k, dtype)


def test_plan_short_rows_edges():
    # one step from 12288 rows: four rows per wave
    assert shape_of(plan(12288, 512, BF16)[1]) == (4, 2, 4, 1, 1, 0)
    assert shape_of(plan(12287, 512, BF16)[1]) == (2, 2, 4, 1, 1, 0)
    # one or two steps below 2048 rows: one row, two slots; from 1024 rows
    # three steps and more take the short-row rule
    assert shape_of(plan(2047, 1024, F16)[1]) == (1, 2, 4, 1, 1, 0)
    assert shape_of(plan(1024, 1536, F16)[1]) == (2, 4, 4, 1, 1, 0)
    assert shape_of(plan(1023, 1536, F16)[1]) == (1, 4, 2, 1, 1, 0)    # below: four slots, two waves
    # 11..12 steps: one row of four slots below 6144 rows, four slices of
    # three from there; off 128-byte lines from 6144 rows: three rows, eight
    # slices of two
    assert shape_of(plan(4096, 5632, F16)[1]) == (1, 4, 2, 1, 1, 0)
    assert shape_of(plan(6144, 5632, F16)[1]) == (2, 3, 4, 4, 1, 0)
    assert shape_of(plan(6144, 5000, BF16)[1]) == (3, 2, 8, 8, 1, 0)
    assert shape_of(plan(6143, 5000, BF16)[1]) == (2, 3, 4, 4, 1, 0)
    # below 1024 rows the earlier rules (one row: four slots in two-wave
    # workgroups for 3..4 steps, eight slots for 5..8 steps above 512 rows)
    assert shape_of(plan(1023, 2048, BF16)[1]) == (1, 4, 2, 1, 1, 0)
    assert shape_of(plan(1023, 3072, BF16)[1]) == (1, 8, 4, 1, 1, 0)
    assert shape_of(plan(1024, 2048, BF16)[1]) == (1, 4, 4, 1, 1, 0)


@pytest.mark.parametrize("n,k,want", [
    # rows 16-byte but not 128-byte aligned, >= 6144 of them, 13..48 steps:
    # three rows per wave, eight slices, batches of two up to 16 steps, three
    # beyond
    (6144, 7000, (3, 2, 8, 8, 1, 0)),
    (18432, 7176, (3, 2, 8, 8, 1, 0)),
    (32768, 8200, (3, 3, 8, 8, 1, 0)),
    (18432, 14000, (3, 3, 8, 8, 1, 0)),
    (18432, 15864, (3, 3, 8, 8, 1, 0)),      # 31 steps
    # from 32 steps (and from 2048 rows): the shifted-window kernel, eight
    # slices of two-slot batches (four-slot beyond 64 steps from 3072 rows)
    (8192, 15880, (2, 2, 8, 8, 3, 0)),
    (8192, 24584, (2, 2, 8, 8, 3, 0)),
    (2048, 16936, (2, 2, 8, 8, 3, 0)),
    (8192, 40040, (2, 4, 8, 8, 3, 0)),
    (2047, 16936, (2, 3, 16, 16, 1, 0)),     # fewer rows: the two-row table (34 steps)
    (6143, 7000, (2, 4, 4, 4, 1, 0)),        # fewer rows: the two-row table (14 steps)
    (18432, 7168, (2, 4, 4, 4, 1, 0)),       # rows on 128-byte lines: the table
])
def test_plan_rows_off_lines(n, k, want):
    for dtype in (F16, BF16):
        assert shape_of(plan(n, k, dtype)[1]) == want, (n, k, dtype)
