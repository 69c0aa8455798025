// libgemv.so: the C ABI declared in include/gemv.h, over the kernels of
// gemv_kernel.h.  Host work per call is argument validation, an O(1) choice
// of a precompiled variant and one launch (TileLang Case Studies, Case B.4:
// everything that does not depend on the call happens at construction).
#include "gemv.h"

#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "gemv_kernel.h"
#include "gemv_shift.h"
#include "gemv_staged.h"
#include "handle.h"

using mbd_host::kDead;
using mbd_host::kMagic;
using mbd_host::kMaxVariants;
using mbd_host::kPolNT;

namespace {

using KernelFn = void (*)(const uint16_t*, const uint16_t*, uint16_t*, int, int, int, int, int, int,
                          int, float, const uint16_t*, float*, unsigned*);

struct Variant {
  gemv_variant_info_t info;
  KernelFn fn[2];   // [dtype]
};

constexpr int kLanesPerWave = 64;

#define MBD_VARIANT_X(R, U, W, S, AM, POL, X)                                       \
  {{R, U, W, S, AM, POL, X, 0},                                                     \
   {&mbd::gemv_kernel<mbd::DT_F16, R, U, W, S, AM, POL, X>,                         \
    &mbd::gemv_kernel<mbd::DT_BF16, R, U, W, S, AM, POL, X>}}
#define MBD_VARIANT(R, U, W, S, AM, POL) MBD_VARIANT_X(R, U, W, S, AM, POL, false)
#define MBD_REALIGN_R(R, U, W, POL)                                                 \
  {{R, U, W, 1, mbd::A_LDS_SHIFTED, POL, 0, 0},                                     \
   {&mbd::gemv_realign_kernel<mbd::DT_F16, R, U, W, POL>,                           \
    &mbd::gemv_realign_kernel<mbd::DT_BF16, R, U, W, POL>}}
#define MBD_REALIGN(U, W, POL) MBD_REALIGN_R(1, U, W, POL)
#define MBD_SHIFT(R, U, W, S)                                                       \
  {{R, U, W, S, mbd::A_SHIFTED, kPolNT, 0, 0},                                      \
   {&mbd::gemv_shift_kernel<mbd::DT_F16, R, U, W, S, kPolNT>,                       \
    &mbd::gemv_shift_kernel<mbd::DT_BF16, R, U, W, S, kPolNT>}}
#define MBD_STAGED(R, U, W, P, LDS)                                                 \
  {{R, U, W, 1, mbd::A_CACHED, kPolNT, 0, 0, P, LDS},                               \
   {&mbd::gemv_staged_kernel<mbd::DT_F16, R, U, W, P, LDS, kPolNT>,                 \
    &mbd::gemv_staged_kernel<mbd::DT_BF16, R, U, W, P, LDS, kPolNT>}}

// The compiled variants: (rows R, unroll U, waves W, splits S, a mode, B
// cache policy).  Row variants (S == 1) give each wave R whole rows; split
// variants let S waves of a workgroup share R rows for small n.
#define NT kPolNT
#define LDS mbd::A_LDS
#define CCH mbd::A_CACHED
const Variant kVariants[] = {
    // 0..11: row variants, a through the caches, non-temporal B
    MBD_VARIANT(1, 2, 4, 1, CCH, NT), MBD_VARIANT(1, 4, 4, 1, CCH, NT),
    MBD_VARIANT(1, 8, 4, 1, CCH, NT), MBD_VARIANT(2, 2, 4, 1, CCH, NT),
    MBD_VARIANT(2, 4, 4, 1, CCH, NT), MBD_VARIANT(2, 8, 4, 1, CCH, NT),
    MBD_VARIANT(4, 2, 4, 1, CCH, NT), MBD_VARIANT(4, 4, 4, 1, CCH, NT),
    MBD_VARIANT(1, 4, 8, 1, CCH, NT), MBD_VARIANT(2, 4, 8, 1, CCH, NT),
    MBD_VARIANT(1, 4, 2, 1, CCH, NT), MBD_VARIANT(2, 4, 1, 1, CCH, NT),
    // 12..19: row variants, a staged in LDS, non-temporal B
    MBD_VARIANT(1, 4, 4, 1, LDS, NT), MBD_VARIANT(1, 8, 4, 1, LDS, NT),
    MBD_VARIANT(2, 2, 4, 1, LDS, NT), MBD_VARIANT(2, 4, 4, 1, LDS, NT),
    MBD_VARIANT(4, 2, 4, 1, LDS, NT), MBD_VARIANT(4, 4, 4, 1, LDS, NT),
    MBD_VARIANT(2, 4, 8, 1, LDS, NT), MBD_VARIANT(4, 2, 8, 1, LDS, NT),
    // 20..31: split variants, a through the caches, non-temporal B
    MBD_VARIANT(1, 2, 8, 2, CCH, NT), MBD_VARIANT(1, 4, 8, 2, CCH, NT),
    MBD_VARIANT(2, 4, 8, 2, CCH, NT), MBD_VARIANT(1, 2, 8, 4, CCH, NT),
    MBD_VARIANT(1, 4, 8, 4, CCH, NT), MBD_VARIANT(2, 4, 8, 4, CCH, NT),
    MBD_VARIANT(1, 2, 8, 8, CCH, NT), MBD_VARIANT(1, 4, 8, 8, CCH, NT),
    MBD_VARIANT(2, 4, 8, 8, CCH, NT), MBD_VARIANT(1, 4, 4, 4, CCH, NT),
    MBD_VARIANT(1, 2, 16, 16, CCH, NT), MBD_VARIANT(1, 4, 16, 16, CCH, NT),
    // 32..37: split across workgroups as well (few rows of many steps: 33
    // up to 96 rows, 37 up to 256)
    MBD_VARIANT_X(1, 4, 8, 8, CCH, NT, true), MBD_VARIANT_X(1, 2, 8, 8, CCH, NT, true),
    MBD_VARIANT_X(1, 4, 4, 4, CCH, NT, true), MBD_VARIANT_X(1, 2, 4, 4, CCH, NT, true),
    MBD_VARIANT_X(2, 4, 8, 4, CCH, NT, true), MBD_VARIANT_X(1, 4, 4, 1, CCH, NT, true),
    // 38..41: rows not 16-byte aligned: line-aligned B granules, a realigned in LDS
    MBD_REALIGN(4, 4, NT), MBD_REALIGN(2, 4, NT), MBD_REALIGN(4, 8, NT), MBD_REALIGN(8, 4, NT),
    // 42: one row per lane, one element per step (the uncoalesced layout; study only)
    {{kLanesPerWave, 1, 4, 1, mbd::A_CACHED, 0, 0, 1},
     {&mbd::gemv_rowlane_kernel<mbd::DT_F16, 4>, &mbd::gemv_rowlane_kernel<mbd::DT_BF16, 4>}},
    // 43..47: more realigning shapes (two rows per trip in 44..46)
    MBD_REALIGN(8, 8, NT), MBD_REALIGN_R(2, 4, 4, NT), MBD_REALIGN_R(2, 4, 8, NT),
    MBD_REALIGN_R(2, 2, 8, NT),
    MBD_REALIGN(2, 8, NT),
    // 48..52: B prefetched P items ahead through register slots (P = 1: none)
    MBD_STAGED(2, 2, 8, 1, false), MBD_STAGED(2, 2, 8, 2, false), MBD_STAGED(2, 2, 8, 3, false),
    MBD_STAGED(2, 4, 8, 2, false), MBD_STAGED(1, 4, 8, 2, false),
    // 53..56: the same through LDS slots filled by buffer loads into LDS
    MBD_STAGED(2, 2, 8, 1, true), MBD_STAGED(2, 2, 8, 2, true), MBD_STAGED(2, 2, 8, 3, true),
    MBD_STAGED(1, 4, 4, 2, true),
    // 57..58: realigning, 16 waves per workgroup (half the staging of a per wave)
    MBD_REALIGN(4, 16, NT), MBD_REALIGN(2, 16, NT),
    // 59: two rows, four slices, one row group per (4-wave) workgroup
    MBD_VARIANT(2, 4, 4, 4, CCH, NT),
    // 60..66: rows not 16-byte aligned: line-aligned B granules, a read
    // through the caches at each row's shift (no staging); two-row shapes
    // take rows 64 apart, which share the shift
    MBD_SHIFT(1, 2, 4, 1), MBD_SHIFT(2, 4, 4, 1), MBD_SHIFT(1, 4, 4, 4), MBD_SHIFT(2, 4, 4, 4),
    MBD_SHIFT(2, 4, 8, 8), MBD_SHIFT(1, 4, 8, 8), MBD_SHIFT(2, 4, 2, 2),
    // 67..69: two rows per wave whose k-slices fill their batch of loads:
    // two steps per batch in eight slices, eight in four or eight slices
    MBD_VARIANT(2, 2, 8, 8, CCH, NT), MBD_VARIANT(2, 8, 4, 4, CCH, NT), MBD_VARIANT(2, 8, 8, 8, CCH, NT),
    // 70..71: the shifted-window kernel with two-slot batches (61 VGPRs, where
    // its four-slot two-row forms take 88: 8 waves per SIMD instead of 5)
    MBD_SHIFT(2, 2, 4, 4), MBD_SHIFT(2, 2, 8, 8),
    // 72..73: two-slot batches over four slices, one or two rows per wave
    // (the plans of 513..895 rows of long rows)
    MBD_VARIANT(1, 2, 4, 4, CCH, NT), MBD_VARIANT(2, 2, 4, 4, CCH, NT),
    // 74..78: two rows per wave, batches of 3, 5 or 6 steps over four or
    // eight slices
    MBD_VARIANT(2, 3, 8, 8, CCH, NT), MBD_VARIANT(2, 6, 8, 8, CCH, NT),
    MBD_VARIANT(2, 5, 4, 4, CCH, NT), MBD_VARIANT(2, 3, 4, 4, CCH, NT),
    MBD_VARIANT(2, 5, 8, 8, CCH, NT),
    // 79..80: three rows per wave, eight slices of two- or three-slot batches
    // (rows that start off 128-byte lines)
    MBD_VARIANT(3, 2, 8, 8, CCH, NT), MBD_VARIANT(3, 3, 8, 8, CCH, NT),
    // 81: two rows, sixteen slices of three-slot batches (rows of 32..52 steps)
    MBD_VARIANT(2, 3, 16, 16, CCH, NT),
};
#undef NT
#undef LDS
#undef CCH
constexpr int kNumVariants = (int)(sizeof(kVariants) / sizeof(kVariants[0]));

size_t lds_bytes(const gemv_variant_info_t& v, int64_t k) {
  const int64_t nsteps = (k + mbd::kStep - 1) / mbd::kStep;
  if (v.a_mode == mbd::A_LDS_SHIFTED) {   // two shifted, zero-padded copies of a
    const int64_t steps =
        ((k + mbd::kLine - 1 + mbd::kStep - 1) / mbd::kStep + v.unroll - 1) / v.unroll * v.unroll;
    const int64_t len = mbd::kPadA + steps * mbd::kStep + 8;
    return (size_t)(4 * len);
  }
  if (v.stages > 0)   // pipelined B: LDS slots of every wave, or none
    return v.b_lds ? (size_t)v.waves * v.stages * v.unroll * v.rows * mbd::kStepBytes : 0;
  size_t b = 0;
  if (v.a_mode == mbd::A_LDS) b += (size_t)nsteps * mbd::kStepBytes;   // (A_SHIFTED: no copy of a)
  if (v.splits > 1) b += (size_t)v.waves * v.rows * sizeof(float);
  return b;
}

// Rows a workgroup covers per trip (layout 1: rows == 64, one per lane).
int64_t rows_per_block(const gemv_variant_info_t& v) { return (int64_t)(v.waves / v.splits) * v.rows; }

// The items dealt out to the row units: rows, or for the shifted-window
// kernel's two-row variants pair slots (slot p: rows 128 (p / 64) + p % 64
// and 64 rows later), 64 per 128 rows or part of them.
bool pairs_rows(const gemv_variant_info_t& v) { return v.a_mode == mbd::A_SHIFTED && v.rows == 2; }
int64_t row_items(const gemv_variant_info_t& v, int64_t n) { return pairs_rows(v) ? 64 * ((n + 127) / 128) : n; }
int64_t items_per_block(const gemv_variant_info_t& v) {
  return pairs_rows(v) ? (int64_t)(v.waves / v.splits) : rows_per_block(v);
}

// Caller scratch of the cross-workgroup split (gemv_run_ws), laid out as
// the kernel header states: the arrival counters, each in a 128-byte line of
// its own, one bank per k-group count; then the fp32 partial sums, row by row
// (k-group q of row i at i * xwg_row_stride(Q) + q).
using mbd::kWsCounterBytes;
using mbd::kWsFloats;
using mbd::kXwgMaxQ;
using mbd::kXwgRanges;
constexpr int64_t kTicketMaxWorkgroups = 512;
static_assert(kWsCounterBytes + kWsFloats * sizeof(float) + mbd::kWsTicketBytes ==
                  (size_t)GEMV_WORKSPACE_BYTES,
              "the header's workspace size is the layout's");

// Shape of a launch plan: a variant shape plus a workgroup count (0 = one
// row range per wave, i.e. no persistence).
struct Plan {
  int rows, unroll, waves, splits, a_mode, policy;
  int grid;
  int kgroups;   // > 1: a cross-workgroup variant with this many k-groups
  int wg_cap = 0;   // > 0: at most this many workgroups per CU (padding their LDS)
};

// Workgroups per CU for the four-wave row plans that measured faster with
// fewer of them resident, on grids of at least four full rounds at that cap:
// two rows x four slices of four slots (the headline's plan; 7 per CU by its
// registers) or of three slots, one row of four slots.  With fewer waves per
// SIMD a load waits behind less of the queue, and the launch's last
// workgroups drain sooner; on smaller grids the cap only idles slots.
// (Graph replay, the same plan with and without its LDS padded to cap the
// workgroups per CU at 5: (18432, 7168) fp16 37.76 -> 37.46 us, bf16 37.81 ->
// 37.65, (57344, 7168) fp16 112.62 -> 111.88, (16384, 5120) bf16 24.80 ->
// 24.63, (32768, 5120) bf16 46.96 -> 46.55, (32768, 2048) bf16 20.01 ->
// 19.90, (12288, 7168) fp16 (4.8 rounds) 26.21 -> 26.08, (24576, 7168) fp16
// 49.82 -> 49.32; with grids of 1.6-3.2 rounds 1.6-1.8% slower, e.g. (4096,
// 7168) bf16 10.60 -> 10.79; one row of eight slots: within 0.25%; at 4 per
// CU the headline took 37.45-37.53, at 3 38.20, and two rows of three slots
// lost 4-7% at 4; eight-wave plans: no gain.)
constexpr int kCapRounds = 4;
int wg_cap_of(const Plan& p) {
  if (p.a_mode != mbd::A_CACHED || p.kgroups > 1 || p.waves != 4 || p.grid != 0) return 0;
  if (p.rows == 2 && p.splits == 4 && (p.unroll == 4 || p.unroll == 3)) return 5;
  if (p.rows == 1 && p.splits == 1 && p.unroll == 4) return 5;
  return 0;
}

int find_variant(const Plan& p) {
  const int x = p.kgroups > 1 ? 1 : 0;
  for (int v = 0; v < kNumVariants; ++v) {
    const gemv_variant_info_t& i = kVariants[v].info;
    if (i.rows == p.rows && i.unroll == p.unroll && i.waves == p.waves && i.splits == p.splits &&
        i.a_mode == p.a_mode && i.b_policy == p.policy && i.cross_wg == x && i.layout == 0 &&
        i.stages == 0)
      return v;
  }
  return -1;
}

// The automatic plan, O(1) per call, in this order:
//  0. rows that do not start on 16-byte boundaries, at least 768 of them,
//     and rows that start on 16-byte but not on 128-byte lines, at least 2048
//     of them, of at least 32 steps:
//     the shifted-window kernel (B in line-aligned granules, a read at each
//     row's shift through the caches; two-row shapes pair rows 64 apart),
//     mostly in its two-slot forms (61 VGPRs: 8 waves per SIMD, where the
//     four-slot two-row forms take 88: 5), by the rows' granule steps
//     nst = ceil((k + 63) / 512) and row count.  From 6144 rows: two rows x
//     four slices of two-slot batches up to 31 steps (four-slot batches at
//     14..15 steps from 12288 rows), eight slices for 32..64 steps, eight
//     slices of four-slot batches beyond; 1024..6143 rows: four slices up to
//     9 steps, eight for 10..64 (and beyond 64 below 3072 rows; four-slot
//     batches above); below 1024 rows: eight slices for 6..48 steps, one row
//     x eight slices beyond.  Rows of at most 4 steps: at most 2 from 8192
//     rows in the realigning kernel (aligned granules of B from each row's
//     128-byte line, a staged twice in LDS), two rows per trip of an
//     eight-wave workgroup; 3, and 4 from 8192 rows, two rows per four-wave
//     workgroup of the shifted-window kernel; the rest one row per wave of
//     it.  Rows of 5 steps from 12288 rows, and below 1024 rows, go to 1.
//     (Graph-replayed sweeps over 78 misaligned shapes, n = 768..49152,
//     k = 1025..32769, every candidate shape of the three misaligned kernels
//     on full and persistent grids: 1.1% off the best compiled plan on
//     average, 3.1% at the 90th percentile, where the previous tier 0, built
//     on the four-slot forms, was 3.5% and 9.6%, up to 16%.  Rows of at most
//     4 steps from 48 shapes drawn at random, below.)
//  1. the misaligned rows tier 0 leaves, of 5 granule steps: from 12288
//     rows the realigning kernel in eight-wave workgroups, two steps per
//     batch, on a persistent grid of 1024 (8192 waves: 32 per CU, one full
//     occupancy); on 768..1023 rows one row per wave in two-wave workgroups
//     with unaligned 16-byte loads.  (Graph replay over random misaligned
//     shapes: within 0.7% of the best compiled plan on the two of 28747 and
//     30066 rows; 2.6% off on average over n = 768..2560, k = 2049..6143
//     bf16 for the two-wave plan.)
//  2. too few rows to give the GPU 2048 waves even with 16 waves per row
//     (n < 128), with rows of at least 32 steps: one row per 8-wave
//     workgroup, eight k-slices.  With a workspace, up to 192 rows of at
//     least 128 steps (256 of at least 256) split k across Q workgroups as
//     well (below).
//  3. (misaligned rows below 768 of them take 4 as it stands, with
//     unaligned 16-byte loads)
//  4. otherwise a through the caches and non-temporal B loads, each wave's
//     (or slice's) steps in a batch of loads no larger than they need, in
//     this order: very long rows (unsplit on 1280..4095 rows, three rows over
//     eight slices from 4096 rows); rows of 12 or 18..24 whole steps on
//     1536..2560 rows unsplit; fewer than 896 rows of at least 20 steps
//     balanced over the CUs; rows off 128-byte lines from 6144 rows of 13..31
//     steps three rows per wave; rows of at most 12 steps from 1024 rows by
//     their step count; two rows per wave on at least 896 rows of 12..96
//     steps from a table by step count; the rest (fewer rows) the earlier
//     bands and the general split -- a row of at most 8 steps to one wave,
//     longer rows split along k inside a workgroup until every wave has at
//     most 4 steps and further while the grid has fewer than 2048 waves.
//     Each branch states its measurements below; over 180 shapes drawn at
//     random (n = 1024..65536, k = 256..65536) the rule is 1% off the best
//     compiled plan on average, 8% at worst.
Plan rule_plan(int64_t n, int64_t k, gemv_dtype_t dtype, size_t max_lds, bool b_aligned,
               bool with_ws) {
  const int64_t nfull0 = k / mbd::kStep;
  const bool misaligned = k > 0 && (k % 8 != 0 || !b_aligned);
  // rows 16-byte aligned that start off 128-byte lines (k not a multiple of
  // 64), at least 2048 of them, of at least 32 steps: the shifted-window
  // kernel of tier 0 too, whose line-aligned granules of B suit them (graph
  // replay, n = 2048..18432, k = 16936..40040 bf16: the best compiled plan
  // or within 2.1%, where the two-row plans were 3-8% behind)
  const bool off_lines = k > 0 && k % mbd::kLine != 0;
  const bool long_off_lines = off_lines && !misaligned && n >= 2048 && (k + mbd::kStep - 1) / mbd::kStep >= 32;
  // 0.
  if ((misaligned && n >= 768) || long_off_lines) {
    const int64_t nst = (k + mbd::kLine - 1 + mbd::kStep - 1) / mbd::kStep;
    auto shift = [](int R, int U, int W, int S) {
      return Plan{R, U, W, S, mbd::A_SHIFTED, kPolNT, 0, 1};
    };
    // misaligned rows of at most four granule steps (k < 1986): at most two
    // from 8192 rows in the realigning kernel, two rows per trip, eight-wave
    // workgroups; three, and four from 8192 rows, two rows per four-wave
    // workgroup of the shifted-window kernel; the rest one row per wave of
    // it.  (Graph replay over 48 shapes drawn at random, n = 768..60051, k =
    // 411..1905, fp16 and bf16: at most two steps from 8192 rows the best
    // compiled plan on all 16, below the best or within 8%; three steps
    // within 6%; four the best from 16136 rows and below 4096.  The tiers
    // below, from an earlier kernel, were 13-47% behind at most two steps.)
    if (misaligned && nst <= 4) {
      const Plan pr = {2, 2, 8, 1, mbd::A_LDS_SHIFTED, kPolNT, 0, 1};
      if (nst <= 2 && n >= 8192 && lds_bytes(kVariants[find_variant(pr)].info, k) <= max_lds) return pr;
      if (nst == 3 || (nst == 4 && n >= 8192)) return shift(2, 4, 4, 1);
      return shift(1, 2, 4, 1);
    }
    if (n < 1024) {
      if (nst >= 6 && nst <= 48) return shift(2, 2, 8, 8);
      if (nst > 48) return shift(1, 4, 8, 8);
    } else if (n < 6144) {
      if (nst >= 4 && nst <= 9) return shift(2, 2, 4, 4);
      if (nst >= 10 && nst <= 64) return shift(2, 2, 8, 8);
      if (nst > 64) return n < 3072 ? shift(2, 2, 8, 8) : shift(2, 4, 8, 8);
    } else if (nst >= 4 && !(nst <= 5 && n >= 12288)) {
      if (nst <= 15 && nst >= 14 && n >= 12288) return shift(2, 4, 4, 4);
      if (nst <= 31) return shift(2, 2, 4, 4);
      if (nst <= 64) return shift(2, 2, 8, 8);
      return shift(2, 4, 8, 8);
    }
  }
  // 1. the misaligned rows tier 0 leaves, of five granule steps: from 12288
  // rows the realigning kernel on a persistent grid of 1024 eight-wave
  // workgroups (8192 waves: 32 per CU), 768..1023 rows one row per wave in
  // two-wave workgroups with unaligned 16-byte loads.
  if (misaligned && n >= 12288) {
    const Plan pr = {1, 2, 8, 1, mbd::A_LDS_SHIFTED, kPolNT, 1024, 1};
    if (lds_bytes(kVariants[find_variant(pr)].info, k) <= max_lds) return pr;
  }
  if (misaligned && n >= 768 && n < 1024) return Plan{1, 4, 2, 1, mbd::A_CACHED, kPolNT, 0, 1};
  // 2. k split over Q workgroups as well, for few rows of many steps -- only
  // with caller scratch for the partials and counters (gemv_run_ws);
  // without it, the in-workgroup split below.  Grids of about 512
  // workgroups (two per CU) measured best, and up to 512 the ticketed
  // combine (one row per workgroup of one row group) takes two round trips
  // off the combine.  So, two steps per wave at most 512 workgroups where
  // that fits: up to 64 rows, one row per 4-wave workgroup, Q = steps / 8,
  // if n Q <= 512; else one row per 8-wave workgroup, Q = 512 / n (at most
  // steps / 16), two load slots per wave, four when a wave has four steps or
  // more.  65..96 rows: four rows per 4-wave workgroup, each wave one row's
  // share of k, Q = 2048 / n (512 workgroups; at most steps / 8).  97..192
  // rows, and up to 256 rows of >= 256 steps: the same shape, Q = steps / 8.
  // Q at most 64.  (Graph replay, every cross-workgroup variant x Q and the
  // in-workgroup plans: 2.7% off the best compiled plan on average over 22
  // shapes of 1..96 rows, 7.4% at worst; 2.5% and 5.9% over 11 shapes of
  // 128..256 rows.  The combine's counters and partials sit in lines of
  // their own, so many workgroups per row do not queue on shared lines.)
  if (with_ws && nfull0 >= 128 && n <= 256) {
    auto fits = [&](int64_t Q) { return n * mbd::xwg_row_stride(Q) <= (int64_t)kWsFloats; };
    if (n <= 64) {
      int64_t Q = nfull0 / 8;
      if (Q > kXwgMaxQ) Q = kXwgMaxQ;
      if (n * Q <= kTicketMaxWorkgroups && fits(Q)) return Plan{1, 2, 4, 4, mbd::A_CACHED, kPolNT, 0, (int)Q};
      Q = nfull0 / 16;
      if (Q > kXwgMaxQ) Q = kXwgMaxQ;
      if (Q > kTicketMaxWorkgroups / n) Q = kTicketMaxWorkgroups / n;
      if (Q < 2) Q = 2;
      const int U = nfull0 / (Q * 8) >= 4 ? 4 : 2;
      if (fits(Q)) return Plan{1, U, 8, 8, mbd::A_CACHED, kPolNT, 0, (int)Q};
    } else if (n <= 96) {
      int64_t Q = nfull0 / 8;
      if (Q > kXwgMaxQ) Q = kXwgMaxQ;
      if (Q > 4 * kTicketMaxWorkgroups / n) Q = 4 * kTicketMaxWorkgroups / n;
      if (Q < 2) Q = 2;
      if (fits(Q)) return Plan{1, 4, 4, 1, mbd::A_CACHED, kPolNT, 0, (int)Q};
    } else if (n <= 192 || nfull0 >= 256) {
      int64_t Q = nfull0 / 8;
      if (Q > kXwgMaxQ) Q = kXwgMaxQ;
      if (fits(Q)) return Plan{1, 4, 4, 1, mbd::A_CACHED, kPolNT, 0, (int)Q};
    }
  }
  // misaligned rows of at least 24 granule steps on 96..319 rows (where the
  // split across workgroups above does not take them): the shifted-window
  // kernel, one row over eight k-slices of four-slot batches (graph replay,
  // random shapes of 137..237 rows, k = 11919..79545: the best compiled plan
  // on all three, where the unaligned loads of the plans below were 6-22%
  // behind; from 49 to 81 rows it was 0-4% either way)
  if (misaligned && n >= 96 && n < 320 && (k + mbd::kLine - 1 + mbd::kStep - 1) / mbd::kStep >= 24)
    return Plan{1, 4, 8, 8, mbd::A_SHIFTED, kPolNT, 0, 1};
  if (n < 128 && nfull0 >= 32) return Plan{1, 4, 8, 8, mbd::A_CACHED, kPolNT, 0, 1};
  // 4.
  const int64_t nfull = k / mbd::kStep;
  // rows of >= 128 steps (k >= 64K) on 1280..2048 rows: one row per wave in
  // two-wave workgroups, no split (graph replay, five shapes in fp16 and
  // bf16: the best compiled plan, 0.9-13.5% ahead of the plans below)
  if (nfull >= 128 && n >= 1280 && n <= 2048) return Plan{1, 4, 2, 1, mbd::A_CACHED, kPolNT, 0, 1};
  // very long rows (k >= 48K) on 1536..4095 rows: no split, two rows per
  // one-wave workgroup (the split's per-slice combine no longer pays); rows
  // of more than 96 steps from 4096 rows: three rows per wave over eight
  // k-slices of three-slot batches (graph replay, n = 4096..8192, k = 51904
  // .. 98304: the best compiled plan or within 1%, where the unsplit plan was
  // up to 14% behind)
  if (nfull >= 96 && n >= 1536 && n < 4096) return Plan{2, 4, 1, 1, mbd::A_CACHED, kPolNT, 0, 1};
  if (k > 96 * mbd::kStep && n >= 4096) return Plan{3, 3, 8, 8, mbd::A_CACHED, kPolNT, 0, 1};
  // rows of 12 or 18..24 whole steps (no partial step) on 1536..2560 rows:
  // no split, one row per wave in two-wave workgroups.  (Graph replay over
  // aligned shapes of n = 1536..8192, k = 6144..16384 with and without a
  // partial step, fp16 and bf16: with the split plans below alone 1.2% off
  // the best compiled plan on average at 2048 rows of 18..24 steps against
  // 1.1% unsplit, and 3-5% behind at 12 steps; from 3072 rows the split
  // plans are as good or better.  With a partial step the unsplit plans lost
  // up to 17%, at k = 11008 on every row count, so they take whole steps
  // only.)
  if (k % mbd::kStep == 0 && (nfull == 12 || (nfull >= 18 && nfull <= 24)) && n >= 1536 &&
      n <= 2560)
    return Plan{1, 4, 2, 1, mbd::A_CACHED, kPolNT, 0, 1};
  const int64_t nsteps = nfull + (k % mbd::kStep != 0 ? 1 : 0);
  // fewer than 896 rows of at least 20 steps: what balances the workgroups
  // over the CUs.  513..831 rows: one row per wave, four slices of two-slot
  // batches (n workgroups, 2-3 per CU); 832..895 rows: the same with two
  // rows per wave (n / 2 workgroups); 320..512 rows: two rows per wave in
  // eight slices, the two-row plan below (at most 256 workgroups, one per
  // CU; fewer than 320 rows would leave too many CUs idle).  (Graph-replayed
  // sweeps over 184 shapes, n = 256..1088, k = 6144..49152, fp16 and bf16:
  // 2.5% off the best compiled plan on average where one row per wave with
  // the general split was 7.7%, up to 34%.)
  if (n > 512 && n < 896 && nsteps >= 20)
    return n < 832 ? Plan{1, 2, 4, 4, mbd::A_CACHED, kPolNT, 0, 1}
                   : Plan{2, 2, 4, 4, mbd::A_CACHED, kPolNT, 0, 1};
  // Rows that start 16-byte but not 128-byte aligned (k not a multiple of
  // 64), at least 6144 of them, of 13..31 steps: three rows per wave, eight
  // k-slices, batches of two (up to 16 steps) or three.  (Graph replay, n =
  // 6144..32768, k = 7000..14000, fp16 and bf16: the best compiled plan or
  // within 3.2%, where the two-row plans below were 2-6% behind; on rows
  // that start on 128-byte lines, and below 6144 rows, three rows per wave
  // do not pay.  Longer ones went to tier 0.)
  if (off_lines && n >= 6144 && nsteps >= 13 && nsteps <= 31)
    return Plan{3, nsteps <= 16 ? 2 : 3, 8, 8, mbd::A_CACHED, kPolNT, 0, 1};
  // Short rows (at most 12 steps) on at least 1024 rows: a batch no larger
  // than the row or the slice needs.  A slot past the wave's steps still
  // issues its B and a loads (out of range, so no memory access, but
  // through the address units all the same), which cost up to 70% where
  // eight-slot batches carried three steps.  1..2 steps: two rows per wave,
  // two slots, from 2048 rows (four rows from 12288 rows of one step), one
  // row below; 3: two rows, four
  // slots; 4: one row, four slots; 5..6: two rows over four slices of two
  // slots; 7..8: one row, eight slots; 9..12: two rows over four slices of
  // three slots -- three rows over eight slices of two on rows off 128-byte
  // lines from 6144 rows, one row of four slots in two-wave workgroups on
  // 2048..6143 rows for 11..12.
  // (Graph replay over 95 shapes, n = 2048..32768, k = 256..6144, fp16 and
  // bf16: 0.8% off the best compiled plan on average, 2.9% at the 90th
  // percentile, where the previous rule -- eight slots for every row of at
  // most 8 steps -- was 12% and 35%, up to 70%.)
  if (n >= 1024 && nsteps <= 12) {
    auto pl = [](int R, int U, int W, int S) { return Plan{R, U, W, S, mbd::A_CACHED, kPolNT, 0, 1}; };
    if (nsteps <= 1 && n >= 2048) return n >= 12288 ? pl(4, 2, 4, 1) : pl(2, 2, 4, 1);
    if (nsteps <= 2 && n >= 2048) return pl(2, 2, 4, 1);
    if (nsteps <= 2) return pl(1, 2, 4, 1);
    if (nsteps <= 3) return pl(2, 4, 4, 1);
    if (nsteps <= 4) return pl(1, 4, 4, 1);
    if (nsteps <= 6) return pl(2, 2, 4, 4);
    if (nsteps <= 8) return pl(1, 8, 4, 1);
    if (off_lines && n >= 6144) return pl(3, 2, 8, 8);
    if (nsteps >= 11 && n >= 2048 && n < 6144) return pl(1, 4, 2, 1);
    return pl(2, 3, 4, 4);
  }
  const int R = ((n >= 896 && k >= 6144) || (n >= 320 && n <= 512 && nsteps >= 20)) ? 2 : 1;
  // rows of one or two steps (k <= 1024): two load slots, not more slots
  // that would only be skipped (measured on MI355X under graph replay:
  // (1024, 1024) 2.75 -> 2.45 us, (256, 512) 2.64 -> 2.35 us)
  if (R == 1 && nsteps <= 2) return Plan{1, 2, 4, 1, mbd::A_CACHED, kPolNT, 0, 1};
  // rows of 3..4 steps: one batch of four slots, two-wave workgroups (graph
  // replay, random shapes of 221..448 rows, k = 1216..1664: the best
  // compiled plan on all four, where one eight-slot batch was 9-11% behind)
  if (R == 1 && nsteps <= 4) return Plan{1, 4, 2, 1, mbd::A_CACHED, kPolNT, 0, 1};
  // up to 512 rows of 5..16 steps, and up to 768 rows of 9..16: four slices
  // in four-wave workgroups, in batches of two up to 8 steps (graph replay,
  // random shapes of 49..432 rows of 5..8 steps: the best compiled plan on
  // all four, where four-slot batches, or one of eight, were 2.6-6.9%
  // behind)
  if (R == 1 && n <= 512 && nsteps >= 5 && nsteps <= 8) return Plan{1, 2, 4, 4, mbd::A_CACHED, kPolNT, 0, 1};
  if (R == 1 && nfull <= 16 && ((n <= 512 && nfull >= 5) || (n <= 768 && nfull > 8)))
    return Plan{1, 4, 4, 4, mbd::A_CACHED, kPolNT, 0, 1};
  // otherwise a row of at most 8 steps goes to one wave, in one batch
  if (R == 1 && nfull <= 8) return Plan{1, 8, 4, 1, mbd::A_CACHED, kPolNT, 0, 1};
  const int smax = R == 1 ? 16 : 8;
  int S = 1;
  while (S < smax && (nfull + S - 1) / S > 4) S *= 2;   // at most 4 steps per wave: one batch
  while (S < smax && ((n + R - 1) / R) * S < 2048 && nfull >= 2 * (2 * S)) S *= 2;
  // Two rows per wave on at least 896 rows of 12..64 steps (nsteps, the
  // partial one included): the k-slices S and the batch U, by the steps.
  // The principle is one batch of loads per slice, U = the slice's share --
  // a batch slot costs registers whether it is used or not (two rows x U = 2
  // / 3 / 4 / 5 / 6 / 8 take 55 / 61 / 73 / 85 / 97 / 121 VGPRs for bf16: 8 /
  // 8 / 6 / 5 / 4 / 4 waves per SIMD) -- with the measured exceptions the
  // table keeps: 25..26 steps take batches of three over eight slices
  // (two batches), 31 steps two-slot batches over four, 14 steps on fewer
  // than 4096 rows eight slices of two, and 32..52 steps sixteen slices of
  // three-slot batches (one or two batches; 16-wave workgroups).  (Graph-
  // replayed sweeps over 266 shapes, n = 1024..16384, k = 6144..32768 with
  // and without a partial step, fp16 and bf16, 16 candidate plans each: 0.4%
  // off the best compiled plan on average, 1.5% at the 90th percentile, 4.2%
  // at worst, where the previous rule, with batches of 2, 4 and 8 only, was
  // 1.6%, 3.5% and 17%; then sixteen slices, on 87 shapes of 24..92 steps:
  // 1.0-2.8% faster than eight at 32..52 steps, (7168, 16384) bf16 35.26 ->
  // 34.49 us.)
  if (R == 2 && n >= 896 && nsteps >= 12 && nsteps <= 64) {
    // {U, S} for nsteps = 12 + i
    static constexpr signed char kTwoRow[53][2] = {
        {3, 4}, {4, 4}, {4, 4}, {2, 8}, {3, 8},                   // 12..16
        {5, 4}, {5, 4}, {5, 4}, {5, 4},                           // 17..20
        {3, 8}, {3, 8}, {3, 8}, {3, 8}, {3, 8}, {3, 8},           // 21..26
        {8, 4}, {8, 4}, {8, 4}, {4, 8}, {2, 4},                   // 27..31
        {3, 16}, {3, 16}, {3, 16}, {3, 16}, {3, 16}, {3, 16},     // 32..37
        {3, 16}, {3, 16}, {3, 16}, {3, 16}, {3, 16}, {3, 16},     // 38..43
        {3, 16}, {3, 16}, {3, 16}, {3, 16}, {3, 16}, {3, 16},     // 44..49
        {3, 16}, {3, 16}, {3, 16},                                // 50..52
        {8, 8}, {8, 8}, {8, 8}, {8, 8},                           // 53..56
        {8, 8}, {8, 8}, {8, 8}, {8, 8}, {8, 8}, {8, 8}, {8, 8}, {8, 8}};  // 57..64
    int U = kTwoRow[nsteps - 12][0], Sl = kTwoRow[nsteps - 12][1];
    if (nsteps == 14 && n < 4096) U = 2, Sl = 8;
    return Plan{2, U, Sl, Sl, mbd::A_CACHED, kPolNT, 0, 1};
  }
  // 65..80 steps on at least 896 rows: eight slices of five-slot batches
  // (two batches each; graph replay, n = 1024..8192, k = 36864..40960: the
  // best compiled plan or within 1.2%, where two-slot batches were 1-5%
  // behind); 81..96 steps: eight slices of three-slot batches
  if (R == 2 && n >= 896 && nsteps >= 65 && nsteps <= 80) return Plan{2, 5, 8, 8, mbd::A_CACHED, kPolNT, 0, 1};
  if (R == 2 && n >= 896 && nsteps >= 81 && nsteps <= 96) return Plan{2, 3, 8, 8, mbd::A_CACHED, kPolNT, 0, 1};
  // Two rows per wave otherwise (320..895 rows, or more than 64 steps): give
  // each k-slice a share that fills its batch of loads -- eight slots for
  // shares of 7-8 steps (25..28 steps over four slices, 49..64 over eight),
  // four for shares of 3-4 (21..24 and 29..34 steps over eight), and two --
  // several batches, at full occupancy -- for the shares in between (15..20
  // steps, 35..48, 65..80; fp16 keeps four slices of four up to 16 steps).
  if (R == 2 && nsteps >= 15 && nsteps <= 80 && !(dtype == GEMV_F16 && nsteps <= 16)) {
    auto two = [](int U, int Sl) { return Plan{2, U, Sl, Sl, mbd::A_CACHED, kPolNT, 0, 1}; };
    if (nsteps <= 20) return two(2, 8);
    if (nsteps >= 25 && nsteps <= 28) return two(8, 4);
    if (nsteps >= 35 && nsteps <= 48) return two(2, 8);
    if (nsteps >= 49 && nsteps <= 64) return two(8, 8);
    if (nsteps >= 65) return two(2, 8);
  }
  const int W = R == 2 ? S : (S == 1 ? 4 : (S <= 8 ? 8 : 16));
  return Plan{R, 4, W, S, mbd::A_CACHED, kPolNT, 0, 1};
}

}  // namespace

static_assert(kNumVariants <= kMaxVariants, "the handle keeps per-variant LDS for kMaxVariants");

// The scratch of gemv_run_noalloc, for callers that cannot allocate: the
// layout of a gemv_run_ws workspace (counters, then partials), one copy per
// GPU, held until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: its device address on each GPU comes from
// hipGetSymbolAddress, once per device, and only that address is used.
static __device__ __align__(256) unsigned char scratch[GEMV_WORKSPACE_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];   // this GPU's copy of `scratch`, once resolved
}  // namespace

// With device `dev` current: the device address of its copy of `scratch`,
// resolved and zero-filled on the first call for that device.
static gemv_status_t scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return GEMV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GEMV_ERR_HIP;
    // the arrival counters start at zero (every completed call leaves them so)
    if (hipMemset(p, 0, (size_t)GEMV_WORKSPACE_BYTES) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess)
      return GEMV_ERR_HIP;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return GEMV_OK;
}

extern "C" const char* gemv_status_string(gemv_status_t s) {
  switch (s) {
    case GEMV_OK: return "GEMV_OK";
    case GEMV_ERR_NULL_HANDLE: return "GEMV_ERR_NULL_HANDLE";
    case GEMV_ERR_INVALID_ARG: return "GEMV_ERR_INVALID_ARG";
    case GEMV_ERR_UNSUPPORTED_DTYPE: return "GEMV_ERR_UNSUPPORTED_DTYPE";
    case GEMV_ERR_MISALIGNED: return "GEMV_ERR_MISALIGNED";
    case GEMV_ERR_ALIASING: return "GEMV_ERR_ALIASING";
    case GEMV_ERR_TOO_LARGE: return "GEMV_ERR_TOO_LARGE";
    case GEMV_ERR_WRONG_DEVICE: return "GEMV_ERR_WRONG_DEVICE";
    case GEMV_ERR_UNSUPPORTED: return "GEMV_ERR_UNSUPPORTED";
    case GEMV_ERR_HIP: return "GEMV_ERR_HIP";
    case GEMV_ERR_OOM: return "GEMV_ERR_OOM";
  }
  return "GEMV_ERR_UNKNOWN";
}

extern "C" int32_t gemv_num_variants(void) { return kNumVariants; }

extern "C" gemv_status_t gemv_variant_info(int32_t v, gemv_variant_info_t* info) {
  if (!info || v < 0 || v >= kNumVariants) return GEMV_ERR_INVALID_ARG;
  *info = kVariants[v].info;
  return GEMV_OK;
}

// Every check of gemv_run that needs neither the handle nor the GPU.
extern "C" gemv_status_t gemv_check_args(const void* B, const void* a, const void* c, int64_t n,
                                         int64_t k, gemv_dtype_t dtype) {
  return gemv_check_args_ex(B, a, c, n, k, dtype, nullptr);
}

extern "C" gemv_status_t gemv_check_args_ex(const void* B, const void* a, const void* c,
                                            int64_t n, int64_t k, gemv_dtype_t dtype,
                                            const gemv_epilogue_t* ep) {
  if (dtype != GEMV_F16 && dtype != GEMV_BF16) return GEMV_ERR_UNSUPPORTED_DTYPE;
  if (n < 0 || k < 0) return GEMV_ERR_INVALID_ARG;
  if (n == 0) return GEMV_OK;
  // B and a are never read when k == 0 (an empty tensor may hand over NULL)
  if (!c || (k > 0 && (!B || !a))) return GEMV_ERR_INVALID_ARG;
  if (((uintptr_t)c | (k > 0 ? ((uintptr_t)B | (uintptr_t)a) : 0u)) & 1u) return GEMV_ERR_MISALIGNED;
  if (n > GEMV_MAX_N || k > GEMV_MAX_K) return GEMV_ERR_TOO_LARGE;
  const uintptr_t c0 = (uintptr_t)c, c1 = c0 + (uintptr_t)n * 2u;
  if (k > 0) {
    const uintptr_t b0 = (uintptr_t)B, b1 = b0 + (uintptr_t)n * (uintptr_t)k * 2u;
    const uintptr_t a0 = (uintptr_t)a, a1 = a0 + (uintptr_t)k * 2u;
    if ((c0 < b1 && b0 < c1) || (c0 < a1 && a0 < c1)) return GEMV_ERR_ALIASING;
  }
  if (ep && ep->bias) {
    const uintptr_t z0 = (uintptr_t)ep->bias, z1 = z0 + (uintptr_t)n * 2u;
    if (z0 & 1u) return GEMV_ERR_MISALIGNED;
    // bias may be c itself (accumulate in place), but must not partly overlap it
    if (z0 != c0 && z0 < c1 && c0 < z1) return GEMV_ERR_ALIASING;
  }
  return GEMV_OK;
}

struct Launch {
  int variant;
  int grid;      // row ranges (workgroups along x; along y with cross_wg)
  int kgroups;   // k-groups (workgroups along x with cross_wg), 1 otherwise
  int flags;     // kernel flags
  size_t lds;    // dynamic LDS per workgroup
};
static_assert(GEMV_FLAG_XCD_CONTIGUOUS == mbd::kFlagXcdContiguous, "flag values agree");

// The shape-dependent part of a launch: validate a variant, grid and
// k-group count against (n, k) and fill in the grid actually launched and
// the dynamic LDS.  Needs no device.
static gemv_status_t shape_launch(int v, int64_t g, int64_t q, int flags, int64_t n, int64_t k,
                                  bool b_aligned, Launch* L) {
  const gemv_variant_info_t& info = kVariants[v].info;
  // the pipelined variants load whole 16-byte granules of aligned rows only
  if (info.stages > 0 && k > 0 && (k % 8 != 0 || !b_aligned)) return GEMV_ERR_UNSUPPORTED;
  const int64_t rb = items_per_block(info);
  const int64_t nrb = (row_items(info, n) + rb - 1) / rb;   // one row range per wave (or workgroup)
  if (g <= 0 || g > nrb) g = nrb;
  // the kernels walk their row ranges, so a smaller grid is always valid;
  // keep the launch's work-items along x (workgroups x threads, a 32-bit
  // field of the dispatch) at most 2^31
  const int64_t gmax = ((int64_t)1 << 31) / ((int64_t)info.waves * kLanesPerWave);
  if (g > gmax) g = gmax;
  if (info.layout == 1 && (int64_t)kLanesPerWave * k * 2 >= ((int64_t)1 << 32))
    return GEMV_ERR_UNSUPPORTED;   // a wave's 64 rows must fit one buffer descriptor
  if (info.cross_wg) {
    if (q <= 0) q = 4;
    if (q > kXwgMaxQ) return GEMV_ERR_UNSUPPORTED;
    // the scratch holds a line-padded row of q partials per row and one
    // counter per row range (a smaller grid is valid: each workgroup walks
    // a longer row range)
    if (g > kXwgRanges) g = kXwgRanges;
    if (n * mbd::xwg_row_stride(q) > (int64_t)kWsFloats) return GEMV_ERR_TOO_LARGE;   // partials beyond the scratch
  } else {
    if (q > 1) return GEMV_ERR_INVALID_ARG;
    q = 1;
  }
  L->variant = v;
  L->grid = (int)g;
  L->kgroups = (int)q;
  L->flags = flags;
  L->lds = lds_bytes(info, k);
  return GEMV_OK;
}

static gemv_status_t resolve(const gemv_handle_s* h, int64_t n, int64_t k, gemv_dtype_t dtype,
                             bool b_aligned, bool with_ws, Launch* L) {
  int v;
  int64_t g, q;
  int flags = 0;
  int cap = 0;   // workgroups per CU (0: what the kernel's resources allow)
  if (h->forced.variant >= 0) {
    v = h->forced.variant;
    g = h->forced.grid;
    q = h->forced.kgroups;
    flags = h->forced.flags;
    // the cross-workgroup split needs the caller's scratch
    if (kVariants[v].info.cross_wg && !with_ws) return GEMV_ERR_UNSUPPORTED;
  } else {
    const Plan p = rule_plan(n, k, dtype, h->max_lds, b_aligned, with_ws);
    v = find_variant(p);
    if (v < 0) return GEMV_ERR_UNSUPPORTED;   // a plan names a variant that is not compiled
    g = p.grid;
    q = p.kgroups;
    cap = wg_cap_of(p);
  }
  gemv_status_t s = shape_launch(v, g, q, flags, n, k, b_aligned, L);
  if (s != GEMV_OK) return s;
  const size_t st = h->static_lds[v][0] > h->static_lds[v][1] ? h->static_lds[v][0] : h->static_lds[v][1];
  if (L->lds + st > h->max_lds) return GEMV_ERR_UNSUPPORTED;
  if (cap > 0 && (int64_t)L->grid >= (int64_t)kCapRounds * cap * h->num_cus) {
    // pad the dynamic LDS so that at most `cap` workgroups fit a CU's LDS
    // (1 KiB below the even share, for the allocation granule)
    const size_t share = h->max_lds / (size_t)cap;
    if (share > st + 1024 && L->lds < share - 1024 - st) L->lds = share - 1024 - st;
  }
  return GEMV_OK;
}

extern "C" gemv_status_t gemv_plan_config(int64_t n, int64_t k, gemv_dtype_t dtype, int32_t b_aligned,
                                          int64_t max_lds, int32_t with_workspace,
                                          gemv_config_t* out) {
  if (!out) return GEMV_ERR_INVALID_ARG;
  if (dtype != GEMV_F16 && dtype != GEMV_BF16) return GEMV_ERR_UNSUPPORTED_DTYPE;
  if (n <= 0 || k < 0 || n > GEMV_MAX_N || k > GEMV_MAX_K || max_lds <= 0) return GEMV_ERR_INVALID_ARG;
  const Plan p = rule_plan(n, k, dtype, (size_t)max_lds, b_aligned != 0, with_workspace != 0);
  const int v = find_variant(p);
  if (v < 0) return GEMV_ERR_UNSUPPORTED;
  Launch L;
  gemv_status_t s = shape_launch(v, p.grid, p.kgroups, 0, n, k, b_aligned != 0, &L);
  if (s != GEMV_OK) return s;
  if (L.lds > (size_t)max_lds) return GEMV_ERR_UNSUPPORTED;
  out->variant = L.variant;
  out->grid = L.grid;
  out->kgroups = L.kgroups;
  out->flags = L.flags;
  return GEMV_OK;
}

extern "C" gemv_status_t gemv_create(gemv_handle_t* out) {
  if (!out) return GEMV_ERR_INVALID_ARG;
  *out = nullptr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return report(nullptr, GEMV_ERR_HIP, "hipGetDevice");
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
    return report(nullptr, GEMV_ERR_HIP, "hipGetDeviceProperties");
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return report(nullptr, GEMV_ERR_UNSUPPORTED, "device is not gfx950");
  int max_lds = 0;
  if (hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
    return report(nullptr, GEMV_ERR_HIP, "hipDeviceGetAttribute(max LDS)");
  void* scr = nullptr;
  const gemv_status_t ss = scratch_address(dev, &scr);
  if (ss != GEMV_OK) return report(nullptr, ss, "hipGetSymbolAddress(scratch)");
  gemv_handle_s* h = (gemv_handle_s*)calloc(1, sizeof(gemv_handle_s));
  if (!h) return GEMV_ERR_OOM;
  h->scratch = scr;
  for (int v = 0; v < kNumVariants; ++v) {
    for (int d = 0; d < 2; ++d) {
      hipFuncAttributes fa;
      const void* fn = (const void*)kVariants[v].fn[d];
      if (hipFuncGetAttributes(&fa, fn) != hipSuccess) {
        free(h);
        return report(nullptr, GEMV_ERR_HIP, "hipFuncGetAttributes");
      }
      h->static_lds[v][d] = fa.sharedSizeBytes;
      const int dyn_max = max_lds - (int)fa.sharedSizeBytes;
      if (dyn_max < 0 ||
          hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, dyn_max) != hipSuccess) {
        free(h);
        return report(nullptr, GEMV_ERR_HIP, "hipFuncSetAttribute(max dynamic LDS)");
      }
    }
  }
  h->magic = kMagic;
  h->device = dev;
  h->num_cus = prop.multiProcessorCount;
  h->max_lds = (size_t)max_lds;
  const char* lg = getenv("GEMV_LOG");
  h->log = lg && strcmp(lg, "1") == 0;
  h->forced.variant = -1;
  h->forced.grid = 0;
  h->forced.kgroups = 0;
  h->forced.flags = 0;
  *out = h;
  return GEMV_OK;
}

extern "C" gemv_status_t gemv_destroy(gemv_handle_t h) {
  if (!h) return GEMV_OK;
  if (h->magic != kMagic) return GEMV_ERR_NULL_HANDLE;
  // the handle holds no device memory: kernels still in flight never read it
  h->magic = kDead;
  free(h);
  return GEMV_OK;
}

extern "C" gemv_status_t gemv_force_config(gemv_handle_t h, const gemv_config_t* cfg) {
  if (!h || h->magic != kMagic) return GEMV_ERR_NULL_HANDLE;
  if (!cfg || cfg->variant < 0) {
    h->forced.variant = -1;
    h->forced.grid = 0;
    h->forced.kgroups = 0;
    h->forced.flags = 0;
    return GEMV_OK;
  }
  if (cfg->variant >= kNumVariants || cfg->grid < 0 || cfg->kgroups < 0 ||
      (cfg->flags & ~GEMV_FLAG_XCD_CONTIGUOUS) != 0 ||
      (!kVariants[cfg->variant].info.cross_wg && cfg->kgroups > 1))
    return report(h, GEMV_ERR_INVALID_ARG, "config");
  h->forced = *cfg;
  return GEMV_OK;
}

extern "C" gemv_status_t gemv_query_config(gemv_handle_t h, int64_t n, int64_t k,
                                           gemv_dtype_t dtype, int32_t with_workspace,
                                           gemv_config_t* out) {
  if (!h || h->magic != kMagic) return GEMV_ERR_NULL_HANDLE;
  if (!out) return GEMV_ERR_INVALID_ARG;
  if (dtype != GEMV_F16 && dtype != GEMV_BF16) return GEMV_ERR_UNSUPPORTED_DTYPE;
  if (n <= 0 || k < 0 || n > GEMV_MAX_N || k > GEMV_MAX_K) return GEMV_ERR_INVALID_ARG;
  Launch L;
  gemv_status_t s = resolve(h, n, k, dtype, true, with_workspace != 0, &L);
  if (s != GEMV_OK) return s;
  out->variant = L.variant;
  out->grid = L.grid;
  out->kgroups = L.kgroups;
  out->flags = L.flags;
  return GEMV_OK;
}

extern "C" gemv_status_t gemv_run(gemv_handle_t h, const void* B, const void* a, void* c,
                                  int64_t n, int64_t k, gemv_dtype_t dtype, hipStream_t stream) {
  return gemv_run_ws(h, B, a, c, n, k, dtype, nullptr, nullptr, 0, stream);
}

extern "C" gemv_status_t gemv_run_ex(gemv_handle_t h, const void* B, const void* a, void* c,
                                     int64_t n, int64_t k, gemv_dtype_t dtype,
                                     const gemv_epilogue_t* ep, hipStream_t stream) {
  return gemv_run_ws(h, B, a, c, n, k, dtype, ep, nullptr, 0, stream);
}

// The workspace checks of gemv_run_ws, after gemv_check_args_ex has passed
// and n > 0: size, alignment, no overlap with B, a, c or the bias.
static gemv_status_t check_workspace(const void* B, const void* a, const void* c, int64_t n,
                                     int64_t k, const gemv_epilogue_t* ep, const void* ws,
                                     size_t ws_bytes) {
  if (!ws) return GEMV_OK;
  if (ws_bytes < (size_t)GEMV_WORKSPACE_BYTES) return GEMV_ERR_INVALID_ARG;
  if ((uintptr_t)ws & 15u) return GEMV_ERR_MISALIGNED;
  const uintptr_t w0 = (uintptr_t)ws, w1 = w0 + (uintptr_t)GEMV_WORKSPACE_BYTES;
  auto hits = [&](const void* p, uintptr_t bytes) {
    const uintptr_t p0 = (uintptr_t)p;
    return p && bytes && p0 < w1 && w0 < p0 + bytes;
  };
  if (hits(c, (uintptr_t)n * 2u) || (k > 0 && (hits(B, (uintptr_t)n * (uintptr_t)k * 2u) ||
                                                hits(a, (uintptr_t)k * 2u))) ||
      (ep && hits(ep->bias, (uintptr_t)n * 2u)))
    return GEMV_ERR_ALIASING;
  return GEMV_OK;
}

extern "C" gemv_status_t gemv_run_ws(gemv_handle_t h, const void* B, const void* a, void* c,
                                     int64_t n, int64_t k, gemv_dtype_t dtype,
                                     const gemv_epilogue_t* ep, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  if (!h || h->magic != kMagic) return report(nullptr, GEMV_ERR_NULL_HANDLE, "gemv_run");
  gemv_status_t s = gemv_check_args_ex(B, a, c, n, k, dtype, ep);
  if (s != GEMV_OK) return report(h, s, "gemv_run arguments");
  if (n == 0) return GEMV_OK;
  s = check_workspace(B, a, c, n, k, ep, workspace, workspace_bytes);
  if (s != GEMV_OK) return report(h, s, "gemv_run_ws workspace");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return report(h, GEMV_ERR_HIP, "hipGetDevice");
  if (dev != h->device) return report(h, GEMV_ERR_WRONG_DEVICE, "gemv_run");
  Launch L;
  s = resolve(h, n, k, dtype, ((uintptr_t)B & 15u) == 0, workspace != nullptr, &L);
  if (s != GEMV_OK)
    return report(h, s, s == GEMV_ERR_TOO_LARGE ? "rows x k-groups (rounded up to 32) exceed the scratch's 2^18 partials"
                                                : "no variant fits (LDS, or scratch for the k-split)");
  const Variant& var = kVariants[L.variant];
  const gemv_variant_info_t& vi = var.info;
  mbd::GemvArgs p;
  p.B = (const uint16_t*)B;
  p.a = (const uint16_t*)a;
  p.c = (uint16_t*)c;
  p.bias = ep ? (const uint16_t*)ep->bias : nullptr;
  // the scratch: the counter bank of this k-group count, then the partials
  p.cnt = workspace ? (unsigned*)workspace + (size_t)(L.kgroups - 1) * kXwgRanges * mbd::kCntStride
                    : nullptr;
  p.ws = workspace ? (float*)((char*)workspace + kWsCounterBytes) : nullptr;
  p.n = (int)n;
  p.k = (int)k;
  p.flags = L.flags | (ep ? mbd::kFlagEpilogue : 0);
  // One row per workgroup of one row group, as the automatic plan's split of
  // up to 96 rows has it, and at most 512 workgroups: the ticketed combine,
  // on its own bank of the scratch (pointed to by ws; the kernel takes its
  // row lines from there).  With more workgroups than that the combiners
  // that wait hold places that workgroups of other rows are queued for: on
  // MI355X the ticketed combine was 2-9% faster up to 384 workgroups, even at
  // 512-768 and 7-14% slower from 1024.
  if (workspace && vi.cross_wg && vi.rows == 1 && vi.waves == vi.splits && L.grid == n &&
      n <= mbd::kTicketRows && (int64_t)L.grid * L.kgroups <= kTicketMaxWorkgroups) {
    p.ws = (float*)((char*)workspace + kWsCounterBytes + kWsFloats * sizeof(float) +
                    mbd::ticket_bank_offset(L.kgroups));
    p.flags |= mbd::kFlagTicket;
  }
  p.alpha = ep ? ep->alpha : 1.0f;
  // balanced shares: rows over the row units, full k-steps over the k-slices
  int64_t units;
  if (vi.a_mode == mbd::A_LDS_SHIFTED || vi.stages > 0)
    units = (int64_t)L.grid * vi.waves;                                         // a wave per unit
  else if (vi.splits == 1 && !vi.cross_wg) units = (int64_t)L.grid * (vi.waves / vi.splits);
  else units = L.grid;                                                          // a workgroup per unit
  const int64_t items = row_items(vi, n);
  p.rows_q = (int)(items / units);
  p.rows_r = (int)(items % units);
  // the k-steps shared out: whole 512-element steps (the partial one goes to
  // the last slice), or for the shifted-window kernel every granule step of
  // the longest row, ceil((k + 63) / 512)
  const int64_t nfull = vi.a_mode == mbd::A_SHIFTED ? (k + mbd::kLine - 1 + mbd::kStep - 1) / mbd::kStep
                                                    : k / mbd::kStep;
  const int64_t nsl = (int64_t)vi.splits * L.kgroups;
  p.slice_q = (int)(nfull / nsl);
  p.slice_r = (int)(nfull % nsl);
  // in the order of the kernels' parameters (MBD_GEMV_PARAMS)
  void* args[] = {(void*)&p.B,       (void*)&p.a,       (void*)&p.c,       (void*)&p.n,
                  (void*)&p.k,       (void*)&p.flags,   (void*)&p.rows_q,  (void*)&p.rows_r,
                  (void*)&p.slice_q, (void*)&p.slice_r, (void*)&p.alpha,   (void*)&p.bias,
                  (void*)&p.ws,      (void*)&p.cnt};
  // the cross-workgroup split's grid is (k-groups, row ranges)
  hipError_t e = hipLaunchKernel((const void*)var.fn[dtype],
                                 vi.cross_wg ? dim3((unsigned)L.kgroups, (unsigned)L.grid)
                                             : dim3((unsigned)L.grid),
                                 dim3((unsigned)(var.info.waves * mbd::kLanes)), args, L.lds, stream);
  if (e != hipSuccess) return report(h, GEMV_ERR_HIP, hipGetErrorString(e));
  return GEMV_OK;
}

extern "C" gemv_status_t gemv_run_noalloc(gemv_handle_t h, const void* B, const void* a, void* c,
                                          int64_t n, int64_t k, gemv_dtype_t dtype,
                                          const gemv_epilogue_t* ep, hipStream_t stream) {
  if (!h || h->magic != kMagic) return report(nullptr, GEMV_ERR_NULL_HANDLE, "gemv_run_noalloc");
  // gemv_run_ws on this GPU's static scratch: validation, plan and launch
  // allocate nothing; a plan needing more partials than the scratch holds
  // (a forced k-split only) is GEMV_ERR_TOO_LARGE
  return gemv_run_ws(h, B, a, c, n, k, dtype, ep, h->scratch, (size_t)GEMV_WORKSPACE_BYTES, stream);
}
