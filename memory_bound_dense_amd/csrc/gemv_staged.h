// The pipelined-B form of the GEMV (TileLang Case Studies, Case B.1, "O3"):
// while one item of B is consumed, the next P - 1 are already on their way.
// Kept for measurement next to gemv_kernel, which issues a group of loads and
// waits for it (latency then is hidden by the other waves of the CU alone).
//
// An item is U 512-element steps of R rows of one wave (R * U wave-loads of
// 1 KiB).  A wave owns a contiguous range of rows and walks it as one flat
// sequence of items, R rows at a time, so the pipeline runs on across row
// boundaries instead of draining at the end of every row.  Two forms of the
// slots:
//   * VIA_LDS = false: P register slots.  The loads write VGPRs; the
//     compiler's wait before an item's first use counts only the loads issued
//     before it, so the later items stay in flight.
//   * VIA_LDS = true: P LDS slots per wave, filled by buffer loads that write
//     LDS directly (the form the pages use: asynchronous copies into shared
//     memory, then shared-memory reads), then read back with ds_read_b128.
//     Each lane reads back exactly the 16 bytes it fetched, so the LDS trip
//     buys no data sharing; it costs LDS space (waves * P * R * U KiB per
//     workgroup) and with it occupancy.
// P = 1 issues each item right before it is used (no overlap), 2 is double,
// 3 triple buffering.  Rows must be 16-byte aligned (k % 8 == 0 and B
// 16-byte aligned); the host rejects other calls for these variants.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemv_kernel.h"

namespace mbd {

// s_waitcnt operand that waits for vmcnt <= n (0..63) and nothing else:
// vmcnt in bits 3:0 and 15:14, expcnt (bits 6:4) and lgkmcnt (bits 11:8) at
// their maxima.
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
constexpr int kWaitVmcnt0 = waitcnt_vm(0);

template <int R, int U, int P>
struct StagedRegs {
  u32x4 b[P][U][R];
  u32x4 a[P][U];
};

// Issue item (rows rbase .. rbase + nrows - 1, group grp) into `slot`.  The
// slot index is a constant once the caller's loops are unrolled, so the
// register slots stay in VGPRs.  A dead issue (past the wave's last item,
// never consumed) keeps the instruction stream -- and so the wait counts --
// the same but gets descriptors of zero range: it touches no memory.
template <int R, int U, int P, bool VIA_LDS, int BPOL>
__device__ __forceinline__ void staged_issue(StagedRegs<R, U, P>& regs, uint8_t* wlds, int slot,
                                             const uint16_t* B, const uint16_t* a, bool live,
                                             int k, int nfull, int rbase, int nrows, int grp,
                                             int lane_off) {
  const __amdgpu_buffer_rsrc_t brsrc =
      make_rsrc(B + (int64_t)rbase * k, live ? (uint32_t)nrows * (uint32_t)k * 2u : 0u);
  const __amdgpu_buffer_rsrc_t arsrc = make_rsrc(a, live ? (uint32_t)k * 2u : 0u);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    // steps past the row's full steps re-load its last full step (it is in
    // flight or cached already); the consumer skips them
    int t = grp * U + u;
    t = t < nfull ? t : nfull - 1;
    t = t > 0 ? t : 0;
    const int off = t * kStepBytes + lane_off;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t soff = (uint32_t)(r < nrows ? r : nrows - 1) * (uint32_t)k * 2u;
      if constexpr (VIA_LDS) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            brsrc,
            (__attribute__((address_space(3))) void*)(wlds + ((slot * U + u) * R + r) * kStepBytes),
            16, off, (int)soff, 0, BPOL);
      } else {
        regs.b[slot][u][r] = __builtin_amdgcn_raw_buffer_load_b128(brsrc, off, soff, BPOL);
      }
    }
    regs.a[slot][u] = __builtin_amdgcn_raw_buffer_load_b128(arsrc, off, 0u, 0);
  }
}

template <int DT, int R, int U, int WAVES, int P, bool VIA_LDS, int BPOL>
__global__ __launch_bounds__(WAVES * kLanes) void gemv_staged_kernel(MBD_GEMV_PARAMS) {
  MBD_GEMV_ARGS;
  static_assert(P >= 1 && P <= 3, "pipeline depth 1..3");
  static_assert((P - 1) * U * R <= 63, "the slot wait must fit vmcnt");
  const uint16_t* __restrict__ B = p.B;
  const uint16_t* __restrict__ a = p.a;
  uint16_t* c = p.c;
  const int k = p.k, flags = p.flags;
  const float alpha = p.alpha;
  const uint16_t* bias = p.bias;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & (kLanes - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane_off = lane * 16;

  const int nfull = k >> 9;
  const int rem = k & (kStep - 1);
  const __amdgpu_buffer_rsrc_t arsrc = make_rsrc(a, (uint32_t)k * 2u);

  const int64_t wg = (flags & kFlagXcdContiguous) ? xcd_unit(blockIdx.x, gridDim.x) : blockIdx.x;
  const int64_t unit = wg * WAVES + wave;
  const int lo = share_start(unit, p.rows_q, p.rows_r);
  const int hi = lo + p.rows_q + (unit < p.rows_r ? 1 : 0);
  if (lo >= hi) return;                    // wave-uniform; the kernel has no barrier

  // items: ntrips trips of R rows, gpt groups of U steps each (one group of
  // nothing but re-loads when k < 512: the trip is then all tail)
  const int gpt = nfull > 0 ? (nfull + U - 1) / U : 1;
  const int ntrips = (hi - lo + R - 1) / R;
  const int nitems = ntrips * gpt;

  uint8_t* wlds = smem + (size_t)wave * (P * U * R * kStepBytes);   // this wave's slots
  StagedRegs<R, U, P> regs;

  // producer cursor (it stops at the last item; the P - 1 issues after it
  // are dead)
  int ptrip = 0, pgrp = 0, pitem = 0;
  // consumer cursor
  int ctrip = 0, cgrp = 0;
  // finished rows wait in lanes (lane j: row fbase + j) and leave in one
  // coalesced store per 64 rows, so no store sits between the loads in flight
  float res = 0.0f;
  int fbase = lo, fcount = 0;
  auto flush = [&]() {
    if (lane < fcount) c[fbase + lane] = to_bits<DT>(res);
    fbase += fcount;
    fcount = 0;
    // the slot waits below count loads only: let the store drain first
    if constexpr (VIA_LDS) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  };
  float acc[R][2];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r][0] = acc[r][1] = 0.0f;

  // issue the producer's item into `slot`, then advance the producer
  auto issue = [&](int slot) {
    const int rb = lo + ptrip * R;
    const int nr = (hi - rb) < R ? (hi - rb) : R;
    const bool live = pitem < nitems;
    staged_issue<R, U, P, VIA_LDS, BPOL>(regs, wlds, slot, B, a, live, k, nfull, rb, nr, pgrp,
                                         lane_off);
    if (pitem < nitems - 1) {
      if (++pgrp == gpt) { pgrp = 0; ++ptrip; }
    }
    ++pitem;
  };

  // prologue: items 0 .. P-2 into slots 0 .. P-2
#pragma unroll
  for (int s = 0; s < P - 1; ++s) issue(s);

  for (int i = 0; i < nitems; i += P) {
#pragma unroll
    for (int s = 0; s < P; ++s) {
      // item i + s + P - 1 into the slot that item i + s - 1 has just freed
      issue((s + P - 1) % P);
      if (i + s < nitems) {
        // consume slot s: item (ctrip, cgrp)
        if constexpr (VIA_LDS) {
          // slot s's copies into LDS have landed once no more loads are
          // outstanding than were surely issued after them: the copies of
          // the P - 1 later items (copies into LDS keep their order; the a
          // loads may be scheduled anywhere, so they are not counted; loads
          // return in order)
          __builtin_amdgcn_s_waitcnt(waitcnt_vm((P - 1) * U * R));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (cgrp * U + u < nfull) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
              u32x4 bv;
              if constexpr (VIA_LDS) {
                bv = *reinterpret_cast<const u32x4*>(wlds + ((s * U + u) * R + r) * kStepBytes + lane_off);
              } else {
                bv = regs.b[s][u][r];
              }
              fma8<DT>(bv, regs.a[s][u], acc[r][0], acc[r][1]);
            }
          }
        }
        if (++cgrp == gpt) {   // the trip's last group: tail, reduce, store
          const int rbase = lo + ctrip * R;
          const int nrows = (hi - rbase) < R ? (hi - rbase) : R;
          if (rem != 0) {
            const __amdgpu_buffer_rsrc_t brsrc =
                make_rsrc(B + (int64_t)rbase * k, (uint32_t)nrows * (uint32_t)k * 2u);
            const int e0 = (nfull * kLanes + lane) * kVec;
            const u32x4 av = load_vec_tail(arsrc, e0, k, 0u);
#pragma unroll
            for (int r = 0; r < R; ++r) {
              const uint32_t soff = (uint32_t)(r < nrows ? r : nrows - 1) * (uint32_t)k * 2u;
              const u32x4 bv = load_vec_tail(brsrc, e0, k, soff);
              fma8<DT>(bv, av, acc[r][0], acc[r][1]);
            }
          }
          if (fcount + R > kLanes) flush();
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const float tot = wave_sum(acc[r][0] + acc[r][1]);
            if (r < nrows && lane == fcount + r) res = finish<DT>(tot, flags, alpha, bias, rbase + r);
            acc[r][0] = acc[r][1] = 0.0f;
          }
          fcount += nrows;
          cgrp = 0;
          ++ctrip;
        }
      }
    }
  }
  flush();
  // no load (into LDS above all) may outlive the wave
  __builtin_amdgcn_s_waitcnt(0);
}

}  // namespace mbd
