// Rows that do not start on a 16-byte boundary (k % 8 != 0, or B itself not
// 16-byte aligned), with the aligned kernel's plan shapes and no staging.
//
// B is read as gemv_realign_kernel reads it: in aligned 16-byte granules
// from the 128-byte line that holds the row's first element, so a wave's
// 1 KiB load covers exactly 8 lines.  Granule v of a row whose first element
// sits o elements into its line (0..63) holds row elements [j0, j0 + 8),
// j0 = 8v - o, so it needs a[j0 .. j0 + 7] -- a window that starts s = o mod 8
// elements before an 8-element boundary of a.  Here every lane reads that
// window straight through the caches, without staging a in LDS:
//   * one 16-byte load at element j0 - (s & 1), a 4-byte aligned address
//     (measured on MI355X, the headline plan with a read 4 bytes off its
//     16-byte grid: 37.94 against 37.86 us), dwords d0..d3, and one 16-bit
//     load of the element after them, d4;
//   * window dword i = (d_{i+1} : d_i) >> (16 * (s & 1)), one v_alignbyte
//     (a shift of 0 for even s: the window is d0..d3).
// The odd form costs 1.2% on that plan, a single 2-byte-aligned 16-byte load
// 2.4%.  s is uniform over a row, so the shift is too.
//
// Buffer loads return a dword only when all of it lies inside the
// descriptor's range (zero otherwise, checked on MI355X).  A lane whose
// granule lies wholly inside the row gets its window right from the loads
// above.  A step is "clean" when every lane's does (all but the row's first
// step when o > 0 and its last one or two): then nothing else happens.  In
// the other steps each lane looks at its own granule, with VALU work only:
//   * elements outside [0, k) are cleared in B (neighbouring rows' data, a
//     NaN included, never reaches the sum) and in a;
//   * the lane whose granule straddles the row's start (j0 = -s, s > 0)
//     takes its window from a[0 .. 7] (loaded once per wave) shifted by the
//     row's s -- its own load, at a negative offset, is not used;
//   * the lane that holds element k - 1 gets it from a scalar copy: for odd
//     k that element shares a dword with the one past the end of a, which
//     the range check returns as zero.
// So every element is read inside its buffer and each product is the exact
// product of the two 16-bit inputs.
//
// Two rows per trip share one window when they share o: rows i and i + 64
// always do (they are 128 k bytes apart).  So with R = 2 a trip takes such a
// pair -- "slot" p stands for rows 128 (p / 64) + p % 64 and 64 rows later,
// the second absent past n -- and, as in the aligned kernel's two-row plans,
// each step reads a once for both rows.  With R = 1 slot p is row p.  Slots
// and k-steps are dealt as in gemv_kernel: balanced ranges per wave (S == 1)
// or per workgroup (S > 1, the S k-slices of a row group summed through LDS
// in slice order); the k-steps shared out are the granule steps of the
// longest row, ceil((k + 63) / 512), steps past a row's own granules reading
// zeros.
#pragma once

#include "gemv_kernel.h"

namespace mbd {

// The window [-s, 8 - s) of a, 0 < s < 8: s zeros, then a[0 .. 7 - s] (the
// granule that straddles a row's start).  a0 holds a[0 .. 7]; s is uniform.
__device__ __forceinline__ u32x4 start_window(const u32x4& a0, int s) {
  uint32_t x0 = a0[0], x1 = a0[1], x2 = a0[2], x3 = a0[3];
  // keep this (and so the wait for a0's load) where it is used, after the
  // group's loads were issued: hoisted to the row's set-up it would hold
  // every wave's first loads back by a memory round trip
  asm volatile("" : "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3));
  u32x4 w = {0u, 0u, 0u, 0u};
  switch (s) {   // dword i of the window holds elements 2i - s, 2i + 1 - s
    case 1: w[0] = x0 << 16; w[1] = __builtin_amdgcn_alignbyte(x1, x0, 2);
            w[2] = __builtin_amdgcn_alignbyte(x2, x1, 2); w[3] = __builtin_amdgcn_alignbyte(x3, x2, 2); break;
    case 2: w[1] = x0; w[2] = x1; w[3] = x2; break;
    case 3: w[1] = x0 << 16; w[2] = __builtin_amdgcn_alignbyte(x1, x0, 2);
            w[3] = __builtin_amdgcn_alignbyte(x2, x1, 2); break;
    case 4: w[2] = x0; w[3] = x1; break;
    case 5: w[2] = x0 << 16; w[3] = __builtin_amdgcn_alignbyte(x1, x0, 2); break;
    case 6: w[3] = x0; break;
    case 7: w[3] = x0 << 16; break;
    default: break;
  }
  return w;
}

// Rows of slot p: R == 1, row p; R == 2, rows 128 (p / 64) + p % 64 and 64
// rows later.
template <int R>
__device__ __forceinline__ int slot_row(int slot, int r) {
  if constexpr (R == 1) {
    return slot;
  } else {
    return ((slot >> 6) << 7) + (slot & 63) + 64 * r;
  }
}

template <int DT, int R, int U, int WAVES, int S, int BPOL>
__global__ __launch_bounds__(WAVES * kLanes) void gemv_shift_kernel(MBD_GEMV_PARAMS) {
  MBD_GEMV_ARGS;
  const uint16_t* __restrict__ B = p.B;
  const uint16_t* __restrict__ a = p.a;
  uint16_t* c = p.c;
  const int n = p.n, k = p.k, flags = p.flags;
  const float alpha = p.alpha;
  const uint16_t* bias = p.bias;
  static_assert(WAVES % S == 0, "splits must divide the waves of a workgroup");
  static_assert(R == 1 || R == 2, "one row, or a pair of rows 64 apart");
  constexpr int G = WAVES / S;   // row groups per workgroup
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float* part = reinterpret_cast<float*>(smem);

  const int lane = threadIdx.x & (kLanes - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rg = wave / S;
  const int sl = wave - rg * S;
  const __amdgpu_buffer_rsrc_t arsrc = make_rsrc(a, (uint32_t)k * 2u);

  // this wave's k-slice: granule steps [t0, t1) of the longest row
  const int t0 = share_start(sl, p.slice_q, p.slice_r);
  const int t1 = t0 + p.slice_q + (sl < p.slice_r ? 1 : 0);

  // a[0 .. 7] (for the granule that straddles a row's start; zeros past k),
  // by the waves whose slice holds step 0, and a[k - 1] (which a dword load
  // misses when k is odd), by those whose slice can hold it -- not by every
  // wave, which would all read the same two lines
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  const u32x4 a_head = t0 == 0 && t1 > 0 ? __builtin_amdgcn_raw_buffer_load_b128(arsrc, 0u, 0u, 0) : zero4;
  const uint32_t a_last = k > 0 && t1 > (k - 1) / kStep
                              ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(arsrc, (uint32_t)(k - 1) * 2u, 0u, 0)
                              : 0u;

  constexpr bool kWaveRanges = S == 1;
  const int64_t wg = (flags & kFlagXcdContiguous) ? xcd_unit(blockIdx.x, gridDim.x) : blockIdx.x;
  const int64_t unit = kWaveRanges ? wg * G + rg : wg;
  const int lo = share_start(unit, p.rows_q, p.rows_r);   // slots
  const int hi = lo + p.rows_q + (unit < p.rows_r ? 1 : 0);
  constexpr int kTrip = kWaveRanges ? 1 : G;
  const int goff = kWaveRanges ? 0 : rg;

  for (int base = lo; base < hi; base += kTrip) {   // trip count uniform in a workgroup when S > 1
    const int slot = base + goff;                    // may lie past hi for S > 1: computed, not stored
    bool live[R];
    __amdgpu_buffer_rsrc_t brsrc[R];
    int o = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int want = slot_row<R>(slot, r);
      live[r] = slot < hi && want < n;
      // a row that is not stored reads the slot's first row (or the last
      // row): the same o, and inside B
      const int r0 = slot_row<R>(slot, 0);
      const int row = live[r] ? want : (slot < hi && r0 < n ? r0 : n - 1);
      const uint16_t* rowp = B + (int64_t)row * k;
      o = (int)(((uintptr_t)rowp >> 1) & (kLine - 1));                // wave-uniform, one o for the rows
      const int nv = k > 0 ? (o + k + kVec - 1) / kVec : 0;           // granules touching the row
      brsrc[r] = make_rsrc(rowp - o, (uint32_t)nv * 16u);
    }
    const int sh = (o & 1) * 2;                                       // bytes to shift the window by
    const int c1 = (k + o) / kStep;                                   // steps below c1 end inside the rows
    float acc[R][2];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r][0] = acc[r][1] = 0.0f;

    for (int t = t0; t < t1; t += U) {
      // every load of the group first (B, then a's dwords and, for odd o,
      // the element after them), so one memory round trip covers the group
      u32x4 bv[U][R], dv[U];
      uint32_t d4[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int st = t + u;
        const bool ok = st < t1;
        const uint32_t boff = ok ? (uint32_t)((st * kLanes + lane) * 16) : kOffsetOutOfRange;
#pragma unroll
        for (int r = 0; r < R; ++r) bv[u][r] = __builtin_amdgcn_raw_buffer_load_b128(brsrc[r], boff, 0u, BPOL);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int st = t + u;
        const bool ok = st < t1;
        // the window starts at j0; read from the dword-aligned element
        // j0 - (o & 1) (j0 and o have the same parity)
        const int e = (st * kLanes + lane) * kVec - o - (o & 1);
        dv[u] = __builtin_amdgcn_raw_buffer_load_b128(arsrc, ok ? (uint32_t)e * 2u : kOffsetOutOfRange, 0u, 0);
        d4[u] = (o & 1) ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(
                              arsrc, ok ? (uint32_t)(e + kVec) * 2u : kOffsetOutOfRange, 0u, 0)
                        : 0u;
      }
      // then slot by slot: join the window, fix up the rows' first step
      // (o > 0) and their last ones lane by lane, multiply and add
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int st = t + u;
        const uint32_t d0 = dv[u][0], d1 = dv[u][1], d2 = dv[u][2], d3 = dv[u][3];
        u32x4 w;
        w[0] = __builtin_amdgcn_alignbyte(d1, d0, sh);
        w[1] = __builtin_amdgcn_alignbyte(d2, d1, sh);
        w[2] = __builtin_amdgcn_alignbyte(d3, d2, sh);
        w[3] = __builtin_amdgcn_alignbyte(d4[u], d3, sh);
        u32x4 b[R];
#pragma unroll
        for (int r = 0; r < R; ++r) b[r] = bv[u][r];
        const bool clean = (st > 0 || o == 0) && st < c1;
        if (!clean) {
          const int j0 = (st * kLanes + lane) * kVec - o;
          // only the rows' step 0 has granules before the row (the loaded
          // window of the one that straddles its start is not used; the
          // others are cleared below); t == 0 there, so only slot 0
          if (u == 0 && st == 0 && j0 < 0) w = start_window(a_head, o & (kVec - 1));
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t m = keep_mask(j0 + 2 * i, k);
            const uint32_t y = w[i];
            w[i] = y & m;
#pragma unroll
            for (int r = 0; r < R; ++r) {
              const uint32_t x = b[r][i];
              b[r][i] = x & m;
            }
          }
          // element k - 1, if in this granule: at position p
          const int pk = k - 1 - j0;
          if (pk >= 0 && pk < kVec) {
            uint32_t al = a_last;
            asm volatile("" : "+v"(al));   // (as in start_window: no early wait)
            const int sh16 = (pk & 1) * 16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t y = w[i];
              w[i] = (pk >> 1) == i ? ((y & ~(0xffffu << sh16)) | (al << sh16)) : y;
            }
          }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) fma8<DT>(b[r], w, acc[r][0], acc[r][1]);
      }
    }

    float tot[R];
#pragma unroll
    for (int r = 0; r < R; ++r) tot[r] = wave_sum(acc[r][0] + acc[r][1]);
    float mine = tot[0];
    bool mine_live = live[0];
#pragma unroll
    for (int r = 1; r < R; ++r) {
      mine = (lane == r) ? tot[r] : mine;
      mine_live = (lane == r) ? live[r] : mine_live;
    }
    bool leader = lane < R && mine_live;   // holds the sum of the slot's row `lane`
    if constexpr (S > 1) {
      if (lane < R) part[(rg * S + sl) * R + lane] = mine;
      __syncthreads();
      leader = leader && sl == 0;
      if (leader) {
        float s2 = 0.0f;
        for (int qq = 0; qq < S; ++qq) s2 += part[(rg * S + qq) * R + lane];
        mine = s2;
      }
      __syncthreads();
    }
    if (leader) {
      const int row = slot_row<R>(slot, lane);
      c[row] = to_bits<DT>(finish<DT>(mine, flags, alpha, bias, row));
    }
  }
}

}  // namespace mbd
