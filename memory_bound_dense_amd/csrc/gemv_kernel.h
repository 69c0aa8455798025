// Dense GEMV kernels for gfx950 (CDNA4): c = B @ a, fp16/bf16 in, fp32 sum.
//
// The product is bound by HBM bandwidth: every element of B is read exactly
// once and used once, about one flop per byte, so the design goal is to keep
// enough 16-byte loads of B in flight on every CU and to do nothing else
// expensive.  No matrix cores: this is not a contraction worth tiling.
//
// gemv_kernel -- the lanes-along-k layout that TileLang Case Studies, Case B,
// shows is the one that coalesces, sized for 64-lane wavefronts:
//   * a workgroup has WAVES wavefronts, arranged as G = WAVES/S row groups
//     times S k-slices;
//   * rows are dealt in balanced contiguous ranges (per wave, or per
//     workgroup when S > 1 or XWG); a wave walks its range R rows at a time,
//     and lane l reads elements [8*(64*t + l), +8) of each of those rows at
//     step t -- one 16-byte load per lane, 1 KiB contiguous per row per wave;
//   * U steps are unrolled, so a wave keeps R*U KiB of B in flight;
//   * a is either staged once per workgroup in LDS (A_LDS; Case B.2 is the
//     shared-memory variant of this choice) or read with the same 16-byte
//     loads through the caches (A_CACHED);
//   * each lane keeps fp32 partial sums; the 64 lane partials of a row are
//     combined with DPP row operations and two cross-row swaps;
//   * with S > 1 the k-slices of a row group are summed through LDS in slice
//     order (fixed order, so results do not depend on timing);
//   * with XWG, Q = gridDim.x workgroups also share a row range along k:
//     each writes its fp32 row partials to the caller's scratch, and the
//     workgroup that arrives last (a device-scope counter per row range)
//     sums the Q partials in a fixed order and writes c;
//   * an optional fused epilogue (alpha, bias) is one FMA before the store.
// gemv_realign_kernel -- rows that do not start on 16-byte boundaries: B in
// aligned granules, a realigned through two shifted LDS copies.
// gemv_rowlane_kernel -- the uncoalesced layout (one row per lane), for
// measurement only.
//
// Loads go through buffer resources: the row base is a wave-uniform 64-bit
// address in SGPRs, the per-row offset an SGPR soffset and the lane offset a
// single VGPR shared by all rows.  Every offset is in bounds by construction;
// the descriptor's range (the wave's rows) is a second fence.  In
// gemv_kernel, rows are only 2-byte aligned when k is not a multiple of 8;
// its 16-byte loads then rely on the unaligned buffer access that ROCm
// enables for compute queues (the realigning kernel needs none).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mbd {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

enum { DT_F16 = 0, DT_BF16 = 1 };
enum { A_LDS = 0, A_CACHED = 1, A_LDS_SHIFTED = 2, A_SHIFTED = 3 };

constexpr int kLanes = 64;
constexpr int kVec = 8;                 // 16-bit elements per 16-byte load
constexpr int kStep = kLanes * kVec;    // elements per row per wave-load
constexpr int kStepBytes = kStep * 2;   // 1 KiB
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)
// A buffer offset beyond every descriptor's range (ranges here are < 2^31
// bytes): a load from it returns zeros without a memory access.
constexpr uint32_t kOffsetOutOfRange = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}

// Element-wise load of the 8-element vector starting at element e0 of a row:
// the full 16 bytes when the vector lies inside the row, otherwise the
// elements below `len` one by one and zeros above.  Only the last vector of a
// row takes the slow branch.
__device__ __forceinline__ u32x4 load_vec_tail(__amdgpu_buffer_rsrc_t rsrc, int e0, int len,
                                               uint32_t soff) {
  if (e0 + kVec <= len) {
    return __builtin_amdgcn_raw_buffer_load_b128(rsrc, e0 * 2, soff, 0);
  }
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  if (e0 < len) {
#pragma unroll
    for (int i = 0; i < kVec; ++i) {
      if (e0 + i < len) {
        uint32_t x = __builtin_amdgcn_raw_buffer_load_b16(rsrc, (e0 + i) * 2, soff, 0);
        w[i >> 1] |= x << ((i & 1) * 16);
      }
    }
  }
  u32x4 v = {w[0], w[1], w[2], w[3]};
  return v;
}

// acc0 += sum of the even products, acc1 += sum of the odd products of the
// 8-element vectors b and a (fp32, each product exact, one rounding per add).
template <int DT>
__device__ __forceinline__ void fma8(const u32x4& b, const u32x4& a, float& acc0, float& acc1) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // Copy the component to a scalar first: a bit_cast applied directly to
    // an ext-vector element reads component 0 whatever the index.
    const uint32_t bw = b[i];
    const uint32_t aw = a[i];
    if constexpr (DT == DT_F16) {
      f16x2 bb = __builtin_bit_cast(f16x2, bw);
      f16x2 aa = __builtin_bit_cast(f16x2, aw);
      acc0 = __builtin_fmaf((float)bb.x, (float)aa.x, acc0);
      acc1 = __builtin_fmaf((float)bb.y, (float)aa.y, acc1);
    } else {
      // bfloat16 is the upper half of a binary32: widening is a shift/mask.
      float blo = __builtin_bit_cast(float, bw << 16);
      float bhi = __builtin_bit_cast(float, bw & 0xffff0000u);
      float alo = __builtin_bit_cast(float, aw << 16);
      float ahi = __builtin_bit_cast(float, aw & 0xffff0000u);
      acc0 = __builtin_fmaf(blo, alo, acc0);
      acc1 = __builtin_fmaf(bhi, ahi, acc1);
    }
  }
}

// One 8-element step of a row: the FMAs above, or, in a PROBE build (a
// measurement aid: the same kernel and launch with the arithmetic taken
// out), an xor-fold of B's bits into the accumulator that keeps B's loads
// alive -- a's loads, left unused, are then dropped by the compiler.
template <int DT, bool PROBE>
__device__ __forceinline__ void accumulate(const u32x4& b, const u32x4& a, float& acc0,
                                           float& acc1) {
  if constexpr (PROBE) {
    const uint32_t x = b[0] ^ b[1] ^ b[2] ^ b[3];
    acc0 = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, acc0) ^ x);
  } else {
    fma8<DT>(b, a, acc0, acc1);
  }
}

// Workgroups are dispatched round-robin over the XCDs (workgroup b runs on
// XCD b % 8).  With kFlagXcdContiguous the row ranges are renumbered so that
// each XCD's workgroups own one contiguous block of rows: XCD x takes units
// [start(x), start(x) + count(x)) with count(x) = G/8 (+1 for x < G % 8).
constexpr int kXcds = 8;
constexpr int kFlagXcdContiguous = 1;
// The fused epilogue (page "Optimizing TileLang Programs", epilogue fusion):
// c = alpha * sum + bias, one fp32 FMA on the row sum before the store.
constexpr int kFlagEpilogue = 2;

// Scratch layout of the cross-workgroup split, shared with the host: each
// arrival counter alone in a 128-byte line (kCntStride words apart), and a
// row's Q partial sums together at row * xwg_row_stride(Q) + q, the stride Q
// rounded up to whole 128-byte lines -- no two rows, and no two counters,
// share a line.  Packed, the counters and partials of neighbouring rows
// shared lines, and the atomics and stores of different workgroups queued
// on them (measured on MI355X: 64 x 65536 bf16 5.40 -> 4.89 us).
// The whole scratch: first the counters, one bank of kXwgRanges per k-group
// count Q = 1..kXwgMaxQ (so that a counter only ever sees one Q), then
// kWsFloats partials.
constexpr int kCntStride = 32;
constexpr int kXwgMaxQ = 64;
constexpr int kXwgRanges = 256;
constexpr size_t kWsCounterBytes = (size_t)kXwgMaxQ * kXwgRanges * kCntStride * sizeof(unsigned);  // 2 MiB
constexpr size_t kWsFloats = (size_t)1 << 18;                                                      // 1 MiB
__host__ __device__ constexpr int64_t xwg_row_stride(int64_t Q) { return (Q + 31) & ~(int64_t)31; }

// The ticketed combine (kFlagTicket: one row per workgroup, one row group)
// has a region of its own after the partials: one bank per Q, kTicketRows
// row lines of ticket_stride(Q) 8-byte words each -- word 0 holds the row's
// ticket counter, word 1 + q the partial of k-group q with its tag in the
// high half.  A line is a whole number of 128-byte lines.
constexpr int kFlagTicket = 4;
constexpr int kTicketRows = 96;
constexpr int kTicketSpins = 1 << 20;   // polls before a waiting combiner gives up
__host__ __device__ constexpr int64_t ticket_stride(int64_t Q) { return (Q + 1 + 15) & ~(int64_t)15; }
constexpr size_t ticket_bank_offset(int Q) {   // bytes from the region's start to bank Q
  size_t b = 0;
  for (int j = 1; j < Q; ++j) b += (size_t)kTicketRows * (size_t)ticket_stride(j) * 8u;
  return b;
}
constexpr size_t kWsTicketBytes = ticket_bank_offset(kXwgMaxQ + 1);
// tickets count 0, 1, ..., Q * M - 1 and wrap to 0, M = floor((2^31 - 1) / Q):
// a multiple of Q, so whole calls keep the counter at a multiple of Q
__host__ __device__ constexpr unsigned ticket_wrap(int Q) {
  return (unsigned)Q * (0x7fffffffu / (unsigned)Q) - 1u;
}

__device__ __forceinline__ int64_t xcd_unit(int64_t b, int64_t G) {
  const int64_t x = b % kXcds, i = b / kXcds;
  const int64_t q = G / kXcds, r = G % kXcds;
  return x * q + (x < r ? x : r) + i;
}

template <int CTRL>
__device__ __forceinline__ float dpp_get(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// Sum over the 64 lanes; every lane receives the same bits.  Each step adds a
// value and its mirror partner, so partial sums stay symmetric in the lanes.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_get<0xB1>(v);    // quad_perm [1,0,3,2]: pairs
  v += dpp_get<0x4E>(v);    // quad_perm [2,3,0,1]: quads
  v += dpp_get<0x141>(v);   // row_half_mirror: groups of 8
  v += dpp_get<0x140>(v);   // row_mirror: rows of 16
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

template <int DT>
__device__ __forceinline__ uint16_t to_bits(float x) {
  if constexpr (DT == DT_F16) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);   // v_cvt_f16_f32, nearest-even
  } else {
    return __builtin_bit_cast(uint16_t, (__bf16)x);     // v_cvt_pk_bf16_f32, nearest-even
  }
}

template <int DT>
__device__ __forceinline__ float widen(uint16_t x) {
  if constexpr (DT == DT_F16) {
    return (float)__builtin_bit_cast(_Float16, x);
  } else {
    return __builtin_bit_cast(float, (uint32_t)x << 16);
  }
}

// The value stored for a row: the sum itself, or alpha * sum (+ bias[row]).
// bias may be c itself: a row's bias is read by the lane that then writes it.
template <int DT>
__device__ __forceinline__ float finish(float s, int flags, float alpha,
                                        const uint16_t* __restrict__ bias, int64_t row) {
  if (!(flags & kFlagEpilogue)) return s;
  return bias ? __builtin_fmaf(alpha, s, widen<DT>(bias[row])) : alpha * s;
}

// Everything a GEMV kernel needs, passed by value (the kernel-argument
// segment is read with scalar loads).  Rows and k-steps are dealt in balanced
// shares worked out on the host, so a wave finds its range with a multiply
// and a min instead of a 64-bit division: share u of U starts at
// u*q + min(u, r) and holds q + (u < r) items, where q = N / U, r = N % U.
struct GemvArgs {
  const uint16_t* B;
  const uint16_t* a;
  uint16_t* c;
  const uint16_t* bias;   // fused epilogue (flags & kFlagEpilogue), may be null
  float* ws;              // cross-workgroup partials (caller scratch)
  unsigned* cnt;          // cross-workgroup arrival counters of this Q
  int n, k, flags;
  float alpha;
  int rows_q, rows_r;     // rows per row unit (per wave, or per workgroup)
  int slice_q, slice_r;   // full 512-element steps per k-slice
};

// The kernels take the fields of GemvArgs as separate arguments, the ones
// every workgroup needs first: the library is built with kernarg preloading,
// so the first 16 dwords (B, a, c, n, k, flags and the row and step shares)
// arrive in SGPRs at wave launch and a workgroup issues its first loads
// without fetching its arguments from memory (measured on MI355X: ~0.3 us of
// a 38 us launch).  A struct argument is not preloaded.
#define MBD_GEMV_PARAMS                                                                  \
  const uint16_t *B_, const uint16_t *a_, uint16_t *c_, int n_, int k_, int flags_,     \
      int rows_q_, int rows_r_, int slice_q_, int slice_r_, float alpha_,               \
      const uint16_t *bias_, float *ws_, unsigned *cnt_
#define MBD_GEMV_ARGS                                                                    \
  const GemvArgs p = {B_, a_, c_, bias_, ws_, cnt_, n_, k_, flags_, alpha_, rows_q_, rows_r_, \
                      slice_q_, slice_r_}

__device__ __forceinline__ int share_start(int64_t u, int q, int r) {
  return (int)(u * q + (u < r ? u : (int64_t)r));
}

template <int DT, int R, int U, int WAVES, int S, int AMODE, int BPOL, bool XWG,
          bool PROBE = false>
__global__ __launch_bounds__(WAVES * kLanes) void gemv_kernel(
    MBD_GEMV_PARAMS) {
  MBD_GEMV_ARGS;
  const uint16_t* __restrict__ B = p.B;
  const uint16_t* __restrict__ a = p.a;
  uint16_t* c = p.c;
  const int k = p.k, flags = p.flags;
  const float alpha = p.alpha;
  const uint16_t* bias = p.bias;
  float* __restrict__ ws = p.ws;
  unsigned* __restrict__ cnt = p.cnt;
  static_assert(WAVES % S == 0, "splits must divide the waves of a workgroup");
  static_assert(!XWG || AMODE == A_CACHED, "a k-chunk per workgroup does not stage all of a");
  constexpr int G = WAVES / S;   // row groups per workgroup
  constexpr int RB = G * R;      // rows per workgroup per row block
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int lane = threadIdx.x & (kLanes - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rg = wave / S;
  const int sl = wave - rg * S;

  const int nfull = k >> 9;              // full 512-element steps
  const int rem = k & (kStep - 1);       // elements of the last, partial step
  const int nsteps = nfull + (rem != 0);
  const __amdgpu_buffer_rsrc_t arsrc = make_rsrc(a, (uint32_t)k * 2u);

  u32x4* a_lds = reinterpret_cast<u32x4*>(smem);
  float* part = reinterpret_cast<float*>(smem + (AMODE == A_LDS ? nsteps * kStepBytes : 0));

  if constexpr (AMODE == A_LDS) {
    // a, zero-padded to whole steps, once per workgroup.
    for (int v = threadIdx.x; v < nsteps * kLanes; v += WAVES * kLanes) {
      a_lds[v] = load_vec_tail(arsrc, v * kVec, k, 0u);
    }
    __syncthreads();
  }

  // this wave's share of the full steps (slice q*S + sl of Q*S); the partial
  // step goes to the last slice
  // With XWG the grid is (Q, row ranges): the Q k-groups of a row range are
  // neighbours in dispatch order, so, workgroups being dealt round robin over
  // the XCDs, k-group q of every row range runs on XCD q mod 8 (for Q a
  // multiple of 8) and each XCD's L2 fetches its own slices of a rather than
  // all of a (measured on MI355X: 1-6% faster on 8..128 rows of 65536..262144
  // columns, the same bits).
  const int Q = XWG ? (int)gridDim.x : 1;
  const int q = XWG ? (int)blockIdx.x : 0;
  const int64_t bx = XWG ? (int64_t)blockIdx.y : (int64_t)blockIdx.x;   // this workgroup's row range
  const int gsl = q * S + sl;
  const int nsl = Q * S;
  const int t0 = share_start(gsl, p.slice_q, p.slice_r);
  const int t1 = t0 + p.slice_q + (gsl < p.slice_r ? 1 : 0);
  (void)nsl;
  const bool tail = (rem != 0) && (gsl == nsl - 1);
  const int lane_off = lane * 16;

  // Rows are dealt out in balanced contiguous ranges, so any grid size is
  // valid and the ranges differ by at most one row.  S == 1: every wave owns
  // a range and walks it R rows at a time.  S > 1: every workgroup owns a
  // range; its row groups take R rows each per trip, its k-slices share them.
  // With XWG the ranges are per workgroup as well (the cross-workgroup
  // combine works on a workgroup's whole range).
  constexpr bool kWaveRanges = S == 1 && !XWG;
  const int64_t wg = (!XWG && (flags & kFlagXcdContiguous)) ? xcd_unit(blockIdx.x, gridDim.x) : bx;
  const int64_t unit = kWaveRanges ? wg * G + rg : wg;
  const int lo = share_start(unit, p.rows_q, p.rows_r);
  const int hi = lo + p.rows_q + (unit < p.rows_r ? 1 : 0);
  constexpr int kTrip = kWaveRanges ? R : RB;
  const int goff = kWaveRanges ? 0 : rg * R;

  // The ticketed combine (below) draws its ticket once the wave's loads of
  // B and a are consumed: its round trip then overlaps the wave's reduction
  // and the workgroup's combine.  (Drawn before the loads, it delays them:
  // the loads' waits count it too, returns being counted in order; drawn
  // between them, the compiler's wait after the branch that issues it is
  // as conservative.)
  [[maybe_unused]] unsigned ticket = 0;
  [[maybe_unused]] float kept = 0.0f;
  [[maybe_unused]] uint64_t* tline = nullptr;   // this row's line in the ticket bank
  [[maybe_unused]] bool take_ticket = false;
  if constexpr (XWG && G == 1) {
    tline = reinterpret_cast<uint64_t*>(ws) + (int64_t)lo * ticket_stride(Q);
    take_ticket = (flags & kFlagTicket) && wave == 0 && lane == 0;
  }
  auto draw_ticket = [&]() {
    if constexpr (XWG && G == 1) {
      if (take_ticket) {
        ticket = __builtin_amdgcn_atomic_inc32(reinterpret_cast<unsigned*>(tline), ticket_wrap(Q),
                                               __ATOMIC_RELAXED, "agent");
        take_ticket = false;
      }
    }
  };

  for (int base = lo; base < hi; base += kTrip) {   // trip count uniform in a workgroup when S > 1
    const int row0 = base + goff;                    // may lie past hi for S > 1: computed, not stored
    const int rbase = row0 < hi ? row0 : hi - 1;
    const int nrows = (hi - rbase) < R ? (hi - rbase) : R;   // >= 1
    const __amdgpu_buffer_rsrc_t brsrc =
        make_rsrc(B + (int64_t)rbase * k, (uint32_t)nrows * (uint32_t)k * 2u);
    uint32_t soff[R];
#pragma unroll
    for (int r = 0; r < R; ++r) soff[r] = (uint32_t)(r < nrows ? r : nrows - 1) * (uint32_t)k * 2u;

    float acc[R][2];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r][0] = acc[r][1] = 0.0f;

    if constexpr (R == 1) {
      // One row per wave: every group in the form of the last group below
      // (slots past the wave's steps load zeros from outside the
      // descriptor's range; the partial step is the slot after step t1 - 1).
      // Measured on MI355X 1-2.5% faster than the two-part loop for these
      // variants; for two rows and more the two-part loop, whose full groups
      // need fewer registers, is faster.
      const int e0 = (nfull * kLanes + lane) * kVec;
      const bool tail_full = tail && e0 + kVec <= k;
      const int tend = t1 + (tail ? 1 : 0);
      for (int t = t0; t < tend; t += U) {
        u32x4 bv[U][R];
        u32x4 av[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int st = t + u;
          const bool ok = st < t1 || (st == t1 && tail_full);
          const uint32_t off = ok ? (uint32_t)(st * kStepBytes + lane_off) : kOffsetOutOfRange;
#pragma unroll
          for (int r = 0; r < R; ++r) bv[u][r] = __builtin_amdgcn_raw_buffer_load_b128(brsrc, off, soff[r], BPOL);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int st = t + u;
          const bool ok = st < t1 || (st == t1 && tail_full);
          if constexpr (AMODE == A_LDS) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            const u32x4 x = a_lds[ok ? st * kLanes + lane : 0];
            av[u] = ok ? x : z;
          } else {
            const uint32_t off = ok ? (uint32_t)(st * kStepBytes + lane_off) : kOffsetOutOfRange;
            av[u] = __builtin_amdgcn_raw_buffer_load_b128(arsrc, off, 0u, 0);
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
          for (int r = 0; r < R; ++r) accumulate<DT, PROBE>(bv[u][r], av[u], acc[r][0], acc[r][1]);
        }
      }
      draw_ticket();
      if (tail && (k & (kVec - 1)) != 0 && e0 < k && e0 + kVec > k) {
        u32x4 ap;
        if constexpr (AMODE == A_LDS) {
          ap = a_lds[nfull * kLanes + lane];
        } else {
          ap = load_vec_tail(arsrc, e0, k, 0u);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) accumulate<DT, PROBE>(load_vec_tail(brsrc, e0, k, soff[r]), ap, acc[r][0], acc[r][1]);
      }
    } else {
      int t = t0;
      for (; t + U <= t1; t += U) {
        u32x4 bv[U][R];
        u32x4 av[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
          for (int r = 0; r < R; ++r) {
            bv[u][r] = __builtin_amdgcn_raw_buffer_load_b128(brsrc, (t + u) * kStepBytes + lane_off,
                                                             soff[r], BPOL);
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if constexpr (AMODE == A_LDS) {
            av[u] = a_lds[(t + u) * kLanes + lane];
          } else {
            av[u] = __builtin_amdgcn_raw_buffer_load_b128(arsrc, (t + u) * kStepBytes + lane_off, 0u, 0);
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
          for (int r = 0; r < R; ++r) accumulate<DT, PROBE>(bv[u][r], av[u], acc[r][0], acc[r][1]);
        }
      }
      // The last, partial group: the remaining full steps (fewer than U) and,
      // on the last slice, the partial step, loaded in one batch -- one round
      // trip, not one per step.  Every slot loads; a slot past them loads from
      // an offset outside the descriptor's range, which returns zeros without
      // touching memory, so the group has no branches (and no registers of its
      // own beyond the main loop's).  a is zeroed there too, so 0 x inf cannot
      // turn into a NaN.
      const int nrem = t1 - t;                           // 0 .. U-1
      if (nrem > 0 || tail) {
        const int e0 = (nfull * kLanes + lane) * kVec;   // this lane's first element of the partial step
        const bool tail_full = tail && e0 + kVec <= k;   // a whole 16-byte vector inside the row
        u32x4 bv[U][R];
        u32x4 av[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int st = t + u;
          const bool ok = u < nrem || (u == nrem && tail_full);
          const uint32_t off = ok ? (uint32_t)(st * kStepBytes + lane_off) : kOffsetOutOfRange;
#pragma unroll
          for (int r = 0; r < R; ++r) bv[u][r] = __builtin_amdgcn_raw_buffer_load_b128(brsrc, off, soff[r], BPOL);
          if constexpr (AMODE == A_LDS) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            const u32x4 x = a_lds[ok ? st * kLanes + lane : 0];
            av[u] = ok ? x : z;
          } else {
            av[u] = __builtin_amdgcn_raw_buffer_load_b128(arsrc, off, 0u, 0);
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
          for (int r = 0; r < R; ++r) accumulate<DT, PROBE>(bv[u][r], av[u], acc[r][0], acc[r][1]);
        }
        // the one vector that straddles k (rows not 16-byte aligned only)
        if (tail && (k & (kVec - 1)) != 0 && e0 < k && e0 + kVec > k) {
          u32x4 ap;
          if constexpr (AMODE == A_LDS) {
            ap = a_lds[nfull * kLanes + lane];
          } else {
            ap = load_vec_tail(arsrc, e0, k, 0u);
          }
#pragma unroll
          for (int r = 0; r < R; ++r) accumulate<DT, PROBE>(load_vec_tail(brsrc, e0, k, soff[r]), ap, acc[r][0], acc[r][1]);
        }
      }
    }

    float tot[R];
#pragma unroll
    for (int r = 0; r < R; ++r) tot[r] = wave_sum(acc[r][0] + acc[r][1]);

    float mine = tot[0];
#pragma unroll
    for (int r = 1; r < R; ++r) mine = (lane == r) ? tot[r] : mine;
    bool leader = lane < R && row0 + lane < hi;   // holds the sum of row row0 + lane
    if constexpr (S > 1) {
      if (lane < R) part[(rg * S + sl) * R + lane] = mine;
      __syncthreads();
      leader = leader && sl == 0;
      if (leader) {
        float s = 0.0f;
        for (int qq = 0; qq < S; ++qq) s += part[(rg * S + qq) * R + lane];
        mine = s;
      }
      __syncthreads();
    }
    if (leader) {
      if constexpr (XWG) {
        if (G == 1 && (flags & kFlagTicket)) {
          kept = mine;   // published below, with its tag
        } else {
          // agent-scope store: written through this XCD's L2 to the point
          // where every XCD sees it
          __hip_atomic_store(&ws[(int64_t)(row0 + lane) * xwg_row_stride(Q) + q], mine,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      } else {
        c[row0 + lane] = to_bits<DT>(finish<DT>(mine, flags, alpha, bias, row0 + lane));
      }
    }
  }

  draw_ticket();   // (drawn above already on the one-row paths that take it)

  if constexpr (XWG) {
    // Publish, count, combine.  Agent-scope accesses are coherent across the
    // XCDs' separate L2s: an agent-scope store is written through to the
    // memory side (sc1), an agent-scope load fetches past L1 and L2 (sc1),
    // and agent-scope atomics on one address are serialised device-wide.  So:
    //  * each leader's partial went out as an agent-scope store above;
    //    s_waitcnt(0) returns once every store of this wave has been
    //    acknowledged, i.e. is visible to any later agent-scope access, and
    //    the barrier makes every wave of the workgroup reach that point
    //    before thread 0 counts the workgroup in (a release without an L2
    //    write-back: the partials never sat dirty in an L2);
    //  * the counter is advanced by a wrapping increment (old >= Q-1 -> 0,
    //    else old + 1).  The workgroup that reads Q-1 is the last of the Q:
    //    the other Q-1 increments were performed before its own, each after
    //    its workgroup's partials were visible;
    //  * that workgroup then reads the Q partials with agent-scope loads,
    //    issued only after its increment returned (an acquire without an L2
    //    invalidate: the loads themselves bypass the caches), and sums them
    //    in k-group order.
    // The wrap leaves the counter at zero after the Q-th increment, in the
    // same atomic step, so a counter goes back to zero whenever whole calls
    // with this Q have completed -- even calls that raced on it (their c is
    // then undefined).  The host gives every Q its own bank of counters, so
    // a counter only ever sees one Q.  (A __threadfence() here compiles to a
    // full L2 write-back and invalidate and made the split 10x slower.)
    if constexpr (G == 1) {
      // One row group: wave 0 made every store of the workgroup's partials,
      // so it alone waits for them, counts the workgroup in and, if last,
      // combines -- no workgroup barrier on this path (the other waves are
      // done).
      if (wave != 0) return;
      if (flags & kFlagTicket) {
        // Ticketed: the workgroup that drew the last ticket of its
        // generation (ticket % Q == Q - 1) combines.  Every other workgroup
        // of that generation drew its ticket before it, so is already
        // running and finishes without waiting on anything: the combiner's
        // wait always ends.  Producers publish {partial, tag} in one 8-byte
        // agent-scope store (single-copy atomic) and leave, with no
        // acknowledgement wait and no second atomic; the combiner polls the
        // other k-groups' words until each carries this generation's tag,
        // then sums lane q = k-group q in the fixed tree, as the counted
        // combine does (same bits).  The tag is the generation + 1, never 0
        // (a cleared word), and the combiner clears its own k-group's word,
        // so every call rewrites all Q words: a word with the current tag
        // was written in this call.  Calls that raced on one workspace draw
        // tickets from one counter; a generation may then lack a k-group,
        // and its combiner gives up after kTicketSpins polls and writes NaN.
        // Each call draws exactly Q tickets, so the counter stays a multiple
        // of Q and later calls are whole generations again.
        const unsigned t = __builtin_amdgcn_readfirstlane(ticket);
        const unsigned gen = t / (unsigned)Q;
        const unsigned tag = gen + 1u;
        const float my = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                                       __builtin_bit_cast(int, kept)));
        if (t - gen * (unsigned)Q != (unsigned)(Q - 1)) {
          if (lane == 0)
            __hip_atomic_store(&tline[1 + q],
                               ((uint64_t)tag << 32) | __builtin_bit_cast(uint32_t, my),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          return;
        }
        float s = 0.0f;
        if (lane == q) {
          s = my;
          __hip_atomic_store(&tline[1 + q], (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else if (lane < Q) {
          uint64_t w = 0;
          int polls = 0;
          do {
            w = __hip_atomic_load(&tline[1 + lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          } while ((uint32_t)(w >> 32) != tag && ++polls < kTicketSpins);
          s = (uint32_t)(w >> 32) == tag ? __builtin_bit_cast(float, (uint32_t)w)
                                         : __builtin_nanf("");
        }
        s = wave_sum(s);
        if (lane == 0) c[lo] = to_bits<DT>(finish<DT>(s, flags, alpha, bias, lo));
        return;
      }
      __builtin_amdgcn_s_waitcnt(0);
      unsigned old = 0;
      if (lane == 0)
        old = __builtin_amdgcn_atomic_inc32(&cnt[bx * kCntStride], (unsigned)(Q - 1),
                                            __ATOMIC_RELAXED, "agent");
      if (__builtin_amdgcn_readfirstlane(old) != (unsigned)(Q - 1)) return;
      for (int r = lo; r < hi; ++r) {
        float s = 0.0f;
        for (int qq = lane; qq < Q; qq += kLanes)
          s += __hip_atomic_load(&ws[(int64_t)r * xwg_row_stride(Q) + qq], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
        s = wave_sum(s);
        if (lane == 0) c[r] = to_bits<DT>(finish<DT>(s, flags, alpha, bias, r));
      }
      return;
    }
    __shared__ int last;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
      last = __builtin_amdgcn_atomic_inc32(&cnt[bx * kCntStride], (unsigned)(Q - 1),
                                           __ATOMIC_RELAXED, "agent") == (unsigned)(Q - 1);
    }
    __syncthreads();
    if (last) {
      // one wave per row: lane j loads partials j, j+64, ... (all lanes at
      // once, so the loads overlap), then the fixed lane tree of wave_sum
      for (int r = lo + wave; r < hi; r += WAVES) {
        float s = 0.0f;
        for (int qq = lane; qq < Q; qq += kLanes)
          s += __hip_atomic_load(&ws[(int64_t)r * xwg_row_stride(Q) + qq], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
        s = wave_sum(s);
        if (lane == 0) c[r] = to_bits<DT>(finish<DT>(s, flags, alpha, bias, r));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Rows that do not start on a 16-byte boundary (k % 8 != 0, or B itself not
// 16-byte aligned).  Instead of unaligned 16-byte loads, B is read in aligned
// 16-byte granules from the 128-byte cache line that holds the row's first
// element, and a is shifted to match: vector v of row i covers row elements
// [8v - o, 8v - o + 8), o = the row's offset in elements from that line
// (0..63), so it needs a[8v - o .. 8v - o + 7].  With line-aligned windows a
// wave's 1 KiB load covers exactly 8 lines, so no line is fetched by two
// loads (16-byte windows straddle 9 lines and refetch the shared one).  LDS
// holds a twice, shifted by 0 and by 1 element behind kPadA zero elements,
// which makes that window start on a 4-byte boundary for either parity of o
// (two ds_read2_b32).  The first and last vectors of a row are masked element
// by element, so nothing from a neighbouring row (a NaN or inf included)
// enters the sum.  A 128-byte line that holds at least one byte of B never
// crosses a page boundary, so the aligned reads past a row's ends stay in
// mapped memory.  Rows are dealt to waves in balanced contiguous ranges, R
// rows per trip.
constexpr int kLine = 64;               // elements per 128-byte line
constexpr int kPadA = kLine;

__device__ __forceinline__ uint32_t keep_mask(int j0, int k) {
  // element j0 in the low half, j0 + 1 in the high half; keep those in [0, k)
  return ((j0 >= 0 && j0 < k) ? 0x0000ffffu : 0u) | ((j0 + 1 >= 0 && j0 + 1 < k) ? 0xffff0000u : 0u);
}

template <int DT, int R, int U, int WAVES, int BPOL>
__global__ __launch_bounds__(WAVES * kLanes) void gemv_realign_kernel(
    MBD_GEMV_PARAMS) {
  MBD_GEMV_ARGS;
  const uint16_t* __restrict__ B = p.B;
  const uint16_t* __restrict__ a = p.a;
  uint16_t* c = p.c;
  const int k = p.k, flags = p.flags;
  const float alpha = p.alpha;
  const uint16_t* bias = p.bias;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & (kLanes - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // copy 0: a_0[kPadA + x] = a[x]; copy 1: a_1[kPadA + x] = a[x - 1]; zeros elsewhere
  // whole groups of U steps are read (masked beyond the row), so the copies
  // cover ceil(steps / U) * U steps
  const int nsteps_max = ((k + kLine - 1 + kStep - 1) / kStep + U - 1) / U * U;
  const int len = kPadA + nsteps_max * kStep + 8;        // elements per copy, a multiple of 8
  uint32_t* a0w = reinterpret_cast<uint32_t*>(smem);      // len / 2 dwords each
  uint32_t* a1w = a0w + len / 2;
  {
    const __amdgpu_buffer_rsrc_t arsrc = make_rsrc(a, (uint32_t)k * 2u);
    u32x4* a0v = reinterpret_cast<u32x4*>(smem);
    const bool a16 = ((uintptr_t)a & 15u) == 0;
    for (int v = threadIdx.x; v < len / kVec; v += WAVES * kLanes) {
      const int e0 = v * kVec - kPadA;                   // a index of the vector's first element
      u32x4 x = {0u, 0u, 0u, 0u};
      if (a16 && e0 >= 0) {
        x = load_vec_tail(arsrc, e0, k, 0u);
      } else {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < kVec; ++i) {
          const int j = e0 + i;
          if (j >= 0 && j < k) {
            uint32_t h = __builtin_amdgcn_raw_buffer_load_b16(arsrc, j * 2, 0u, 0);
            w[i >> 1] |= h << ((i & 1) * 16);
          }
        }
        x[0] = w[0]; x[1] = w[1]; x[2] = w[2]; x[3] = w[3];
      }
      a0v[v] = x;
    }
    __syncthreads();
    for (int w = threadIdx.x; w < len / 2; w += WAVES * kLanes) {
      const uint32_t cur = a0w[w];
      const uint32_t prev = w > 0 ? a0w[w - 1] : 0u;
      a1w[w] = (cur << 16) | (prev >> 16);               // a_1[x] = a_0[x - 1]
    }
    __syncthreads();
  }

  const int64_t wg = (flags & kFlagXcdContiguous) ? xcd_unit(blockIdx.x, gridDim.x) : blockIdx.x;
  const int64_t unit = wg * WAVES + wave;
  const int lo = share_start(unit, p.rows_q, p.rows_r);
  const int hi = lo + p.rows_q + (unit < p.rows_r ? 1 : 0);

  // R rows per trip (their loads issued together); a second row past the
  // range end repeats the first and is not stored.
  for (int row0 = lo; row0 < hi; row0 += R) {
    const uint16_t* basep[R];       // 16-byte aligned start of each row's granules
    const uint32_t* aw[R];          // the a copy that matches the row's offset
    int o[R], nv[R], abase[R], tmid[R];
    int nsteps = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = row0 + r < hi ? row0 + r : row0;
      const uint16_t* rowp = B + (int64_t)row * k;
      o[r] = (int)(((uintptr_t)rowp >> 1) & (kLine - 1));  // wave-uniform
      nv[r] = k > 0 ? (o[r] + k + kVec - 1) / kVec : 0;    // granules touching the row
      basep[r] = rowp - o[r];                              // 128-byte aligned
      aw[r] = (o[r] & 1) ? a1w : a0w;
      // dword of the a copy lined up with element 0 of granule v: (8v - o + (o & 1) + kPadA) / 2
      abase[r] = (kPadA - o[r] + (o[r] & 1)) >> 1;
      tmid[r] = ((k + o[r]) / kVec) / kLanes;              // steps [1, tmid) need no masks
      const int ns = (nv[r] + kLanes - 1) / kLanes;
      nsteps = ns > nsteps ? ns : nsteps;
    }
    float acc[R][2];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r][0] = acc[r][1] = 0.0f;

    // The steps in groups of U, all loads of a group issued together.  A row's
    // group is "clean" when every granule in it lies inside the row; the
    // others (the row's first granules when o != 0, its last full granules
    // and beyond) are masked after the load.  Granules at or past nv lie
    // outside the descriptor's range: the hardware returns them without a
    // memory access, and the mask clears them whatever they hold.
    for (int t = 0; t < nsteps; t += U) {
      u32x4 bv[R][U], av[R][U];
      bool clean[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        clean[r] = (t > 0 || o[r] == 0) && (t + U <= tmid[r]);
        const __amdgpu_buffer_rsrc_t brsrc = make_rsrc(basep[r], (uint32_t)nv[r] * 16u);
#pragma unroll
        for (int u = 0; u < U; ++u)
          bv[r][u] = __builtin_amdgcn_raw_buffer_load_b128(brsrc, ((t + u) * kLanes + lane) * 16, 0u,
                                                           BPOL);
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int d = abase[r] + ((t + u) * kLanes + lane) * 4;
          av[r][u][0] = aw[r][d]; av[r][u][1] = aw[r][d + 1];
          av[r][u][2] = aw[r][d + 2]; av[r][u][3] = aw[r][d + 3];
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (!clean[r]) {
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int j0 = ((t + u) * kLanes + lane) * kVec - o[r];   // row element of the granule start
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t w = bv[r][u][i];
              bv[r][u][i] = w & keep_mask(j0 + 2 * i, k);
            }
          }
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int u = 0; u < U; ++u) fma8<DT>(bv[r][u], av[r][u], acc[r][0], acc[r][1]);
      }
    }

#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float tot = wave_sum(acc[r][0] + acc[r][1]);
      const int row = row0 + r;
      if (lane == 0 && row < hi) c[row] = to_bits<DT>(finish<DT>(tot, flags, alpha, bias, row));
    }
  }
}

// ---------------------------------------------------------------------------
// The uncoalesced layout, kept for measurement only (TileLang Case Studies,
// Case B "Root Cause": the thread index that varies fastest within a warp
// walked the rows, so neighbouring lanes read addresses a row apart).  Here
// lane l of a wave owns one row and walks k one element at a time: the 64
// loads of one wave instruction land 2k bytes apart.  Never chosen by the
// automatic plan.
template <int DT, int WAVES>
__global__ __launch_bounds__(WAVES * kLanes) void gemv_rowlane_kernel(
    MBD_GEMV_PARAMS) {
  MBD_GEMV_ARGS;
  const uint16_t* __restrict__ B = p.B;
  const uint16_t* __restrict__ a = p.a;
  uint16_t* c = p.c;
  const int n = p.n, k = p.k, flags = p.flags;
  const float alpha = p.alpha;
  const uint16_t* bias = p.bias;
  const int lane = threadIdx.x & (kLanes - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const __amdgpu_buffer_rsrc_t arsrc = make_rsrc(a, (uint32_t)k * 2u);
  // rows of this wave: [row0, row0 + 64); the descriptor starts at row0
  for (int64_t row0 = ((int64_t)blockIdx.x * WAVES + wave) * kLanes; row0 < n;
       row0 += (int64_t)gridDim.x * WAVES * kLanes) {
    const int nrows = (n - row0) < kLanes ? (int)(n - row0) : kLanes;
    const int r = lane < nrows ? lane : nrows - 1;
    const __amdgpu_buffer_rsrc_t brsrc =
        make_rsrc(B + row0 * k, (uint32_t)nrows * (uint32_t)k * 2u);
    const uint32_t roff = (uint32_t)r * (uint32_t)k * 2u;
    float acc = 0.0f;
    for (int j = 0; j < k; ++j) {
      const uint32_t bb = __builtin_amdgcn_raw_buffer_load_b16(brsrc, roff + j * 2, 0u, 0);
      const uint32_t aa = __builtin_amdgcn_raw_buffer_load_b16(arsrc, j * 2, 0u, 0);
      float bf, af;
      if constexpr (DT == DT_F16) {
        bf = (float)__builtin_bit_cast(_Float16, (uint16_t)bb);
        af = (float)__builtin_bit_cast(_Float16, (uint16_t)aa);
      } else {
        bf = __builtin_bit_cast(float, bb << 16);
        af = __builtin_bit_cast(float, aa << 16);
      }
      acc = __builtin_fmaf(bf, af, acc);
    }
    if (lane < nrows) c[row0 + lane] = to_bits<DT>(finish<DT>(acc, flags, alpha, bias, row0 + lane));
  }
}

}  // namespace mbd
