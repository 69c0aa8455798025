// One decode step of gated linear attention for gfx950 (TileLang Case
// Studies, Case D "Background"), per (batch, head):
//
//     S_new = diag(exp(gk)) S + outer(k, v)        S: DK x DV, float32
//     o     = scale * q^T S_new                    o: DV, 16-bit dtype
//
// Like the GEMV this is bound by HBM: the state is read once and written once
// (8 bytes per element) and everything else is a few KiB.  The pages' kernel
// (Case D) streams state tiles through shared memory with TMA pipelines in
// two passes; here one pass does both: every lane owns 4 consecutive state
// columns of a column block and walks the rows of the head, so each state
// element is loaded once (16-byte buffer load), updated in registers, stored
// once (16-byte buffer store) and folded into its column's partial of o in
// the same step.  There is no second pass over the state and no shared tile
// to race on.  The row groups' partials of o are summed through LDS in a
// fixed order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemv_kernel.h"

namespace mbd {

constexpr int kGlaThreads = 256;

// LPR lanes per row, 4 columns each: a column block of 4*LPR columns and
// kGlaThreads/LPR row groups.  Workgroup b handles head b / nblk and column
// block b % nblk.  S_out may equal S_in (each 16 bytes are read, then written,
// by one lane).
// STAGE: exp(gk), k and q of the head are computed once per workgroup into
// LDS (3 * dk floats of dynamic LDS) instead of being loaded -- and exp taken
// -- by every lane of a row group for every row; the host picks it when the
// head is short enough for that LDS to stay small.
template <int DT, int LPR, int ROWS = 4, int LPOL = 0, int SPOL = 0, bool STAGE = false>
// Parameters in the order a workgroup needs them: the first 14 dwords
// (everything up to q) are preloaded into SGPRs at wave launch, so no load
// of the trip waits on a kernel-argument fetch; o and scale, needed only at
// the end, are fetched from the argument segment.
__global__ __launch_bounds__(kGlaThreads) void gla_decode_kernel(
    const float* S_in, float* S_out, int dk, int dv, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ gk, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ q, uint16_t* __restrict__ o, float scale) {
  constexpr int CW = 4 * LPR;                 // columns per block
  constexpr int RG = kGlaThreads / LPR;       // row groups
  const int nblk = (dv + CW - 1) / CW;        // column blocks per head
  __shared__ float part[RG][CW];

  const int t = threadIdx.x;
  const int c4 = t % LPR;
  const int rg = t / LPR;
  const int64_t head = blockIdx.x / nblk;
  const int blk = blockIdx.x - (int)(head * nblk);
  const int j0 = blk * CW + c4 * 4;           // first column of this lane
  const bool active = j0 < dv;                // dv % 4 == 0: a lane's 4 columns are all in or all out

  const int64_t rowbase = head * dk;          // row index of the head's first state row
  const __amdgpu_buffer_rsrc_t sin_r =
      make_rsrc(S_in + rowbase * dv, (uint32_t)dk * (uint32_t)dv * 4u);
  const __amdgpu_buffer_rsrc_t sout_r =
      make_rsrc(S_out + rowbase * dv, (uint32_t)dk * (uint32_t)dv * 4u);

  // ROWS rows per trip, their loads issued together, and the next trip's
  // loads issued before this trip's update (a lane only ever rewrites the 16
  // bytes it has itself read, so this is safe in place too).  The first
  // trip's loads, and v, are issued before the staging below, so their
  // latency overlaps it.  Rows past dk load from outside the descriptor's
  // range (zeros, no memory access) and are not stored.  LPOL / SPOL:
  // cache-policy bits of the state loads / stores.
  constexpr int kRows = ROWS;
  constexpr int kTrip = kRows * RG;
  auto load_trip = [&](int i0, u32x4 (&sv)[kRows]) {
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int i = i0 + r * RG;
      const uint32_t off = i < dk ? ((uint32_t)i * (uint32_t)dv + (uint32_t)j0) * 4u : kOffsetOutOfRange;
      sv[r] = __builtin_amdgcn_raw_buffer_load_b128(sin_r, off, 0u, LPOL);
    }
  };
  // Without staging, the row scalars (gk, k, q) of a trip travel with its
  // state rows: loaded a trip ahead, as raw 16-bit values, through buffer
  // descriptors whose range is the head's dk rows -- a row past dk (every
  // row when dk == 0) reads zero with no memory access -- so no branch holds
  // a load back and nothing waits on one memory round trip before issuing
  // the next.  (With both behind conditions the compiler waited for the
  // state before the loop and for each row's scalars in turn: several round
  // trips where one suffices.)  A zero row gives e = 1, k = q = 0 and a
  // zero state: its update is computed and dropped by the selects below.
  const __amdgpu_buffer_rsrc_t gk_r = make_rsrc(gk + rowbase, (uint32_t)dk * 2u);
  const __amdgpu_buffer_rsrc_t k_r = make_rsrc(k + rowbase, (uint32_t)dk * 2u);
  const __amdgpu_buffer_rsrc_t q_r = make_rsrc(q + rowbase, (uint32_t)dk * 2u);
  auto load_scalars = [&](int i0, uint16_t (&sg)[kRows], uint16_t (&sk)[kRows],
                          uint16_t (&sq)[kRows]) {
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int i = i0 + r * RG;
      const uint32_t off = i < dk ? (uint32_t)i * 2u : kOffsetOutOfRange;
      sg[r] = __builtin_amdgcn_raw_buffer_load_b16(gk_r, off, 0u, 0);
      sk[r] = __builtin_amdgcn_raw_buffer_load_b16(k_r, off, 0u, 0);
      sq[r] = __builtin_amdgcn_raw_buffer_load_b16(q_r, off, 0u, 0);
    }
  };
  u32x4 cur[kRows];
  uint16_t cg[kRows], ck[kRows], cq[kRows];
  float vj[4] = {0.f, 0.f, 0.f, 0.f};
  if (active) {
    load_trip(rg, cur);
    if constexpr (!STAGE) load_scalars(rg, cg, ck, cq);
    // v through a descriptor over the head's dv values whose range is empty
    // when dk == 0 (the inputs other than o may then be null buffers): a
    // load that reads nothing there, rather than a branch around it -- a
    // branch made the compiler widen v inside it, and so wait for every load
    // issued before v (the first trip's state rows) before the loop
    const __amdgpu_buffer_rsrc_t v_r =
        make_rsrc(v + (dk > 0 ? head * dv : 0), dk > 0 ? (uint32_t)dv * 2u : 0u);
    const auto vv = __builtin_amdgcn_raw_buffer_load_b64(v_r, (uint32_t)j0 * 2u, 0u, 0);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      vj[c] = widen<DT>((uint16_t)(vv[c >> 1] >> (16 * (c & 1))));
  }

  extern __shared__ float gla_rows[];        // STAGE: e[0..dk), k[dk..2dk), q[2dk..3dk)
  if constexpr (STAGE) {
    for (int i = t; i < dk; i += kGlaThreads) {
      gla_rows[i] = expf(widen<DT>(gk[rowbase + i]));
      gla_rows[dk + i] = widen<DT>(k[rowbase + i]);
      gla_rows[2 * dk + i] = widen<DT>(q[rowbase + i]);
    }
    __syncthreads();
  }

  float oacc[4] = {0.f, 0.f, 0.f, 0.f};
  if (active) {
    for (int i0 = rg; i0 < dk; i0 += kTrip) {
      // The next trip's loads go out before this trip waits on anything.
      // Without staging they are issued unconditionally (state rows past dk
      // come from outside the descriptor's range: no memory access), and
      // the update below is branch-free, so no branch holds a load back.
      // With staging the loads are conditional and the update branches per
      // row (measured on MI355X: 0.6-4.6% faster there than the
      // unconditional form; without staging the unconditional form is 6%
      // faster at 32 heads).
      const bool more = i0 + kTrip < dk;
      u32x4 nxt[kRows];
      uint16_t ng[kRows], nk[kRows], nq[kRows];
      if constexpr (STAGE) {
        if (more) load_trip(i0 + kTrip, nxt);
      } else {
        load_trip(i0 + kTrip, nxt);
        load_scalars(i0 + kTrip, ng, nk, nq);
      }
      float e[kRows], ki[kRows], qi[kRows];
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        if constexpr (STAGE) {
          const int i = i0 + r * RG;
          if (i < dk) {
            e[r] = gla_rows[i];
            ki[r] = gla_rows[dk + i];
            qi[r] = gla_rows[2 * dk + i];
          }
        } else {
          e[r] = expf(widen<DT>(cg[r]));
          ki[r] = widen<DT>(ck[r]);
          qi[r] = widen<DT>(cq[r]);
        }
      }
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        const int i = i0 + r * RG;
        if constexpr (STAGE) {
          if (i < dk) {
            u32x4 nv;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const uint32_t w = cur[r][c];
              const float sn = __builtin_fmaf(ki[r], vj[c], e[r] * __builtin_bit_cast(float, w));
              nv[c] = __builtin_bit_cast(uint32_t, sn);
              oacc[c] = __builtin_fmaf(qi[r], sn, oacc[c]);
            }
            __builtin_amdgcn_raw_buffer_store_b128(
                nv, sout_r, ((uint32_t)i * (uint32_t)dv + (uint32_t)j0) * 4u, 0u, SPOL);
          }
        } else {
          // every slot is updated (a row past dk holds zero scalars and a
          // zero state) and kept by a select; only the store is conditional
          const bool live = i < dk;
          u32x4 nv;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const uint32_t w = cur[r][c];
            const float sn = __builtin_fmaf(ki[r], vj[c], e[r] * __builtin_bit_cast(float, w));
            nv[c] = __builtin_bit_cast(uint32_t, sn);
            const float acc = __builtin_fmaf(qi[r], sn, oacc[c]);
            oacc[c] = live ? acc : oacc[c];
          }
          if (live)
            __builtin_amdgcn_raw_buffer_store_b128(
                nv, sout_r, ((uint32_t)i * (uint32_t)dv + (uint32_t)j0) * 4u, 0u, SPOL);
        }
      }
      if constexpr (STAGE) {
        if (more) {
#pragma unroll
          for (int r = 0; r < kRows; ++r) cur[r] = nxt[r];
        }
      } else {
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
          cur[r] = nxt[r];
          cg[r] = ng[r];
          ck[r] = nk[r];
          cq[r] = nq[r];
        }
      }
    }
  }

#pragma unroll
  for (int c = 0; c < 4; ++c) part[rg][c4 * 4 + c] = oacc[c];
  __syncthreads();
  if (t < CW) {
    const int j = blk * CW + t;
    if (j < dv) {
      float s = 0.0f;
      for (int r = 0; r < RG; ++r) s += part[r][t];
      o[head * dv + j] = to_bits<DT>(scale * s);
    }
  }
}

}  // namespace mbd
