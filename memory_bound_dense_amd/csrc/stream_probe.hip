// Measurement aids (include/stream_probe.h), not the GEMV path:
//  * mbd_stream_read -- how fast this GPU reads a buffer it does not reuse:
//    every wave streams one contiguous share of the buffer with 16-byte
//    loads, U wave-loads (U KiB) in flight, folds what it read into one word
//    with a DPP wave reduction and writes it -- no per-workgroup serial tail;
//  * mbd_stream_copy -- the read + write counterpart (a state update's mix);
//  * mbd_gemv_probe -- the GEMV kernel itself, built with its arithmetic
//    taken out (gemv_kernel's PROBE flag: the same B loads, grid, k-slices,
//    wave and workgroup reductions and stores; the FMAs replaced by an
//    xor-fold, so a is never read), for the plan shapes the automatic plan
//    uses on rows that start on 16-byte boundaries.  Its time is what the
//    GEMV's access pattern costs on its own.
#include "stream_probe.h"

#include <hip/hip_runtime.h>

#include "gemv_kernel.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / mbd::kLanes;
constexpr uint32_t kBlock = 1024;   // bytes of one wave-load (64 lanes x 16 B)

__device__ __forceinline__ uint32_t wave_add(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false);
  v += (uint32_t)__shfl_xor((int)v, 16, 64);
  v += (uint32_t)__shfl_xor((int)v, 32, 64);
  return v;
}

// Wave w of the grid's W waves owns 1 KiB blocks [w*q + min(w, r), +q + (w < r))
// of the nblk blocks (q = nblk / W, r = nblk % W), and reads them U at a
// time; a slot past its share loads from outside its descriptor's range
// (zeros, no memory access).
template <int U, int POL>
__global__ __launch_bounds__(kThreads) void stream_read(const uint8_t* __restrict__ src,
                                                        uint64_t nblk, uint32_t* __restrict__ out) {
  const uint64_t W = (uint64_t)gridDim.x * kWaves;
  const uint64_t w = (uint64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const uint64_t q = nblk / W, r = nblk % W;
  const uint64_t lo = w * q + (w < r ? w : r);
  const uint32_t cnt = (uint32_t)(q + (w < r ? 1 : 0));
  const __amdgpu_buffer_rsrc_t rs = mbd::make_rsrc(src + lo * kBlock, cnt * kBlock);
  const uint32_t lane_off = (threadIdx.x & 63u) * 16u;
  uint32_t acc = 0;
  for (uint32_t t = 0; t < cnt; t += U) {
    mbd::u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t off = t + u < cnt ? (t + u) * kBlock + lane_off : mbd::kOffsetOutOfRange;
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0u, POL);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc += v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  acc = wave_add(acc);
  if ((threadIdx.x & 63u) == 0) out[w] = acc;
}

// Streaming copy: each workgroup copies 16 KiB per loop trip, every 16-byte
// vector read and written once.
constexpr int kCopyUnroll = 4;
template <int POL>
__global__ __launch_bounds__(kThreads) void stream_copy(const uint8_t* __restrict__ src,
                                                        uint8_t* __restrict__ dst, uint64_t nvec) {
  const uint64_t per = (uint64_t)kThreads * kCopyUnroll;
  const uint64_t nchunks = nvec / per;
  for (uint64_t ch = blockIdx.x; ch < nchunks; ch += gridDim.x) {
    const uint64_t base = ch * per;
    __amdgpu_buffer_rsrc_t r = mbd::make_rsrc(src + base * 16u, kThreads * kCopyUnroll * 16);
    __amdgpu_buffer_rsrc_t w = mbd::make_rsrc(dst + base * 16u, kThreads * kCopyUnroll * 16);
    mbd::u32x4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, ((uint32_t)u * kThreads + threadIdx.x) * 16u, 0u, POL);
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
      __builtin_amdgcn_raw_buffer_store_b128(v[u], w, ((uint32_t)u * kThreads + threadIdx.x) * 16u, 0u, POL);
  }
}

using ReadFn = void (*)(const uint8_t*, uint64_t, uint32_t*);
template <int U>
ReadFn read_fn(int nt) {
  return nt ? &stream_read<U, 2> : &stream_read<U, 0>;
}

// The GEMV kernel in its PROBE build, for the plan shapes (R, U, W, S,
// cross-workgroup) the automatic plan takes on 16-byte aligned rows.
using GemvFn = void (*)(const uint16_t*, const uint16_t*, uint16_t*, int, int, int, int, int, int,
                        int, float, const uint16_t*, float*, unsigned*);
struct ProbeShape {
  int rows, unroll, waves, splits, xwg;
  GemvFn fn;
};
#define MBD_PROBE(R, U, W, S, X)                                                     \
  {R, U, W, S, X,                                                                    \
   &mbd::gemv_kernel<mbd::DT_F16, R, U, W, S, mbd::A_CACHED, 2, (bool)X, true>}
const ProbeShape kProbeShapes[] = {
    MBD_PROBE(1, 2, 4, 1, 0), MBD_PROBE(1, 4, 4, 1, 0), MBD_PROBE(1, 8, 4, 1, 0),
    MBD_PROBE(2, 4, 4, 4, 0), MBD_PROBE(2, 4, 8, 8, 0), MBD_PROBE(2, 4, 8, 4, 0),
    MBD_PROBE(1, 4, 4, 4, 0), MBD_PROBE(1, 4, 8, 8, 0), MBD_PROBE(2, 4, 1, 1, 0),
    MBD_PROBE(1, 4, 2, 1, 0), MBD_PROBE(1, 4, 8, 8, 1), MBD_PROBE(2, 2, 8, 8, 0),
    MBD_PROBE(2, 8, 4, 4, 0), MBD_PROBE(2, 8, 8, 8, 0), MBD_PROBE(1, 2, 4, 4, 0),
    MBD_PROBE(2, 2, 4, 4, 0), MBD_PROBE(1, 2, 8, 8, 1), MBD_PROBE(1, 4, 4, 1, 1),
    MBD_PROBE(2, 3, 8, 8, 0), MBD_PROBE(2, 5, 4, 4, 0), MBD_PROBE(2, 5, 8, 8, 0),
    MBD_PROBE(2, 6, 8, 8, 0), MBD_PROBE(2, 3, 4, 4, 0), MBD_PROBE(3, 2, 8, 8, 0),
    MBD_PROBE(3, 3, 8, 8, 0), MBD_PROBE(2, 2, 4, 1, 0), MBD_PROBE(2, 4, 4, 1, 0),
    MBD_PROBE(4, 2, 4, 1, 0), MBD_PROBE(1, 2, 4, 4, 0), MBD_PROBE(1, 2, 4, 4, 1),
    MBD_PROBE(2, 3, 16, 16, 0),
};
#undef MBD_PROBE

}  // namespace

extern "C" int mbd_stream_copy(const void* src, void* dst, size_t bytes, int grid, int nontemporal,
                               hipStream_t stream) {
  if (!src || !dst || bytes == 0 || (bytes % (kThreads * kCopyUnroll * 16)) != 0 ||
      (((uintptr_t)src | (uintptr_t)dst) % 16) != 0 || grid < 0)
    return -1;
  const uint8_t* s8 = (const uint8_t*)src;
  uint8_t* d8 = (uint8_t*)dst;
  if (s8 < d8 + bytes && d8 < s8 + bytes) return -1;
  const uint64_t nvec = bytes / 16;
  const uint64_t per_wg = (uint64_t)kThreads * kCopyUnroll;
  uint64_t g = grid > 0 ? (uint64_t)grid : nvec / per_wg;
  if (g > (1u << 20)) g = 1u << 20;
  if (g < 1) g = 1;
  if (nontemporal)
    hipLaunchKernelGGL(stream_copy<2>, dim3((unsigned)g), dim3(kThreads), 0, stream, s8, d8, nvec);
  else
    hipLaunchKernelGGL(stream_copy<0>, dim3((unsigned)g), dim3(kThreads), 0, stream, s8, d8, nvec);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

extern "C" int mbd_stream_read(const void* src, size_t bytes, uint32_t* out, int out_len, int grid,
                               int unroll, int nontemporal, hipStream_t stream, int* launched) {
  if (!src || !out || out_len < kWaves || bytes == 0 || (bytes % kBlock) != 0 ||
      ((uintptr_t)src % 16) != 0 || grid < 0)
    return -1;
  ReadFn fn;
  switch (unroll) {
    case 2: fn = read_fn<2>(nontemporal); break;
    case 4: fn = read_fn<4>(nontemporal); break;
    case 8: fn = read_fn<8>(nontemporal); break;
    case 16: fn = read_fn<16>(nontemporal); break;
    default: return -1;
  }
  const uint64_t nblk = bytes / kBlock;
  // default grid: one batch of `unroll` wave-loads per wave
  uint64_t g = grid > 0 ? (uint64_t)grid : (nblk + (uint64_t)kWaves * unroll - 1) / ((uint64_t)kWaves * unroll);
  if (g > (1u << 22)) g = 1u << 22;
  if (g < 1) g = 1;
  if (g * kWaves > (uint64_t)out_len) return -1;
  // a wave's share must fit one buffer descriptor (< 2^31 bytes)
  if ((nblk / (g * kWaves) + 1) * kBlock >= (1ull << 31)) return -1;
  if (launched) *launched = (int)g;
  const uint8_t* s8 = (const uint8_t*)src;
  void* args[] = {(void*)&s8, (void*)&nblk, (void*)&out};
  hipError_t e = hipLaunchKernel((const void*)fn, dim3((unsigned)g), dim3(kThreads), args, 0, stream);
  return e == hipSuccess ? 0 : -2;
}

extern "C" int mbd_gemv_probe_has(int rows, int unroll, int waves, int splits, int xwg) {
  for (const ProbeShape& p : kProbeShapes)
    if (p.rows == rows && p.unroll == unroll && p.waves == waves && p.splits == splits && p.xwg == xwg)
      return 1;
  return 0;
}

extern "C" int mbd_gemv_probe(int rows, int unroll, int waves, int splits, int xwg, const void* B,
                              int64_t n, int64_t k, void* out, void* workspace, int grid,
                              int kgroups, hipStream_t stream) {
  const ProbeShape* ps = nullptr;
  for (const ProbeShape& p : kProbeShapes)
    if (p.rows == rows && p.unroll == unroll && p.waves == waves && p.splits == splits && p.xwg == xwg)
      ps = &p;
  if (!ps || !B || !out || n <= 0 || k <= 0 || k % 8 != 0 || ((uintptr_t)B % 16) != 0 ||
      n > (1 << 30) || k > (1 << 27) || grid <= 0 ||
      (xwg ? (!workspace || kgroups < 1 || kgroups > mbd::kXwgMaxQ ||
              n * mbd::xwg_row_stride(kgroups) > (int64_t)mbd::kWsFloats || grid > mbd::kXwgRanges)
           : kgroups != 1))
    return -1;
  // the row ranges and k-slices exactly as gemv_run_ws deals them; the
  // workspace (xwg) is laid out as gemv_run_ws's: the counter banks, then
  // the partials
  const int64_t rb = (int64_t)(waves / splits) * rows;
  if ((int64_t)grid > (n + rb - 1) / rb) return -1;
  const int64_t units = (splits == 1 && !xwg) ? (int64_t)grid * (waves / splits) : grid;
  int rows_q = (int)(n / units), rows_r = (int)(n % units);
  const int64_t nfull = k / mbd::kStep, nsl = (int64_t)splits * kgroups;
  int slice_q = (int)(nfull / nsl), slice_r = (int)(nfull % nsl);
  const uint16_t* Bp = (const uint16_t*)B;
  const uint16_t* ap = Bp;   // never read in the PROBE build
  uint16_t* cp = (uint16_t*)out;
  const uint16_t* bias = nullptr;
  unsigned* cnt =
      xwg ? (unsigned*)workspace + (size_t)(kgroups - 1) * mbd::kXwgRanges * mbd::kCntStride : nullptr;
  float* ws = xwg ? (float*)((char*)workspace + mbd::kWsCounterBytes) : nullptr;
  int ni = (int)n, ki = (int)k, flags = 0;
  float alpha = 1.0f;
  void* args[] = {(void*)&Bp,      (void*)&ap,      (void*)&cp,      (void*)&ni,
                  (void*)&ki,      (void*)&flags,   (void*)&rows_q,  (void*)&rows_r,
                  (void*)&slice_q, (void*)&slice_r, (void*)&alpha,   (void*)&bias,
                  (void*)&ws,      (void*)&cnt};
  const size_t lds = splits > 1 ? (size_t)waves * rows * sizeof(float) : 0;
  // the cross-workgroup split's grid is (k-groups, row ranges), as gemv_run_ws launches it
  hipError_t e = hipLaunchKernel((const void*)ps->fn, xwg ? dim3((unsigned)kgroups, (unsigned)grid)
                                                          : dim3((unsigned)grid),
                                 dim3((unsigned)(waves * mbd::kLanes)), args, lds, stream);
  return e == hipSuccess ? 0 : -2;
}
