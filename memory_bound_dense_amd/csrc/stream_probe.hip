// Streaming-read probe: how fast can this GPU read a buffer it does not
// reuse?  Every lane reads 16-byte vectors, a workgroup-stride loop covers the
// buffer, and each workgroup folds what it read into one checksum so the
// loads cannot be dropped.  Measurement aid only (include/stream_probe.h).
#include "stream_probe.h"

#include <hip/hip_runtime.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int kRsrcWord3 = 0x00020000;

// xcd != 0: workgroup b (dispatched to XCD b % 8) reads the chunks of a
// contiguous eighth of the buffer instead of every gridDim-th chunk.
template <int POL>
__global__ __launch_bounds__(kThreads) void stream_read(const uint8_t* __restrict__ src,
                                                        uint64_t nvec, uint32_t* __restrict__ out,
                                                        int xcd) {
  uint32_t acc = 0;
  const uint64_t per = (uint64_t)kThreads * kUnroll;
  const uint64_t nchunks = nvec / per;
  uint64_t first = blockIdx.x, step = gridDim.x, stop = nchunks;
  if (xcd && gridDim.x % 8 == 0) {
    // XCD x = blockIdx % 8 owns chunks [x*nchunks/8, (x+1)*nchunks/8)
    const uint64_t x = blockIdx.x % 8, i = blockIdx.x / 8, g8 = gridDim.x / 8;
    const uint64_t lo = x * nchunks / 8, hi = (x + 1) * nchunks / 8;
    first = lo + i;
    step = g8;
    stop = hi;
  }
  for (uint64_t ch = first; ch < stop; ch += step) {
    const uint64_t base = ch * per;
    // one descriptor per whole 16 KiB chunk (the host only accepts whole
    // chunks), so every offset below is inside the buffer
    __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(src + base * 16u), (short)0, kThreads * kUnroll * 16, kRsrcWord3);
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t off = ((uint32_t)u * kThreads + threadIdx.x) * 16u;
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0u, POL);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t x0 = v[u][0], x1 = v[u][1], x2 = v[u][2], x3 = v[u][3];
      acc += x0 ^ x1 ^ x2 ^ x3;
    }
  }
  __shared__ uint32_t red[kThreads];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
    for (int i = 0; i < kThreads; ++i) s += red[i];
    out[blockIdx.x] = s;
  }
}

// Streaming copy: the same chunk walk, each 16-byte vector read and written
// once (read + write traffic, the mix of a state update).
template <int POL>
__global__ __launch_bounds__(kThreads) void stream_copy(const uint8_t* __restrict__ src,
                                                        uint8_t* __restrict__ dst, uint64_t nvec) {
  const uint64_t per = (uint64_t)kThreads * kUnroll;
  const uint64_t nchunks = nvec / per;
  for (uint64_t ch = blockIdx.x; ch < nchunks; ch += gridDim.x) {
    const uint64_t base = ch * per;
    __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(src + base * 16u), (short)0, kThreads * kUnroll * 16, kRsrcWord3);
    __amdgpu_buffer_rsrc_t w = __builtin_amdgcn_make_buffer_rsrc(
        dst + base * 16u, (short)0, kThreads * kUnroll * 16, kRsrcWord3);
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, ((uint32_t)u * kThreads + threadIdx.x) * 16u, 0u, POL);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      __builtin_amdgcn_raw_buffer_store_b128(v[u], w, ((uint32_t)u * kThreads + threadIdx.x) * 16u, 0u, POL);
  }
}

}  // namespace

extern "C" int mbd_stream_copy(const void* src, void* dst, size_t bytes, int grid, int nontemporal,
                               hipStream_t stream) {
  if (!src || !dst || bytes == 0 || (bytes % (kThreads * kUnroll * 16)) != 0 ||
      (((uintptr_t)src | (uintptr_t)dst) % 16) != 0 || grid < 0)
    return -1;
  const uint8_t* s8 = (const uint8_t*)src;
  uint8_t* d8 = (uint8_t*)dst;
  if (s8 < d8 + bytes && d8 < s8 + bytes) return -1;
  const uint64_t nvec = bytes / 16;
  const uint64_t per_wg = (uint64_t)kThreads * kUnroll;
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
                               int nontemporal, int xcd, hipStream_t stream, int* launched) {
  if (!src || !out || out_len < 1 || bytes == 0 || (bytes % (kThreads * kUnroll * 16)) != 0 ||
      ((uintptr_t)src % 16) != 0 || grid < 0)
    return -1;
  const uint64_t nvec = bytes / 16;
  const uint64_t per_wg = (uint64_t)kThreads * kUnroll;
  uint64_t g = grid > 0 ? (uint64_t)grid : (nvec + per_wg - 1) / per_wg;
  if (g > (1u << 20)) g = 1u << 20;
  if (g < 1) g = 1;
  if (g > (uint64_t)out_len) return -1;
  if (launched) *launched = (int)g;
  if (nontemporal)
    hipLaunchKernelGGL(stream_read<2>, dim3((unsigned)g), dim3(kThreads), 0, stream,
                       (const uint8_t*)src, nvec, out, xcd);
  else
    hipLaunchKernelGGL(stream_read<0>, dim3((unsigned)g), dim3(kThreads), 0, stream,
                       (const uint8_t*)src, nvec, out, xcd);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
