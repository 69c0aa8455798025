// libgemv.so, continued: one GLA decode step (include/gla_decode.h) over the
// kernel of gla_kernel.h, on a handle made by gemv_create.
#include "gla_decode.h"

#include "gla_kernel.h"
#include "handle.h"

using mbd_host::kMagic;
using mbd_host::kPolNT;

namespace {

bool overlaps(uintptr_t p0, size_t b0, uintptr_t p1, size_t b1) {
  return b0 && b1 && p0 < p1 + b1 && p1 < p0 + b0;
}

}  // namespace

extern "C" gemv_status_t gla_check_args(const void* q, const void* k, const void* v,
                                        const void* gk, const float* S_in, const float* S_out,
                                        const void* o, int64_t bh, int64_t dk, int64_t dv,
                                        gemv_dtype_t dtype) {
  if (dtype != GEMV_F16 && dtype != GEMV_BF16) return GEMV_ERR_UNSUPPORTED_DTYPE;
  if (bh < 0 || dk < 0 || dv < 0) return GEMV_ERR_INVALID_ARG;
  if (bh == 0 || dv == 0) return GEMV_OK;
  if (dv % 4 != 0) return GEMV_ERR_INVALID_ARG;
  if (!o || (dk > 0 && (!q || !k || !v || !gk || !S_in || !S_out))) return GEMV_ERR_INVALID_ARG;
  const uintptr_t u16 = (uintptr_t)o | (dk > 0 ? ((uintptr_t)q | (uintptr_t)k | (uintptr_t)v |
                                                   (uintptr_t)gk) : 0u);
  if (u16 & 1u) return GEMV_ERR_MISALIGNED;
  if (dk > 0 && (((uintptr_t)S_in | (uintptr_t)S_out) & 15u)) return GEMV_ERR_MISALIGNED;
  if (dk > 65536 || dv > 65536 || dk * dv > ((int64_t)1 << 28) || bh > ((int64_t)1 << 30))
    return GEMV_ERR_TOO_LARGE;
  const size_t ob = (size_t)bh * dv * 2;
  if (dk > 0) {
    const size_t sb = (size_t)bh * dk * dv * 4, kb = (size_t)bh * dk * 2, vb = (size_t)bh * dv * 2;
    const uintptr_t si = (uintptr_t)S_in, so = (uintptr_t)S_out;
    if (si != so && overlaps(si, sb, so, sb)) return GEMV_ERR_ALIASING;
    const uintptr_t small[4] = {(uintptr_t)q, (uintptr_t)k, (uintptr_t)gk, (uintptr_t)v};
    const size_t sizes[4] = {kb, kb, kb, vb};
    for (int i = 0; i < 4; ++i) {
      if (overlaps(small[i], sizes[i], so, sb) || overlaps(small[i], sizes[i], (uintptr_t)o, ob))
        return GEMV_ERR_ALIASING;
    }
    if (overlaps((uintptr_t)o, ob, si, sb) || overlaps((uintptr_t)o, ob, so, sb))
      return GEMV_ERR_ALIASING;
  }
  return GEMV_OK;
}

namespace {

// Heads of at most this many rows stage exp(gk), k and q in LDS (6 KiB).
constexpr int64_t kGlaStageRows = 512;

using GlaFn = void (*)(const float*, float*, int, int, const uint16_t*, const uint16_t*,
                       const uint16_t*, const uint16_t*, uint16_t*, float);

}  // namespace

extern "C" gemv_status_t gla_decode_step(gemv_handle_t h, const void* q, const void* k,
                                         const void* v, const void* gk, const float* S_in,
                                         float* S_out, void* o, int64_t bh, int64_t dk, int64_t dv,
                                         float scale, gemv_dtype_t dtype, hipStream_t stream) {
  if (!h || h->magic != kMagic) return report(nullptr, GEMV_ERR_NULL_HANDLE, "gla_decode_step");
  gemv_status_t s = gla_check_args(q, k, v, gk, S_in, S_out, o, bh, dk, dv, dtype);
  if (s != GEMV_OK) return report(h, s, "gla_decode_step arguments");
  if (bh == 0 || dv == 0) return GEMV_OK;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return report(h, GEMV_ERR_HIP, "hipGetDevice");
  if (dev != h->device) return report(h, GEMV_ERR_WRONG_DEVICE, "gla_decode_step");
  // The widest column block (8, 16 or 32 lanes x 4 columns) that still gives
  // >= 16 workgroups per CU; state loads and stores non-temporal (measured on
  // MI355X: ~13% faster than the default policy).  Heads of at most
  // kGlaStageRows rows get exp(gk), k and q staged once per workgroup in LDS
  // when the grid has at least one workgroup per CU.
  static const GlaFn fns[2][2][3] = {
      {{&mbd::gla_decode_kernel<mbd::DT_F16, 8, 4, kPolNT, kPolNT, false>,
        &mbd::gla_decode_kernel<mbd::DT_F16, 16, 4, kPolNT, kPolNT, false>,
        &mbd::gla_decode_kernel<mbd::DT_F16, 32, 4, kPolNT, kPolNT, false>},
       {&mbd::gla_decode_kernel<mbd::DT_F16, 8, 4, kPolNT, kPolNT, true>,
        &mbd::gla_decode_kernel<mbd::DT_F16, 16, 4, kPolNT, kPolNT, true>,
        &mbd::gla_decode_kernel<mbd::DT_F16, 32, 4, kPolNT, kPolNT, true>}},
      {{&mbd::gla_decode_kernel<mbd::DT_BF16, 8, 4, kPolNT, kPolNT, false>,
        &mbd::gla_decode_kernel<mbd::DT_BF16, 16, 4, kPolNT, kPolNT, false>,
        &mbd::gla_decode_kernel<mbd::DT_BF16, 32, 4, kPolNT, kPolNT, false>},
       {&mbd::gla_decode_kernel<mbd::DT_BF16, 8, 4, kPolNT, kPolNT, true>,
        &mbd::gla_decode_kernel<mbd::DT_BF16, 16, 4, kPolNT, kPolNT, true>,
        &mbd::gla_decode_kernel<mbd::DT_BF16, 32, 4, kPolNT, kPolNT, true>}}};
  int sel = 0;
  const int64_t want = 16 * (int64_t)h->num_cus;
  for (int c = 2; c >= 0; --c) {
    const int64_t cw = 4 * (8 << c);
    if (bh * ((dv + cw - 1) / cw) >= want || c == 0) { sel = c; break; }
  }
  const int64_t cw = 4 * (8 << sel);
  const int64_t nblk = (dv + cw - 1) / cw;   // the kernel derives the same count from dv
  const int64_t grid = bh * nblk;
  // staging pays once the grid covers every CU; below that a workgroup's
  // wait for the staged rows sits on the critical path of a latency-bound
  // launch (measured on MI355X, 128 x 128 heads: 32 heads 3.50 us without
  // against 3.89 us with; 128 heads 4.84 against 4.71)
  // (dk == 0, o the empty sum, runs in either form: neither reads a row
  // scalar, a state row or v then, so those inputs may be null)
  const int stage = (dk <= kGlaStageRows && grid >= h->num_cus) ? 1 : 0;
  const size_t lds = stage ? (size_t)(3 * dk) * sizeof(float) : 0;
  // one workgroup per (head, column block); its work-items along x (a 32-bit
  // field of the dispatch) are kept at most 2^31
  if (grid > ((int64_t)1 << 31) / mbd::kGlaThreads) return report(h, GEMV_ERR_TOO_LARGE, "gla grid");
  const uint16_t *qp = (const uint16_t*)q, *kp = (const uint16_t*)k, *vp = (const uint16_t*)v,
                 *gp = (const uint16_t*)gk;
  uint16_t* op = (uint16_t*)o;
  int dki = (int)dk, dvi = (int)dv;
  void* args[] = {(void*)&S_in, (void*)&S_out, (void*)&dki, (void*)&dvi, (void*)&vp,
                  (void*)&gp,   (void*)&kp,    (void*)&qp,  (void*)&op,  (void*)&scale};
  hipError_t e = hipLaunchKernel((const void*)fns[dtype][stage][sel], dim3((unsigned)grid),
                                 dim3(mbd::kGlaThreads), args, lds, stream);
  if (e != hipSuccess) return report(h, GEMV_ERR_HIP, hipGetErrorString(e));
  return GEMV_OK;
}
