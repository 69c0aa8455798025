/*
 * gla_decode.h -- one decode step of gated linear attention (GLA), in
 * libgemv.so next to the GEMV (same handle, same status codes, include/gemv.h).
 *
 * Operation (TileLang Case Studies, Case D "Background"), for each of bh
 * independent (batch, head) pairs h:
 *
 *     S_new[h] = diag(exp(gk[h])) S[h] + outer(k[h], v[h])
 *     o[h]     = scale * q[h]^T S_new[h]
 *
 * Shapes and types: q, k, gk are (bh, dk) and v is (bh, dv), dense, of the
 * 16-bit dtype; the state S is float32 (bh, dk, dv), row-major (row i = the
 * dk index, contiguous along dv); o is (bh, dv) of the dtype.  The state is
 * updated in fp32 (exp from the device math library, one FMA per element)
 * and stored as float32; o is summed in fp32 over dk in a fixed order and
 * rounded once (nearest-even) into the dtype.  The pages do not state the
 * state's precision: float32 state and a 16-bit o are this library's reading.
 *
 * Pointers are caller-owned device pointers on the handle's GPU.  S_out may
 * be S_in (the state updated in place) but must not partly overlap it; o must
 * not overlap any input or the state.  S_in and S_out must be 16-byte
 * aligned and dv a multiple of 4; the 16-bit arrays need 2-byte alignment.
 *
 * Like gemv_run: host validation, one kernel enqueued on `stream`, no
 * allocation, no synchronisation; on any error nothing is launched.
 * bh == 0 or dv == 0 is a no-op; dk == 0 writes o = 0 (the empty sum).
 * Limits: dk, dv <= 65536, dk * dv <= 2^28, bh <= 2^30 (GEMV_ERR_TOO_LARGE);
 * gla_decode_step also returns GEMV_ERR_TOO_LARGE when bh times the number of
 * column blocks it picks (ceil(dv / 32) to ceil(dv / 128)) exceeds 2^23.
 */
#ifndef MBD_GLA_DECODE_H
#define MBD_GLA_DECODE_H

#include "gemv.h"

#ifdef __cplusplus
extern "C" {
#endif

gemv_status_t gla_decode_step(gemv_handle_t h, const void* q, const void* k, const void* v,
                              const void* gk, const float* S_in, float* S_out, void* o,
                              int64_t bh, int64_t dk, int64_t dv, float scale, gemv_dtype_t dtype,
                              hipStream_t stream);

/* The host checks of gla_decode_step, in its order (no handle, no GPU). */
gemv_status_t gla_check_args(const void* q, const void* k, const void* v, const void* gk,
                             const float* S_in, const float* S_out, const void* o, int64_t bh,
                             int64_t dk, int64_t dv, gemv_dtype_t dtype);

#ifdef __cplusplus
}
#endif

#endif /* MBD_GLA_DECODE_H */
