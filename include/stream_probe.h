/*
 * stream_probe.h -- measurement aids shipped next to libgemv.so, in their own
 * library (libmbd_probe.so).  None of them is part of the GEMV path.
 *
 * TileLang Case Studies, Case C discusses the gap between a GPU's rated and
 * its achievable bandwidth for a GEMV; these calls measure the achievable
 * side on this GPU: a plain streaming read (and copy) of a device buffer, and
 * the GEMV kernel itself with its arithmetic taken out, so that the cost of
 * the GEMV's access pattern can be told from the cost of its arithmetic.
 * Every call enqueues on `stream` and returns 0, -1 on a bad argument (nothing
 * launched), or -2 if the launch failed.
 */
#ifndef MBD_STREAM_PROBE_H
#define MBD_STREAM_PROBE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes at device address `src` (16-byte aligned; bytes a
 * non-zero multiple of 1 KiB) with 16-byte loads: `grid` workgroups of four
 * 64-lane waves (0 = one batch of `unroll` KiB per wave, capped at 2^22
 * workgroups); each wave reads one contiguous share of the buffer (shares
 * differ by at most 1 KiB), `unroll` (2, 4, 8 or 16) wave-loads of 1 KiB at a
 * time, folds them into one word with a wave reduction and writes it to
 * out[wave] (out holds out_len >= 4 * grid words).  `nontemporal` != 0 marks
 * the loads non-temporal.  *launched receives the grid used (may be NULL). */
int mbd_stream_read(const void* src, size_t bytes, uint32_t* out, int out_len, int grid, int unroll,
                    int nontemporal, hipStream_t stream, int* launched);

/* Copy `bytes` bytes from src to dst (both 16-byte aligned, not
 * overlapping; bytes a non-zero multiple of 16 KiB) with 16-byte loads and
 * stores: the read + write counterpart of mbd_stream_read.  `grid`
 * workgroups of 256 lanes, 16 KiB per workgroup per loop trip (0 = one trip
 * per workgroup). */
int mbd_stream_copy(const void* src, void* dst, size_t bytes, int grid, int nontemporal,
                    hipStream_t stream);

/* 1 if mbd_gemv_probe has a build of the GEMV plan shape (rows, unroll,
 * waves, splits, cross-workgroup) -- the shapes the automatic plan takes for
 * rows on 16-byte boundaries -- else 0. */
int mbd_gemv_probe_has(int rows, int unroll, int waves, int splits, int xwg);

/* The GEMV kernel of that plan shape with its arithmetic taken out: the same
 * launch as gemv_run_ws makes for a (n, k) B at device address B (16-byte
 * aligned, k % 8 == 0) with `grid` workgroups and `kgroups` k-groups -- the
 * same B loads, row ranges, k-slices, reductions, cross-workgroup combine
 * (through `workspace`, laid out and zero-filled as for gemv_run_ws; NULL
 * when xwg == 0) and one 2-byte store per row into `out` (n elements) -- but
 * each 16-byte vector of B is xor-folded instead of multiplied by a, and a is
 * never read.  The values written are meaningless. */
int mbd_gemv_probe(int rows, int unroll, int waves, int splits, int xwg, const void* B, int64_t n,
                   int64_t k, void* out, void* workspace, int grid, int kgroups, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif
