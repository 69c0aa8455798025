/*
 * stream_probe.h -- measurement aid shipped next to libgemv.so: a plain
 * streaming read of a device buffer, to measure the HBM read bandwidth this
 * GPU delivers in practice (the ceiling a bandwidth-bound kernel such as the
 * GEMV can approach; TileLang Case Studies, Case C discusses the gap between
 * the rated and the achievable bandwidth of a GEMV).
 *
 * It is not part of the GEMV path.  Library: libmbd_probe.so.
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
 * non-zero multiple of 16 KiB) with 16-byte loads, `grid` workgroups of 256
 * lanes that each read 16 KiB per loop trip (0 = one trip per workgroup,
 * capped at 2^20 workgroups),
 * `nontemporal` != 0 marks the loads non-temporal; `xcd_contiguous` != 0
 * (with a grid that is a multiple of 8) lets the workgroups of each XCD read
 * one contiguous eighth of the buffer instead of every grid-th chunk.  Each workgroup writes one
 * 32-bit checksum to out[blockIdx] (out holds >= the launched grid; pass
 * out_len to bound it).  Enqueued on `stream`; returns 0 on success, -1 on a
 * bad argument, -2 if the launch failed.  *launched receives the grid used
 * (may be NULL). */
int mbd_stream_read(const void* src, size_t bytes, uint32_t* out, int out_len, int grid,
                    int nontemporal, int xcd_contiguous, hipStream_t stream, int* launched);

/* Copy `bytes` bytes from src to dst (both 16-byte aligned, not
 * overlapping; bytes a non-zero multiple of 16 KiB) with 16-byte loads and
 * stores: the read + write counterpart of mbd_stream_read.  `grid` as there
 * (0 = one trip per workgroup).  Returns 0, -1 on a bad argument, -2 if the
 * launch failed. */
int mbd_stream_copy(const void* src, void* dst, size_t bytes, int grid, int nontemporal,
                    hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif
