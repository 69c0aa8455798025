/*
 * gemv.h -- C ABI of the MI355X (gfx950) dense GEMV library, libgemv.so.
 *
 * Operation (TileLang Case Studies, Case B "Background"): the dense
 * matrix-vector product
 *
 *     c[i] = sum_{j=0}^{k-1} B[i][j] * a[j],      0 <= i < n,
 *
 * with B an (n, k) matrix, a a (k,) vector and c an (n,) vector, all of one
 * 16-bit floating-point dtype (IEEE binary16 or bfloat16).  Products are
 * summed in fp32 and each c[i] is rounded once, to nearest-even, into the
 * dtype.  The pages leave the accumulation type and the output rounding
 * unstated; fp32 accumulation and round-to-nearest-even are this library's
 * reading.  IEEE special values propagate (NaN in -> NaN out, inf*0 -> NaN,
 * overflow -> inf); subnormals are kept.
 *
 * Layout.  B is row-major and dense: row i starts at element i*k (leading
 * dimension == k, no stride argument), as in Case B where lanes that walk k
 * read one contiguous span of a row.  a and c are dense vectors.  Every
 * pointer is a device pointer on the handle's GPU and needs 2-byte (element)
 * alignment only; 16-byte alignment of rows is not required.
 *
 * Ownership.  B, a and c belong to the caller.  The library never allocates,
 * frees or keeps them past the call.  c must hold n elements and must not
 * overlap B or a.  The handle belongs to the library and is released by
 * gemv_destroy.
 *
 * Asynchrony.  gemv_run validates its arguments on the host, enqueues one
 * kernel on `stream` and returns; it allocates nothing and never
 * synchronises.  c is valid once the stream reaches that point; B, a and c
 * must stay alive until then.  All set-up (device query, kernel attributes)
 * happens in gemv_create, so a call costs one launch (TileLang Case Studies,
 * Case B.4: build once at construction, only launch per call).
 *
 * Errors.  Every function returns a gemv_status_t; nothing throws, aborts or
 * prints (unless the environment variable GEMV_LOG=1, which prints one line
 * per rejected call to stderr).  On any error no kernel is launched and c is
 * left untouched.  Validation order in gemv_run: handle, dtype, n >= 0 and
 * k >= 0, n == 0 (success, no launch), null pointers (c always, B and a when
 * k > 0; with k == 0 neither is read), alignment, size limits, overlap of c
 * with B or a, current device == handle device; then the launch, whose
 * failure is GEMV_ERR_HIP.
 *
 * Scratch.  The handle owns no device memory.  gemv_run and gemv_run_ex use
 * none: for few rows they split k inside a workgroup.  Splitting k across
 * workgroups as well (faster for a few long rows, e.g. 64 rows of 65536)
 * needs device scratch for the partial sums and arrival counters, which the
 * caller brings to gemv_run_ws (GEMV_WORKSPACE_BYTES).
 *
 * Threading.  The handle is read-only after gemv_create (gemv_force_config,
 * a benchmarking aid, aside), so gemv_run and gemv_run_ex calls on one handle
 * may run concurrently on different streams.  gemv_run_ws calls may too, as
 * long as calls that can overlap on the GPU use different workspaces.
 */
#ifndef MBD_GEMV_H
#define MBD_GEMV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct gemv_handle_s* gemv_handle_t;

typedef enum {
  GEMV_F16 = 0,   /* IEEE-754 binary16 */
  GEMV_BF16 = 1   /* bfloat16 (upper half of binary32) */
} gemv_dtype_t;

typedef enum {
  GEMV_OK = 0,
  GEMV_ERR_NULL_HANDLE = 1,       /* handle is NULL or already destroyed */
  GEMV_ERR_INVALID_ARG = 2,       /* negative size, NULL pointer, bad config */
  GEMV_ERR_UNSUPPORTED_DTYPE = 3, /* dtype is not GEMV_F16 / GEMV_BF16 */
  GEMV_ERR_MISALIGNED = 4,        /* a pointer is not 2-byte aligned */
  GEMV_ERR_ALIASING = 5,          /* c overlaps B or a */
  GEMV_ERR_TOO_LARGE = 6,         /* n > 2^30 or k > 2^27, or a forced k-split
                                     across workgroups whose partials (n x
                                     k-groups rounded up to 32) exceed the
                                     scratch */
  GEMV_ERR_WRONG_DEVICE = 7,      /* current HIP device != the handle's */
  GEMV_ERR_UNSUPPORTED = 8,       /* no kernel for this GPU / configuration */
  GEMV_ERR_HIP = 9,               /* a HIP runtime call failed */
  GEMV_ERR_OOM = 10               /* host allocation of the handle failed */
} gemv_status_t;

/* Largest sizes gemv_run accepts. */
#define GEMV_MAX_N 1073741824LL
#define GEMV_MAX_K 134217728LL

/* Bytes of caller scratch that gemv_run_ws needs for its cross-workgroup
 * k-split: 2 MiB of arrival counters (64 banks of 256, one bank per k-group
 * count, one counter per 128-byte line), 1 MiB of fp32 partial sums (n rows x
 * k-groups rounded up to a multiple of 32 <= 2^18), and 1.92 MiB of ticket
 * lines (64 banks of 96 rows: the split with one row per workgroup). */
#define GEMV_WORKSPACE_BYTES 5160960LL

/* Create a handle bound to the current HIP device.  Queries the device (it
 * must be a gfx950), sets kernel attributes and fixes the variant table; it
 * allocates host memory for the handle only.  *out receives the handle, or
 * NULL on error. */
gemv_status_t gemv_create(gemv_handle_t* out);

/* c = B @ a on `stream` (0 = the null stream).  B: n*k elements, row-major;
 * a: k elements; c: n elements; all of `dtype`, on the handle's device.
 * n == 0 is a no-op; k == 0 writes zeros (the empty sum) into c. */
gemv_status_t gemv_run(gemv_handle_t h, const void* B, const void* a, void* c,
                       int64_t n, int64_t k, gemv_dtype_t dtype, hipStream_t stream);

/* The fused epilogue (page "Optimizing TileLang Programs", epilogue fusion:
 * post-operations applied in registers before the single write of c):
 *     c[i] = round_to_dtype( alpha * sum_j B[i][j] a[j] + bias[i] )
 * computed as one fp32 FMA on the fp32 row sum (alpha * sum without bias).
 * bias: n elements of the same dtype (2-byte aligned) or NULL; it may be c
 * itself (accumulate in place) but must not partly overlap c. */
typedef struct {
  float alpha;
  const void* bias;
} gemv_epilogue_t;

/* gemv_run with an epilogue; ep == NULL is exactly gemv_run.  Validation as
 * gemv_run, then the bias checks (GEMV_ERR_MISALIGNED, GEMV_ERR_ALIASING). */
gemv_status_t gemv_run_ex(gemv_handle_t h, const void* B, const void* a, void* c,
                          int64_t n, int64_t k, gemv_dtype_t dtype, const gemv_epilogue_t* ep,
                          hipStream_t stream);

/* gemv_run_ex with caller scratch, which lets the plan split k across
 * workgroups where that is faster (few rows of many columns: the Q
 * workgroups that share a row range each write fp32 partials; the last to
 * arrive, told by an arrival counter, sums them in a fixed order, so results
 * do not depend on timing).  Pages: TileLang Case Studies, Case B.3 (few rows
 * underfill the GPU) and Case C (split-k plus a reduction).
 *   workspace:       NULL (then exactly gemv_run_ex), or device memory on the
 *                    handle's device, 16-byte aligned, at least
 *                    workspace_bytes >= GEMV_WORKSPACE_BYTES (else
 *                    GEMV_ERR_INVALID_ARG / GEMV_ERR_MISALIGNED), overlapping
 *                    none of B, a, c and bias (GEMV_ERR_ALIASING).  Owned by
 *                    the caller; the library keeps no reference after the
 *                    call's kernel completes.
 *   contents:        zero-filled once before its first use (e.g. hipMemset);
 *                    from then on every completed call leaves it in a state
 *                    the next call accepts (each arrival counter at zero or
 *                    at a multiple of the call's k-group count, every
 *                    published partial tagged with a finished generation),
 *                    so it needs no clearing between calls.
 *   concurrency:     calls that may overlap on the GPU need different
 *                    workspaces; overlapping calls on one workspace race (c
 *                    undefined, possibly NaN: a combining workgroup that
 *                    finds a partial missing gives up after a bounded number
 *                    of polls), though the workspace is back in such a state
 *                    once those calls have completed.
 * Validation as gemv_run_ex, then (n > 0) the workspace checks above. */
gemv_status_t gemv_run_ws(gemv_handle_t h, const void* B, const void* a, void* c,
                          int64_t n, int64_t k, gemv_dtype_t dtype, const gemv_epilogue_t* ep,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * gemv_run_ws with the library's own static scratch in place of a caller
 * workspace -- GEMV_WORKSPACE_BYTES per GPU, in the library's image, its
 * device address resolved and zero-filled by gemv_create on each GPU and
 * held until the process ends.  The call allocates nothing (no hipMalloc,
 * no allocating library routine) and never synchronises.  Every call on one
 * GPU shares that GPU's scratch: calls that may overlap on the GPU (other
 * streams, other handles, other threads) race -- their c is undefined --
 * so issue them on one stream or order them; gemv_run_ws with a workspace
 * per stream has no such limit.  A forced k-split across workgroups whose
 * partials (n x k-groups rounded up to 32) exceed the scratch's 2^18 is
 * GEMV_ERR_TOO_LARGE; the automatic plan never needs more.  Otherwise as
 * gemv_run_ws. */
gemv_status_t gemv_run_noalloc(gemv_handle_t h, const void* B, const void* a, void* c,
                               int64_t n, int64_t k, gemv_dtype_t dtype,
                               const gemv_epilogue_t* ep, hipStream_t stream);

/* Every check gemv_run makes that needs neither a handle nor a GPU, in the
 * same order and with the same result: GEMV_OK means gemv_run would go on to
 * the device check and the launch (or return GEMV_OK at once when n == 0).
 * Pure host arithmetic on the pointer values; nothing is dereferenced. */
gemv_status_t gemv_check_args(const void* B, const void* a, const void* c, int64_t n, int64_t k,
                              gemv_dtype_t dtype);

/* The same for gemv_run_ex (ep may be NULL). */
gemv_status_t gemv_check_args_ex(const void* B, const void* a, const void* c, int64_t n, int64_t k,
                                 gemv_dtype_t dtype, const gemv_epilogue_t* ep);

/* Release the handle.  NULL is a no-op.  Kernels already enqueued do not
 * read the handle, so they may still be running. */
gemv_status_t gemv_destroy(gemv_handle_t h);

/* Static, human-readable name of a status code. */
const char* gemv_status_string(gemv_status_t s);

/* ---- kernel variants (for benchmarking and tuning; Case C: profile with a
 *      fixed configuration, never with autotuning inside the trace) ------- */

/* Shape of one compiled kernel variant.  A workgroup has `waves` 64-lane
 * wavefronts arranged as (waves / splits) row groups x `splits` k-slices; a
 * row group owns `rows` consecutive rows; each wave streams its rows of B
 * with 16-byte loads along k, `unroll` 512-element steps per loop trip.
 * a_mode 0: a is staged once per workgroup in LDS; 1: a is read through the
 * cache hierarchy with the same 16-byte loads; 2: for rows that do not start
 * on a 16-byte boundary, B is read in aligned 16-byte granules starting at
 * the 128-byte line that holds each row's first element, and a is staged in
 * LDS twice (shifted by 0 and 1 element) to line up with them; 3: the same
 * granules of B, and a read through the caches at each row's shift (a 4-byte
 * aligned 16-byte load and a 2-byte load per granule, joined by a shift).
 * splits > 1 sums the k-slices of a row group in a fixed order through LDS
 * (deterministic). */
typedef struct {
  int32_t rows;
  int32_t unroll;
  int32_t waves;
  int32_t splits;
  int32_t a_mode;
  int32_t b_policy;   /* cache-policy bits of the B loads (0 = default) */
  int32_t cross_wg;   /* 1: kgroups workgroups share each row range along k,
                         combining through the caller's scratch: runs only
                         from gemv_run_ws with a workspace */
  int32_t layout;     /* 0: lanes along k (coalesced); 1: one row per lane,
                         one element per step -- the uncoalesced layout of
                         TileLang Case Studies, Case B, kept for measurement
                         and never chosen automatically */
  int32_t stages;     /* 0: the plain loop (a wave issues a group of loads,
                         then waits for it); 1..3: the pipelined-B form of
                         TileLang Case Studies, Case B.1, kept for measurement
                         and never chosen automatically -- each wave keeps
                         `stages` - 1 items of `unroll` steps x `rows` rows in
                         flight while it consumes one (1 = sequential,
                         2 = double, 3 = triple buffering); it needs 16-byte
                         aligned rows (k % 8 == 0, B 16-byte aligned) and
                         returns GEMV_ERR_UNSUPPORTED otherwise */
  int32_t b_lds;      /* stages > 0: 1 = the slots are in LDS, filled by
                         buffer loads that write LDS directly; 0 = registers */
} gemv_variant_info_t;

typedef struct {
  int32_t variant;    /* index in [0, gemv_num_variants()), or -1 = automatic */
  int32_t grid;       /* workgroups per k-group; 0 = one row range per wave
                         (per workgroup when splits > 1 or cross_wg) */
  int32_t kgroups;    /* cross_wg variants: workgroups sharing a row range
                         along k (0 = automatic); other variants: 0 or 1 */
  int32_t flags;      /* GEMV_FLAG_* bits */
} gemv_config_t;

/* Workgroups are dispatched round-robin over the GPU's 8 XCDs.  With this
 * flag the row ranges are renumbered so that the workgroups of one XCD own
 * one contiguous block of rows (measured: no gain for the automatic plans,
 * a gain for some persistent grids).  Variants with cross_wg ignore it: their
 * k-groups are what is dealt over the XCDs. */
#define GEMV_FLAG_XCD_CONTIGUOUS 1

/* Number of compiled variants. */
int32_t gemv_num_variants(void);

/* Describe variant `v`; GEMV_ERR_INVALID_ARG if out of range or info NULL. */
gemv_status_t gemv_variant_info(int32_t v, gemv_variant_info_t* info);

/* Force a configuration on every later gemv_run of this handle (NULL or
 * variant -1 restores automatic selection).  Not thread-safe with concurrent
 * gemv_run calls on the same handle.  A cross_wg variant then runs only
 * from gemv_run_ws with a workspace (elsewhere GEMV_ERR_UNSUPPORTED). */
gemv_status_t gemv_force_config(gemv_handle_t h, const gemv_config_t* cfg);

/* The configuration gemv_run would use for (n, k, dtype) on this handle,
 * for a 16-byte-aligned B (gemv_run also looks at B's alignment), without
 * (with_workspace == 0: gemv_run, gemv_run_ex) or with (gemv_run_ws with a
 * workspace) caller scratch.  grid is reported as the number of workgroups
 * actually launched. */
gemv_status_t gemv_query_config(gemv_handle_t h, int64_t n, int64_t k, gemv_dtype_t dtype,
                                int32_t with_workspace, gemv_config_t* out);

/* The configuration the automatic plan picks for (n, k, dtype), worked out on
 * the host alone -- no handle, no device, no HIP call -- for a device whose
 * per-workgroup LDS limit is `max_lds` bytes (163840 on MI355X) and a B that
 * is (b_aligned != 0) or is not 16-byte aligned, and without (with_workspace
 * == 0) or with caller scratch (see gemv_query_config).  It is the rule gemv_run
 * applies (TileLang Case Studies, Case B.4: the choice is fixed host logic,
 * not per-call tuning), so tools and CPU tests can inspect it; on a real
 * handle gemv_query_config gives the same answer (it also checks the LDS the
 * kernels declare statically).  grid is the number of workgroups launched.
 * Errors: GEMV_ERR_INVALID_ARG (out NULL, n <= 0, k < 0, sizes above the
 * limits, max_lds <= 0), GEMV_ERR_UNSUPPORTED_DTYPE, GEMV_ERR_UNSUPPORTED (no
 * compiled variant fits). */
gemv_status_t gemv_plan_config(int64_t n, int64_t k, gemv_dtype_t dtype, int32_t b_aligned,
                               int64_t max_lds, int32_t with_workspace, gemv_config_t* out);

#ifdef __cplusplus
}
#endif

#endif /* MBD_GEMV_H */
