// libgemv.so: the C ABI declared in include/gemv.h, over the kernels of
// gemv_kernel.h.  Host work per call is argument validation, an O(1) choice
// of a precompiled variant and one launch (TileLang Case Studies, Case B.4:
// everything that does not depend on the call happens at construction).
#include "gemv.h"

#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gemv_kernel.h"

namespace {

using KernelFn = void (*)(const uint16_t*, const uint16_t*, uint16_t*, int, int);

struct Variant {
  gemv_variant_info_t info;
  KernelFn fn[2];   // [dtype]
};

// Cache-policy bits of the B loads on gfx950: bit 1 marks the access
// non-temporal (B has no reuse within a call).
constexpr int kPolNT = 2;

#define MBD_VARIANT(R, U, W, S, AM, POL)                                            \
  {{R, U, W, S, AM, POL},                                                           \
   {&mbd::gemv_kernel<mbd::DT_F16, R, U, W, S, AM, POL>,                            \
    &mbd::gemv_kernel<mbd::DT_BF16, R, U, W, S, AM, POL>}}

// The compiled variants: (rows R, unroll U, waves W, splits S, a mode, B
// cache policy).  Row variants (S == 1) give each wave R whole rows; split
// variants let S waves of a workgroup share R rows for small n.
#define NT kPolNT
#define LDS mbd::A_LDS
#define CCH mbd::A_CACHED
const Variant kVariants[] = {
    // 0..11: row variants, a through the caches, non-temporal B
    MBD_VARIANT(1, 2, 4, 1, CCH, NT), MBD_VARIANT(1, 4, 4, 1, CCH, NT),
    MBD_VARIANT(1, 8, 4, 1, CCH, NT), MBD_VARIANT(2, 2, 4, 1, CCH, NT),
    MBD_VARIANT(2, 4, 4, 1, CCH, NT), MBD_VARIANT(2, 8, 4, 1, CCH, NT),
    MBD_VARIANT(4, 2, 4, 1, CCH, NT), MBD_VARIANT(4, 4, 4, 1, CCH, NT),
    MBD_VARIANT(1, 4, 8, 1, CCH, NT), MBD_VARIANT(2, 4, 8, 1, CCH, NT),
    MBD_VARIANT(1, 4, 2, 1, CCH, NT), MBD_VARIANT(2, 4, 1, 1, CCH, NT),
    // 12..19: row variants, a staged in LDS, non-temporal B
    MBD_VARIANT(1, 4, 4, 1, LDS, NT), MBD_VARIANT(1, 8, 4, 1, LDS, NT),
    MBD_VARIANT(2, 2, 4, 1, LDS, NT), MBD_VARIANT(2, 4, 4, 1, LDS, NT),
    MBD_VARIANT(4, 2, 4, 1, LDS, NT), MBD_VARIANT(4, 4, 4, 1, LDS, NT),
    MBD_VARIANT(2, 4, 8, 1, LDS, NT), MBD_VARIANT(4, 2, 8, 1, LDS, NT),
    // 20..23: default cache policy (for comparison)
    MBD_VARIANT(1, 4, 4, 1, CCH, 0), MBD_VARIANT(2, 4, 4, 1, CCH, 0),
    MBD_VARIANT(2, 4, 4, 1, LDS, 0), MBD_VARIANT(4, 2, 4, 1, LDS, 0),
    // 24..29: other cache-policy bits on one shape (sc0 = 1, sc1 = 16)
    MBD_VARIANT(2, 4, 4, 1, CCH, 1), MBD_VARIANT(2, 4, 4, 1, CCH, 3),
    MBD_VARIANT(2, 4, 4, 1, CCH, 16), MBD_VARIANT(2, 4, 4, 1, CCH, 18),
    MBD_VARIANT(2, 4, 4, 1, CCH, 17), MBD_VARIANT(2, 4, 4, 1, CCH, 19),
    // 30..41: split variants, a through the caches, non-temporal B
    MBD_VARIANT(1, 2, 8, 2, CCH, NT), MBD_VARIANT(1, 4, 8, 2, CCH, NT),
    MBD_VARIANT(2, 4, 8, 2, CCH, NT), MBD_VARIANT(1, 2, 8, 4, CCH, NT),
    MBD_VARIANT(1, 4, 8, 4, CCH, NT), MBD_VARIANT(2, 4, 8, 4, CCH, NT),
    MBD_VARIANT(1, 2, 8, 8, CCH, NT), MBD_VARIANT(1, 4, 8, 8, CCH, NT),
    MBD_VARIANT(2, 4, 8, 8, CCH, NT), MBD_VARIANT(1, 4, 4, 4, CCH, NT),
    MBD_VARIANT(1, 2, 16, 16, CCH, NT), MBD_VARIANT(1, 4, 16, 16, CCH, NT),
};
#undef NT
#undef LDS
#undef CCH
constexpr int kNumVariants = (int)(sizeof(kVariants) / sizeof(kVariants[0]));

size_t lds_bytes(const gemv_variant_info_t& v, int64_t k) {
  const int64_t nsteps = (k + mbd::kStep - 1) / mbd::kStep;
  size_t b = 0;
  if (v.a_mode == mbd::A_LDS) b += (size_t)nsteps * mbd::kStepBytes;
  if (v.splits > 1) b += (size_t)v.waves * v.rows * sizeof(float);
  return b;
}

int64_t rows_per_block(const gemv_variant_info_t& v) { return (int64_t)(v.waves / v.splits) * v.rows; }

// Shape of a launch plan: a variant shape plus a workgroup count (0 = one
// row range per wave, i.e. no persistence).
struct Plan {
  int rows, unroll, waves, splits, a_mode, policy;
  int grid;
};

// Measured on MI355X for the listed workload shapes (several plans lie
// within a few per cent of each other on these; the fastest median is kept).
struct TunedShape {
  int64_t n, k;
  Plan plan;
};
const TunedShape kTuned[] = {
    {4096, 11008, {1, 4, 4, 4, mbd::A_CACHED, kPolNT, 0}},
    {4096, 14336, {1, 4, 4, 1, mbd::A_CACHED, kPolNT, 512}},
};

int find_variant(const Plan& p) {
  for (int v = 0; v < kNumVariants; ++v) {
    const gemv_variant_info_t& i = kVariants[v].info;
    if (i.rows == p.rows && i.unroll == p.unroll && i.waves == p.waves && i.splits == p.splits &&
        i.a_mode == p.a_mode && i.b_policy == p.policy)
      return v;
  }
  return -1;
}

// The general rule, for shapes without a measured entry:
//  * rows whose start is not 16-byte aligned (k % 8 != 0): one row per wave
//    and a staged in LDS, which keeps the texture path free for the
//    unaligned B loads;
//  * otherwise a through the caches and non-temporal B loads; two rows per
//    wave when both n and k are large;
//  * k is split inside a workgroup while every wave still streams at least
//    8 KiB of B, and further (down to two 512-element steps per slice) while
//    the grid has fewer than 4096 waves.
Plan rule_plan(int64_t n, int64_t k, size_t max_lds) {
  if (k % 8 != 0) {
    Plan p = {1, 4, 4, 1, mbd::A_LDS, kPolNT, 0};
    if (lds_bytes(kVariants[find_variant(p)].info, k) > max_lds) p.a_mode = mbd::A_CACHED;
    return p;
  }
  const int64_t nfull = k / mbd::kStep;
  const int R = (n >= 4096 && k >= 6144) ? 2 : 1;
  const int64_t row_bytes = 2 * k * R;
  const int smax = R == 1 ? 16 : 8;
  int S = 1;
  while (S < smax && row_bytes / (2 * S) >= 8192 && nfull >= 2 * (2 * S)) S *= 2;
  while (S < smax && ((n + R - 1) / R) * S < 4096 && nfull >= 2 * (2 * S)) S *= 2;
  const int W = S == 1 ? 4 : (S <= 8 ? 8 : 16);
  return Plan{R, 4, W, S, mbd::A_CACHED, kPolNT, 0};
}

Plan auto_plan(int64_t n, int64_t k, size_t max_lds) {
  for (const TunedShape& t : kTuned)
    if (t.n == n && t.k == k) return t.plan;
  return rule_plan(n, k, max_lds);
}

constexpr uint32_t kMagic = 0x47454d56u;   // "GEMV"
constexpr uint32_t kDead = 0xdeadbeefu;

}  // namespace

struct gemv_handle_s {
  uint32_t magic;
  int device;
  int num_cus;
  size_t max_lds;
  int log;
  gemv_config_t forced;
};

static gemv_status_t report(const gemv_handle_s* h, gemv_status_t s, const char* what) {
  int log = h ? h->log : (getenv("GEMV_LOG") && strcmp(getenv("GEMV_LOG"), "1") == 0);
  if (log && s != GEMV_OK) fprintf(stderr, "gemv: %s: %s\n", gemv_status_string(s), what);
  return s;
}

extern "C" const char* gemv_status_string(gemv_status_t s) {
  switch (s) {
    case GEMV_OK: return "GEMV_OK";
    case GEMV_ERR_NULL_HANDLE: return "GEMV_ERR_NULL_HANDLE";
    case GEMV_ERR_INVALID_ARG: return "GEMV_ERR_INVALID_ARG";
    case GEMV_ERR_UNSUPPORTED_DTYPE: return "GEMV_ERR_UNSUPPORTED_DTYPE";
    case GEMV_ERR_MISALIGNED: return "GEMV_ERR_MISALIGNED";
    case GEMV_ERR_ALIASING: return "GEMV_ERR_ALIASING";
    case GEMV_ERR_TOO_LARGE: return "GEMV_ERR_TOO_LARGE";
    case GEMV_ERR_WRONG_DEVICE: return "GEMV_ERR_WRONG_DEVICE";
    case GEMV_ERR_UNSUPPORTED: return "GEMV_ERR_UNSUPPORTED";
    case GEMV_ERR_HIP: return "GEMV_ERR_HIP";
    case GEMV_ERR_OOM: return "GEMV_ERR_OOM";
  }
  return "GEMV_ERR_UNKNOWN";
}

extern "C" int32_t gemv_num_variants(void) { return kNumVariants; }

extern "C" gemv_status_t gemv_variant_info(int32_t v, gemv_variant_info_t* info) {
  if (!info || v < 0 || v >= kNumVariants) return GEMV_ERR_INVALID_ARG;
  *info = kVariants[v].info;
  return GEMV_OK;
}

// Every check of gemv_run that needs neither the handle nor the GPU.
extern "C" gemv_status_t gemv_check_args(const void* B, const void* a, const void* c, int64_t n,
                                         int64_t k, gemv_dtype_t dtype) {
  if (dtype != GEMV_F16 && dtype != GEMV_BF16) return GEMV_ERR_UNSUPPORTED_DTYPE;
  if (n < 0 || k < 0) return GEMV_ERR_INVALID_ARG;
  if (n == 0) return GEMV_OK;
  // B and a are never read when k == 0 (an empty tensor may hand over NULL)
  if (!c || (k > 0 && (!B || !a))) return GEMV_ERR_INVALID_ARG;
  if (((uintptr_t)c | (k > 0 ? ((uintptr_t)B | (uintptr_t)a) : 0u)) & 1u) return GEMV_ERR_MISALIGNED;
  if (n > GEMV_MAX_N || k > GEMV_MAX_K) return GEMV_ERR_TOO_LARGE;
  const uintptr_t c0 = (uintptr_t)c, c1 = c0 + (uintptr_t)n * 2u;
  if (k > 0) {
    const uintptr_t b0 = (uintptr_t)B, b1 = b0 + (uintptr_t)n * (uintptr_t)k * 2u;
    const uintptr_t a0 = (uintptr_t)a, a1 = a0 + (uintptr_t)k * 2u;
    if ((c0 < b1 && b0 < c1) || (c0 < a1 && a0 < c1)) return GEMV_ERR_ALIASING;
  }
  return GEMV_OK;
}

static gemv_status_t resolve(const gemv_handle_s* h, int64_t n, int64_t k, int* variant,
                             int* grid, size_t* lds) {
  int v;
  int64_t g;
  if (h->forced.variant >= 0) {
    v = h->forced.variant;
    g = h->forced.grid;
  } else {
    const Plan p = auto_plan(n, k, h->max_lds);
    v = find_variant(p);
    if (v < 0) return GEMV_ERR_UNSUPPORTED;   // a plan names a variant that is not compiled
    g = p.grid;
  }
  const gemv_variant_info_t& info = kVariants[v].info;
  const int64_t rb = rows_per_block(info);
  const int64_t nrb = (n + rb - 1) / rb;       // one row range per wave (or workgroup)
  if (g <= 0 || g > nrb) g = nrb;
  // the kernels walk their row ranges, so a smaller grid is always valid;
  // keep the launch's work-item count well inside 32 bits
  const int64_t gmax = (int64_t)1 << 24;
  if (g > gmax) g = gmax;
  const size_t l = lds_bytes(info, k);
  if (l > h->max_lds) return GEMV_ERR_UNSUPPORTED;
  *variant = v;
  *grid = (int)g;
  *lds = l;
  return GEMV_OK;
}

extern "C" gemv_status_t gemv_create(gemv_handle_t* out) {
  if (!out) return GEMV_ERR_INVALID_ARG;
  *out = nullptr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return report(nullptr, GEMV_ERR_HIP, "hipGetDevice");
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
    return report(nullptr, GEMV_ERR_HIP, "hipGetDeviceProperties");
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return report(nullptr, GEMV_ERR_UNSUPPORTED, "device is not gfx950");
  int max_lds = 0;
  if (hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
    return report(nullptr, GEMV_ERR_HIP, "hipDeviceGetAttribute(max LDS)");
  for (int v = 0; v < kNumVariants; ++v) {
    for (int d = 0; d < 2; ++d) {
      if (hipFuncSetAttribute((const void*)kVariants[v].fn[d],
                              hipFuncAttributeMaxDynamicSharedMemorySize, max_lds) != hipSuccess)
        return report(nullptr, GEMV_ERR_HIP, "hipFuncSetAttribute");
    }
  }
  gemv_handle_s* h = (gemv_handle_s*)calloc(1, sizeof(gemv_handle_s));
  if (!h) return GEMV_ERR_OOM;
  h->magic = kMagic;
  h->device = dev;
  h->num_cus = prop.multiProcessorCount;
  h->max_lds = (size_t)max_lds;
  const char* lg = getenv("GEMV_LOG");
  h->log = lg && strcmp(lg, "1") == 0;
  h->forced.variant = -1;
  h->forced.grid = 0;
  *out = h;
  return GEMV_OK;
}

extern "C" gemv_status_t gemv_destroy(gemv_handle_t h) {
  if (!h) return GEMV_OK;
  if (h->magic != kMagic) return GEMV_ERR_NULL_HANDLE;
  h->magic = kDead;
  free(h);
  return GEMV_OK;
}

extern "C" gemv_status_t gemv_force_config(gemv_handle_t h, const gemv_config_t* cfg) {
  if (!h || h->magic != kMagic) return GEMV_ERR_NULL_HANDLE;
  if (!cfg || cfg->variant < 0) {
    h->forced.variant = -1;
    h->forced.grid = 0;
    return GEMV_OK;
  }
  if (cfg->variant >= kNumVariants || cfg->grid < 0) return report(h, GEMV_ERR_INVALID_ARG, "config");
  h->forced = *cfg;
  return GEMV_OK;
}

extern "C" gemv_status_t gemv_query_config(gemv_handle_t h, int64_t n, int64_t k,
                                           gemv_dtype_t dtype, gemv_config_t* out) {
  if (!h || h->magic != kMagic) return GEMV_ERR_NULL_HANDLE;
  if (!out) return GEMV_ERR_INVALID_ARG;
  if (dtype != GEMV_F16 && dtype != GEMV_BF16) return GEMV_ERR_UNSUPPORTED_DTYPE;
  if (n <= 0 || k < 0 || n > GEMV_MAX_N || k > GEMV_MAX_K) return GEMV_ERR_INVALID_ARG;
  int v, g;
  size_t l;
  gemv_status_t s = resolve(h, n, k, &v, &g, &l);
  if (s != GEMV_OK) return s;
  out->variant = v;
  out->grid = g;
  return GEMV_OK;
}

extern "C" gemv_status_t gemv_run(gemv_handle_t h, const void* B, const void* a, void* c,
                                  int64_t n, int64_t k, gemv_dtype_t dtype, hipStream_t stream) {
  if (!h || h->magic != kMagic) return report(nullptr, GEMV_ERR_NULL_HANDLE, "gemv_run");
  gemv_status_t s = gemv_check_args(B, a, c, n, k, dtype);
  if (s != GEMV_OK) return report(h, s, "gemv_run arguments");
  if (n == 0) return GEMV_OK;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return report(h, GEMV_ERR_HIP, "hipGetDevice");
  if (dev != h->device) return report(h, GEMV_ERR_WRONG_DEVICE, "gemv_run");
  int v, grid;
  size_t lds;
  s = resolve(h, n, k, &v, &grid, &lds);
  if (s != GEMV_OK) return report(h, s, "no variant fits (LDS)");
  const Variant& var = kVariants[v];
  const uint16_t* Bp = (const uint16_t*)B;
  const uint16_t* ap = (const uint16_t*)a;
  uint16_t* cp = (uint16_t*)c;
  int ni = (int)n, ki = (int)k;
  void* args[] = {(void*)&Bp, (void*)&ap, (void*)&cp, (void*)&ni, (void*)&ki};
  hipError_t e = hipLaunchKernel((const void*)var.fn[dtype], dim3((unsigned)grid),
                                 dim3((unsigned)(var.info.waves * mbd::kLanes)), args, lds, stream);
  if (e != hipSuccess) return report(h, GEMV_ERR_HIP, hipGetErrorString(e));
  return GEMV_OK;
}
