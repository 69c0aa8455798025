// Internal to libgemv.so: the handle shared by the GEMV (gemv.hip) and the
// GLA decode step (gla.hip), and error reporting.
#pragma once

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gemv.h"

namespace mbd_host {

// Cache-policy bits of a buffer access on gfx950: bit 1 marks it
// non-temporal (streamed data with no reuse within a call).
constexpr int kPolNT = 2;

constexpr uint32_t kMagic = 0x47454d56u;   // "GEMV"
constexpr uint32_t kDead = 0xdeadbeefu;
constexpr int kMaxVariants = 96;

}  // namespace mbd_host

struct gemv_handle_s {
  uint32_t magic;
  int device;
  int num_cus;
  size_t max_lds;
  int log;
  gemv_config_t forced;
  void* scratch;       // device address of this GPU's copy of the library's static scratch
  size_t static_lds[mbd_host::kMaxVariants][2];   // LDS each kernel declares statically
};

// Returns s; with GEMV_LOG=1 also prints what failed.
static inline gemv_status_t report(const gemv_handle_s* h, gemv_status_t s, const char* what) {
  int log = h ? h->log : (getenv("GEMV_LOG") && strcmp(getenv("GEMV_LOG"), "1") == 0);
  if (log && s != GEMV_OK) fprintf(stderr, "gemv: %s: %s\n", gemv_status_string(s), what);
  return s;
}
