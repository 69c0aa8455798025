/* A plain C (C99) caller of the library: the public headers compile as C
 * and every declared entry point links from libgemv.so.  Without a GPU it
 * exercises only the calls that need no device (argument checks, the host
 * plan, the variant table, status strings); gemv_create must then fail
 * cleanly.  Prints one "name value" line per check for the driving test. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gemv.h"
#include "gla_decode.h"

int main(void) {
  /* every entry point, taken by address: a missing export fails the link */
  void* fns[] = {(void*)&gemv_create,        (void*)&gemv_run,          (void*)&gemv_run_ex,
                 (void*)&gemv_run_ws,        (void*)&gemv_run_noalloc,
                 (void*)&gemv_destroy,       (void*)&gemv_status_string, (void*)&gemv_check_args,
                 (void*)&gemv_check_args_ex, (void*)&gemv_num_variants,  (void*)&gemv_variant_info,
                 (void*)&gemv_force_config,  (void*)&gemv_query_config,  (void*)&gemv_plan_config,
                 (void*)&gla_decode_step,    (void*)&gla_check_args};
  int linked = 0;
  for (size_t i = 0; i < sizeof(fns) / sizeof(fns[0]); ++i) linked += fns[i] != NULL;
  printf("linked %d\n", linked);

  printf("status0 %s\n", gemv_status_string(GEMV_OK));
  printf("status5 %s\n", gemv_status_string(GEMV_ERR_ALIASING));

  /* fake, well-separated device addresses: the checks never dereference */
  const void* B = (const void*)(uintptr_t)(1ull << 32);
  const void* a = (const void*)(uintptr_t)(1ull << 34);
  const void* c = (const void*)(uintptr_t)(1ull << 36);
  printf("check_ok %d\n", (int)gemv_check_args(B, a, c, 4, 8, GEMV_F16));
  printf("check_misaligned %d\n",
         (int)gemv_check_args((const char*)B + 1, a, c, 4, 8, GEMV_F16));
  printf("check_too_large %d\n", (int)gemv_check_args(B, a, c, GEMV_MAX_N + 1, 8, GEMV_BF16));

  gemv_config_t cfg;
  memset(&cfg, 0, sizeof cfg);
  gemv_status_t s = gemv_plan_config(18432, 7168, GEMV_F16, 1, 163840, 0, &cfg);
  gemv_variant_info_t info;
  memset(&info, 0, sizeof info);
  if (s == GEMV_OK) s = gemv_variant_info(cfg.variant, &info);
  printf("plan_status %d\n", (int)s);
  printf("plan_shape R%d U%d W%d S%d grid %d\n", info.rows, info.unroll, info.waves, info.splits,
         cfg.grid);
  printf("variants %d\n", (int)gemv_num_variants());
  gemv_config_t xw;
  memset(&xw, 0, sizeof xw);
  s = gemv_plan_config(64, 65536, GEMV_BF16, 1, 163840, 1, &xw);
  printf("plan_ws_kgroups %d %d\n", (int)s, xw.kgroups);
  printf("workspace_bytes %lld\n", (long long)GEMV_WORKSPACE_BYTES);

  printf("gla_check %d\n", (int)gla_check_args((const void*)(uintptr_t)(1ull << 40), a, c,
                                               (const void*)(uintptr_t)(1ull << 38),
                                               (const float*)(uintptr_t)(1ull << 41),
                                               (const float*)(uintptr_t)(1ull << 41),
                                               (const void*)(uintptr_t)(1ull << 42), 32, 128, 128,
                                               GEMV_BF16));

  gemv_handle_t h = NULL;
  s = gemv_create(&h);
  /* no GPU: a clean error and no handle; with a GPU: a handle, destroyed */
  printf("create %s %s\n", s == GEMV_OK ? "ok" : "error", h ? "handle" : "null");
  printf("run_ws_null_handle %d\n",
         (int)gemv_run_ws(NULL, B, a, (void*)c, 4, 8, GEMV_F16, NULL, NULL, 0, 0));
  printf("run_noalloc_null_handle %d\n",
         (int)gemv_run_noalloc(NULL, B, a, (void*)c, 4, 8, GEMV_F16, NULL, 0));
  printf("destroy %d\n", (int)gemv_destroy(h));
  return 0;
}
