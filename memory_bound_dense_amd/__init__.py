"""MI355X-native dense GEMV, c = B @ a (fp16/bf16 in, fp32 sum).

The compute lives in libgemv.so (HIP kernels for gfx950 behind a C ABI,
include/gemv.h); this package is its ctypes binding.
"""
from ._lib import (EXPORTS, GEMV_BF16, GEMV_F16, GEMV_OK, Gemv, GemvError, GlaDecode,
                   gemv_check_args, gla_check_args, gla_decode_step,
                   gemv_check_args_ex, gemv_create, gemv_destroy, gemv_force_config,
                   gemv_num_variants, gemv_plan_config, gemv_query_config, gemv_run,
                   gemv_run_ex, gemv_run_noalloc, gemv_run_ws, gemv_status_string, gemv_variant_info, load)

__all__ = ["EXPORTS", "GEMV_BF16", "GEMV_F16", "GEMV_OK", "Gemv", "GemvError", "GlaDecode",
           "gla_check_args", "gla_decode_step", "gemv_check_args",
           "gemv_check_args_ex", "gemv_create", "gemv_destroy", "gemv_force_config",
           "gemv_num_variants", "gemv_plan_config", "gemv_query_config", "gemv_run", "gemv_run_ex",
           "gemv_run_noalloc", "gemv_run_ws",
           "gemv_status_string", "gemv_variant_info", "load"]
