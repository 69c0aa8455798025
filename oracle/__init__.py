"""CPU oracle for the dense GEMV c = B @ a (TileLang Case Studies, Case B).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product library and its Python
binding never do.  It shares no code with the HIP path.

Everything here works on raw 16-bit patterns (numpy ``uint16`` arrays) so the
oracle and the GPU consume exactly the same input bits.  The arithmetic lives
in ``gemv_ref.c`` (exact decode, fp64 sum, one round-to-nearest-even); this
module only marshals arrays through ctypes.

Dtype codes: 0 = fp16 (IEEE binary16), 1 = bf16.
"""
import ctypes
import os

import numpy as np

from . import build as _build

F16 = 0
BF16 = 1

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB) or any(
            os.path.getmtime(_build.LIB) < os.path.getmtime(src) for src in _build.SRCS):
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.oracle_decode.argtypes = [ctypes.c_int, ctypes.c_uint16]
    lib.oracle_decode.restype = ctypes.c_double
    lib.oracle_encode.argtypes = [ctypes.c_int, ctypes.c_double]
    lib.oracle_encode.restype = ctypes.c_uint16
    lib.oracle_decode_array.argtypes = [ctypes.c_int, u16p, dp, ctypes.c_int64]
    lib.oracle_decode_array.restype = None
    lib.oracle_encode_array.argtypes = [ctypes.c_int, dp, u16p, ctypes.c_int64]
    lib.oracle_encode_array.restype = None
    lib.oracle_gemv.argtypes = [ctypes.c_int, u16p, u16p, ctypes.c_int64, ctypes.c_int64,
                                u16p, dp, dp, dp]
    lib.oracle_gemv.restype = ctypes.c_int
    lib.oracle_gemv_epilogue.argtypes = [ctypes.c_int, u16p, u16p, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_float, u16p, u16p, dp, dp, dp]
    lib.oracle_gemv_epilogue.restype = ctypes.c_int
    fp = ctypes.POINTER(ctypes.c_float)
    lib.oracle_gla_decode.argtypes = [ctypes.c_int, u16p, u16p, u16p, u16p, fp, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_int64, ctypes.c_float, fp, u16p,
                                      dp, dp, dp]
    lib.oracle_gla_decode.restype = ctypes.c_int
    _lib = lib
    return lib


def _u16(x):
    x = np.ascontiguousarray(x, dtype=np.uint16)
    return x, x.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16))


def _f64(x):
    x = np.ascontiguousarray(x, dtype=np.float64)
    return x, x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def decode(dtype: int, bits) -> np.ndarray:
    """Exact value (float64) of each 16-bit pattern."""
    bits, p = _u16(bits)
    out = np.empty(bits.shape, dtype=np.float64)
    _load().oracle_decode_array(dtype, p, out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                bits.size)
    return out


def encode(dtype: int, x) -> np.ndarray:
    """Round each float64 to the nearest `dtype` value, ties to even."""
    x, p = _f64(x)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_encode_array(dtype, p, out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)),
                                x.size)
    return out


def gemv(dtype: int, B, a):
    """c = B @ a on 16-bit patterns.

    B: (n, k) uint16 patterns, a: (k,) uint16 patterns.
    Returns (c_bits uint16 (n,), s float64 (n,) the unrounded fp64 sum,
    abs float64 (n,) = sum_j |B_ij a_j|).
    """
    B = np.ascontiguousarray(B, dtype=np.uint16)
    a = np.ascontiguousarray(a, dtype=np.uint16)
    if B.ndim != 2 or a.ndim != 1 or B.shape[1] != a.shape[0]:
        raise ValueError("oracle.gemv: B must be (n, k) and a (k,), got %s and %s"
                         % (B.shape, a.shape))
    n, k = B.shape
    c = np.empty(n, dtype=np.uint16)
    s = np.empty(n, dtype=np.float64)
    ab = np.empty(n, dtype=np.float64)
    scratch = np.empty(max(k, 1), dtype=np.float64)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    dp = ctypes.POINTER(ctypes.c_double)
    rc = _load().oracle_gemv(dtype, B.ctypes.data_as(u16p), a.ctypes.data_as(u16p), n, k,
                             c.ctypes.data_as(u16p), s.ctypes.data_as(dp), ab.ctypes.data_as(dp),
                             scratch.ctypes.data_as(dp))
    if rc != 0:
        raise ValueError("oracle.gemv: bad argument")
    return c, s, ab


def gemv_epilogue(dtype: int, B, a, alpha: float, bias=None):
    """c = round(alpha * (B @ a) + bias) on 16-bit patterns; alpha is taken as
    a float32 value, bias (n,) uint16 patterns or None.
    Returns (c_bits, y float64 = alpha*s + bias before rounding, abs = sum_j |B_ij a_j|)."""
    import numpy as np
    B = np.ascontiguousarray(B, dtype=np.uint16)
    a = np.ascontiguousarray(a, dtype=np.uint16)
    if B.ndim != 2 or a.ndim != 1 or B.shape[1] != a.shape[0]:
        raise ValueError("oracle.gemv_epilogue: B must be (n, k) and a (k,)")
    n, k = B.shape
    u16p = ctypes.POINTER(ctypes.c_uint16)
    dp = ctypes.POINTER(ctypes.c_double)
    bp = None
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.uint16)
        if bias.shape != (n,):
            raise ValueError("oracle.gemv_epilogue: bias must be (n,)")
        bp = bias.ctypes.data_as(u16p)
    c = np.empty(n, dtype=np.uint16)
    y = np.empty(n, dtype=np.float64)
    ab = np.empty(n, dtype=np.float64)
    scratch = np.empty(max(k, 1), dtype=np.float64)
    rc = _load().oracle_gemv_epilogue(dtype, B.ctypes.data_as(u16p), a.ctypes.data_as(u16p), n, k,
                                      float(np.float32(alpha)), bp, c.ctypes.data_as(u16p),
                                      y.ctypes.data_as(dp), ab.ctypes.data_as(dp),
                                      scratch.ctypes.data_as(dp))
    if rc != 0:
        raise ValueError("oracle.gemv_epilogue: bad argument")
    return c, y, ab


def gla_decode(dtype: int, q, k, v, gk, S, scale: float):
    """One GLA decode step (TileLang Case Studies, Case D):
    S_new = diag(exp(gk)) S + outer(k, v), o = scale * q^T S_new, per head.

    q, k, gk: (BH, DK) uint16 patterns; v: (BH, DV) patterns; S: (BH, DK, DV)
    float32.  Returns (S_new float32, o uint16 patterns (BH, DV), S_new before
    rounding (float64), o before rounding (float64), |scale| sum_i |q_i S_new|)."""
    import numpy as np
    q, k, v, gk = (np.ascontiguousarray(x, dtype=np.uint16) for x in (q, k, v, gk))
    S = np.ascontiguousarray(S, dtype=np.float32)
    bh, dk, dv = S.shape
    if q.shape != (bh, dk) or k.shape != (bh, dk) or gk.shape != (bh, dk) or v.shape != (bh, dv):
        raise ValueError("oracle.gla_decode: shapes do not match S %s" % (S.shape,))
    u16p = ctypes.POINTER(ctypes.c_uint16)
    fp = ctypes.POINTER(ctypes.c_float)
    dp = ctypes.POINTER(ctypes.c_double)
    Sn = np.empty_like(S)
    o = np.empty((bh, dv), dtype=np.uint16)
    s64 = np.empty(S.shape, dtype=np.float64)
    o64 = np.empty((bh, dv), dtype=np.float64)
    oabs = np.empty((bh, dv), dtype=np.float64)
    rc = _load().oracle_gla_decode(dtype, q.ctypes.data_as(u16p), k.ctypes.data_as(u16p),
                                   v.ctypes.data_as(u16p), gk.ctypes.data_as(u16p),
                                   S.ctypes.data_as(fp), bh, dk, dv, float(np.float32(scale)),
                                   Sn.ctypes.data_as(fp), o.ctypes.data_as(u16p),
                                   s64.ctypes.data_as(dp), o64.ctypes.data_as(dp),
                                   oabs.ctypes.data_as(dp))
    if rc != 0:
        raise ValueError("oracle.gla_decode: bad argument")
    return Sn, o, s64, o64, oabs
