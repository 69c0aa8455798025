"""ctypes binding of libgemv.so (include/gemv.h).

Argument marshalling only: every step of the product runs in the library's
HIP kernels.  The functions keep the C names and return the C status codes;
``Gemv`` wraps a handle for torch tensors (torch supplies device memory and
streams) and raises ``GemvError`` on any status other than GEMV_OK.

There is no fallback: if the library is missing or cannot be loaded, every
entry point raises.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgemv.so")

GEMV_F16 = 0
GEMV_BF16 = 1

GEMV_OK = 0
GEMV_ERR_NULL_HANDLE = 1
GEMV_ERR_INVALID_ARG = 2
GEMV_ERR_UNSUPPORTED_DTYPE = 3
GEMV_ERR_MISALIGNED = 4
GEMV_ERR_ALIASING = 5
GEMV_ERR_TOO_LARGE = 6
GEMV_ERR_WRONG_DEVICE = 7
GEMV_ERR_UNSUPPORTED = 8
GEMV_ERR_HIP = 9
GEMV_ERR_OOM = 10

GEMV_FLAG_XCD_CONTIGUOUS = 1

GEMV_MAX_N = 1073741824
GEMV_MAX_K = 134217728
GEMV_WORKSPACE_BYTES = 5160960

# every symbol include/gemv.h and include/gla_decode.h declare
EXPORTS = ("gemv_create", "gemv_run", "gemv_run_ex", "gemv_run_ws", "gemv_run_noalloc",
           "gemv_destroy",
           "gemv_status_string",
           "gemv_check_args", "gemv_check_args_ex", "gemv_num_variants", "gemv_variant_info",
           "gemv_force_config", "gemv_query_config", "gemv_plan_config", "gla_decode_step",
           "gla_check_args")


class GemvError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        super().__init__("%s%s" % (gemv_status_string(status), (": " + what) if what else ""))


class gemv_variant_info_t(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int32), ("unroll", ctypes.c_int32), ("waves", ctypes.c_int32),
                ("splits", ctypes.c_int32), ("a_mode", ctypes.c_int32),
                ("b_policy", ctypes.c_int32), ("cross_wg", ctypes.c_int32),
                ("layout", ctypes.c_int32), ("stages", ctypes.c_int32),
                ("b_lds", ctypes.c_int32)]


class gemv_epilogue_t(ctypes.Structure):
    _fields_ = [("alpha", ctypes.c_float), ("bias", ctypes.c_void_p)]


class gemv_config_t(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int32), ("grid", ctypes.c_int32),
                ("kgroups", ctypes.c_int32), ("flags", ctypes.c_int32)]


_lib = None


def load():
    """Load libgemv.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libgemv.so is not built (%s); run "
                           "`python -m memory_bound_dense_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    st = ctypes.c_int
    lib.gemv_create.argtypes = [ctypes.POINTER(vp)]
    lib.gemv_create.restype = st
    lib.gemv_run.argtypes = [vp, vp, vp, vp, i64, i64, ctypes.c_int, vp]
    lib.gemv_run.restype = st
    lib.gemv_run_ex.argtypes = [vp, vp, vp, vp, i64, i64, ctypes.c_int,
                                ctypes.POINTER(gemv_epilogue_t), vp]
    lib.gemv_run_ex.restype = st
    lib.gemv_run_ws.argtypes = [vp, vp, vp, vp, i64, i64, ctypes.c_int,
                                ctypes.POINTER(gemv_epilogue_t), vp, ctypes.c_size_t, vp]
    lib.gemv_run_ws.restype = st
    lib.gemv_run_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, ctypes.c_int,
                                     ctypes.POINTER(gemv_epilogue_t), vp]
    lib.gemv_run_noalloc.restype = st
    lib.gemv_check_args_ex.argtypes = [vp, vp, vp, i64, i64, ctypes.c_int,
                                       ctypes.POINTER(gemv_epilogue_t)]
    lib.gemv_check_args_ex.restype = st
    lib.gemv_destroy.argtypes = [vp]
    lib.gemv_destroy.restype = st
    lib.gemv_status_string.argtypes = [st]
    lib.gemv_status_string.restype = ctypes.c_char_p
    lib.gemv_check_args.argtypes = [vp, vp, vp, i64, i64, ctypes.c_int]
    lib.gemv_check_args.restype = st
    lib.gemv_num_variants.argtypes = []
    lib.gemv_num_variants.restype = i32
    lib.gemv_variant_info.argtypes = [i32, ctypes.POINTER(gemv_variant_info_t)]
    lib.gemv_variant_info.restype = st
    lib.gemv_force_config.argtypes = [vp, ctypes.POINTER(gemv_config_t)]
    lib.gemv_force_config.restype = st
    lib.gemv_query_config.argtypes = [vp, i64, i64, ctypes.c_int, i32,
                                      ctypes.POINTER(gemv_config_t)]
    lib.gemv_query_config.restype = st
    lib.gemv_plan_config.argtypes = [i64, i64, ctypes.c_int, i32, i64, i32,
                                     ctypes.POINTER(gemv_config_t)]
    lib.gemv_plan_config.restype = st
    lib.gla_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, ctypes.c_float,
                                    ctypes.c_int, vp]
    lib.gla_decode_step.restype = st
    lib.gla_check_args.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, ctypes.c_int]
    lib.gla_check_args.restype = st
    _lib = lib
    return lib


# ---- the C entry points, same names ------------------------------------------

def gemv_create():
    """Returns (status, handle) -- handle is a ctypes.c_void_p."""
    h = ctypes.c_void_p()
    s = load().gemv_create(ctypes.byref(h))
    return s, h


def gemv_run(h, B, a, c, n, k, dtype, stream=None):
    """B, a, c: device addresses (ints); stream: hipStream_t as int or None."""
    return load().gemv_run(h, B, a, c, n, k, dtype, stream)


def gemv_run_ex(h, B, a, c, n, k, dtype, alpha=1.0, bias=None, stream=None):
    """gemv_run with the epilogue c = alpha * (B @ a) + bias (bias: address or None)."""
    ep = gemv_epilogue_t(alpha, bias)
    return load().gemv_run_ex(h, B, a, c, n, k, dtype, ctypes.byref(ep), stream)


def gemv_run_ws(h, B, a, c, n, k, dtype, workspace, workspace_bytes=GEMV_WORKSPACE_BYTES,
                alpha=None, bias=None, stream=None):
    """gemv_run_ex with caller scratch (workspace: a device address or None);
    no epilogue when alpha and bias are both None."""
    ep = None
    if alpha is not None or bias is not None:
        ep = ctypes.byref(gemv_epilogue_t(1.0 if alpha is None else alpha, bias))
    return load().gemv_run_ws(h, B, a, c, n, k, dtype, ep, workspace, workspace_bytes, stream)


def gemv_run_noalloc(h, B, a, c, n, k, dtype, alpha=None, bias=None, stream=None):
    """gemv_run_ws on the library's static scratch (allocates nothing); no
    epilogue when alpha and bias are both None."""
    ep = None
    if alpha is not None or bias is not None:
        ep = ctypes.byref(gemv_epilogue_t(1.0 if alpha is None else alpha, bias))
    return load().gemv_run_noalloc(h, B, a, c, n, k, dtype, ep, stream)


def gemv_check_args_ex(B, a, c, n, k, dtype, alpha=None, bias=None):
    if alpha is None and bias is None:
        return load().gemv_check_args_ex(B, a, c, n, k, dtype, None)
    ep = gemv_epilogue_t(1.0 if alpha is None else alpha, bias)
    return load().gemv_check_args_ex(B, a, c, n, k, dtype, ctypes.byref(ep))


def gemv_destroy(h):
    return load().gemv_destroy(h)


def gemv_status_string(s):
    return load().gemv_status_string(s).decode()


def gemv_check_args(B, a, c, n, k, dtype):
    return load().gemv_check_args(B, a, c, n, k, dtype)


def gemv_num_variants():
    return load().gemv_num_variants()


def gemv_variant_info(v):
    info = gemv_variant_info_t()
    s = load().gemv_variant_info(v, ctypes.byref(info))
    return s, info


def gemv_force_config(h, variant=-1, grid=0, kgroups=0, flags=0):
    if variant is None:
        return load().gemv_force_config(h, None)
    cfg = gemv_config_t(variant, grid, kgroups, flags)
    return load().gemv_force_config(h, ctypes.byref(cfg))


def gemv_query_config(h, n, k, dtype, with_workspace=0):
    cfg = gemv_config_t()
    s = load().gemv_query_config(h, n, k, dtype, int(with_workspace), ctypes.byref(cfg))
    return s, cfg


def gemv_plan_config(n, k, dtype, b_aligned=1, max_lds=160 * 1024, with_workspace=0):
    """The automatic plan for a shape, on the host alone (no device)."""
    cfg = gemv_config_t()
    s = load().gemv_plan_config(n, k, dtype, int(b_aligned), max_lds, int(with_workspace),
                                ctypes.byref(cfg))
    return s, cfg


def gla_decode_step(h, q, k, v, gk, S_in, S_out, o, bh, dk, dv, scale, dtype, stream=None):
    """One GLA decode step (include/gla_decode.h); all pointers are addresses."""
    return load().gla_decode_step(h, q, k, v, gk, S_in, S_out, o, bh, dk, dv, scale, dtype, stream)


def gla_check_args(q, k, v, gk, S_in, S_out, o, bh, dk, dv, dtype):
    return load().gla_check_args(q, k, v, gk, S_in, S_out, o, bh, dk, dv, dtype)


# ---- torch-tensor convenience ------------------------------------------------

def _dtype_code(t):
    import torch
    if t.dtype == torch.float16:
        return GEMV_F16
    if t.dtype == torch.bfloat16:
        return GEMV_BF16
    raise GemvError(GEMV_ERR_UNSUPPORTED_DTYPE, str(t.dtype))


def _check_devices(tensors, device):
    """Every tensor on `device`, a GPU: the library takes raw addresses and
    cannot tell a host address from a device one, so a CPU tensor (or one on
    another GPU) is refused here, before anything is launched."""
    if device.type != "cuda":
        raise GemvError(GEMV_ERR_INVALID_ARG, "tensors must be on a GPU, got %s" % device)
    for t in tensors:
        if t is not None and t.device != device:
            raise GemvError(GEMV_ERR_INVALID_ARG, "tensors on %s and %s" % (device, t.device))


class Gemv:
    """One handle on the current device.  ``gemv(B, a, c)`` enqueues c = B @ a
    on the current torch stream (or ``stream``); tensors must be dense and on
    the handle's GPU.  With ``workspace=True`` the object also owns caller
    scratch (GEMV_WORKSPACE_BYTES, zero-filled once) and calls gemv_run_ws,
    whose plan may split k across workgroups; calls through one such object
    must then not overlap on the GPU (one stream, or ordered by events)."""

    def __init__(self, workspace=False):
        self.h = None
        self.ws = None
        s, h = gemv_create()
        if s != GEMV_OK:
            raise GemvError(s, "gemv_create")
        self.h = h
        if workspace:
            import torch
            self.ws = torch.zeros(GEMV_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
            torch.cuda.synchronize()     # zero-filled before any stream uses it

    def close(self):
        if self.h is not None:
            gemv_destroy(self.h)
            self.h = None
        self.ws = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def force_config(self, variant=-1, grid=0, kgroups=0, flags=0):
        s = gemv_force_config(self.h, variant, grid, kgroups, flags)
        if s != GEMV_OK:
            raise GemvError(s, "gemv_force_config")

    def query_config(self, n, k, dtype, with_workspace=None):
        """(variant, grid, kgroups) of the plan a call would launch; by default
        for the entry point this object calls (with or without scratch)."""
        if with_workspace is None:
            with_workspace = self.ws is not None
        s, cfg = gemv_query_config(self.h, n, k, dtype, with_workspace)
        if s != GEMV_OK:
            raise GemvError(s, "gemv_query_config")
        return cfg.variant, cfg.grid, cfg.kgroups

    def __call__(self, B, a, c, stream=None, alpha=None, bias=None, use_workspace=True):
        """c = B @ a, or c = alpha * (B @ a) + bias when alpha or bias is given
        (bias: an (n,) tensor of the same dtype, possibly c itself).
        use_workspace=False calls gemv_run / gemv_run_ex even when the object
        owns scratch."""
        import torch
        if B.dim() != 2 or a.dim() != 1 or c.dim() != 1:
            raise GemvError(GEMV_ERR_INVALID_ARG, "B must be 2-D, a and c 1-D")
        n, k = B.shape
        if a.shape[0] != k or c.shape[0] != n:
            raise GemvError(GEMV_ERR_INVALID_ARG, "shapes B%s a%s c%s" % (
                tuple(B.shape), tuple(a.shape), tuple(c.shape)))
        if not (B.is_contiguous() and a.is_contiguous() and c.is_contiguous()):
            raise GemvError(GEMV_ERR_INVALID_ARG, "tensors must be contiguous")
        _check_devices((a, c, bias), B.device)
        dt = _dtype_code(B)
        if a.dtype != B.dtype or c.dtype != B.dtype:
            raise GemvError(GEMV_ERR_UNSUPPORTED_DTYPE, "B, a and c must share one dtype")
        bp = None
        if bias is not None:
            if bias.dim() != 1 or bias.shape[0] != n or bias.dtype != B.dtype or \
                    not bias.is_contiguous():
                raise GemvError(GEMV_ERR_INVALID_ARG, "bias must be a dense (n,) tensor of B's dtype")
            bp = bias.data_ptr()
        if stream is None:
            stream = torch.cuda.current_stream(B.device).cuda_stream
        if self.ws is not None and use_workspace:
            if self.ws.device != B.device:
                raise GemvError(GEMV_ERR_INVALID_ARG, "the workspace is on %s" % self.ws.device)
            s = gemv_run_ws(self.h, B.data_ptr(), a.data_ptr(), c.data_ptr(), n, k, dt,
                            self.ws.data_ptr(), self.ws.numel(), alpha, bp, stream)
        elif alpha is None and bias is None:
            s = gemv_run(self.h, B.data_ptr(), a.data_ptr(), c.data_ptr(), n, k, dt, stream)
        else:
            s = gemv_run_ex(self.h, B.data_ptr(), a.data_ptr(), c.data_ptr(), n, k, dt,
                            1.0 if alpha is None else float(alpha), bp, stream)
        if s != GEMV_OK:
            raise GemvError(s, "gemv_run")
        return c


class GlaDecode:
    """One GLA decode step on torch tensors, through a Gemv handle:
    S_out = diag(exp(gk)) S_in + outer(k, v); o = scale * q^T S_out, per head.
    q, k, gk: (bh, dk); v: (bh, dv); S_in, S_out: float32 (bh, dk, dv), S_out may
    be S_in; o: (bh, dv) of q's dtype."""

    def __init__(self, gemv=None):
        self.g = gemv if gemv is not None else Gemv()

    def __call__(self, q, k, v, gk, S_in, S_out, o, scale, stream=None):
        import torch
        bh, dk = q.shape
        dv = v.shape[1]
        for t, shape in ((k, (bh, dk)), (gk, (bh, dk)), (v, (bh, dv)), (o, (bh, dv)),
                         (S_in, (bh, dk, dv)), (S_out, (bh, dk, dv))):
            if tuple(t.shape) != shape or not t.is_contiguous():
                raise GemvError(GEMV_ERR_INVALID_ARG, "shape/contiguity of a GLA argument")
        _check_devices((k, v, gk, S_in, S_out, o), q.device)
        dt = _dtype_code(q)
        if any(t.dtype != q.dtype for t in (k, v, gk, o)) or S_in.dtype != torch.float32 or \
                S_out.dtype != torch.float32:
            raise GemvError(GEMV_ERR_UNSUPPORTED_DTYPE, "q, k, v, gk, o share a 16-bit dtype; S is float32")
        if stream is None:
            stream = torch.cuda.current_stream(q.device).cuda_stream
        s = gla_decode_step(self.g.h, q.data_ptr(), k.data_ptr(), v.data_ptr(), gk.data_ptr(),
                            S_in.data_ptr(), S_out.data_ptr(), o.data_ptr(), bh, dk, dv,
                            float(scale), dt, stream)
        if s != GEMV_OK:
            raise GemvError(s, "gla_decode_step")
        return o
