"""ctypes binding of libmbd_probe.so (include/stream_probe.h): measurement
aids, not part of the GEMV path -- a plain streaming read and copy of a
device buffer (the HBM bandwidth the GPU delivers in practice), and the GEMV
kernel with its arithmetic taken out (what its access pattern costs alone)."""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmbd_probe.so")
READ_BLOCK = 1024    # mbd_stream_read sizes are multiples of this
CHUNK = 16384        # mbd_stream_copy sizes are multiples of this

_lib = None


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmbd_probe.so is not built; run "
                               "`python -m memory_bound_dense_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        lib.mbd_stream_read.argtypes = [vp, ctypes.c_size_t, vp, i32, i32, i32, i32, vp,
                                        ctypes.POINTER(ctypes.c_int)]
        lib.mbd_stream_read.restype = i32
        lib.mbd_stream_copy.argtypes = [vp, vp, ctypes.c_size_t, i32, i32, vp]
        lib.mbd_stream_copy.restype = i32
        lib.mbd_gemv_probe_has.argtypes = [i32, i32, i32, i32, i32]
        lib.mbd_gemv_probe_has.restype = i32
        lib.mbd_gemv_probe.argtypes = [i32, i32, i32, i32, i32, vp, i64, i64, vp, vp, i32, i32, vp]
        lib.mbd_gemv_probe.restype = i32
        _lib = lib
    return _lib


def stream_read(src_ptr, nbytes, out_ptr, out_len, grid=0, unroll=8, nontemporal=True,
                stream=None):
    """Enqueue one streaming read; returns the workgroup count launched."""
    launched = ctypes.c_int(0)
    rc = load().mbd_stream_read(src_ptr, nbytes, out_ptr, out_len, grid, unroll,
                                int(bool(nontemporal)), stream, ctypes.byref(launched))
    if rc != 0:
        raise RuntimeError("mbd_stream_read failed (%d)" % rc)
    return launched.value


def stream_copy(src_ptr, dst_ptr, nbytes, grid=0, nontemporal=True, stream=None):
    """Enqueue one streaming copy of nbytes (a multiple of CHUNK)."""
    rc = load().mbd_stream_copy(src_ptr, dst_ptr, nbytes, grid, int(bool(nontemporal)), stream)
    if rc != 0:
        raise RuntimeError("mbd_stream_copy failed (%d)" % rc)


def gemv_probe_has(info):
    """Whether the arithmetic-free GEMV build exists for a variant's shape."""
    return bool(load().mbd_gemv_probe_has(info.rows, info.unroll, info.waves, info.splits,
                                          info.cross_wg)) and info.a_mode == 1 and \
        info.layout == 0 and info.stages == 0


def gemv_probe(info, B_ptr, n, k, out_ptr, workspace_ptr, grid, kgroups, stream=None):
    """Enqueue the GEMV launch of variant shape `info` without its arithmetic."""
    rc = load().mbd_gemv_probe(info.rows, info.unroll, info.waves, info.splits, info.cross_wg,
                               B_ptr, n, k, out_ptr, workspace_ptr, grid, kgroups, stream)
    if rc != 0:
        raise RuntimeError("mbd_gemv_probe failed (%d)" % rc)
