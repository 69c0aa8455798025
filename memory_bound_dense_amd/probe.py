"""ctypes binding of libmbd_probe.so (include/stream_probe.h): a plain
streaming read of a device buffer, used to measure the HBM read bandwidth the
GPU delivers in practice.  Not part of the GEMV path."""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmbd_probe.so")
CHUNK = 16384   # bytes per workgroup per loop trip; sizes must be multiples

_lib = None


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmbd_probe.so is not built; run "
                               "`python -m memory_bound_dense_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        lib.mbd_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.POINTER(ctypes.c_int)]
        lib.mbd_stream_read.restype = ctypes.c_int
        lib.mbd_stream_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        lib.mbd_stream_copy.restype = ctypes.c_int
        _lib = lib
    return _lib


def stream_read(src_ptr, nbytes, out_ptr, out_len, grid=0, nontemporal=True, stream=None,
                xcd_contiguous=False):
    """Enqueue one streaming read; returns the workgroup count launched."""
    launched = ctypes.c_int(0)
    rc = load().mbd_stream_read(src_ptr, nbytes, out_ptr, out_len, grid, int(bool(nontemporal)),
                                int(bool(xcd_contiguous)), stream, ctypes.byref(launched))
    if rc != 0:
        raise RuntimeError("mbd_stream_read failed (%d)" % rc)
    return launched.value


def stream_copy(src_ptr, dst_ptr, nbytes, grid=0, nontemporal=True, stream=None):
    """Enqueue one streaming copy of nbytes (a multiple of CHUNK)."""
    rc = load().mbd_stream_copy(src_ptr, dst_ptr, nbytes, grid, int(bool(nontemporal)), stream)
    if rc != 0:
        raise RuntimeError("mbd_stream_copy failed (%d)" % rc)
