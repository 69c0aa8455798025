"""The C ABI without a GPU: the library loads, exports every declared symbol,
and rejects every bad argument with the documented status before any launch.
"""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

import memory_bound_dense_amd as mbd
from memory_bound_dense_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", "gemv.h"), os.path.join(ROOT, "include", "gla_decode.h")]


def _declared_functions():
    names = set()
    for hdr in HEADERS:
        text = open(hdr).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**((?:gemv|gla)_\w+)\s*\(", text,
                                flags=re.M))
    return sorted(names)


def test_header_declares_the_binding_exports():
    assert _declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for code in range(0, 11):
        s = mbd.gemv_status_string(code)
        assert s.startswith("GEMV_"), s
    assert mbd.gemv_status_string(0) == "GEMV_OK"
    assert mbd.gemv_status_string(5) == "GEMV_ERR_ALIASING"
    assert mbd.gemv_status_string(99) == "GEMV_ERR_UNKNOWN"


def test_variant_table():
    nv = mbd.gemv_num_variants()
    assert nv >= 4
    for v in range(nv):
        s, info = mbd.gemv_variant_info(v)
        assert s == mbd.GEMV_OK
        assert info.rows >= 1 and info.unroll >= 1 and info.waves >= 1
        assert info.splits >= 1 and info.waves % info.splits == 0
        assert info.a_mode in (0, 1, 2, 3)
        assert info.cross_wg in (0, 1)
        if info.cross_wg:
            assert info.a_mode == 1      # a k-chunk per workgroup reads a through the caches
        if info.a_mode == 2:
            assert info.rows in (1, 2) and not info.cross_wg
        if info.a_mode == 3:
            assert info.rows in (1, 2) and not info.cross_wg and info.stages == 0
        assert info.layout in (0, 1)
        if info.layout == 1:
            assert info.rows == 64 and info.splits == 1 and not info.cross_wg
        assert 0 <= info.stages <= 3 and info.b_lds in (0, 1)
        if info.stages:
            # pipelined B: cached a, one wave per row range, no split
            assert info.a_mode == 1 and info.splits == 1 and not info.cross_wg
            assert info.layout == 0
        else:
            assert info.b_lds == 0
    assert mbd.gemv_variant_info(nv)[0] == _lib.GEMV_ERR_INVALID_ARG
    assert mbd.gemv_variant_info(-1)[0] == _lib.GEMV_ERR_INVALID_ARG


def test_null_handle_rejected():
    assert mbd.gemv_run(None, 256, 512, 1 << 20, 4, 8, 0, None) == _lib.GEMV_ERR_NULL_HANDLE
    assert mbd.gemv_run_ws(None, 256, 512, 1 << 20, 4, 8, 0, 1 << 30) == _lib.GEMV_ERR_NULL_HANDLE
    assert mbd.gemv_force_config(None, 0, 0) == _lib.GEMV_ERR_NULL_HANDLE
    assert mbd.gemv_query_config(None, 4, 8, 0)[0] == _lib.GEMV_ERR_NULL_HANDLE
    assert mbd.gemv_destroy(None) == mbd.GEMV_OK


def test_binding_refuses_tensors_off_the_gpu():
    """The library takes raw addresses and cannot tell host memory from
    device memory: the binding refuses CPU tensors, and tensors on another
    device than B's (q's for GLA), before any call into the library."""
    import torch
    g = mbd.Gemv.__new__(mbd.Gemv)       # no handle: the device check comes first
    g.h, g.ws = None, None
    B = torch.zeros((4, 8), dtype=torch.float16)
    a = torch.zeros(8, dtype=torch.float16)
    c = torch.zeros(4, dtype=torch.float16)
    with pytest.raises(mbd.GemvError) as e:
        g(B, a, c)
    assert e.value.status == _lib.GEMV_ERR_INVALID_ARG and "GPU" in str(e.value)
    gpu = torch.device("cuda", 0)
    for t in (a, torch.empty(8, dtype=torch.float16, device="meta")):
        with pytest.raises(mbd.GemvError) as e:
            _lib._check_devices((t,), gpu)
        assert e.value.status == _lib.GEMV_ERR_INVALID_ARG
    _lib._check_devices((None,), gpu)     # an absent bias is fine
    gla = mbd.GlaDecode(gemv=g)
    q = torch.zeros((2, 4), dtype=torch.bfloat16)
    S = torch.zeros((2, 4, 4), dtype=torch.float32)
    v = torch.zeros((2, 4), dtype=torch.bfloat16)
    with pytest.raises(mbd.GemvError) as e:
        gla(q, q, v, q, S, S, v, 1.0)
    assert e.value.status == _lib.GEMV_ERR_INVALID_ARG


def test_create_without_gpu_fails_cleanly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    s, h = mbd.gemv_create()
    assert s in (_lib.GEMV_ERR_HIP, _lib.GEMV_ERR_UNSUPPORTED)
    assert not h.value


# Fake, well-separated device addresses: gemv_check_args never dereferences.
B0, A0, C0 = 1 << 32, 1 << 34, 1 << 36


@pytest.mark.parametrize("args,expect", [
    ((B0, A0, C0, 4, 8, 0), _lib.GEMV_OK),
    ((B0, A0, C0, 4, 8, 1), _lib.GEMV_OK),
    ((B0, A0, C0, 4, 8, 2), _lib.GEMV_ERR_UNSUPPORTED_DTYPE),
    ((B0, A0, C0, 4, 8, -1), _lib.GEMV_ERR_UNSUPPORTED_DTYPE),
    ((B0, A0, C0, -1, 8, 0), _lib.GEMV_ERR_INVALID_ARG),
    ((B0, A0, C0, 4, -8, 0), _lib.GEMV_ERR_INVALID_ARG),
    ((0, 0, 0, 0, 8, 0), _lib.GEMV_OK),                     # n == 0: no-op before pointer checks
    ((0, A0, C0, 4, 8, 0), _lib.GEMV_ERR_INVALID_ARG),      # null B
    ((B0, A0, 0, 4, 8, 0), _lib.GEMV_ERR_INVALID_ARG),      # null c
    ((B0, 0, C0, 4, 8, 0), _lib.GEMV_ERR_INVALID_ARG),      # null a with k > 0
    ((B0, 0, C0, 4, 0, 0), _lib.GEMV_OK),                   # a unused when k == 0
    ((0, 0, C0, 4, 0, 0), _lib.GEMV_OK),                    # nor B
    ((B0 + 1, A0 + 1, C0, 4, 0, 0), _lib.GEMV_OK),          # nor their alignment
    ((B0, A0, 0, 4, 0, 0), _lib.GEMV_ERR_INVALID_ARG),      # c is written: never NULL
    ((B0 + 1, A0, C0, 4, 8, 0), _lib.GEMV_ERR_MISALIGNED),
    ((B0, A0 + 1, C0, 4, 8, 0), _lib.GEMV_ERR_MISALIGNED),
    ((B0, A0, C0 + 1, 4, 8, 0), _lib.GEMV_ERR_MISALIGNED),
    ((B0 + 2, A0 + 6, C0 + 14, 4, 8, 0), _lib.GEMV_OK),     # 2-byte alignment is enough
    ((B0, A0, C0, 2 ** 30 + 1, 8, 0), _lib.GEMV_ERR_TOO_LARGE),
    ((B0, A0, C0, 4, 2 ** 27 + 1, 0), _lib.GEMV_ERR_TOO_LARGE),
    ((B0, A0, C0, 4, 2 ** 27, 0), _lib.GEMV_OK),
    ((B0, A0, B0 + 16, 4, 8, 0), _lib.GEMV_ERR_ALIASING),   # c inside B
    ((B0, A0, B0 - 6, 4, 8, 0), _lib.GEMV_ERR_ALIASING),    # c straddles B's start
    ((B0, A0, B0 - 8, 4, 8, 0), _lib.GEMV_OK),              # c ends where B starts
    ((B0, A0, B0 + 64, 4, 8, 0), _lib.GEMV_OK),             # c starts where B ends
    ((B0, A0, A0 + 2, 4, 8, 0), _lib.GEMV_ERR_ALIASING),    # c overlaps a
])
def test_check_args(args, expect):
    assert mbd.gemv_check_args(*args) == expect


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError):
        _lib.load()


@pytest.mark.parametrize("bias,expect", [
    (None, _lib.GEMV_OK),
    (1 << 38, _lib.GEMV_OK),
    ((1 << 38) + 1, _lib.GEMV_ERR_MISALIGNED),
    (C0, _lib.GEMV_OK),                      # bias == c: accumulate in place
    (C0 + 2, _lib.GEMV_ERR_ALIASING),        # partial overlap with c
    (C0 - 6, _lib.GEMV_ERR_ALIASING),
    (C0 - 8, _lib.GEMV_OK),                  # ends where c starts (n = 4)
])
def test_check_args_epilogue(bias, expect):
    assert mbd.gemv_check_args_ex(B0, A0, C0, 4, 8, 0, 0.5, bias) == expect
    # the plain checks still come first
    assert mbd.gemv_check_args_ex(B0 + 1, A0, C0, 4, 8, 0, 0.5, bias) == _lib.GEMV_ERR_MISALIGNED
    assert mbd.gemv_check_args_ex(B0, A0, C0, 4, 8, 0) == _lib.GEMV_OK



# GLA decode step: fake, well-separated addresses (16-byte aligned state)
Q0, K0, V0, G0, S0, S1, O0 = (1 << 40) + 0, (1 << 40) + (1 << 30), (1 << 40) + (2 << 30), \
    (1 << 40) + (3 << 30), 1 << 41, (1 << 41) + (1 << 34), 1 << 42


@pytest.mark.parametrize("args,expect", [
    ((Q0, K0, V0, G0, S0, S1, O0, 32, 128, 128, 1), _lib.GEMV_OK),
    ((Q0, K0, V0, G0, S0, S0, O0, 32, 128, 128, 1), _lib.GEMV_OK),         # in place
    ((Q0, K0, V0, G0, S0, S0 + 16, O0, 32, 128, 128, 1), _lib.GEMV_ERR_ALIASING),
    ((Q0, K0, V0, G0, S0, S1, S1 + 64, 32, 128, 128, 1), _lib.GEMV_ERR_ALIASING),   # o in the state
    ((Q0, K0, V0, G0, S0, S1, Q0 + 2, 32, 128, 128, 1), _lib.GEMV_ERR_ALIASING),    # o over q
    ((Q0, K0, V0, G0, S0, S1, O0, 32, 128, 126, 1), _lib.GEMV_ERR_INVALID_ARG),    # dv % 4
    ((Q0, K0, V0, G0, S0 + 8, S1, O0, 32, 128, 128, 1), _lib.GEMV_ERR_MISALIGNED),
    ((Q0 + 1, K0, V0, G0, S0, S1, O0, 32, 128, 128, 1), _lib.GEMV_ERR_MISALIGNED),
    ((Q0, K0, V0, G0, S0, S1, O0, 32, 128, 128, 2), _lib.GEMV_ERR_UNSUPPORTED_DTYPE),
    ((Q0, K0, V0, G0, S0, S1, O0, -1, 128, 128, 1), _lib.GEMV_ERR_INVALID_ARG),
    ((0, 0, 0, 0, 0, 0, 0, 0, 128, 128, 1), _lib.GEMV_OK),                  # bh == 0: no-op
    ((0, 0, 0, 0, 0, 0, O0, 32, 0, 128, 1), _lib.GEMV_OK),                  # dk == 0: only o
    ((0, K0, V0, G0, S0, S1, O0, 32, 128, 128, 1), _lib.GEMV_ERR_INVALID_ARG),
    ((Q0, K0, V0, G0, S0, S1, O0, 32, 65537, 4, 1), _lib.GEMV_ERR_TOO_LARGE),
    ((Q0, K0, V0, G0, S0, S1, O0, 32, 32768, 16384, 1), _lib.GEMV_ERR_TOO_LARGE),
])
def test_gla_check_args(args, expect):
    assert mbd.gla_check_args(*args) == expect


def test_gla_null_handle():
    assert mbd.gla_decode_step(None, Q0, K0, V0, G0, S0, S1, O0, 1, 4, 4, 1.0, 0) == \
        _lib.GEMV_ERR_NULL_HANDLE


def test_plain_c_consumer(tmp_path):
    """The headers compile as C99 and a C program links every entry point
    from the library and calls the host-only ones (tests/c_abi/consumer.c)."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lib_dir = os.path.dirname(_lib.LIB_PATH)
    exe = str(tmp_path / "consumer")
    build = subprocess.run(
        [cc, "-std=c99", "-Wall", "-Werror", "-isystem", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__",
         "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi", "consumer.c"),
         "-L", lib_dir, "-lgemv", "-Wl,-rpath," + lib_dir, "-o", exe],
        capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stderr
    out = dict(line.split(" ", 1) for line in run.stdout.splitlines())
    assert out["linked"] == str(len(_lib.EXPORTS))
    assert out["status0"] == "GEMV_OK" and out["status5"] == "GEMV_ERR_ALIASING"
    assert out["check_ok"] == str(_lib.GEMV_OK)
    assert out["check_misaligned"] == str(_lib.GEMV_ERR_MISALIGNED)
    assert out["check_too_large"] == str(_lib.GEMV_ERR_TOO_LARGE)
    assert out["plan_status"] == str(_lib.GEMV_OK)
    assert out["plan_shape"] == "R2 U4 W4 S4 grid 9216"      # the headline's plan
    assert out["variants"] == str(mbd.gemv_num_variants())
    assert out["plan_ws_kgroups"] == "%d 8" % _lib.GEMV_OK   # 64 x 65536: 8 k-groups with scratch
    assert out["workspace_bytes"] == str(_lib.GEMV_WORKSPACE_BYTES)
    assert out["run_ws_null_handle"] == str(_lib.GEMV_ERR_NULL_HANDLE)
    assert out["run_noalloc_null_handle"] == str(_lib.GEMV_ERR_NULL_HANDLE)
    assert out["gla_check"] == str(_lib.GEMV_OK)
    import torch
    if torch.cuda.is_available():
        assert out["create"] == "ok handle"
    else:
        assert out["create"] == "error null"
    assert out["destroy"] == str(_lib.GEMV_OK)
