"""The C ABI's validation layer under the address and undefined-behaviour
sanitizers, on the CPU. api.cpp (argument checks) and plan.cpp (launch plans
and workspace sizes) are built with g++ -fsanitize=address,undefined into a
library whose kernel launchers are stubs (tests/asan/launch_stubs.cpp) that
record each call. In a child process with the sanitizer runtime preloaded:
  * every case of tests/test_abi.py runs against that library (a sanitizer
    report aborts the child, so the test fails), and
  * valid calls of every entry point reach their launcher with the arguments
    they were given (the workspace pointer included; the allocation-free
    grouped GEMM gets the library's own array).
Skipped where g++ or its sanitizer runtime is missing, or where another
library is already preloaded into this process tree."""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mpgemm_token_absmax_amd", "csrc")
ROCM_INC = "/opt/rocm/include"


@pytest.fixture(scope="module")
def asan_lib(tmp_path_factory):
    gxx = shutil.which("g++")
    if not gxx or not os.path.isdir(ROCM_INC):
        pytest.skip("g++ or the HIP headers are missing")
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("a library is already preloaded; the sanitizer runtime is not added to it")
    libasan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True,
                             text=True).stdout.strip()
    if not os.path.isabs(libasan) or not os.path.exists(libasan):
        pytest.skip("libasan.so not found")
    out = tmp_path_factory.mktemp("asan") / "libbitlinear_asan.so"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROCM_INC}", "-Wall", "-Werror",
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(ROOT, "tests", "asan", "launch_stubs.cpp"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return str(out), libasan


def _run_child(asan_lib, code):
    lib, libasan = asan_lib
    env = dict(os.environ, LD_PRELOAD=libasan, BL_ASAN_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", textwrap.dedent(code)], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
    return r.stdout


def test_abi_cases_under_sanitizers(asan_lib):
    out = _run_child(asan_lib, """
        import os, sys
        sys.path.insert(0, os.getcwd())
        import mpgemm_token_absmax_amd._lib as L
        L.LIB_PATH = os.environ["BL_ASAN_LIB"]
        import pytest
        sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", "tests/test_abi.py",
                              "-k", "not probe_library"]))
    """)
    assert "passed" in out and "failed" not in out, out[-2000:]


def test_valid_calls_reach_the_launchers(asan_lib):
    _run_child(asan_lib, """
        import ctypes, os, sys
        sys.path.insert(0, os.getcwd())
        import mpgemm_token_absmax_amd._lib as L
        L.LIB_PATH = os.environ["BL_ASAN_LIB"]
        lib = L.lib()
        raw = ctypes.CDLL(os.environ["BL_ASAN_LIB"])
        raw.blstub_calls.restype = ctypes.c_longlong
        raw.blstub_last_name.restype = ctypes.c_char_p
        raw.blstub_last.argtypes = [ctypes.POINTER(ctypes.c_longlong), ctypes.POINTER(ctypes.c_void_p)]
        A, B, C, D, E, F = (0x10000 * i for i in range(1, 7))

        def last(expect_name):
            n0 = last.calls
            last.calls = raw.blstub_calls()
            assert last.calls == n0 + 1, (expect_name, last.calls, n0)
            assert raw.blstub_last_name().decode() == expect_name, raw.blstub_last_name()
            v = (ctypes.c_longlong * 4)()
            ws = ctypes.c_void_p()
            raw.blstub_last(v, ctypes.byref(ws))
            return list(v), ws.value
        last.calls = raw.blstub_calls()

        ok = L.BL_OK
        assert lib.bl_quantize_act(A, 3, 64, 64, B, C, None, None) == ok
        assert last("quantize_act")[0][:3] == [3, 0, 64]
        ws = lib.bl_quantize_act_tensor_workspace(3)
        assert lib.bl_quantize_act_tensor(A, 3, 64, 64, B, C, None, D, ws, None) == ok
        assert last("quantize_act_tensor")[1] == D
        assert lib.bl_rmsnorm_quant(A, None, B, ctypes.c_float(1e-5), 2, 64, 64, None, C, D, None, None) == ok
        last("rmsnorm_quant")
        need = lib.bl_pack_i2s_workspace(64, 256)
        assert lib.bl_pack_i2s(A, L.BL_W_F32, 64, 256, B, C, D, need, None) == ok
        assert last("pack_f32")[1] == D
        assert lib.bl_pack_i2s(A, L.BL_W_TERNARY_I8, 64, 256, B, None, None, 0, None) == ok
        last("pack_ternary")
        assert lib.bl_gemv(A, B, 640, 2560, C, D, 4, E, L.BL_OUT_BF16, None) == ok
        assert last("gemv")[0][:3] == [4, 640, 2560]
        # the GEMM: with a workspace of exactly the size asked for, and without one
        need = lib.bl_gemm_workspace(64, 2560, 6912)
        assert need > 0
        assert lib.bl_gemm(A, B, 2560, 6912, C, D, None, 64, E, L.BL_OUT_BF16, F, need, None) == ok
        v, wsp = last("gemm")
        assert v[:3] == [64, 2560, 6912] and wsp == F
        assert lib.bl_gemm(A, B, 2560, 6912, C, D, None, 64, E, L.BL_OUT_BF16, None, 0, None) == ok
        assert last("gemm")[1] is None
        P = L.GemmProblem
        arr = (P * 3)(P(A, B, 2560, E, 2), P(A, B, 0, None, 2), P(A, B, 640, F, 1))
        Ns = (ctypes.c_int64 * 3)(2560, 0, 640)
        need = lib.bl_gemm_group_workspace(Ns, 3, 6912, 64)
        assert need > 0
        assert lib.bl_gemm_group(arr, 3, 6912, C, D, None, 64, A, need, None) == ok
        v, wsp = last("gemm_group")
        assert v == [64, 2560, 6912, 2] and wsp == A        # the N == 0 problem is dropped
        assert lib.bl_gemm_group_noalloc(arr, 3, 6912, C, D, None, 64, None) == ok
        v, wsp = last("gemm_group")
        assert v == [64, 2560, 6912, 2] and wsp not in (None, 0)
        D_ = L.DecodeProblem
        darr = (D_ * 2)(D_(A, B, 640, 2560, C, 2560, None, None, E, 2),
                        D_(A, B, 2560, 2560, C, 2560, None, None, F, 2))
        assert lib.bl_decode_group(darr, 2, 1, None) == ok
        assert last("decode_group")[0] == [1, 640, 2560, 2]
        assert lib.bl_decode_norm_group(darr, 2, None, D, ctypes.c_float(1e-5), None, None) == ok
        last("decode_norm_group")
        t3 = (D_ * 1)(D_(A, B, 64, 336, C, 336, None, None, E, 2))
        assert lib.bl_decode_group_t3(t3, 1, 1, None) == ok
        last("decode_group_t3")
        print("reached every launcher")
    """)
