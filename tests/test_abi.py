"""C ABI checks that need no GPU: the library loads, exports every function
include/bitlinear.h declares, and rejects bad arguments before launching
anything (every call below fails validation, so no kernel is enqueued)."""
import ctypes
import os
import re

import pytest

from mpgemm_token_absmax_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitlinear.h")

A16 = 0x10000          # fake, 16-byte aligned device addresses (never dereferenced)
B16 = 0x20000
C16 = 0x30000
D16 = 0x40000
E16 = 0x50000


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bl_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libbitlinear.so not built (run __graft_entry__.build())")
    return L.lib()


def test_exports_every_declared_symbol(lib):
    declared = header_functions()
    assert set(declared) == set(L.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.bl_abi_version() == 4
    for s in (L.BL_OK, L.BL_ERR_NULL, L.BL_ERR_SHAPE, L.BL_ERR_ALIGN, L.BL_ERR_DTYPE,
              L.BL_ERR_WORKSPACE, L.BL_ERR_HIP, L.BL_ERR_ALIAS):
        assert lib.bl_status_string(s)
    assert lib.bl_status_string(12345) == b"unknown status"


def test_quantize_validation(lib):
    f = lib.bl_quantize_act
    assert f(A16, 2, 6, 6, B16, C16, None, None) == L.BL_ERR_SHAPE        # K % 4
    assert f(A16, -1, 8, 8, B16, C16, None, None) == L.BL_ERR_SHAPE
    assert f(A16, 2, 8, 4, B16, C16, None, None) == L.BL_ERR_SHAPE        # ldx < K
    assert f(None, 2, 8, 8, B16, C16, None, None) == L.BL_ERR_NULL
    assert f(A16, 2, 8, 8, None, C16, None, None) == L.BL_ERR_NULL
    assert f(A16, 2, 8, 8, B16, None, None, None) == L.BL_ERR_NULL
    assert f(A16 + 8, 2, 8, 8, B16, C16, None, None) == L.BL_ERR_ALIGN
    assert f(A16, 2, 8, 8, B16 + 4, C16, None, None) == L.BL_ERR_ALIGN
    assert f(A16, 2, 8, 8, B16, C16 + 2, None, None) == L.BL_ERR_ALIGN
    assert f(A16, 2, 8, 10, B16, C16, None, None) == L.BL_ERR_ALIGN       # ldx % 4
    assert f(None, 0, 8, 8, None, None, None, None) == L.BL_OK            # M == 0: nothing to do
    # qsum (token sums) is optional; when given it must be 4-byte aligned and
    # 127*K must fit int32
    assert f(A16, 2, 8, 8, B16, C16, D16 + 2, None) == L.BL_ERR_ALIGN
    assert f(A16, 2, 1 << 25, 1 << 25, B16, C16, D16, None) == L.BL_ERR_SHAPE


def test_pack_validation(lib):
    f = lib.bl_pack_i2s
    ws = lib.bl_pack_i2s_workspace(64, 64)
    assert ws > 0 and ws % 16 == 0
    assert lib.bl_pack_i2s_workspace(0, 64) == 0
    assert f(A16, 0, 4, 6, B16, C16, D16, ws, None) == L.BL_ERR_SHAPE
    assert f(A16, 7, 4, 8, B16, C16, D16, ws, None) == L.BL_ERR_DTYPE
    assert f(A16, 0, 0, 8, B16, C16, D16, ws, None) == L.BL_ERR_SHAPE   # empty fp32: no gamma
    assert f(None, 0, 64, 64, B16, C16, D16, ws, None) == L.BL_ERR_NULL
    assert f(A16, 0, 64, 64, B16, None, D16, ws, None) == L.BL_ERR_NULL
    assert f(A16, 0, 64, 64, B16, C16, None, ws, None) == L.BL_ERR_WORKSPACE
    assert f(A16, 0, 64, 64, B16, C16, D16, ws - 1, None) == L.BL_ERR_WORKSPACE
    assert f(A16 + 4, 0, 64, 64, B16, C16, D16, ws, None) == L.BL_ERR_ALIGN
    assert f(A16, 0, 64, 64, B16 + 1, C16, D16, ws, None) == L.BL_ERR_ALIGN
    assert f(A16, 0, 1 << 30, 1 << 10, B16, C16, D16, 1 << 40, None) == L.BL_ERR_SHAPE
    assert f(None, 1, 64, 64, B16, None, None, 0, None) == L.BL_ERR_NULL
    assert f(A16, 1, 64, 64, B16 + 8, None, None, 0, None) == L.BL_ERR_ALIGN
    assert f(None, 1, 0, 64, None, None, None, 0, None) == L.BL_OK     # empty ternary pack


@pytest.mark.parametrize("name", ["bl_gemv", "bl_gemm"])
def test_matmul_validation(lib, name):
    fn = getattr(lib, name)

    def call(packed=A16, gamma=B16, N=64, K=64, q=C16, d=D16, M=2, y=E16, yt=1, qsum=None):
        if name == "bl_gemv":
            return fn(packed, gamma, N, K, q, d, M, y, yt, None)
        return fn(packed, gamma, N, K, q, d, qsum, M, y, yt, None, 0, None)

    assert call(K=6) == L.BL_ERR_SHAPE
    assert call(N=-1) == L.BL_ERR_SHAPE
    assert call(M=-3) == L.BL_ERR_SHAPE
    assert call(yt=3) == L.BL_ERR_DTYPE
    assert call(y=None) == L.BL_ERR_NULL
    assert call(packed=None) == L.BL_ERR_NULL
    assert call(q=None) == L.BL_ERR_NULL
    assert call(gamma=None) == L.BL_ERR_NULL
    assert call(d=None) == L.BL_ERR_NULL
    assert call(packed=A16 + 4) == L.BL_ERR_ALIGN
    assert call(q=C16 + 1) == L.BL_ERR_ALIGN
    assert call(y=E16 + 8) == L.BL_ERR_ALIGN
    assert call(gamma=B16 + 2) == L.BL_ERR_ALIGN
    assert call(K=132108) == L.BL_ERR_SHAPE           # 127*K >= 2^24 with a float output
    assert call(M=0) == L.BL_OK and call(N=0) == L.BL_OK
    assert call(M=0, y=None, packed=None, q=None) == L.BL_OK
    if name == "bl_gemv":
        assert call(M=17) == L.BL_ERR_SHAPE           # gemv covers M <= 16 only
    else:
        assert lib.bl_gemm_workspace(2048, 8192, 8192) == 0
        assert call(qsum=E16 + 0x1002) == L.BL_ERR_ALIGN   # token sums: 4-byte aligned


def test_status_to_exception(lib):
    with pytest.raises(L.BitLinearError) as e:
        L.check("bl_gemv", L.BL_ERR_SHAPE)
    assert e.value.status == L.BL_ERR_SHAPE
    assert "shape" in str(e.value)


def test_decode_group_validation(lib):
    P = L.DecodeProblem

    def prob(**kw):
        base = dict(packed=A16, gamma=B16, N=64, K=256, x=C16, ldx=256, q=None, d=None, y=E16,
                    ytype=2)
        base.update(kw)
        return P(**base)

    def call(probs, M=1):
        arr = (P * max(1, len(probs)))(*probs)
        return lib.bl_decode_group(arr, len(probs), M, None)

    assert call([prob()] * 9) == L.BL_ERR_SHAPE            # more than 8 problems
    assert call([prob()], M=17) == L.BL_ERR_SHAPE           # more than 16 tokens
    assert call([prob(K=260, ldx=260)]) == L.BL_ERR_SHAPE   # K % 64
    assert call([prob(ldx=128)]) == L.BL_ERR_SHAPE          # ldx < K
    assert call([prob(ytype=5)]) == L.BL_ERR_DTYPE
    assert call([prob(packed=None)]) == L.BL_ERR_NULL
    assert call([prob(x=None)]) == L.BL_ERR_NULL
    assert call([prob(gamma=None)]) == L.BL_ERR_NULL
    assert call([prob(), prob(y=None)]) == L.BL_ERR_NULL     # the second problem is checked too
    assert call([prob(x=C16 + 8)]) == L.BL_ERR_ALIGN
    assert call([prob(q=D16 + 4)]) == L.BL_ERR_ALIGN
    assert call([prob(d=D16 + 2)]) == L.BL_ERR_ALIGN
    assert call([prob(ldx=258)]) == L.BL_ERR_ALIGN
    assert call([prob(K=132160, ldx=132160)]) == L.BL_ERR_SHAPE   # fp32-exact bound
    assert call([prob(K=65600, ldx=65600, ytype=0)]) == L.BL_ERR_SHAPE   # K <= 65536
    assert call([prob()], M=2) == L.BL_ERR_NULL             # several tokens need q and d
    assert call([prob(q=D16)], M=2) == L.BL_ERR_NULL
    assert call([], M=1) == L.BL_OK
    assert call([prob()], M=0) == L.BL_OK
    assert call([prob(N=0, packed=None, y=None)]) == L.BL_OK      # nothing to compute
    assert lib.bl_decode_group(None, 1, 1, None) == L.BL_ERR_NULL


def test_decode_group_t3_validation(lib):
    """The base-3 group takes the I2_S group's rules except K % 16 (not 64)."""
    P = L.DecodeProblem

    def prob(**kw):
        base = dict(packed=A16, gamma=B16, N=64, K=336, x=C16, ldx=336, q=None, d=None, y=E16,
                    ytype=2)
        base.update(kw)
        return P(**base)

    def call(probs, M=1):
        arr = (P * max(1, len(probs)))(*probs)
        return lib.bl_decode_group_t3(arr, len(probs), M, None)

    assert call([prob()] * 9) == L.BL_ERR_SHAPE
    assert call([prob()], M=17) == L.BL_ERR_SHAPE
    assert call([prob(K=344, ldx=344)]) == L.BL_ERR_SHAPE   # K % 16
    assert call([prob(ldx=320)]) == L.BL_ERR_SHAPE          # ldx < K
    assert call([prob(K=65552, ldx=65552, ytype=0)]) == L.BL_ERR_SHAPE   # K <= 65536
    assert call([prob(N=1 << 33, K=65536, ldx=65536, ytype=0)]) == L.BL_ERR_SHAPE   # 2^40 bytes
    assert call([prob(ytype=3)]) == L.BL_ERR_DTYPE
    assert call([prob(packed=None)]) == L.BL_ERR_NULL
    assert call([prob(x=None)]) == L.BL_ERR_NULL
    assert call([prob(), prob(gamma=None)]) == L.BL_ERR_NULL
    assert call([prob()], M=3) == L.BL_ERR_NULL             # several tokens need q and d
    assert call([prob(packed=A16 + 4)]) == L.BL_ERR_ALIGN
    assert call([prob(y=E16 + 8)]) == L.BL_ERR_ALIGN
    assert call([prob(ldx=338)]) == L.BL_ERR_ALIGN
    assert call([], M=1) == L.BL_OK
    assert call([prob(N=0, packed=None, y=None)]) == L.BL_OK
    assert lib.bl_decode_group_t3(None, 1, 1, None) == L.BL_ERR_NULL


def test_gemm_group_validation(lib):
    P = L.GemmProblem

    def prob(**kw):
        base = dict(packed=A16, gamma=B16, N=64, y=E16, ytype=2)
        base.update(kw)
        return P(**base)

    def call(probs, K=256, q=C16, d=D16, M=32, qsum=None, ws=None, ws_bytes=0):
        arr = (P * max(1, len(probs)))(*probs)
        return lib.bl_gemm_group(arr, len(probs), K, q, d, qsum, M, ws, ws_bytes, None)

    assert call([prob()] * 9) == L.BL_ERR_SHAPE            # more than 8 problems
    assert call([prob()], K=6) == L.BL_ERR_SHAPE
    assert call([prob()], M=-1) == L.BL_ERR_SHAPE
    assert call([prob(N=-2)]) == L.BL_ERR_SHAPE
    assert call([prob(ytype=3)]) == L.BL_ERR_DTYPE
    assert call([prob(), prob(y=None)]) == L.BL_ERR_NULL    # every problem is checked
    assert call([prob(packed=None)]) == L.BL_ERR_NULL
    assert call([prob(gamma=None)]) == L.BL_ERR_NULL
    assert call([prob()], q=None) == L.BL_ERR_NULL
    assert call([prob()], d=None) == L.BL_ERR_NULL
    assert call([prob(packed=A16 + 4)]) == L.BL_ERR_ALIGN
    assert call([prob(y=E16 + 2)]) == L.BL_ERR_ALIGN
    assert call([prob()], q=C16 + 8) == L.BL_ERR_ALIGN
    assert call([prob()], K=132108) == L.BL_ERR_SHAPE      # fp32-exact bound
    assert call([prob()], qsum=E16 + 0x1001) == L.BL_ERR_ALIGN
    assert call([], M=4) == L.BL_OK
    assert call([prob()], M=0) == L.BL_OK
    assert call([prob(N=0, packed=None, y=None)]) == L.BL_OK
    assert lib.bl_gemm_group(None, 1, 256, C16, D16, None, 4, None, 0, None) == L.BL_ERR_NULL
    # a workspace, when given, must hold the split's partial sums and be aligned
    Ns = (ctypes.c_int64 * 2)(2560, 640)
    need = lib.bl_gemm_group_workspace(Ns, 2, 6912, 64)
    assert need > 0
    two = [prob(N=2560), prob(N=640)]
    assert call(two, K=6912, M=64, ws=A16, ws_bytes=need - 1) == L.BL_ERR_WORKSPACE
    assert call(two, K=6912, M=64, ws=A16 + 8, ws_bytes=need) == L.BL_ERR_ALIGN


def test_gemm_workspace_sizes(lib):
    """bl_gemm_workspace / bl_gemm_group_workspace: the split-K partial sums
    ([splits][M][N] int32) of launches whose tiles leave CUs idle (fewer than
    256 blocks) and whose K is at least 32 steps of 128; 0 where the call runs
    unsplit (enough tiles, short K, the GEMV path at M <= 16, the generic path
    at K % 64 != 0, empty shapes)."""
    ws = lib.bl_gemm_workspace
    for M, N, K in ((64, 2560, 6912), (300, 1000, 8192), (512, 640, 8192), (17, 40, 256 * 16)):
        b = ws(M, N, K)
        assert b > 0 and b % (4 * M * N) == 0, (M, N, K, b)
        assert 2 <= b // (4 * M * N) <= 8
    assert ws(2048, 28672, 8192) == 0          # fills the chip unsplit
    assert ws(2048, 1024, 8192) == 0           # 256 blocks of 64 x 128
    assert ws(512, 2560, 2560) == 0            # 20 K steps: not worth splitting
    assert ws(16, 2560, 2560) == 0             # GEMV path
    assert ws(512, 2560, 2600) == 0            # K % 64 != 0: generic kernel
    assert ws(512, 2560, 256) == 0             # 2 K steps: too short to split
    assert ws(0, 2560, 2560) == 0 and ws(512, 0, 2560) == 0 and ws(512, 2560, 0) == 0
    G = lib.bl_gemm_group_workspace
    N1 = (ctypes.c_int64 * 1)(2560)
    assert G(N1, 1, 6912, 64) == ws(64, 2560, 6912) > 0
    N3 = (ctypes.c_int64 * 3)(2560, 0, 640)     # N == 0 problems add nothing
    N2 = (ctypes.c_int64 * 2)(2560, 640)
    assert G(N3, 3, 6912, 64) == G(N2, 2, 6912, 64) > 0
    assert G(None, 1, 6912, 64) == 0 and G(N1, 9, 6912, 64) == 0
    # bl_gemm: a given workspace must be large enough and aligned (NULL: unsplit)
    need = ws(64, 2560, 6912)
    f = lib.bl_gemm
    args = (A16, B16, 2560, 6912, C16, D16, None, 64, E16, 2)
    assert f(*args, A16, need - 16, None) == L.BL_ERR_WORKSPACE
    assert f(*args, A16 + 4, need, None) == L.BL_ERR_ALIGN


def test_probe_library_exports_and_validation():
    """The benchmark's measurement aids: libblprobe.so exports what
    include/bl_probe.h declares and rejects bad arguments before launching."""
    path = os.path.join(ROOT, "mpgemm_token_absmax_amd", "libblprobe.so")
    if not os.path.exists(path):
        pytest.skip("libblprobe.so not built (run __graft_entry__.build())")
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "bl_probe.h")).read(),
                  flags=re.S)
    declared = sorted(set(re.findall(r"\b(blp_\w+)\s*\(", text)))
    assert declared == ["blp_empty", "blp_stream_read"]
    probe = ctypes.CDLL(path)
    f = probe.blp_stream_read
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert f(A16, 4096, 0, B16, None) == -1            # no blocks
    assert f(A16, 4100, 4, B16, None) == -1            # bytes not a multiple of 16 * blocks
    assert f(A16 + 8, 4096, 4, B16, None) == -1        # misaligned source
    assert f(None, 4096, 4, B16, None) == -1
    assert f(A16, 4096, 4, None, None) == -1
    probe.blp_empty.argtypes = [ctypes.c_int, ctypes.c_void_p]
    assert probe.blp_empty(0, None) == -1


def test_quantize_tensor_validation(lib):
    f = lib.bl_quantize_act_tensor
    ws = lib.bl_quantize_act_tensor_workspace(2)
    assert ws == 16 and lib.bl_quantize_act_tensor_workspace(0) == 0
    assert lib.bl_quantize_act_tensor_workspace(5) == 32
    # (x, M, K, ldx, q, d, qsum, ws, ws_bytes, stream)
    assert f(A16, 2, 6, 6, B16, C16, None, D16, ws, None) == L.BL_ERR_SHAPE       # K % 4
    assert f(A16, 2, 8, 4, B16, C16, None, D16, ws, None) == L.BL_ERR_SHAPE       # ldx < K
    assert f(None, 2, 8, 8, B16, C16, None, D16, ws, None) == L.BL_ERR_NULL
    assert f(A16, 2, 8, 8, B16, None, None, D16, ws, None) == L.BL_ERR_NULL
    assert f(A16, 2, 8, 8, B16, C16, None, None, ws, None) == L.BL_ERR_WORKSPACE
    assert f(A16, 2, 8, 8, B16, C16, None, D16, ws - 1, None) == L.BL_ERR_WORKSPACE
    assert f(A16, 2, 8, 8, B16, C16, None, D16 + 4, ws, None) == L.BL_ERR_ALIGN
    assert f(A16 + 8, 2, 8, 8, B16, C16, None, D16, ws, None) == L.BL_ERR_ALIGN
    assert f(A16, 2, 8, 10, B16, C16, None, D16, ws, None) == L.BL_ERR_ALIGN     # ldx % 4
    assert f(None, 0, 8, 8, None, None, None, None, 0, None) == L.BL_OK            # M == 0
    assert f(A16, 2, 8, 8, B16, C16, E16 + 2, D16, ws, None) == L.BL_ERR_ALIGN    # qsum


def test_rmsnorm_quant_validation(lib):
    f = lib.bl_rmsnorm_quant
    F16 = 0x60000
    # (x, r, g, eps, M, K, ldx, h_out, q, d, qsum)
    ok = (A16, B16, C16, 1e-5, 2, 8, 8, E16, F16, D16, None)

    def call(**kw):
        names = ("x", "r", "g", "eps", "M", "K", "ldx", "h", "q", "d", "qsum")
        a = dict(zip(names, ok))
        a.update(kw)
        return f(*(a[n] for n in names), None)

    assert call(K=6, ldx=6) == L.BL_ERR_SHAPE                 # K % 4
    assert call(ldx=4) == L.BL_ERR_SHAPE                      # ldx < K
    assert call(M=-1) == L.BL_ERR_SHAPE
    assert call(eps=-1e-6) == L.BL_ERR_SHAPE
    assert call(eps=float("nan")) == L.BL_ERR_SHAPE
    assert call(eps=float("inf")) == L.BL_ERR_SHAPE
    assert call(x=None) == L.BL_ERR_NULL
    assert call(g=None) == L.BL_ERR_NULL
    assert call(q=None) == L.BL_ERR_NULL
    assert call(d=None) == L.BL_ERR_NULL
    assert call(x=A16 + 8) == L.BL_ERR_ALIGN
    assert call(r=B16 + 8) == L.BL_ERR_ALIGN
    assert call(g=C16 + 8) == L.BL_ERR_ALIGN
    assert call(h=E16 + 8) == L.BL_ERR_ALIGN
    assert call(q=F16 + 4) == L.BL_ERR_ALIGN
    assert call(d=D16 + 2) == L.BL_ERR_ALIGN
    assert call(ldx=10) == L.BL_ERR_ALIGN                     # ldx % 4
    assert call(qsum=D16 + 2) == L.BL_ERR_ALIGN
    # h_out may be x or r exactly, but must not partly overlap either
    assert call(h=A16 + 16) == L.BL_ERR_ALIAS
    assert call(h=B16 + 16) == L.BL_ERR_ALIAS
    assert call(h=B16 - 16) == L.BL_ERR_ALIAS
    assert call(M=0, x=None, g=None, q=None, d=None) == L.BL_OK
    assert lib.bl_status_string(L.BL_ERR_ALIAS)


def test_t3_validation(lib):
    assert lib.bl_pack_t3_row_bytes(0) == 0
    assert lib.bl_pack_t3_row_bytes(16) == 64 and lib.bl_pack_t3_row_bytes(320) == 64
    assert lib.bl_pack_t3_row_bytes(336) == 128 and lib.bl_pack_t3_row_bytes(2560) == 512
    p = lib.bl_pack_t3
    assert p(A16, L.BL_W_TERNARY_I8, 2, 20, B16, None, None, 0, None) == L.BL_ERR_SHAPE  # K % 16
    assert p(A16, 7, 2, 32, B16, None, None, 0, None) == L.BL_ERR_DTYPE
    assert p(None, L.BL_W_TERNARY_I8, 2, 32, B16, None, None, 0, None) == L.BL_ERR_NULL
    assert p(A16 + 4, L.BL_W_TERNARY_I8, 2, 32, B16, None, None, 0, None) == L.BL_ERR_ALIGN
    assert p(A16, L.BL_W_F32, 2, 32, B16, C16, None, 0, None) == L.BL_ERR_WORKSPACE
    assert p(A16, L.BL_W_F32, 0, 32, B16, C16, D16, 1 << 20, None) == L.BL_ERR_SHAPE
    assert p(A16, L.BL_W_F32, 2, 32, B16, None, D16, 1 << 20, None) == L.BL_ERR_NULL
    assert p(None, L.BL_W_TERNARY_I8, 0, 32, None, None, None, 0, None) == L.BL_OK
    g = lib.bl_gemv_t3
    # (packed, gamma, N, K, q, d, M, y, ytype)
    assert g(A16, B16, 8, 20, C16, D16, 1, E16, L.BL_OUT_BF16, None) == L.BL_ERR_SHAPE   # K % 16
    assert g(A16, B16, 8, 32, C16, D16, 17, E16, L.BL_OUT_BF16, None) == L.BL_ERR_SHAPE  # M > 16
    assert g(A16, B16, 8, 32, C16, D16, 1, None, L.BL_OUT_BF16, None) == L.BL_ERR_NULL
    assert g(None, B16, 8, 32, C16, D16, 1, E16, L.BL_OUT_BF16, None) == L.BL_ERR_NULL
    assert g(A16, None, 8, 32, C16, D16, 1, E16, L.BL_OUT_F32, None) == L.BL_ERR_NULL
    assert g(A16, B16, 8, 32, C16, D16, 1, E16, 9, None) == L.BL_ERR_DTYPE
    assert g(A16 + 8, B16, 8, 32, C16, D16, 1, E16, L.BL_OUT_BF16, None) == L.BL_ERR_ALIGN
    assert g(A16, B16, 8, 1 << 18, C16, D16, 1, E16, L.BL_OUT_F32, None) == L.BL_ERR_SHAPE
    assert g(None, None, 8, 32, None, None, 0, None, L.BL_OUT_BF16, None) == L.BL_OK     # M == 0


def test_decode_norm_group_validation(lib):
    f = lib.bl_decode_norm_group
    P = L.DecodeProblem

    def probs(*specs):
        arr = (P * len(specs))()
        for i, (N, K, x) in enumerate(specs):
            arr[i] = P(A16 + 0x1000 * i, B16, N, K, x, K, None, None, 0x80000 + 0x1000 * i,
                       L.BL_OUT_BF16)
        return arr

    X, G, R, H = 0x90000, 0xA0000, 0xB0000, 0xC0000
    ok = probs((64, 256, X), (32, 256, X))
    assert f(ok, 9, R, G, 1e-5, H, None) == L.BL_ERR_SHAPE
    assert f(ok, 2, R, G, -1.0, H, None) == L.BL_ERR_SHAPE
    assert f(ok, 2, R, None, 1e-5, H, None) == L.BL_ERR_NULL
    assert f(probs((64, 256, X), (32, 512, X)), 2, R, G, 1e-5, H, None) == L.BL_ERR_SHAPE  # K differs
    assert f(probs((64, 256, X), (32, 256, X + 0x400)), 2, R, G, 1e-5, H, None) == L.BL_ERR_SHAPE
    assert f(probs((64, 96, X)), 1, R, G, 1e-5, H, None) == L.BL_ERR_SHAPE      # K % 64
    assert f(probs((64, 32832, X)), 1, R, G, 1e-5, H, None) == L.BL_ERR_SHAPE   # K > 32768
    assert f(probs((64, 256, X)), 1, R + 8, G, 1e-5, H, None) == L.BL_ERR_ALIGN
    assert f(probs((64, 256, X)), 1, R, G, 1e-5, X + 16, None) == L.BL_ERR_ALIAS
    assert f(probs((64, 256, X)), 1, R, G, 1e-5, R, None) == L.BL_ERR_ALIAS   # no in-place here
    assert f(None, 0, None, None, 0.0, None, None) == L.BL_OK
