"""bl_gemm_group_noalloc through the C ABI: the grouped GEMM whose split-K
partial sums go to the library's own device array. Its outputs must equal
bl_gemm_group's with a workspace of its own, byte for byte, on two calls in
a row (the second smaller, over what the first left in the array), and the
oracle's."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from mpgemm_token_absmax_amd import _lib as L

pytestmark = pytest.mark.gpu

GAMMA = np.float32(W.GAMMA_DRAWN)
OUT = {"bf16": (L.BL_OUT_BF16, torch.bfloat16), "f32": (L.BL_OUT_F32, torch.float32),
       "i32": (L.BL_OUT_I32, torch.int32)}


def _case(M, K, Ns, seed):
    import mpgemm_token_absmax_amd as bl
    q = W.int8_codes(seed, M, K)
    d = W.positive_scales(seed + 1, M)
    ts = [W.ternary_drawn(seed + 2 + i, n, K, 0.35) for i, n in enumerate(Ns)]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    probs = [dict(packed=bl.pack_i2s(dev(t)), gamma=dev(np.array([GAMMA], np.float32)),
                  out_dtype=("bf16", "i32", "f32")[i % 3]) for i, t in enumerate(ts)]
    qs = dev(oracle.token_sums(q).astype(np.int32))
    return q, d, ts, dev(q), dev(d), qs, probs


def _noalloc(lib, probs, qd, dd, qs, M, K):
    arr = (L.GemmProblem * len(probs))()
    ys = []
    for i, p in enumerate(probs):
        ytype, tdt = OUT[p["out_dtype"]]
        N = p["packed"].shape[0]
        y = torch.full((M, N), 7, dtype=tdt, device="cuda")
        arr[i] = L.GemmProblem(p["packed"].data_ptr(), p["gamma"].data_ptr(), N, y.data_ptr(), ytype)
        ys.append(y)
    st = lib.bl_gemm_group_noalloc(arr, len(probs), K, qd.data_ptr(), dd.data_ptr(), qs.data_ptr(),
                                   M, torch.cuda.current_stream().cuda_stream)
    assert st == L.BL_OK, L.status_string(st)
    return ys


def test_gemm_group_noalloc_matches_workspace_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mpgemm_token_absmax_amd as bl
    lib = bl.lib()
    # the first group splits K into the array (15.7 MB of partial sums), the
    # second, smaller one (K % 128 == 64) splits over what the first left there
    for M, K, Ns, seed in ((128, 6912, (2560, 640, 640), 500), (100, 4160, (300, 1000), 600)):
        q, d, ts, qd, dd, qs, probs = _case(M, K, Ns, seed)
        need = lib.bl_gemm_group_workspace((ctypes_int64 := __import__("ctypes").c_int64 * len(Ns))(*Ns),
                                           len(Ns), K, M)
        assert 0 < need <= L.BL_GEMM_NOALLOC_SCRATCH_BYTES
        ys = _noalloc(lib, probs, qd, dd, qs, M, K)
        ref = bl.GemmGroup(probs, qd, dd, qsum=qs)()
        torch.cuda.synchronize()
        for p, y, r, t in zip(probs, ys, ref, ts):
            a = y.view(torch.uint8).cpu().numpy()
            b = r.view(torch.uint8).cpu().numpy()
            assert np.array_equal(a, b), (M, K, p["out_dtype"])
            if p["out_dtype"] == "i32":
                assert np.array_equal(y.cpu().numpy().astype(np.int64), oracle.mpgemm_acc(q, t))
