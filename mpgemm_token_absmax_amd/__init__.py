"""Ternary BitLinear mpGEMM on AMD Instinct MI355X (gfx950).

Python binding of libbitlinear.so (C ABI: include/bitlinear.h). The functions
here take and return torch tensors on the GPU, pass their device pointers and
torch's current stream to the library, and do nothing else: every step of the
computation runs in the library's HIP kernels. PyTorch provides device memory
and streams only.

    q, d        = quantize_act(x_bf16)              # per-token absmax int8
    q, d        = quantize_act_tensor(x_bf16)       # one absmax scale for all tokens
    h, q, d     = rmsnorm_quant(x, g, eps, residual=r)  # fused add + RMSNorm + quantize
    packed, g   = pack_i2s(w_fp32)                  # absmean ternary -> 2-bit I2_S
    packed      = pack_i2s(w_ternary_int8)          # pack only (caller keeps gamma)
    y           = gemv(packed, g, q, d)             # M <= 16 tokens
    y           = gemm(packed, g, q, d)             # any M (int8 MFMA)
    p3, g       = pack_t3(w_fp32)                   # base-3, 5 weights per byte (1.6 bpw)
    y           = gemv_t3(p3, g, q, d)              # M <= 16 over the base-3 packing
    ys          = gemm_group([dict(packed=.., gamma=..), ...], q, d)
                                                    # GEMMs sharing one q, fewest launches
    ys          = decode_group([dict(packed=.., gamma=.., x=..), ...])
                                                    # fused quantize + GEMV, one launch
    ys          = NormDecodeGroup([dict(packed=.., gamma=..), ...], x, g, eps, residual=r)()
                                                    # + residual add and RMSNorm, one launch
"""
from __future__ import annotations

import ctypes

import torch

from ._lib import (BL_OUT_BF16, BL_OUT_F32, BL_OUT_I32, BL_W_F32, BL_W_TERNARY_I8, MAX_GROUP,
                   BitLinearError, DecodeProblem, GemmProblem, check, lib, status_string)

__all__ = ["quantize_act", "quantize_act_tensor", "rmsnorm_quant", "pack_i2s", "pack_i2s_workspace",
           "pack_t3", "gemv_t3", "gemv", "gemm",
           "gemm_workspace", "gemm_group", "GemmGroup", "decode_group", "DecodeGroup",
           "decode_group_t3", "DecodeGroupT3",
           "NormDecodeGroup",
           "BitLinearError", "status_string",
           "lib", "OUT_TYPES"]

OUT_TYPES = {"i32": (BL_OUT_I32, torch.int32), "f32": (BL_OUT_F32, torch.float32),
             "bf16": (BL_OUT_BF16, torch.bfloat16)}


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype, ndim: int):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D")


def _sums(qsum, with_sums, M, device):
    """The token-sum output buffer: the given one, a new int32 [M], or None."""
    if qsum is not None:
        _need(qsum, "qsum", torch.int32, 1)
        if qsum.shape[0] != M or not qsum.is_contiguous():
            raise ValueError("qsum must be a contiguous int32 [M]")
        return qsum
    return torch.empty((M,), dtype=torch.int32, device=device) if with_sums else None


def quantize_act(x: torch.Tensor, q: torch.Tensor | None = None, d: torch.Tensor | None = None,
                 qsum: torch.Tensor | None = None, with_sums: bool = False):
    """x: bf16 [M][K] (row stride x.stride(0)) -> (q int8 [M][K], d fp32 [M]),
    plus qsum int32 [M] (the token sums of q, for gemm / gemm_group) when
    with_sums is set or a qsum buffer is given."""
    _need(x, "x", torch.bfloat16, 2)
    if x.stride(1) != 1:
        raise ValueError("x rows must be contiguous")
    M, K = x.shape
    if q is None:
        q = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if d is None:
        d = torch.empty((M,), dtype=torch.float32, device=x.device)
    qs = _sums(qsum, with_sums, M, x.device)
    check("bl_quantize_act", lib().bl_quantize_act(_ptr(x), M, K, x.stride(0), _ptr(q), _ptr(d),
                                                   _ptr(qs), _stream(x.device)))
    return (q, d) if qs is None else (q, d, qs)


def quantize_act_tensor(x: torch.Tensor, q: torch.Tensor | None = None,
                        d: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                        qsum: torch.Tensor | None = None, with_sums: bool = False):
    """x: bf16 [M][K] -> (q int8 [M][K], d fp32 [M]) with ONE scale for the
    whole tensor (every d[t] equal); qsum as in quantize_act."""
    _need(x, "x", torch.bfloat16, 2)
    if x.stride(1) != 1:
        raise ValueError("x rows must be contiguous")
    M, K = x.shape
    if q is None:
        q = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if d is None:
        d = torch.empty((M,), dtype=torch.float32, device=x.device)
    nws = int(lib().bl_quantize_act_tensor_workspace(M))
    if workspace is None:
        workspace = torch.empty((max(nws, 16),), dtype=torch.uint8, device=x.device)
    qs = _sums(qsum, with_sums, M, x.device)
    check("bl_quantize_act_tensor",
          lib().bl_quantize_act_tensor(_ptr(x), M, K, x.stride(0), _ptr(q), _ptr(d), _ptr(qs),
                                       _ptr(workspace), workspace.numel(), _stream(x.device)))
    return (q, d) if qs is None else (q, d, qs)


def rmsnorm_quant(x: torch.Tensor, g: torch.Tensor, eps: float, residual: torch.Tensor | None = None,
                  h_out: torch.Tensor | None = None, q: torch.Tensor | None = None,
                  d: torch.Tensor | None = None, write_h: bool = True,
                  qsum: torch.Tensor | None = None, with_sums: bool = False):
    """Residual add + RMSNorm + per-token absmax int8 in one kernel.

    x, residual: bf16 [M][K] with the same row stride; g: bf16 [K]. Returns
    (h, q, d): h = bf16(x + residual) (x itself without a residual; None when
    write_h is False and no h_out is given), q int8 [M][K], d fp32 [M]; and
    qsum int32 [M] as a fourth item when with_sums is set or qsum is given.
    h_out may be residual itself (in-place update of the residual stream).
    """
    _need(x, "x", torch.bfloat16, 2)
    _need(g, "g", torch.bfloat16, 1)
    if x.stride(1) != 1 or g.stride(0) != 1:
        raise ValueError("x rows and g must be contiguous")
    M, K = x.shape
    if g.shape[0] != K:
        raise ValueError("g must have K entries")
    for t, name in ((residual, "residual"), (h_out, "h_out")):
        if t is not None:
            _need(t, name, torch.bfloat16, 2)
            if tuple(t.shape) != (M, K) or t.stride() != x.stride():
                raise ValueError(f"{name} must match x's shape and strides")
    if h_out is None and write_h and residual is not None:     # x's row stride
        h_out = torch.empty_strided((M, K), x.stride(), dtype=torch.bfloat16, device=x.device)
    if q is None:
        q = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if d is None:
        d = torch.empty((M,), dtype=torch.float32, device=x.device)
    qs = _sums(qsum, with_sums, M, x.device)
    check("bl_rmsnorm_quant",
          lib().bl_rmsnorm_quant(_ptr(x), _ptr(residual), _ptr(g), float(eps), M, K, x.stride(0),
                                 _ptr(h_out), _ptr(q), _ptr(d), _ptr(qs), _stream(x.device)))
    h = h_out if h_out is not None else (x if residual is None and write_h else None)
    return (h, q, d) if qs is None else (h, q, d, qs)


def pack_i2s_workspace(N: int, K: int) -> int:
    return int(lib().bl_pack_i2s_workspace(N, K))


def pack_i2s(w: torch.Tensor, packed: torch.Tensor | None = None,
             gamma: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """fp32 [N][K] -> (packed uint8 [N][K/4], gamma fp32 [1]) (absmean ternarize + pack);
    int8 ternary [N][K] -> packed uint8 [N][K/4] (pack only)."""
    if not isinstance(w, torch.Tensor) or not w.is_cuda or w.dim() != 2:
        raise TypeError("w must be a 2-D CUDA tensor")
    if not w.is_contiguous():
        raise ValueError("w must be contiguous")
    N, K = w.shape
    if K % 4:
        raise ValueError("K must be a multiple of 4")
    if packed is None:
        packed = torch.empty((N, K // 4), dtype=torch.uint8, device=w.device)
    s = _stream(w.device)
    if w.dtype == torch.float32:
        if gamma is None:
            gamma = torch.empty((1,), dtype=torch.float32, device=w.device)
        nws = pack_i2s_workspace(N, K)
        if workspace is None:
            workspace = torch.empty((max(nws, 16),), dtype=torch.uint8, device=w.device)
        check("bl_pack_i2s", lib().bl_pack_i2s(_ptr(w), BL_W_F32, N, K, _ptr(packed),
                                               _ptr(gamma), _ptr(workspace),
                                               workspace.numel(), s))
        return packed, gamma
    if w.dtype == torch.int8:
        check("bl_pack_i2s", lib().bl_pack_i2s(_ptr(w), BL_W_TERNARY_I8, N, K, _ptr(packed),
                                               None, None, 0, s))
        return packed
    raise TypeError("w must be float32 or int8")


def pack_t3(w: torch.Tensor, packed: torch.Tensor | None = None,
            gamma: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """As pack_i2s, into the base-3 format (five weights per byte): packed is
    uint8 [N][64*ceil(K/320)]. K % 16 == 0."""
    if not isinstance(w, torch.Tensor) or not w.is_cuda or w.dim() != 2:
        raise TypeError("w must be a 2-D CUDA tensor")
    if not w.is_contiguous():
        raise ValueError("w must be contiguous")
    N, K = w.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    if packed is None:
        packed = torch.empty((N, int(lib().bl_pack_t3_row_bytes(K))), dtype=torch.uint8,
                             device=w.device)
    s = _stream(w.device)
    if w.dtype == torch.float32:
        if gamma is None:
            gamma = torch.empty((1,), dtype=torch.float32, device=w.device)
        nws = pack_i2s_workspace(N, K)
        if workspace is None:
            workspace = torch.empty((max(nws, 16),), dtype=torch.uint8, device=w.device)
        check("bl_pack_t3", lib().bl_pack_t3(_ptr(w), BL_W_F32, N, K, _ptr(packed), _ptr(gamma),
                                             _ptr(workspace), workspace.numel(), s))
        return packed, gamma
    if w.dtype == torch.int8:
        check("bl_pack_t3", lib().bl_pack_t3(_ptr(w), BL_W_TERNARY_I8, N, K, _ptr(packed),
                                             None, None, 0, s))
        return packed
    raise TypeError("w must be float32 or int8")


def gemv_t3(packed: torch.Tensor, gamma: torch.Tensor, q: torch.Tensor, d: torch.Tensor,
            out_dtype: str = "bf16", out: torch.Tensor | None = None) -> torch.Tensor:
    """y[M][N] for M <= 16 tokens over base-3 packed weights."""
    _need(packed, "packed", torch.uint8, 2)
    _need(q, "q", torch.int8, 2)
    N, RB = packed.shape
    M, K = q.shape
    if RB != int(lib().bl_pack_t3_row_bytes(K)):
        raise ValueError(f"packed [{N}][{RB}] does not match q [{M}][{K}]")
    ytype, tdt = OUT_TYPES[out_dtype]
    if ytype != BL_OUT_I32:
        _need(gamma, "gamma", torch.float32, 1)
        _need(d, "d", torch.float32, 1)
    if out is None:
        out = torch.empty((M, N), dtype=tdt, device=q.device)
    elif out.dtype != tdt or tuple(out.shape) != (M, N) or not out.is_contiguous():
        raise ValueError("out has the wrong dtype, shape or layout")
    check("bl_gemv_t3", lib().bl_gemv_t3(_ptr(packed), _ptr(gamma), N, K, _ptr(q), _ptr(d), M,
                                         _ptr(out), ytype, _stream(q.device)))
    return out


def _matmul_args(packed, gamma, q, d, out, out_dtype):
    _need(packed, "packed", torch.uint8, 2)
    _need(q, "q", torch.int8, 2)
    N, KB = packed.shape
    M, K = q.shape
    if KB * 4 != K:
        raise ValueError(f"packed [{N}][{KB}] does not match q [{M}][{K}]")
    ytype, tdt = OUT_TYPES[out_dtype]
    if ytype != BL_OUT_I32:
        _need(gamma, "gamma", torch.float32, 1)
        _need(d, "d", torch.float32, 1)
    if out is None:
        out = torch.empty((M, N), dtype=tdt, device=q.device)
    elif out.dtype != tdt or tuple(out.shape) != (M, N) or not out.is_contiguous():
        raise ValueError("out has the wrong dtype, shape or layout")
    return N, K, M, ytype, out


def gemv(packed: torch.Tensor, gamma: torch.Tensor, q: torch.Tensor, d: torch.Tensor,
         out_dtype: str = "bf16", out: torch.Tensor | None = None) -> torch.Tensor:
    """y[M][N] for M <= 16 tokens (decode path)."""
    N, K, M, ytype, out = _matmul_args(packed, gamma, q, d, out, out_dtype)
    check("bl_gemv", lib().bl_gemv(_ptr(packed), _ptr(gamma), N, K, _ptr(q), _ptr(d), M,
                                   _ptr(out), ytype, _stream(q.device)))
    return out


def gemm_workspace(M: int, N: int, K: int) -> int:
    return int(lib().bl_gemm_workspace(M, N, K))


def _qsum_in(qsum, M):
    if qsum is not None:
        _need(qsum, "qsum", torch.int32, 1)
        if qsum.shape[0] != M or not qsum.is_contiguous():
            raise ValueError("qsum must be a contiguous int32 [M]")
    return qsum


def gemm(packed: torch.Tensor, gamma: torch.Tensor, q: torch.Tensor, d: torch.Tensor,
         out_dtype: str = "bf16", out: torch.Tensor | None = None,
         workspace: torch.Tensor | None = None, qsum: torch.Tensor | None = None,
         split: bool = True) -> torch.Tensor:
    """y[M][N] for any M (prefill path, int8 MFMA). qsum: the token sums of q
    (from quantize_act(..., with_sums=True)); with them the kernel runs on
    offset weights, same results. split: give the call a workspace (the one
    passed, or a new one) so that small launches split K; same results."""
    N, K, M, ytype, out = _matmul_args(packed, gamma, q, d, out, out_dtype)
    qsum = _qsum_in(qsum, M)
    nws = gemm_workspace(M, N, K)
    if not split:
        workspace = None
    elif nws and workspace is None:
        workspace = torch.empty((nws,), dtype=torch.uint8, device=q.device)
    check("bl_gemm", lib().bl_gemm(_ptr(packed), _ptr(gamma), N, K, _ptr(q), _ptr(d), _ptr(qsum), M,
                                   _ptr(out), ytype, _ptr(workspace),
                                   0 if workspace is None else workspace.numel(),
                                   _stream(q.device)))
    return out


class GemmGroup:
    """A prepared bl_gemm_group call over one quantized input (q int8 [M][K],
    d fp32 [M]): the descriptor array is built once, so repeated calls (or a
    graph capture) only pass pointers.

    problems: list of dicts with keys packed (uint8 [N][K/4]), gamma (fp32 [1])
    and optional y (output [M][N]) and out_dtype. split: give the calls the
    workspace with which small launches split K (the outputs are the same
    without it): `workspace` when given (uint8, large enough; groups whose
    calls run one after another on one stream may share one), else a new one."""

    def __init__(self, problems, q: torch.Tensor, d: torch.Tensor, out_dtype: str = "bf16",
                 qsum: torch.Tensor | None = None, split: bool = True,
                 workspace: torch.Tensor | None = None):
        if not 1 <= len(problems) <= MAX_GROUP:
            raise ValueError(f"1..{MAX_GROUP} problems per group")
        _need(q, "q", torch.int8, 2)
        _need(d, "d", torch.float32, 1)
        M, K = q.shape
        self.qsum = _qsum_in(qsum, M)
        arr = (GemmProblem * len(problems))()
        self.problems = []
        for i, p in enumerate(problems):
            packed = p["packed"]
            _need(packed, "packed", torch.uint8, 2)
            N, KB = packed.shape
            if KB * 4 != K:
                raise ValueError(f"packed [{N}][{KB}] does not match q [{M}][{K}]")
            ytype, tdt = OUT_TYPES[p.get("out_dtype", out_dtype)]
            gamma = p.get("gamma")
            if ytype != BL_OUT_I32:
                _need(gamma, "gamma", torch.float32, 1)
            y = p.get("y")
            if y is None:
                y = torch.empty((M, N), dtype=tdt, device=q.device)
            elif y.dtype != tdt or tuple(y.shape) != (M, N) or not y.is_contiguous():
                raise ValueError("y has the wrong dtype, shape or layout")
            arr[i] = GemmProblem(packed.data_ptr(), _ptr(gamma), N, y.data_ptr(), ytype)
            self.problems.append(dict(p, y=y))
        self.q, self.d, self.M, self.K = q, d, M, K
        self._arr = arr
        Ns = (ctypes.c_int64 * len(problems))(*[p["packed"].shape[0] for p in self.problems])
        nws = int(lib().bl_gemm_group_workspace(Ns, len(problems), K, M)) if split else 0
        if nws and workspace is not None:
            _need(workspace, "workspace", torch.uint8, 1)
            if workspace.numel() < nws:
                raise ValueError(f"workspace holds {workspace.numel()} bytes, {nws} needed")
        elif nws:
            workspace = torch.empty((nws,), dtype=torch.uint8, device=q.device)
        self.workspace = workspace if nws else None

    @property
    def outputs(self):
        return [p["y"] for p in self.problems]

    def __call__(self):
        ws = self.workspace
        check("bl_gemm_group", lib().bl_gemm_group(self._arr, len(self.problems), self.K,
                                                   self.q.data_ptr(), self.d.data_ptr(),
                                                   _ptr(self.qsum), self.M, _ptr(ws),
                                                   0 if ws is None else ws.numel(),
                                                   _stream(self.q.device)))
        return self.outputs


def gemm_group(problems, q: torch.Tensor, d: torch.Tensor, out_dtype: str = "bf16",
               qsum: torch.Tensor | None = None, split: bool = True):
    """GEMMs of several projections over the same quantized input q, d
    (qsum: optional token sums of q, as in gemm; split: as in GemmGroup).
    Returns the list of outputs y."""
    return GemmGroup(problems, q, d, out_dtype, qsum, split)()


class DecodeGroup:
    """A prepared bl_decode_group call: the descriptor array is built once, so
    repeated calls (or a graph capture) only pass pointers.

    problems: list of dicts with keys packed (uint8 [N][K/4]), gamma (fp32 [1]),
    x (bf16 [M][K]), and optional y (output), q (int8 [M][K]) and d (fp32 [M])
    buffers; out_dtype applies to every y that is allocated here."""

    _fn = "bl_decode_group"

    def _row_bytes(self, K: int) -> int:
        return K // 4

    def __init__(self, problems, out_dtype: str = "bf16"):
        if not 1 <= len(problems) <= MAX_GROUP:
            raise ValueError(f"1..{MAX_GROUP} problems per group")
        self.problems = []
        arr = (DecodeProblem * len(problems))()
        M = None
        for i, p in enumerate(problems):
            packed, x = p["packed"], p["x"]
            _need(packed, "packed", torch.uint8, 2)
            _need(x, "x", torch.bfloat16, 2)
            if x.stride(1) != 1:
                raise ValueError("x rows must be contiguous")
            N, KB = packed.shape
            Mi, K = x.shape
            if KB != self._row_bytes(K):
                raise ValueError("packed does not match x")
            M = Mi if M is None else M
            if Mi != M:
                raise ValueError("all problems of a group share M")
            ytype, tdt = OUT_TYPES[p.get("out_dtype", out_dtype)]
            y = p.get("y")
            if y is None:
                y = torch.empty((M, N), dtype=tdt, device=x.device)
            elif y.dtype != tdt or tuple(y.shape) != (M, N) or not y.is_contiguous():
                raise ValueError("y has the wrong dtype, shape or layout")
            q, d, gamma = p.get("q"), p.get("d"), p.get("gamma")
            if M > 1 and (q is None or d is None):     # several tokens stage their codes
                q = torch.empty((M, K), dtype=torch.int8, device=x.device) if q is None else q
                d = torch.empty((M,), dtype=torch.float32, device=x.device) if d is None else d
            arr[i] = DecodeProblem(packed.data_ptr(), _ptr(gamma), N, K, x.data_ptr(),
                                   x.stride(0), _ptr(q), _ptr(d), y.data_ptr(), ytype)
            self.problems.append(dict(p, y=y, q=q, d=d))
        self.M = M
        self._arr = arr
        self._device = problems[0]["x"].device

    @property
    def outputs(self):
        return [p["y"] for p in self.problems]

    def __call__(self):
        check(self._fn, getattr(lib(), self._fn)(self._arr, len(self.problems), self.M,
                                                 _stream(self._device)))
        return self.outputs


class DecodeGroupT3(DecodeGroup):
    """A prepared bl_decode_group_t3 call: DecodeGroup over base-3 packed
    weights (packed: uint8 [N][64*ceil(K/320)] from pack_t3; K % 16 == 0)."""

    _fn = "bl_decode_group_t3"

    def _row_bytes(self, K: int) -> int:
        return 64 * ((K + 319) // 320) if K > 0 else 0


class NormDecodeGroup(DecodeGroup):
    """A prepared bl_decode_norm_group call: one token's residual add, RMSNorm
    and quantize, then every problem's GEMV, in one launch.

    x: bf16 [1][K], the input every problem reads; g: bf16 [K] norm weight;
    residual: bf16 [1][K] or None; h_out: bf16 [1][K] or None (receives
    bf16(x + residual); must not overlap x or residual). problems: dicts with
    packed, gamma and optional y, q, d, out_dtype."""

    def __init__(self, problems, x, g, eps: float, residual=None, h_out=None,
                 out_dtype: str = "bf16"):
        _need(x, "x", torch.bfloat16, 2)
        if x.shape[0] != 1 or not x.is_contiguous():
            raise ValueError("x must be one contiguous token [1][K]")
        super().__init__([dict(p, x=x) for p in problems], out_dtype)
        K = x.shape[1]
        _need(g, "g", torch.bfloat16, 1)
        if g.shape[0] != K or not g.is_contiguous():
            raise ValueError("g must be contiguous [K]")
        for t, name in ((residual, "residual"), (h_out, "h_out")):
            if t is not None:
                _need(t, name, torch.bfloat16, 2)
                if tuple(t.shape) != (1, K) or not t.is_contiguous():
                    raise ValueError(f"{name} must be contiguous [1][K]")
        self.x, self.g, self.eps, self.residual, self.h_out = x, g, float(eps), residual, h_out

    def __call__(self):
        check("bl_decode_norm_group",
              lib().bl_decode_norm_group(self._arr, len(self.problems), _ptr(self.residual),
                                         _ptr(self.g), self.eps, _ptr(self.h_out),
                                         _stream(self._device)))
        return self.outputs


def decode_group(problems, out_dtype: str = "bf16"):
    """One fused launch: quantize each problem's bf16 x per token, GEMV, dequant.
    Returns the list of outputs y."""
    return DecodeGroup(problems, out_dtype)()


def decode_group_t3(problems, out_dtype: str = "bf16"):
    """decode_group over base-3 packed weights (pack_t3). Returns the outputs y."""
    return DecodeGroupT3(problems, out_dtype)()
