"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bar: bit-exact packed bytes, gamma, quantized activations, int32 accumulators
and fp32 outputs (the fp32 epilogue fl32(fl32(acc) * fl32(gamma*d)) is a
defined single-rounding formula); fp32 also within 1e-6 relative of the fp64
y_ref = acc*gamma*d; bf16 bit-exact to the round-to-nearest-even of that fp32
value and within 1 bf16 ulp of y_ref rounded directly from fp64.

Inputs come from the seeded generators in workloads.py, never from the GPU.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

GAMMA = np.float32(W.GAMMA_DRAWN)


def _bl():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mpgemm_token_absmax_amd as bl
    bl.lib()                   # fails loudly if the library is missing
    return bl


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return dev(bits.view(np.int16)).view(torch.bfloat16)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def check_outputs(acc_ref, gamma, d, y_i32=None, y_f32=None, y_bf16=None, rows=None, cols=None):
    """Compare GPU outputs (the full [M][N] arrays, or the entries (rows, cols))
    with the oracle's accumulators acc_ref ([M][N], or [S] at the entries)."""
    if rows is None:
        A, D = np.asarray(acc_ref), np.asarray(d)
        sel = (lambda a: a)
    else:
        A, D = np.asarray(acc_ref)[:, None], np.asarray(d)[rows]
        sel = (lambda a: a[rows, cols][:, None])
    if y_i32 is not None:
        assert np.array_equal(sel(y_i32).astype(np.int64), A), "int32 accumulators differ"
    y32_ref = oracle.dequant_f32(A, gamma, D)
    y64_ref = oracle.dequant_f64(A, gamma, D)
    if y_f32 is not None:
        got = sel(y_f32)
        assert np.array_equal(got.view(np.uint32), y32_ref.view(np.uint32)), "fp32 outputs differ"
        assert np.array_equal(y64_ref == 0, got == 0)
        nz = y64_ref != 0
        rel = np.abs(got.astype(np.float64)[nz] - y64_ref[nz]) / np.abs(y64_ref[nz])
        assert rel.size == 0 or rel.max() <= 1e-6, rel.max()
    if y_bf16 is not None:
        got = sel(y_bf16)
        exp = oracle.round_f64_to_bf16_bits(y32_ref.astype(np.float64))
        assert np.array_equal(got, exp), "bf16 outputs differ from RNE(fp32)"
        direct = oracle.round_f64_to_bf16_bits(y64_ref)
        g_i = got.astype(np.int32)
        r_i = direct.astype(np.int32)
        same_sign = (g_i & 0x8000) == (r_i & 0x8000)
        within = np.abs((g_i & 0x7FFF) - (r_i & 0x7FFF)) <= 1
        assert np.all((g_i == r_i) | (same_sign & within)), "bf16 more than 1 ulp from y_ref"


def run_all_outputs(bl, fn, packed_d, gamma_d, q_d, d_d):
    outs = {}
    for name in ("i32", "f32", "bf16"):
        outs[name] = host(fn(packed_d, gamma_d, q_d, d_d, out_dtype=name))
    return outs


# ---------------------------------------------------------------------------
# quantize_act
# ---------------------------------------------------------------------------

QUANT_SHAPES = [(1, 4), (1, 64), (3, 260), (16, 1024), (17, 2560), (5, 6912), (4, 11008),
                (2, 28672), (3, 36000), (64, 4096), (1, 8), (1, 32768), (2, 32776), (6, 520)]


@pytest.mark.parametrize("M,K", QUANT_SHAPES, ids=[f"M{m}K{k}" for m, k in QUANT_SHAPES])
def test_quantize_parity(M, K):
    bl = _bl()
    say(f"quantize M={M} K={K}")
    x = W.activations_bf16(100 + M * 7 + K, M, K, outlier_frac=0.01, outlier_scale=20.0)
    q_ref, d_ref = oracle.quantize_act_absmax(x)
    q, d = bl.quantize_act(dev_bf16(x))
    q2, d2, qs = bl.quantize_act(dev_bf16(x), with_sums=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(q), q_ref)
    assert np.array_equal(host(d).view(np.uint32), d_ref.view(np.uint32))
    # the token sums ride along without changing q or d
    assert torch.equal(q2, q) and torch.equal(d2, d)
    assert np.array_equal(host(qs), oracle.token_sums(q_ref))


def test_quantize_special_rows_and_stride():
    bl = _bl()
    say("quantize special rows + ldx > K")
    import pins
    rows = []
    for name in ("e1_quant_basic.json", "e2_quant_ties.json"):
        g = pins.golden(name)
        r = np.zeros(8, dtype=np.float32)
        r[:len(g["x"][0])] = g["x"][0]
        rows.append(r)
    rows += [np.zeros(8, np.float32), np.full(8, -3.0, np.float32),
             np.array([0, 0, 0, 0, 0, 9, 0, 0], np.float32), np.full(8, 2.0**-100, np.float32),
             np.array([1e30, -1e30, 1, -1, 0, 2, 3, 4], np.float32)]
    x = W.f32_to_bf16_bits(np.stack(rows))
    # embed in a wider buffer: row stride 24 elements
    wide = np.zeros((x.shape[0], 24), dtype=np.uint16)
    wide[:, 8:16] = x
    q_ref, d_ref = oracle.quantize_act_absmax(x)
    xd = dev_bf16(wide)[:, 8:16]            # base 16-byte aligned, rows 8-byte aligned
    assert xd.stride(0) == 24
    q, d = bl.quantize_act(xd)
    torch.cuda.synchronize()
    assert np.array_equal(host(q), q_ref)
    assert np.array_equal(host(d).view(np.uint32), d_ref.view(np.uint32))
    # row stride 12 (not a multiple of 8 elements): the 8-byte load path
    wide12 = np.zeros((x.shape[0], 12), dtype=np.uint16)
    wide12[:, :8] = x
    x12 = dev_bf16(wide12)[:, :8]
    q12, d12, s12 = bl.quantize_act(x12, with_sums=True)
    _, _, s24 = bl.quantize_act(xd, with_sums=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(q12), q_ref)
    assert np.array_equal(host(d12).view(np.uint32), d_ref.view(np.uint32))
    assert np.array_equal(host(s12), oracle.token_sums(q_ref))
    assert np.array_equal(host(s24), oracle.token_sums(q_ref))
    # the golden q values themselves
    assert host(q)[0, :4].tolist() == [-127, 32, 16, 95]
    assert host(q)[1, :6].tolist() == [127, 62, -62, 0, 2, -2]


QUANT_TENSOR_SHAPES = [(1, 64), (3, 260), (17, 2560), (5, 6912), (2, 28672), (3, 36000),
                       (64, 4096), (2048, 8192), (300, 8), (1, 4)]


@pytest.mark.parametrize("M,K", QUANT_TENSOR_SHAPES, ids=[f"M{m}K{k}" for m, k in QUANT_TENSOR_SHAPES])
def test_quantize_tensor_parity(M, K):
    """One scale over all tokens: bit-exact q and d against the oracle (both
    the 16-byte path and the any-K path)."""
    bl = _bl()
    say(f"quantize per tensor M={M} K={K}")
    x = W.activations_bf16(700 + M * 7 + K, M, K, outlier_frac=0.01, outlier_scale=20.0)
    if M > 2:
        x[M // 2] = 0                                  # a zero token keeps the shared scale
    q_ref, d_ref = oracle.quantize_act_absmax_tensor(x)
    q, d, qs = bl.quantize_act_tensor(dev_bf16(x), with_sums=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(q), q_ref)
    assert np.array_equal(host(d).view(np.uint32), d_ref.view(np.uint32))
    assert np.array_equal(host(qs), oracle.token_sums(q_ref))


def test_quantize_tensor_special():
    bl = _bl()
    say("quantize per tensor: golden e8, zero tensor, strided rows")
    import pins
    g = pins.golden("e8_quant_tensor.json")
    xg = pins.bf16_bits(g["x"])
    q, d = bl.quantize_act_tensor(dev_bf16(xg))
    torch.cuda.synchronize()
    assert host(q).tolist() == g["q"]
    assert host(d).view(np.uint32).tolist() == g["d_bits"]
    z, dz = bl.quantize_act_tensor(dev_bf16(np.zeros((4, 16), np.uint16)))
    torch.cuda.synchronize()
    assert not host(z).any() and not host(dz).any()
    x = W.activations_bf16(71, 6, 24, 0.0, 1.0)
    for ldx in (32, 28):                               # 16-byte path, then the any-K path
        wide = np.zeros((6, ldx), np.uint16)
        wide[:, :24] = x
        qs, ds = bl.quantize_act_tensor(dev_bf16(wide)[:, :24])
        q_ref, d_ref = oracle.quantize_act_absmax_tensor(x)
        torch.cuda.synchronize()
        assert np.array_equal(host(qs), q_ref)
        assert np.array_equal(host(ds).view(np.uint32), d_ref.view(np.uint32))


def test_config3_prefill_per_tensor_scale():
    """2B-layer prefill (512 tokens) with one activation scale per layer input:
    per-tensor quantize then bl_gemm_group, every output against the oracle."""
    bl = _bl()
    cfg = W.LAYERS[3]
    by = {p.name: p for p in cfg.projs}
    for names in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",)):
        inps = [W.proj_inputs(cfg, by[n], 512) for n in names]
        x = inps[0].x_bf16
        say(f"config 3 per-tensor group {names}")
        q_ref, d_ref = oracle.quantize_act_absmax_tensor(x)
        q, d = bl.quantize_act_tensor(dev_bf16(x))
        probs = [dict(packed=bl.pack_i2s(dev(inp.w_tern)),
                      gamma=dev(np.array([inp.gamma], np.float32)), out_dtype="bf16")
                 for inp in inps]
        ys = bl.gemm_group(probs, q, d)
        torch.cuda.synchronize()
        assert np.array_equal(host(q), q_ref)
        assert np.array_equal(host(d).view(np.uint32), d_ref.view(np.uint32))
        for inp, y in zip(inps, ys):
            acc = oracle.mpgemm_acc_f64blas(q_ref, inp.w_tern)
            check_outputs(acc, np.float32(inp.gamma), d_ref, y_bf16=host(y))


def test_quantize_empty():
    bl = _bl()
    say("quantize empty")
    q, d = bl.quantize_act(torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda"))
    assert q.shape == (0, 64) and d.shape == (0,)
    q, d = bl.quantize_act(torch.zeros((3, 0), dtype=torch.bfloat16, device="cuda"))
    qs = torch.full((3,), 7, dtype=torch.int32, device="cuda")
    bl.quantize_act(torch.zeros((3, 0), dtype=torch.bfloat16, device="cuda"), qsum=qs)
    torch.cuda.synchronize()
    assert host(d).tolist() == [0.0, 0.0, 0.0]
    assert host(qs).tolist() == [0, 0, 0]


# ---------------------------------------------------------------------------
# residual add + RMSNorm + quantize
# ---------------------------------------------------------------------------

def check_norm(x, r, g, eps, h, q, d, rows=None):
    """GPU h, q, d (full [M] arrays) against the oracle on `rows` (all by
    default), every one bit-exact: the mean square is the correctly rounded
    one on both sides."""
    rows = np.arange(x.shape[0]) if rows is None else np.asarray(rows)
    h_ref, q_ref, d_ref = oracle.rmsnorm_quant(x[rows], None if r is None else r[rows], g, eps)
    if h is not None:
        assert np.array_equal(h[rows], h_ref), "h differs"
    assert np.array_equal(q[rows], q_ref), "codes differ"
    assert np.array_equal(d[rows].view(np.uint32), d_ref.view(np.uint32)), "scales differ"


def midpoint_batch(seed, K, n_per_kind=2, scales=(0, -50, 40)):
    """Rows of K bf16 values whose exact mean square is an fp32 rounding
    midpoint ("tie") or lies 2^-80 (relative) above or below one, at several
    magnitudes (tests/midpoint_rows.py), each checked here to be what it
    claims against the oracle's exact mean square."""
    from fractions import Fraction
    import midpoint_rows as MR
    rng = np.random.default_rng(seed)
    rows, kinds = [], []
    for kind in ("tie", "above", "below"):
        for se in scales:
            got = 0
            for _ in range(8):
                row = MR.midpoint_row(rng, K, kind, se, background=got % 2 == 0)
                if row is None:
                    continue
                ms = oracle.norm._mean_square(oracle.widen_bf16(row))
                f = oracle.round_fraction_to_f32(ms)
                lo, hi = np.nextafter(f, np.float32(0)), np.nextafter(f, np.float32(np.inf))
                mids = [(Fraction(float(lo)) + Fraction(float(f))) / 2,
                        (Fraction(float(f)) + Fraction(float(hi))) / 2]
                dist = min(abs(ms - m) for m in mids)
                assert (dist == 0) == (kind == "tie") and dist <= ms * Fraction(1, 2 ** 70)
                rows.append(row)
                kinds.append(kind)
                got += 1
                if got == n_per_kind:
                    break
    return np.stack(rows), kinds


@pytest.mark.parametrize("K,ldx", [(64, 64), (2560, 2560), (8192, 8192), (4100, 4100),
                                   (2560, 2564), (40000, 40000)])
def test_rmsnorm_quant_midpoints(K, ldx):
    """Tokens whose exact mean square sits on an fp32 rounding midpoint or
    2^-80 beside one, where an fp64 sum of squares alone would round the
    wrong way: every code and scale bit-exact, through the register-row
    kernel (K % 8 == 0, K <= 32768) and the generic one, with and without a
    residual (a zero residual keeps h = x)."""
    bl = _bl()
    x, kinds = midpoint_batch(4000 + K, K)
    M = x.shape[0]
    say(f"rmsnorm_quant midpoints K={K} ldx={ldx} rows={M} kinds={kinds}")
    g = W.f32_to_bf16_bits((1.0 + 0.1 * W.rng(K).standard_normal(K)).astype(np.float32))
    for r in (None, np.zeros_like(x)):
        h, q, d = _norm_run(bl, x, r, g, 0.0 if r is None else 1e-30, ldx,
                            "none" if r is None else "new")
        check_norm(x, r, g, 0.0 if r is None else 1e-30, h, q, d)


@pytest.mark.parametrize("K", [2560, 4096, 8192])
def test_decode_norm_group_midpoints(K):
    """The one-token decode launch with the norm folded in, on midpoint
    tokens: each token's q, d and outputs bit-exact against the oracle."""
    bl = _bl()
    x, kinds = midpoint_batch(4100 + K, K, n_per_kind=1, scales=(0, -40))
    g = W.f32_to_bf16_bits((1.0 + 0.1 * W.rng(K + 1).standard_normal(K)).astype(np.float32))
    t = W.ternary_drawn(K + 7, 96, K, 0.4)
    packed = bl.pack_i2s(dev(t))
    gam = dev(np.array([GAMMA], np.float32))
    say(f"decode_norm_group midpoints K={K} tokens={x.shape[0]}")
    for i in range(x.shape[0]):
        xi = x[i:i + 1]
        q = torch.empty((1, K), dtype=torch.int8, device="cuda")
        d = torch.empty((1,), dtype=torch.float32, device="cuda")
        (y,) = bl.NormDecodeGroup([dict(packed=packed, gamma=gam, q=q, d=d, out_dtype="f32")],
                                  dev_bf16(xi), dev_bf16(g), 0.0)()
        torch.cuda.synchronize()
        _, q_ref, d_ref = oracle.rmsnorm_quant(xi, None, g, 0.0)
        assert np.array_equal(host(q), q_ref), (i, kinds[i])
        assert host(d).view(np.uint32)[0] == d_ref.view(np.uint32)[0], (i, kinds[i])
        check_outputs(oracle.mpgemm_acc(q_ref, t), GAMMA, d_ref, y_f32=host(y))


# (M, K, ldx, residual, h mode, eps): h mode "new" (a fresh h_out), "none"
# (no h_out), "in_r" (h_out is r), "in_x" (h_out is x). K % 8 == 0 with
# ldx % 8 == 0 and K <= 32768 takes the register-row kernel (256 threads up to
# K = 8192, 1024 above); the rest the generic three-pass kernel.
NORM_CASES = [
    (1, 2560, 2560, True, "new", 1e-5), (5, 2560, 2560, True, "in_r", 1e-5),
    (3, 4096, 4096, False, "none", 1e-6), (2, 6912, 6912, True, "new", 1e-5),
    (2, 8192, 8192, True, "in_x", 1e-5), (3, 11008, 11008, True, "new", 1e-6),
    (2, 28672, 28672, False, "none", 1e-5), (1, 32768, 32768, True, "new", 0.0),
    (7, 40, 40, True, "new", 1e-5), (3, 8, 8, False, "none", 1e-5),
    (2, 2560, 2568, True, "new", 1e-5), (64, 1024, 1024, True, "new", 1e-5),
    (4, 36, 36, True, "new", 1e-5), (3, 2564, 2568, True, "in_r", 1e-5),
    (2, 2560, 2564, False, "none", 1e-5), (2, 32776, 32776, True, "new", 1e-5),
    (1, 4, 4, False, "none", 1e-5), (2, 40000, 40004, True, "in_r", 1e-6),
]


def _norm_run(bl, x, r, g, eps, ldx, mode):
    M, K = x.shape
    def padded(a):
        wide = np.zeros((M, ldx), np.uint16)
        wide[:, :K] = a
        return dev_bf16(wide)[:, :K]
    xd = padded(x)
    rd = None if r is None else padded(r)
    gd = dev_bf16(g)
    h_out = {"new": None, "none": None, "in_r": rd, "in_x": xd}[mode]
    h, q, d, qs = bl.rmsnorm_quant(xd, gd, eps, residual=rd, h_out=h_out, write_h=mode != "none",
                                   with_sums=True)
    torch.cuda.synchronize()
    # the token sums are those of the codes written
    assert np.array_equal(host(qs), oracle.token_sums(host(q)))
    return (None if h is None else host(h)), host(q), host(d)


@pytest.mark.parametrize("M,K,ldx,res,mode,eps", NORM_CASES,
                         ids=[f"M{c[0]}K{c[1]}ld{c[2]}{'r' if c[3] else ''}-{c[4]}" for c in NORM_CASES])
def test_rmsnorm_quant_parity(M, K, ldx, res, mode, eps):
    bl = _bl()
    say(f"rmsnorm_quant M={M} K={K} ldx={ldx} residual={res} h={mode} eps={eps}")
    x, r, g = W.norm_inputs(900 + 3 * M + K, M, K, outlier_frac=0.01, outlier_scale=20.0)
    if not res:
        r = None
    h, q, d = _norm_run(bl, x, r, g, eps, ldx, mode)
    check_norm(x, r, g, eps, h if mode != "none" else None, q, d)


def test_rmsnorm_quant_golden_and_special():
    bl = _bl()
    say("rmsnorm_quant golden e9 + special rows")
    import pins
    for c in pins.golden("e9_rmsnorm_quant.json")["cases"]:
        x = pins.bf16_bits([c["x"]])
        r = None if c["r"] is None else pins.bf16_bits([c["r"]])
        h, q, d = _norm_run(bl, x, r, pins.bf16_bits(c["g"]), c["eps"], 4,
                            "new" if r is not None else "none")
        assert q[0].tolist() == c["q"], c["derivation"]
        assert int(d.view(np.uint32)[0]) == c["d_bits"], c["derivation"]
        if r is not None:
            assert h[0].tolist() == c["h_bits"], c["derivation"]
    # zero rows (eps 0 and > 0), a residual that cancels x, a single spike,
    # tiny and large magnitudes; both kernels (K = 64 and K = 68)
    for K in (64, 68):
        x, r, g = W.norm_inputs(31 + K, 8, K)
        x[0] = 0
        r[0] = 0
        r[1] = x[1] ^ np.uint16(0x8000)                      # x + r = 0 exactly
        x[2] = 0
        r[2] = 0
        x[2, 5] = W.f32_to_bf16_bits(np.array([7.0], np.float32))[0]
        x[3] = W.f32_to_bf16_bits(np.full(K, 2.0 ** -60, np.float32))
        r[3] = 0
        x[4] = W.f32_to_bf16_bits(np.full(K, 1.0e18, np.float32))
        r[4] = 0
        for eps in (0.0, 1e-6):
            h, q, d = _norm_run(bl, x, r, g, eps, K, "new")
            check_norm(x, r, g, eps, h, q, d)
            assert not q[:2].any() and not d[:2].any()


def test_rmsnorm_quant_empty():
    bl = _bl()
    say("rmsnorm_quant empty")
    g = torch.ones(64, dtype=torch.bfloat16, device="cuda")
    h, q, d = bl.rmsnorm_quant(torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda"), g, 1e-5)
    assert q.shape == (0, 64) and d.shape == (0,)
    g0 = torch.ones(0, dtype=torch.bfloat16, device="cuda")
    h, q, d = bl.rmsnorm_quant(torch.zeros((3, 0), dtype=torch.bfloat16, device="cuda"), g0, 1e-5)
    torch.cuda.synchronize()
    assert host(d).tolist() == [0.0, 0.0, 0.0]


@pytest.mark.parametrize("cid,M,n_rows", [(3, 512, 48), (5, 2048, 24)])
def test_rmsnorm_quant_prefill_sampled(cid, M, n_rows):
    """Full prefill shapes (2B layer: 512 x 2560; 100B layer: 2048 x 8192)
    with the configs' outlier channels and the residual stream updated in
    place, as in a decoder layer: sampled tokens against the oracle, and the
    whole h against the residual add done once on the CPU."""
    bl = _bl()
    cfg = W.LAYERS[cid]
    K = cfg.projs[0].K
    say(f"rmsnorm_quant config {cid}: M={M} K={K}")
    x, r, g = W.norm_inputs(5000 + cid, M, K, cfg.outlier_frac, cfg.outlier_scale)
    h, q, d = _norm_run(bl, x, r, g, 1e-5, K, "in_r")
    rows = np.sort(W.rng(77 + cid).permutation(M)[:n_rows])
    rows[0], rows[-1] = 0, M - 1
    check_norm(x, r, g, 1e-5, None, q, d, rows=rows)
    xs = oracle.widen_bf16(x)
    rs = oracle.widen_bf16(r)
    h_all = oracle.norm._bf16_rne_from_f32((xs + rs).astype(np.float32))
    assert np.array_equal(h, h_all)


# ---------------------------------------------------------------------------
# pack_i2s
# ---------------------------------------------------------------------------

PACK_SHAPES = [(1, 4), (3, 12), (2, 20), (16, 64), (17, 260), (640, 2560), (1024, 1024),
               (33, 4096)]


@pytest.mark.parametrize("N,K", PACK_SHAPES, ids=[f"N{n}K{k}" for n, k in PACK_SHAPES])
def test_pack_f32_parity(N, K):
    bl = _bl()
    say(f"pack f32 N={N} K={K}")
    w = W.weights_f32_normal(200 + N + K, N, K)
    t_ref, g_ref = oracle.ternarize_absmean(w)
    p_ref = oracle.pack_i2s(t_ref)
    packed, gamma = bl.pack_i2s(dev(w))
    torch.cuda.synchronize()
    assert host(gamma).view(np.uint32)[0] == np.float32(g_ref).view(np.uint32)
    assert np.array_equal(host(packed), p_ref)


def _tiles_with_ties(N, K, seed):
    """Rows whose |w| values are a permutation of a pattern with mean exactly 1,
    so gamma = 1, t = 0.5 and every +-0.5 sits exactly on the threshold."""
    base = np.array([2.0, 0.5, 0.5, 1.0, 0.0, 0.5, 1.5, 2.0], dtype=np.float32)  # mean 1
    r = W.rng(seed)
    w = np.empty((N, K), dtype=np.float32)
    for n in range(N):
        row = np.resize(base, K)
        w[n] = r.permutation(row) * np.where(r.random(K) < 0.5, -1, 1)
    return w


@pytest.mark.parametrize("case", ["ties", "huge_small", "subnormal", "spread", "golden_e3",
                                  "golden_e4"])
def test_pack_f32_adversarial(case):
    bl = _bl()
    say(f"pack f32 adversarial {case}")
    r = W.rng(31)
    if case == "ties":
        w = _tiles_with_ties(12, 64, 5)
    elif case == "huge_small":
        w = np.array([[2.0**60] + [1.0] * 1023 + [2.0**-20] * 64], dtype=np.float32)
    elif case == "subnormal":
        w = np.array([[1e-45, 3e-45, 1.0, 2.0**-126, 2.0**-130, 0.1, 0.3, 0.0]], np.float32)
    elif case == "spread":
        w = (r.standard_normal((4, 500)) * np.exp2(r.integers(-60, 60, (4, 500)))).astype(
            np.float32)
    elif case == "golden_e3":
        w = np.array([[7.0, 1.0, 0.0, 0.0]], np.float32)
    else:  # e4's 12 weights laid out as 3 x 4
        w = np.array([[0.75, -0.25, 0.125, -1.0], [0.0, 0.375, -0.75, 0.25],
                      [-0.125, 1.0, 0.0, -0.375]], np.float32)
    t_ref, g_ref = oracle.ternarize_absmean(w)
    packed, gamma = bl.pack_i2s(dev(w))
    torch.cuda.synchronize()
    assert host(gamma).view(np.uint32)[0] == np.float32(g_ref).view(np.uint32), (
        host(gamma)[0], g_ref)
    assert np.array_equal(host(packed), oracle.pack_i2s(t_ref))
    if case == "ties":
        assert g_ref == 1.0 and np.any(np.abs(w) == 0.5)


@pytest.mark.parametrize("N,K", [(1, 4), (5, 12), (7, 36), (64, 256), (300, 2560)])
def test_pack_ternary_parity(N, K):
    bl = _bl()
    say(f"pack ternary N={N} K={K}")
    t = W.ternary_drawn(300 + N, N, K, 0.4)
    packed = bl.pack_i2s(dev(t))
    torch.cuda.synchronize()
    assert np.array_equal(host(packed), oracle.pack_i2s(t))
    # values outside {-1, 0, 1} are taken by their sign
    wide = (t.astype(np.int16) * W.rng(7).integers(1, 100, t.shape)).clip(-128, 127).astype(
        np.int8)
    packed2 = bl.pack_i2s(dev(wide))
    torch.cuda.synchronize()
    assert np.array_equal(host(packed2), oracle.pack_i2s(np.sign(wide).astype(np.int8)))


# ---------------------------------------------------------------------------
# gemv / gemm on generated int8 activations
# ---------------------------------------------------------------------------

def _mm_case(M, N, K, seed, zero_rows=()):
    q = W.int8_codes(seed, M, K, zero_rows)
    q[0, :min(K, 8)] = 127              # extremes
    if M > 1:
        q[1, :min(K, 8)] = -127
    t = W.ternary_drawn(seed + 1, N, K, 0.35)
    if N > 2:
        t[2, :] = 1                       # all +1 row: acc = sum of q
    d = W.positive_scales(seed + 2, M, zero_rows)
    return q, t, d


def _run_mm(bl, fn_name, M, N, K, seed, zero_rows=()):
    say(f"{fn_name} M={M} N={N} K={K} seed={seed}")
    q, t, d = _mm_case(M, N, K, seed, zero_rows)
    acc = oracle.mpgemm_acc(q, t)
    packed = bl.pack_i2s(dev(t))
    gd = dev(np.array([GAMMA], np.float32))
    fn = getattr(bl, fn_name)
    outs = run_all_outputs(bl, fn, packed, gd, dev(q), dev(d))
    torch.cuda.synchronize()
    check_outputs(acc, GAMMA, d, outs["i32"], outs["f32"], outs["bf16"])
    if fn_name == "gemm":
        # with the token sums the kernel runs on offset weights: same bits
        qs = dev(oracle.token_sums(q).astype(np.int32))
        for name in ("i32", "f32", "bf16"):
            y = host(bl.gemm(packed, gd, dev(q), dev(d), out_dtype=name, qsum=qs))
            assert np.array_equal(y.view(np.uint8), outs[name].view(np.uint8)), name
    return outs


GEMV_CASES = [(1, 1, 64), (1, 5, 4), (1, 17, 12), (1, 100, 320), (1, 640, 2560), (2, 33, 256),
              (3, 16, 1024), (4, 129, 576), (5, 64, 2560), (8, 300, 260), (15, 17, 6912),
              (16, 128, 4096), (16, 3, 64), (1, 2049, 256), (16, 2100, 512)]


@pytest.mark.parametrize("M,N,K", GEMV_CASES, ids=[f"M{m}N{n}K{k}" for m, n, k in GEMV_CASES])
def test_gemv_parity(M, N, K):
    bl = _bl()
    _run_mm(bl, "gemv", M, N, K, seed=1000 + M * 31 + N * 7 + K, zero_rows=(M - 1,) if M > 2
            else ())


GEMM_CASES = [(17, 1, 64), (17, 130, 256), (33, 17, 4), (64, 64, 2560), (100, 640, 320),
              (128, 128, 256), (129, 257, 576), (300, 100, 1024), (512, 640, 2560),
              (65, 48, 6912), (1, 40, 256), (16, 40, 256), (200, 33, 260), (2048, 1100, 320)]


@pytest.mark.parametrize("M,N,K", GEMM_CASES, ids=[f"M{m}N{n}K{k}" for m, n, k in GEMM_CASES])
def test_gemm_parity(M, N, K):
    bl = _bl()
    _run_mm(bl, "gemm", M, N, K, seed=2000 + M * 31 + N * 7 + K, zero_rows=(M - 2,) if M > 3
            else ())


GROUP_CASES = [
    # (M, K, [N per problem], [out dtype per problem]); the first case has a
    # problem big enough for the 128x256-tile launch next to small ones
    (512, 128, [16484, 640, 0, 33], ["bf16", "f32", "bf16", "i32"]),
    (300, 1024, [100, 257], ["f32", "bf16"]),
    (2048, 256, [1024, 1024, 8192], ["bf16", "bf16", "i32"]),
    (40, 260, [7, 64], ["f32", "i32"]),          # K % 64 != 0
    (9, 512, [50, 3], ["bf16", "f32"]),           # M <= 16
    # two big problems of >= 32768 rows together: the 256x128-tile launch,
    # each problem alone the 128x256 one
    (300, 256, [16400, 16400], ["bf16", "i32"]),
]


@pytest.mark.parametrize("M,K,Ns,outs", GROUP_CASES,
                         ids=[f"M{c[0]}K{c[1]}N{'-'.join(map(str, c[2]))}" for c in GROUP_CASES])
def test_gemm_group_parity(M, K, Ns, outs):
    """Every problem of a group against the oracle, and bit-identical to the
    same problem run alone through bl_gemm."""
    bl = _bl()
    seed = 3000 + M + K
    say(f"gemm_group M={M} K={K} N={Ns} outs={outs}")
    q = W.int8_codes(seed, M, K, (M - 1,))
    d = W.positive_scales(seed + 1, M, (M - 1,))
    qd, dd = dev(q), dev(d)
    probs, refs = [], []
    for i, (N, o) in enumerate(zip(Ns, outs)):
        t = W.ternary_drawn(seed + 10 + i, N, K, 0.3 + 0.05 * i)
        g = np.float32(GAMMA * (1 + i))
        probs.append(dict(packed=bl.pack_i2s(dev(t)), gamma=dev(np.array([g], np.float32)),
                          out_dtype=o))
        refs.append((t, g))
    ys = bl.gemm_group(probs, qd, dd)
    alone = [bl.gemm(p["packed"], p["gamma"], qd, dd, out_dtype=p["out_dtype"]) for p in probs]
    qs = dev(oracle.token_sums(q).astype(np.int32))
    ys_off = [y.clone() for y in bl.gemm_group(probs, qd, dd, qsum=qs)]
    torch.cuda.synchronize()
    for (t, g), o, y, y1, y2 in zip(refs, outs, ys, alone, ys_off):
        assert torch.equal(y, y1), "group output differs from the single-problem call"
        assert torch.equal(y, y2), "offset-weight (token sums) output differs"
        acc = oracle.mpgemm_acc_f64blas(q, t) if M * t.shape[0] * K > 2e8 else \
            oracle.mpgemm_acc(q, t)
        check_outputs(acc, g, d, **{f"y_{o}": host(y)})


@pytest.mark.parametrize("M,N,K", [(17, 640, 2560), (31, 300, 320), (33, 2560, 6912),
                                   (33, 1024, 8192)])
def test_gemv_equals_gemm(M, N, K):
    """The MFMA GEMM at its smallest token counts (M > 16, so bl_gemm runs
    k_gemm_i2s) against bl_gemv over the same tokens in slices of at most 16:
    byte-identical for every output type, with and without the token sums,
    and both equal to the oracle; a repeated GEMM gives the same bytes."""
    bl = _bl()
    say(f"gemv == gemm M={M} N={N} K={K}")
    q, t, d = _mm_case(M, N, K, 79 + M)
    acc = oracle.mpgemm_acc(q, t)
    packed = bl.pack_i2s(dev(t))
    gd = dev(np.array([GAMMA], np.float32))
    qd, dd = dev(q), dev(d)
    qs = dev(oracle.token_sums(q).astype(np.int32))
    for name in ("i32", "f32", "bf16"):
        y_mm = host(bl.gemm(packed, gd, qd, dd, out_dtype=name))
        y_off = host(bl.gemm(packed, gd, qd, dd, out_dtype=name, qsum=qs))
        y_again = host(bl.gemm(packed, gd, qd, dd, out_dtype=name, qsum=qs))
        parts = [host(bl.gemv(packed, gd, qd[t0:t0 + 16], dd[t0:t0 + 16], out_dtype=name))
                 for t0 in range(0, M, 16)]
        torch.cuda.synchronize()
        y_mv = np.concatenate(parts, axis=0)
        assert np.array_equal(y_mm.view(np.uint8), y_mv.view(np.uint8)), name
        assert np.array_equal(y_off.view(np.uint8), y_mv.view(np.uint8)), name
        assert np.array_equal(y_again.view(np.uint8), y_off.view(np.uint8)), name
        kw = {"i32": "y_i32", "f32": "y_f32", "bf16": "y_bf16"}[name]
        check_outputs(acc, GAMMA, d, **{kw: y_mm})


SPLIT_CASES = [(64, 2560, 6912), (17, 40, 4096), (100, 300, 4160), (300, 1000, 8192),
               (512, 640, 8192), (33, 4000, 6912)]


@pytest.mark.parametrize("M,N,K", SPLIT_CASES, ids=[f"M{m}N{n}K{k}" for m, n, k in SPLIT_CASES])
def test_gemm_split_k(M, N, K):
    """Launches whose tiles leave CUs idle and whose K is long split K over the
    workspace and add the int32 partials in a second launch: byte-identical to
    the unsplit launch (no workspace) for every output type, with and without
    the token sums (K % 128 == 64 tails included), and equal to the oracle."""
    bl = _bl()
    nws = bl.gemm_workspace(M, N, K)
    say(f"gemm split-K M={M} N={N} K={K} workspace={nws}")
    assert nws > 0
    q, t, d = _mm_case(M, N, K, 301 + M)
    acc = oracle.mpgemm_acc(q, t) if M * N * K < 4e8 else oracle.mpgemm_acc_f64blas(q, t)
    packed = bl.pack_i2s(dev(t))
    gd = dev(np.array([GAMMA], np.float32))
    qd, dd = dev(q), dev(d)
    qs = dev(oracle.token_sums(q).astype(np.int32))
    ws = torch.full((nws,), 0x5A, dtype=torch.uint8, device="cuda")   # stale bytes in it
    for name in ("i32", "f32", "bf16"):
        for qsum in (None, qs):
            y_split = host(bl.gemm(packed, gd, qd, dd, out_dtype=name, qsum=qsum, workspace=ws))
            y_plain = host(bl.gemm(packed, gd, qd, dd, out_dtype=name, qsum=qsum, split=False))
            torch.cuda.synchronize()
            assert np.array_equal(y_split.view(np.uint8), y_plain.view(np.uint8)), name
        kw = {"i32": "y_i32", "f32": "y_f32", "bf16": "y_bf16"}[name]
        check_outputs(acc, GAMMA, d, **{kw: y_split})


def test_gemm_group_split_k():
    """A group whose small problems split K next to one that fills the chip
    unsplit, and a group of small problems that split together (the 2B-class
    {q,k,v} shapes at 128 tokens and K = 6912): byte-identical to the group
    without a workspace and to bl_gemm per problem."""
    bl = _bl()
    for M, K, Ns in ((1024, 4096, (16384, 64, 256)), (128, 6912, (2560, 640, 640))):
        say(f"gemm_group split-K M={M} K={K} Ns={Ns}")
        q, _, d = _mm_case(M, 8, K, 400 + M)
        qd, dd = dev(q), dev(d)
        qs = dev(oracle.token_sums(q).astype(np.int32))
        probs = [dict(packed=bl.pack_i2s(dev(W.ternary_drawn(410 + i, n, K, 0.35))),
                      gamma=dev(np.array([GAMMA], np.float32)), out_dtype=ot)
                 for i, (n, ot) in enumerate(zip(Ns, ("bf16", "i32", "f32")))]
        g_split = bl.GemmGroup(probs, qd, dd, qsum=qs)
        assert g_split.workspace is not None
        ys = [host(y) for y in g_split()]
        ys_plain = [host(y) for y in bl.GemmGroup(probs, qd, dd, qsum=qs, split=False)()]
        torch.cuda.synchronize()
        for p, a, b in zip(probs, ys, ys_plain):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
            one = host(bl.gemm(p["packed"], p["gamma"], qd, dd, out_dtype=p["out_dtype"]))
            assert np.array_equal(a.view(np.uint8), one.view(np.uint8))


def test_k_zero_and_empty():
    bl = _bl()
    say("K == 0 and empty M/N")
    q = torch.zeros((3, 0), dtype=torch.int8, device="cuda")
    packed = torch.zeros((5, 0), dtype=torch.uint8, device="cuda")
    gd = dev(np.array([GAMMA], np.float32))
    dd = dev(np.ones(3, np.float32))
    for fn in (bl.gemv, bl.gemm):
        y = fn(packed, gd, q, dd, out_dtype="f32")
        torch.cuda.synchronize()
        assert np.all(host(y) == 0) and y.shape == (3, 5)
    y = bl.gemm(torch.zeros((0, 16), dtype=torch.uint8, device="cuda"), gd,
                torch.zeros((4, 64), dtype=torch.int8, device="cuda"), dd[:1].repeat(4))
    assert y.shape == (4, 0)


# ---------------------------------------------------------------------------
# fused decode group (quantize + GEMV + dequant in one launch)
# ---------------------------------------------------------------------------

def _decode_group_case(bl, M, shapes, seed, with_qd=True, out_types=None):
    say(f"decode_group M={M} shapes={shapes} with_qd={with_qd}")
    probs, refs = [], []
    for i, (N, K) in enumerate(shapes):
        x = W.activations_bf16(seed + 10 * i, M, K, outlier_frac=0.01, outlier_scale=20.0)
        if M > 2:
            x[M - 1] = 0                                  # an all-zero token
        t = W.ternary_drawn(seed + 10 * i + 1, N, K, 0.4)
        ot = (out_types or ["bf16", "f32", "i32"])[i % len(out_types or ["bf16", "f32", "i32"])]
        p = dict(packed=bl.pack_i2s(dev(t)), gamma=dev(np.array([GAMMA], np.float32)),
                 x=dev_bf16(x), out_dtype=ot)
        if with_qd:
            p["q"] = torch.empty((M, K), dtype=torch.int8, device="cuda")
            p["d"] = torch.empty((M,), dtype=torch.float32, device="cuda")
        probs.append(p)
        refs.append((x, t, ot))
    grp = bl.DecodeGroup(probs)
    ys = grp()
    torch.cuda.synchronize()
    for p, y, (x, t, ot) in zip(probs, ys, refs):
        q_ref, d_ref = oracle.quantize_act_absmax(x)
        acc = oracle.mpgemm_acc(q_ref, t)
        if with_qd:
            assert np.array_equal(host(p["q"]), q_ref)
            assert np.array_equal(host(p["d"]).view(np.uint32), d_ref.view(np.uint32))
        kw = {"i32": "y_i32", "f32": "y_f32", "bf16": "y_bf16"}[ot]
        check_outputs(acc, GAMMA, d_ref, **{kw: host(y)})
        # identical to the unfused calls
        q, d = bl.quantize_act(p["x"])
        y2 = bl.gemv(p["packed"], p["gamma"], q, d, out_dtype=ot)
        torch.cuda.synchronize()
        assert np.array_equal(host(y2).view(np.uint8), host(y).view(np.uint8))
    return grp


@pytest.mark.parametrize("M", [1, 2, 3, 4, 16])
def test_decode_group_parity(M):
    bl = _bl()
    _decode_group_case(bl, M, [(100, 320), (640, 2560), (33, 64), (2049, 256), (5, 6912)],
                       seed=40 + M)


def test_decode_group_one_token_long_k():
    """One-token groups whose parts need 4 and 8 x chunks per lane, with a
    K % 256 != 0 tail, K of exactly 16384, and the 16-wave block at the
    largest K the call takes (65536)."""
    bl = _bl()
    _decode_group_case(bl, 1, [(33, 16384), (17, 4160), (3, 1088), (20, 64)], seed=77)
    _decode_group_case(bl, 1, [(3, 65536), (9, 40960)], seed=78, out_types=["f32", "bf16"])


@pytest.mark.parametrize("K", [9024, 11008, 13824, 16384, 20032, 24576, 27648, 32768])
def test_decode_group_one_token_batches(K):
    """One-token groups whose waves walk 5 to 8 steps in a single load batch:
    8 waves per block at K = 9024, 11008 (the 7B-class {down}), 13824 and
    16384, 16 waves at K = 20032, 24576, 27648 and 32768 (ragged last steps
    included)."""
    bl = _bl()
    _decode_group_case(bl, 1, [(33, K), (17, K)], seed=700 + K % 97)


def test_decode_group_wide():
    """One-token groups with a problem of >= 8192 rows take the whole-line
    kernel: one batch per wave at K = 512, 2560, 4160 (K % 512 != 0) and 8192
    (waves without steps at the small K), small problems riding in the same
    launch, a ragged last row block, and two batches per wave at K = 28672."""
    bl = _bl()
    _decode_group_case(bl, 1, [(8192, 8192)], seed=90)
    _decode_group_case(bl, 1, [(8200, 4160), (1000, 4160)], seed=91)
    _decode_group_case(bl, 1, [(8192, 2560), (640, 2560), (640, 2560)], seed=92,
                       out_types=["bf16", "i32", "f32"])
    _decode_group_case(bl, 1, [(9000, 512), (16, 64)], seed=93)
    _decode_group_case(bl, 1, [(8193, 28672)], seed=94, out_types=["i32"])
    # four steps per wave with x staged by direct-to-LDS loads: the 100B-class
    # shape, and a ragged last step (K % 512 != 0) with a ragged row block
    _decode_group_case(bl, 1, [(28672, 8192)], seed=98, out_types=["i32"])
    _decode_group_case(bl, 1, [(8200, 7936), (300, 7936)], seed=99, out_types=["f32", "bf16"])


def test_decode_group_one_token_large_groups():
    """One-token groups of at least 256 16-row tiles, as the layers stream
    them: three problems whose row counts are not multiples of 16 (ragged
    last row blocks in every problem), partial last steps (K % 512 != 0 and
    K % 256 != 0), eight problems in one launch, the 7B-class groups, the
    x chunks of a 24576-long row, launches that issue their weights after
    the activation row (several load batches per wave), no q and d outputs,
    and an i32 output without gamma."""
    bl = _bl()
    _decode_group_case(bl, 1, [(4100, 1088), (2000, 1088), (100, 1088)], seed=130)
    _decode_group_case(bl, 1, [(4096, 4096)] * 3, seed=131, out_types=["bf16"])
    _decode_group_case(bl, 1, [(11008, 4096), (11008, 4096)], seed=132, out_types=["bf16"])
    _decode_group_case(bl, 1, [(4096, 11008)], seed=133, out_types=["f32"])
    _decode_group_case(bl, 1, [(520, 512)] * 8, seed=134)
    _decode_group_case(bl, 1, [(5000, 320), (3001, 320)], seed=135, with_qd=False)
    _decode_group_case(bl, 1, [(4100, 24576)], seed=136, out_types=["i32"])
    # weights issued after the row maximum or the codes (launches of >= 512
    # and >= 1024 blocks), with several load batches per wave
    _decode_group_case(bl, 1, [(4096, 36864)] * 2, seed=139, out_types=["i32", "f32"])
    _decode_group_case(bl, 1, [(16384, 16896)], seed=140, out_types=["bf16"])
    N, K = 4111, 2112
    say(f"decode_group i32 without gamma N={N} K={K}")
    x = W.activations_bf16(137, 1, K, outlier_frac=0.01, outlier_scale=20.0)
    t = W.ternary_drawn(138, N, K, 0.4)
    (y,) = bl.decode_group([dict(packed=bl.pack_i2s(dev(t)), x=dev_bf16(x))], out_dtype="i32")
    torch.cuda.synchronize()
    q_ref, _ = oracle.quantize_act_absmax(x)
    assert np.array_equal(host(y), oracle.mpgemm_acc(q_ref, t).astype(np.int32))


def test_decode_group_tokens_large_groups():
    """2-4-token groups of at least 512 16-row blocks, whose weights are
    issued after the row maxima: the 7B-class {q,k,v} at 4 tokens (one load
    batch), and 3 tokens over two 24576-long problems (two batches per wave,
    more than 64 KB of LDS)."""
    bl = _bl()
    _decode_group_case(bl, 4, [(4096, 4096)] * 3, seed=141, out_types=["bf16"])
    _decode_group_case(bl, 3, [(4096, 24576)] * 2, seed=142, out_types=["f32", "i32"])


def test_decode_group_wide_longest_k():
    """The 16-wave whole-line block at the largest K the call takes (65536):
    byte-identical to quantize + bl_gemv, sampled rows against the oracle."""
    bl = _bl()
    N, K = 8208, 65536
    say(f"decode_group wide N={N} K={K}")
    x = W.activations_bf16(95, 1, K, outlier_frac=0.01, outlier_scale=20.0)
    t = W.ternary_drawn(96, N, K, 0.4)
    packed = bl.pack_i2s(dev(t))
    gamma = dev(np.array([GAMMA], np.float32))
    (y,) = bl.decode_group([dict(packed=packed, gamma=gamma, x=dev_bf16(x))], out_dtype="f32")
    q, d = bl.quantize_act(dev_bf16(x))
    y2 = bl.gemv(packed, gamma, q, d, out_dtype="f32")
    torch.cuda.synchronize()
    assert np.array_equal(host(y).view(np.uint32), host(y2).view(np.uint32))
    q_ref, d_ref = oracle.quantize_act_absmax(x)
    rows = np.unique(np.concatenate([W.rng(97).integers(0, N, 40), [0, 15, 16, N - 17, N - 1]]))
    acc = oracle.mpgemm_acc(q_ref, t[rows])
    check_outputs(acc, GAMMA, d_ref, y_f32=host(y)[:, rows])


# ---------------------------------------------------------------------------
# base-3 weights, five per byte
# ---------------------------------------------------------------------------

T3_PACK_SHAPES = [(1, 16), (3, 320), (5, 336), (17, 2560), (7, 4160), (640, 2560), (9, 28672)]


@pytest.mark.parametrize("N,K", T3_PACK_SHAPES, ids=[f"N{n}K{k}" for n, k in T3_PACK_SHAPES])
def test_pack_t3_parity(N, K):
    """Packed bytes bit-exact against the oracle, from int8 ternary weights and
    from fp32 weights (same gamma and ternary values as the I2_S packing)."""
    bl = _bl()
    say(f"pack_t3 N={N} K={K}")
    t = W.ternary_drawn(300 + N + K, N, K, 0.4)
    got = bl.pack_t3(dev(t))
    torch.cuda.synchronize()
    assert np.array_equal(host(got), oracle.pack_t3(t))
    w = W.weights_f32_normal(400 + N + K, N, K)
    p3, g3 = bl.pack_t3(dev(w))
    p2, g2 = bl.pack_i2s(dev(w))
    torch.cuda.synchronize()
    t_ref = oracle.ternarize_absmean(w)[0]
    assert host(g3).view(np.uint32)[0] == host(g2).view(np.uint32)[0]
    assert np.array_equal(host(p3), oracle.pack_t3(t_ref))


T3_GEMV_CASES = [(1, 1, 16), (1, 5, 320), (1, 17, 336), (2, 33, 2560), (4, 100, 4160),
                 (16, 64, 1296), (1, 640, 6912), (3, 300, 8192), (1, 129, 28672), (16, 40, 65536)]


@pytest.mark.parametrize("M,N,K", T3_GEMV_CASES, ids=[f"M{m}N{n}K{k}" for m, n, k in T3_GEMV_CASES])
def test_gemv_t3_parity(M, N, K):
    """Every output type against the oracle, and byte-identical to bl_gemv on
    the I2_S packing of the same weights."""
    bl = _bl()
    say(f"gemv_t3 M={M} N={N} K={K}")
    x = W.activations_bf16(500 + M + N, M, K, outlier_frac=0.01, outlier_scale=20.0)
    if M > 2:
        x[1] = 0
    t = W.ternary_drawn(600 + N + K, N, K, 0.4)
    q, d = bl.quantize_act(dev_bf16(x))
    p3 = bl.pack_t3(dev(t))
    p2 = bl.pack_i2s(dev(t))
    gamma = dev(np.array([GAMMA], np.float32))
    q_ref, d_ref = oracle.quantize_act_absmax(x)
    acc = oracle.mpgemm_acc(q_ref, t)
    for ot in ("i32", "f32", "bf16"):
        y3 = bl.gemv_t3(p3, gamma, q, d, out_dtype=ot)
        y2 = bl.gemv(p2, gamma, q, d, out_dtype=ot)
        torch.cuda.synchronize()
        kw = {"i32": "y_i32", "f32": "y_f32", "bf16": "y_bf16"}[ot]
        if ot != "f32" or 127 * K < 2 ** 24:
            check_outputs(acc, GAMMA, d_ref, **{kw: host(y3)})
        assert np.array_equal(host(y3).view(np.uint8), host(y2).view(np.uint8))


def test_gemv_t3_empty_and_zero_k():
    bl = _bl()
    say("gemv_t3 empty / K = 0")
    gamma = dev(np.array([GAMMA], np.float32))
    q = torch.zeros((2, 0), dtype=torch.int8, device="cuda")
    d = torch.ones(2, dtype=torch.float32, device="cuda")
    p3 = torch.zeros((5, 0), dtype=torch.uint8, device="cuda")
    y = bl.gemv_t3(p3, gamma, q, d, out_dtype="f32")
    torch.cuda.synchronize()
    assert host(y).shape == (2, 5) and not host(y).any()
    y0 = bl.gemv_t3(torch.zeros((0, 64), dtype=torch.uint8, device="cuda"), gamma,
                    torch.zeros((1, 16), dtype=torch.int8, device="cuda"), d[:1])
    assert y0.shape == (1, 0)


def _decode_group_t3_case(bl, M, shapes, seed, with_qd=True, out_types=None, zero_x=False):
    say(f"decode_group_t3 M={M} shapes={shapes} with_qd={with_qd}")
    ots = out_types or ["bf16", "f32", "i32"]
    probs, refs = [], []
    for i, (N, K) in enumerate(shapes):
        x = W.activations_bf16(seed + 10 * i, M, K, outlier_frac=0.01, outlier_scale=20.0)
        if zero_x or M > 2:
            x[M - 1] = 0                                  # an all-zero token
        t = W.ternary_drawn(seed + 10 * i + 1, N, K, 0.4)
        ot = ots[i % len(ots)]
        p = dict(packed=bl.pack_t3(dev(t)), gamma=dev(np.array([GAMMA], np.float32)),
                 x=dev_bf16(x), out_dtype=ot)
        if with_qd:
            p["q"] = torch.full((M, K), 99, dtype=torch.int8, device="cuda")
            p["d"] = torch.full((M,), -1.0, dtype=torch.float32, device="cuda")
        probs.append(p)
        refs.append((x, t, ot))
    ys = bl.DecodeGroupT3(probs)()
    torch.cuda.synchronize()
    for p, y, (x, t, ot) in zip(probs, ys, refs):
        q_ref, d_ref = oracle.quantize_act_absmax(x)
        acc = oracle.mpgemm_acc(q_ref, t)
        if with_qd:
            assert np.array_equal(host(p["q"]), q_ref)
            assert np.array_equal(host(p["d"]).view(np.uint32), d_ref.view(np.uint32))
        kw = {"i32": "y_i32", "f32": "y_f32", "bf16": "y_bf16"}[ot]
        check_outputs(acc, GAMMA, d_ref, **{kw: host(y)})
        # identical to quantize + the base-3 GEMV, and to the I2_S decode group
        q, d = bl.quantize_act(p["x"])
        y2 = bl.gemv_t3(p["packed"], p["gamma"], q, d, out_dtype=ot)
        torch.cuda.synchronize()
        assert np.array_equal(host(y2).view(np.uint8), host(y).view(np.uint8))
        K = x.shape[1]
        if K % 64 == 0:
            (y3,) = bl.decode_group([dict(packed=bl.pack_i2s(dev(t)), gamma=p["gamma"], x=p["x"],
                                          out_dtype=ot)])
            torch.cuda.synchronize()
            assert np.array_equal(host(y3).view(np.uint8), host(y).view(np.uint8))


def test_decode_group_t3_one_token():
    """One launch per group at M == 1, through every block configuration:
    one segment per wave (K = 16 with a single step, 336, 2560), 2-4 segments
    (6912, 4160 with an odd step count), 8 waves (12800) and two load batches
    (28672), small problems riding with large ones, ragged row blocks, and
    every output type."""
    bl = _bl()
    _decode_group_t3_case(bl, 1, [(2560, 2560), (640, 2560), (640, 2560)], seed=1200)
    _decode_group_t3_case(bl, 1, [(17, 336), (1, 16), (33, 1296)], seed=1210)
    _decode_group_t3_case(bl, 1, [(2560, 6912), (1000, 4160)], seed=1220,
                          out_types=["bf16", "i32"])
    _decode_group_t3_case(bl, 1, [(100, 12800), (16, 320)], seed=1230, out_types=["f32"])
    _decode_group_t3_case(bl, 1, [(8192, 28672)], seed=1240, with_qd=False)
    _decode_group_t3_case(bl, 1, [(129, 8192)], seed=1250, zero_x=True)


def test_decode_group_t3_longest_k():
    """The 16-wave block (more than 64 KB of LDS) at K = 65536 and 61456."""
    bl = _bl()
    _decode_group_t3_case(bl, 1, [(24, 65536), (9, 61456)], seed=1260, out_types=["f32", "bf16"])


@pytest.mark.parametrize("M", [2, 3, 16])
def test_decode_group_t3_tokens(M):
    """Several tokens: quantize pass, then the base-3 GEMV per problem."""
    bl = _bl()
    _decode_group_t3_case(bl, M, [(100, 320), (33, 1296), (640, 2560)], seed=1270 + M)


@pytest.mark.parametrize("M", [1, 3])
def test_decode_group_t3_graph_replay(M):
    """HIP-graph replays of the base-3 decode group (one fused launch at one
    token; quantize + GEMV launches at three) give the eager result every time."""
    bl = _bl()
    say(f"decode_group_t3 graph replay M={M}")
    probs = []
    for i, (N, K) in enumerate([(2560, 2560), (640, 2560), (33, 1296)]):
        x = W.activations_bf16(1400 + 10 * i + M, M, K, outlier_frac=0.01, outlier_scale=20.0)
        t = W.ternary_drawn(1401 + 10 * i, N, K, 0.4)
        probs.append(dict(packed=bl.pack_t3(dev(t)), gamma=dev(np.array([GAMMA], np.float32)),
                          x=dev_bf16(x), out_dtype="bf16"))
    grp = bl.DecodeGroupT3(probs)
    ref = [host(y).copy() for y in grp()]
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        grp()
    for _ in range(3):
        for y in grp.outputs:
            y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for y, r in zip(grp.outputs, ref):
            assert np.array_equal(host(y), r)


def test_decode_group_t3_zero_k():
    """A K == 0 problem gives zeros (and a zero scale) next to a normal one."""
    bl = _bl()
    say("decode_group_t3 K = 0")
    x0 = torch.zeros((1, 0), dtype=torch.bfloat16, device="cuda")
    d0 = torch.full((1,), 5.0, dtype=torch.float32, device="cuda")
    y0 = torch.full((1, 7), 3.0, dtype=torch.float32, device="cuda")
    t = W.ternary_drawn(1290, 40, 336, 0.4)
    x = W.activations_bf16(1291, 1, 336)
    gamma = dev(np.array([GAMMA], np.float32))
    ys = bl.decode_group_t3([dict(packed=torch.zeros((7, 0), dtype=torch.uint8, device="cuda"),
                                  gamma=gamma, x=x0, y=y0, d=d0, out_dtype="f32"),
                             dict(packed=bl.pack_t3(dev(t)), gamma=gamma, x=dev_bf16(x),
                                  out_dtype="f32")])
    torch.cuda.synchronize()
    assert not host(ys[0]).any() and host(d0)[0] == 0.0
    q_ref, d_ref = oracle.quantize_act_absmax(x)
    check_outputs(oracle.mpgemm_acc(q_ref, t), GAMMA, d_ref, y_f32=host(ys[1]))


NORM_GROUP_CASES = [
    ("qkv_2b", [(2560, 2560), (640, 2560), (640, 2560)], True, 1e-5),
    ("gate_up_2b", [(6912, 2560), (6912, 2560)], True, 1e-6),
    ("down_2b_subnorm", [(2560, 6912)], False, 1e-5),
    ("7b", [(4096, 4096), (11008, 4096)], True, 1e-5),
    ("100b_q", [(8192, 8192), (1024, 8192)], True, 1e-5),
    ("k32768_16waves", [(64, 32768), (17, 32768)], True, 0.0),
    ("tiny", [(33, 64), (5, 64)], False, 1e-5),
    ("k_tail", [(40, 4160)], True, 1e-5),
]


@pytest.mark.parametrize("name,shapes,res,eps", NORM_GROUP_CASES, ids=[c[0] for c in NORM_GROUP_CASES])
def test_decode_norm_group_parity(name, shapes, res, eps):
    """Residual add + RMSNorm + quantize + GEMV in one launch: h, q, d and
    every output against the oracle, and byte-identical to bl_rmsnorm_quant
    followed by bl_gemv."""
    bl = _bl()
    K = shapes[0][1]
    say(f"decode_norm_group {name}: shapes={shapes} residual={res} eps={eps}")
    x, r, g = W.norm_inputs(1100 + K, 1, K, outlier_frac=0.01, outlier_scale=20.0)
    if not res:
        r = None
    xd, gd = dev_bf16(x), dev_bf16(g)
    rd = None if r is None else dev_bf16(r)
    hd = torch.empty_like(xd) if res else None
    probs, ts = [], []
    for i, (N, _) in enumerate(shapes):
        t = W.ternary_drawn(1200 + N + i, N, K, 0.4)
        ts.append(t)
        probs.append(dict(packed=bl.pack_i2s(dev(t)), gamma=dev(np.array([GAMMA], np.float32)),
                          q=torch.empty((1, K), dtype=torch.int8, device="cuda"),
                          d=torch.empty((1,), dtype=torch.float32, device="cuda"),
                          out_dtype=("bf16", "f32", "i32")[i % 3]))
    grp = bl.NormDecodeGroup(probs, xd, gd, eps, residual=rd, h_out=hd)
    ys = grp()
    h_ref, q_ref, d_ref = oracle.rmsnorm_quant(x, r, g, eps)
    # the unfused path: fused norm kernel, then the GEMV over its codes
    h2, q2, d2 = bl.rmsnorm_quant(xd, gd, eps, residual=rd)
    torch.cuda.synchronize()
    if res:
        assert np.array_equal(host(hd), h_ref)
    for p, y, t in zip(grp.problems, ys, ts):
        ot = p["out_dtype"]
        assert np.array_equal(host(p["q"]), q_ref)
        assert host(p["d"]).view(np.uint32)[0] == d_ref.view(np.uint32)[0]
        acc = oracle.mpgemm_acc(q_ref, t)
        kw = {"i32": "y_i32", "f32": "y_f32", "bf16": "y_bf16"}[ot]
        check_outputs(acc, GAMMA, d_ref, **{kw: host(y)})
        y2 = bl.gemv(p["packed"], p["gamma"], q2, d2, out_dtype=ot)
        torch.cuda.synchronize()
        assert np.array_equal(host(y2).view(np.uint8), host(y).view(np.uint8))


def test_decode_norm_group_graph_replay():
    """Graph replays of the fused norm decode give the eager result every time."""
    bl = _bl()
    K = 2560
    say("decode_norm_group graph replay")
    x, r, g = W.norm_inputs(1300, 1, K)
    t = W.ternary_drawn(1301, 640, K, 0.4)
    grp = bl.NormDecodeGroup([dict(packed=bl.pack_i2s(dev(t)),
                                   gamma=dev(np.array([GAMMA], np.float32)))],
                             dev_bf16(x), dev_bf16(g), 1e-5, residual=dev_bf16(r))
    ref = host(grp()[0]).copy()
    s = torch.cuda.Stream()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=s):
        grp()
    for _ in range(3):
        grp.outputs[0].zero_()
        gr.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(grp.outputs[0]), ref)


def test_decode_group_tokens_long_k():
    """Several tokens (quantize launch + GEMV over the codes) at the largest K."""
    bl = _bl()
    _decode_group_case(bl, 2, [(3, 65536), (40, 64)], seed=79, out_types=["i32", "bf16"])
    _decode_group_case(bl, 16, [(17, 28672)], seed=80, out_types=["f32"])


def test_decode_group_two_row_tiles():
    """5..16 tokens in launches with at least 256 blocks of 32 rows: each wave
    of the code GEMV takes two row tiles (ragged last tiles, a small problem
    inside a large group)."""
    bl = _bl()
    _decode_group_case(bl, 16, [(8200, 1024), (600, 2048)], seed=120, out_types=["bf16", "i32"])
    _decode_group_case(bl, 5, [(8193, 4096)], seed=121, out_types=["f32"])
    _decode_group_case(bl, 12, [(4100, 3072), (4100, 3072), (31, 3072)], seed=122)


@pytest.mark.parametrize("pad", [8, 4])
def test_decode_group_tokens_strided_x(pad):
    """2..4 tokens with x rows further apart than K: a row stride that keeps
    every row 16-byte aligned (pad 8) quantizes in the GEMV launch, pad 4 takes
    the quantize launch + code GEMV; both against the oracle and the unfused
    calls."""
    bl = _bl()
    for M, shapes, seed in ((3, [(100, 320), (640, 2560), (33, 6912)], 110),
                            (4, [(2560, 2560), (7, 27648)], 111)):
        say(f"decode_group strided x M={M} pad={pad} shapes={shapes}")
        probs, refs = [], []
        for i, (N, K) in enumerate(shapes):
            x = W.activations_bf16(seed + 10 * i, M, K, outlier_frac=0.01, outlier_scale=20.0)
            wide = np.zeros((M, K + pad), dtype=x.dtype)
            wide[:, :K] = x
            wide[:, K:] = x[:, :pad]                        # junk past K must be ignored
            xd = dev_bf16(wide)[:, :K]
            t = W.ternary_drawn(seed + 10 * i + 1, N, K, 0.4)
            probs.append(dict(packed=bl.pack_i2s(dev(t)), gamma=dev(np.array([GAMMA], np.float32)),
                              x=xd, out_dtype="f32",
                              q=torch.empty((M, K), dtype=torch.int8, device="cuda"),
                              d=torch.empty((M,), dtype=torch.float32, device="cuda")))
            refs.append((x, t))
        ys = bl.DecodeGroup(probs)()
        torch.cuda.synchronize()
        for p, y, (x, t) in zip(probs, ys, refs):
            q_ref, d_ref = oracle.quantize_act_absmax(x)
            assert np.array_equal(host(p["q"]), q_ref)
            assert np.array_equal(host(p["d"]).view(np.uint32), d_ref.view(np.uint32))
            check_outputs(oracle.mpgemm_acc(q_ref, t), GAMMA, d_ref, y_f32=host(y))


def test_decode_group_chunked_k_and_no_qd():
    """K larger than one LDS chunk (several chunks per block), q/d not requested."""
    bl = _bl()
    _decode_group_case(bl, 16, [(300, 11008), (64, 4096)], seed=60)
    _decode_group_case(bl, 4, [(130, 28672)], seed=61, with_qd=False)
    _decode_group_case(bl, 1, [(17, 28672), (8, 64), (1, 128)], seed=62, out_types=["f32"])


def test_decode_group_repeat_and_graph():
    """Repeated calls and HIP-graph replays give the eager result every time."""
    bl = _bl()
    grp = _decode_group_case(bl, 1, [(2560, 2560), (640, 2560)], seed=63)
    ref = [host(y).copy() for y in grp.outputs]
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        grp()
    for _ in range(3):
        for y in grp.outputs:
            y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for y, r in zip(grp.outputs, ref):
            assert np.array_equal(host(y), r)


def test_config2_layer_decode_groups():
    """BitNet-2B-like layer at batch 1 through the fused decode groups of a real
    decoder layer: {q, k, v}, {o}, {gate, up}, {down}."""
    bl = _bl()
    cfg = W.LAYERS[2]
    groups = [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)]
    by_name = {p.name: p for p in cfg.projs}
    for names in groups:
        probs, refs = [], []
        for nm in names:
            inp = W.proj_inputs(cfg, by_name[nm], 1)
            probs.append(dict(packed=bl.pack_i2s(dev(inp.w_tern)),
                              gamma=dev(np.array([inp.gamma], np.float32)),
                              x=dev_bf16(inp.x_bf16), out_dtype="bf16"))
            refs.append(inp)
        say(f"config 2 decode group {names}")
        ys = bl.decode_group(probs)
        torch.cuda.synchronize()
        for y, inp in zip(ys, refs):
            q_ref, d_ref = oracle.quantize_act_absmax(inp.x_bf16)
            acc = oracle.mpgemm_acc(q_ref, inp.w_tern)
            check_outputs(acc, np.float32(inp.gamma), d_ref, y_bf16=host(y))


# ---------------------------------------------------------------------------
# full pipelines at the layer shapes
# ---------------------------------------------------------------------------

def _pipeline(bl, cfg, proj, M, p_zero_override=None, sample=None):
    """x -> quantize -> (pack) -> gemv/gemm, each stage checked against the oracle."""
    inp = W.proj_inputs(cfg, proj, M, p_zero_override=p_zero_override)
    say(f"config {cfg.cid} {proj.name} M={M} K={proj.K} N={proj.N}")
    q_ref, d_ref = oracle.quantize_act_absmax(inp.x_bf16)
    q, d = bl.quantize_act(dev_bf16(inp.x_bf16))
    if inp.w_f32 is not None:
        t_ref, g_ref = oracle.ternarize_absmean(inp.w_f32)
        packed, gd = bl.pack_i2s(dev(inp.w_f32))
    else:
        t_ref, g_ref = inp.w_tern, np.float32(inp.gamma)
        packed = bl.pack_i2s(dev(inp.w_tern))
        gd = dev(np.array([g_ref], np.float32))
    fn = bl.gemv if M <= 16 else bl.gemm
    y = fn(packed, gd, q, d, out_dtype="bf16")
    y32 = fn(packed, gd, q, d, out_dtype="f32")
    torch.cuda.synchronize()
    assert np.array_equal(host(q), q_ref)
    assert np.array_equal(host(d).view(np.uint32), d_ref.view(np.uint32))
    if inp.w_f32 is not None:
        assert host(gd).view(np.uint32)[0] == np.float32(g_ref).view(np.uint32)
        assert np.array_equal(host(packed), oracle.pack_i2s(t_ref))
    if sample is None:
        acc = oracle.mpgemm_acc(q_ref, t_ref) if M * proj.N * proj.K < 4e8 else \
            oracle.mpgemm_acc_f64blas(q_ref, t_ref)
        check_outputs(acc, g_ref, d_ref, None, host(y32), host(y))
    else:
        r = W.rng(sample)
        rows = np.concatenate([r.integers(0, M, 256), [0, M - 1]])
        cols = np.concatenate([r.integers(0, proj.N, 256), [proj.N - 1, 0]])
        acc = oracle.mpgemm_acc_entries(q_ref, t_ref, rows, cols)
        check_outputs(acc, g_ref, d_ref, None, host(y32), host(y), rows=rows, cols=cols)
        # two full tokens and two full output features
        yb = host(y32)
        for tok in (0, M // 2):
            acc_row = oracle.mpgemm_acc(q_ref[tok:tok + 1], t_ref)
            check_outputs(acc_row, g_ref, d_ref[tok:tok + 1], None, yb[tok:tok + 1])
        for n in (1, proj.N // 3):
            acc_col = oracle.mpgemm_acc(q_ref, t_ref[n:n + 1])
            check_outputs(acc_col, g_ref, d_ref, None, yb[:, n:n + 1])


@pytest.mark.parametrize("cid,M", [(1, 1), (2, 1), (4, 1), (4, 4), (4, 16), (3, 512)])
def test_layer_configs(cid, M):
    bl = _bl()
    cfg = W.LAYERS[cid]
    for proj in cfg.projs:
        _pipeline(bl, cfg, proj, M)


def test_config4_sparse_variant():
    """7B layer with ternary weights drawn at P(0) = 0.65."""
    bl = _bl()
    cfg = W.LAYERS[4]
    for proj in cfg.projs:
        _pipeline(bl, cfg, proj, 1, p_zero_override=0.65)


def test_config5_grouped_sampled():
    """100B-class layer at 2048 tokens through bl_gemm_group: {q, k, v} and
    {gate, up} share one quantized input; sampled entries against the oracle,
    full outputs equal to the per-projection bl_gemm."""
    bl = _bl()
    cfg = W.LAYERS[5]
    by = {p.name: p for p in cfg.projs}
    for names in (("q", "k", "v"), ("gate", "up")):
        K = by[names[0]].K
        inps = [W.proj_inputs(cfg, by[n], 2048) for n in names]
        x = inps[0].x_bf16
        say(f"config 5 group {names} K={K}")
        q_ref, d_ref = oracle.quantize_act_absmax(x)
        # the benchmark's form: token sums from the quantizer, offset weights
        q, d, qs = bl.quantize_act(dev_bf16(x), with_sums=True)
        probs = []
        for inp in inps:
            probs.append(dict(packed=bl.pack_i2s(dev(inp.w_tern)),
                              gamma=dev(np.array([inp.gamma], np.float32)), out_dtype="f32"))
        ys = bl.gemm_group(probs, q, d, qsum=qs)
        torch.cuda.synchronize()
        assert np.array_equal(host(q), q_ref)
        assert np.array_equal(host(qs), oracle.token_sums(q_ref))
        for n, inp, pr, y in zip(names, inps, probs, ys):
            y1 = bl.gemm(pr["packed"], pr["gamma"], q, d, out_dtype="f32")
            assert torch.equal(y, y1), n
            r = W.rng(6000 + by[n].index)
            rows = np.concatenate([r.integers(0, 2048, 256), [0, 2047]])
            cols = np.concatenate([r.integers(0, by[n].N, 256), [by[n].N - 1, 0]])
            acc = oracle.mpgemm_acc_entries(q_ref, inp.w_tern, rows, cols)
            check_outputs(acc, np.float32(inp.gamma), d_ref, None, host(y), rows=rows, cols=cols)
            del y1


def test_config5_sampled():
    """100B-class layer at 2048 tokens: every stage at full size; the GEMM checked
    on sampled entries, two full tokens and two full output features."""
    bl = _bl()
    cfg = W.LAYERS[5]
    for proj in cfg.projs:
        _pipeline(bl, cfg, proj, 2048, sample=5000 + proj.index)
