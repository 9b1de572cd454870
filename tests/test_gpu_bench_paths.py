"""GPU parity of exactly the launches bench.py times, at its shapes: the
bench's own builders make the launches (decode groups of the layer, grouped
GEMMs over one quantized input with token sums), and every output element is
compared with the oracle on the same seeded inputs.

Bar (as in test_gpu_parity): the int32 accumulators bit-exact, bf16 outputs
bit-exact to the round-to-nearest-even of the fp32 epilogue
fl32(fl32(acc) * fl32(gamma * d)) and within 1 bf16 ulp of the fp64 value.
Large contractions use the oracle's fp64-BLAS sum, exact because every
partial sum is an integer below 2^53; it is pinned against the int64 sum on
the CPU (tests/pins.py)."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from test_gpu_parity import _bl, check_outputs, dev, host, say

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

pytestmark = pytest.mark.gpu


def _acc(q, t):
    """Exact accumulators, by column blocks of the weights (bounded memory)."""
    out = np.empty((q.shape[0], t.shape[0]), dtype=np.int64)
    step = max(1, (1 << 25) // max(1, t.shape[1]))
    for n0 in range(0, t.shape[0], step):
        out[:, n0:n0 + step] = oracle.mpgemm_acc_f64blas(q, t[n0:n0 + step])
    return out


def _check_cols(acc, gamma, d, y_bf16=None, y_i32=None, step=4096):
    for n0 in range(0, acc.shape[1], step):
        sl = slice(n0, n0 + step)
        check_outputs(acc[:, sl], gamma, d,
                      y_i32=None if y_i32 is None else y_i32[:, sl],
                      y_bf16=None if y_bf16 is None else y_bf16[:, sl])


_WREF = {}


def _weights_ref(cfg, proj, p_zero_override=None):
    """The oracle's ternary weights and gamma of one projection (cached: the
    7B-class layer's absmean ternarization takes seconds on the host)."""
    key = (cfg.cid, proj.name, p_zero_override)
    if key not in _WREF:
        _WREF[key] = _weights_ref_uncached(cfg, proj, p_zero_override)
    return _WREF[key]


def _weights_ref_uncached(cfg, proj, p_zero_override):
    inp = W.proj_inputs(cfg, proj, 1, with_acts=False, p_zero_override=p_zero_override)
    if inp.w_f32 is not None:
        t, g = oracle.ternarize_absmean(inp.w_f32)
        return t, np.float32(g)
    return inp.w_tern, np.float32(inp.gamma)


def _decode_layer(cid, M, p_zero_override=None):
    """One layer copy of the bench's decode stream (bench.decode_layers with
    R = 1): the four fused launches run in layer order, then every projection's
    bf16 output is checked in full; packed bytes and gamma against the
    oracle's ternarization."""
    bl = _bl()
    cfg = W.LAYERS[cid]
    say(f"bench decode path: {cfg.name} M={M} p_zero={p_zero_override}")
    layers, ys = bench.decode_layers(torch, bl, W, torch.device("cuda", 0), cfg, M, R=1,
                                     p_zero_override=p_zero_override)
    for f in layers[0]:
        f()
    torch.cuda.synchronize()
    probs = [p for launch in layers[0] for p in launch.problems]
    for proj in cfg.projs:
        t_ref, g_ref = _weights_ref(cfg, proj, p_zero_override)
        x = W.activations_bf16(W.seed_for(cid, proj.index, 1), M, proj.K,
                               cfg.outlier_frac, cfg.outlier_scale)
        q_ref, d_ref = oracle.quantize_act_absmax(x)
        p = next(pp for pp in probs if pp["y"] is ys[proj.name])
        assert host(p["gamma"]).view(np.uint32)[0] == g_ref.view(np.uint32), proj.name
        assert np.array_equal(host(p["packed"]), oracle.pack_i2s(t_ref)), proj.name
        if M > 1:                       # the codes the launch staged (or wrote) for the GEMV
            assert np.array_equal(host(p["q"]), q_ref), proj.name
            assert np.array_equal(host(p["d"]).view(np.uint32), d_ref.view(np.uint32)), proj.name
        _check_cols(_acc(q_ref, t_ref), g_ref, d_ref, y_bf16=host(ys[proj.name]))


@pytest.mark.parametrize("M", [1, 4, 16])
def test_config4_decode_stream_path(M):
    _decode_layer(4, M)


def test_config4_sparse_decode_stream_path():
    _decode_layer(4, 1, p_zero_override=0.65)


def test_config2_decode_stream_path():
    _decode_layer(2, 1)


def test_config1_gemv_path():
    """The 1024 x 1024 GEMV as bench.single_gemv_workload launches it."""
    bl = _bl()
    cfg = W.LAYERS[1]
    proj = cfg.projs[0]
    inp = W.proj_inputs(cfg, proj, 1)
    packed, gamma = bl.pack_i2s(dev(inp.w_f32))
    y = torch.empty((1, proj.N), dtype=torch.bfloat16, device="cuda")
    bl.DecodeGroup([dict(packed=packed, gamma=gamma, x=dev(inp.x_bf16.view(np.int16)).view(torch.bfloat16),
                         y=y)])()
    torch.cuda.synchronize()
    t_ref, g_ref = oracle.ternarize_absmean(inp.w_f32)
    q_ref, d_ref = oracle.quantize_act_absmax(inp.x_bf16)
    assert host(gamma).view(np.uint32)[0] == np.float32(g_ref).view(np.uint32)
    check_outputs(oracle.mpgemm_acc(q_ref, t_ref), np.float32(g_ref), d_ref, y_bf16=host(y))


def _prefill_group(cid, M, names):
    """One group of the bench's prefill layer (bench.build_prefill):
    bl_quantize_act with token sums, then bl_gemm_group on offset weights;
    codes, scales and token sums bit-exact, every bf16 output and (from the
    same launch configuration with int32 outputs) every accumulator."""
    bl = _bl()
    cfg = W.LAYERS[cid]
    say(f"bench prefill path: {cfg.name} M={M} group={names}")
    _, _, G = bench.build_prefill(torch, bl, W, torch.device("cuda", 0), cid=cid, M=M,
                                  groups=(names,))
    e = G[0]
    bl.quantize_act(e["x"], e["q"], e["d"], qsum=e["qs"])
    e["group"]()
    acc_grp = bl.GemmGroup([dict(p, y=None, out_dtype="i32") for p in e["group"].problems],
                           e["q"], e["d"], qsum=e["qs"])
    acc_outs = acc_grp()
    torch.cuda.synchronize()
    by = {p.name: p for p in cfg.projs}
    x = W.proj_inputs(cfg, by[names[0]], M).x_bf16
    q_ref, d_ref = oracle.quantize_act_absmax(x)
    assert np.array_equal(host(e["q"]), q_ref)
    assert np.array_equal(host(e["d"]).view(np.uint32), d_ref.view(np.uint32))
    assert np.array_equal(host(e["qs"]), oracle.token_sums(q_ref))
    for n, p, a in zip(names, e["group"].problems, acc_outs):
        t_ref, g_ref = _weights_ref(cfg, by[n])
        acc = _acc(q_ref, t_ref)
        _check_cols(acc, g_ref, d_ref, y_bf16=host(p["y"]), y_i32=host(a))
        del acc
    del G, acc_grp, acc_outs
    torch.cuda.empty_cache()


@pytest.mark.parametrize("names", W.LAYER_GROUPS, ids=["+".join(g) for g in W.LAYER_GROUPS])
def test_config3_prefill_path(names):
    _prefill_group(3, 512, names)


@pytest.mark.parametrize("names", W.LAYER_GROUPS, ids=["+".join(g) for g in W.LAYER_GROUPS])
def test_config5_prefill_path(names):
    """The 100B-class layer at 2048 tokens, every element of every projection."""
    _prefill_group(5, 2048, names)
