"""Benchmark of the ternary BitLinear hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

Headline (the JSON `value`): decode GEMV packed-weight GB/s on a stream of 32
distinct 7B-class layers (hidden 4096, FFN 11008, 32 heads; ternary weights
from fp32 N(0, 0.02) by the absmean rule) at batch 1. One step = one layer:
for each of its 7 projections (q, k, v, o, gate, up, down) the per-token
absmax int8 quantization of the bf16 input and the I2_S GEMV with the bf16
dequant fused into the store, issued as one fused launch per group of
projections that do not depend on each other in a decoder layer: {q,k,v},
{o}, {gate,up}, {down}. Step i runs layer copy i mod 32 (32 * 50.6 MB =
1.62 GB, six times the 256 MB Infinity Cache), so every step streams its
weights from HBM, as decoding one token through a 32-layer model does.
Weight packing is the offline conversion and is done before timing; inputs
are resident in HBM. Exactly --steps steps are timed: the --warmup steps and
then the --steps steps are each captured into one HIP graph (the rotation
continues across them) and replayed once, between two synchronizations.

Also on the same JSON line:
  roofline       the fused one-token decode kernels of that step: packed bytes
                 per launch over the mean launch interval of the timed steps
                 (HIP events on the replay stream), against 8 TB/s; `traffic`
                 from rocprofv3 counters while the kernel sources are unchanged;
  roofline_gemm  the prefill GEMM (k_gemm_i2s) on the 100B-class layer at 2048
                 tokens, int8 ops per second against 5.0 POP/s;
  configs        every workload: the 1024 x 1024 GEMV, the BitNet-2B-like
                 layer at batch 1 and at 512 tokens, the 7B-class layer at 1,
                 4 and 16 tokens (and with 65% zero weights), the 100B-class
                 layer at 2048 tokens;
  cpu_baseline   the CPU oracle timed per workload on this host, on one core
                 and on all cores (row shards in worker processes), with the
                 GPU / oracle ratio.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_7b_stream_traffic.json")
DECODE_SOURCES = ("mpgemm_token_absmax_amd/csrc/gemv_i2s.hip",
                  "mpgemm_token_absmax_amd/csrc/common.hpp",
                  "mpgemm_token_absmax_amd/csrc/launch.hpp")
ROTATE = 32                       # distinct layer copies of a decode stream


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by a plain-kernel calibration), or
    None when the decode kernels' sources changed since the counters were taken."""
    import hashlib
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        h = hashlib.sha256()
        for rel in DECODE_SOURCES:
            with open(os.path.join(ROOT, rel), "rb") as f:
                h.update(f.read())
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != h.hexdigest():
        return None
    return rec.get("traffic_bytes_per_launch")


# ------------------------------------------------------------- graph helpers

def capture_fns(torch, stream, fns):
    """HIP graph of the given launch callables, captured on `stream`."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for f in fns:
            f()
    return g


def upload_graph(g, stream):
    """hipGraphUpload of an instantiated graph on `stream`, so that its first
    replay (the timed one) does not also do the upload work; a no-op where the
    graph object does not expose its executable."""
    import ctypes
    if g is None or not hasattr(g, "raw_cuda_graph_exec"):
        return
    exe = g.raw_cuda_graph_exec()
    if not exe:
        return
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipGraphUpload.restype = ctypes.c_int
    hip.hipGraphUpload.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    err = hip.hipGraphUpload(ctypes.c_void_p(exe), ctypes.c_void_p(stream.cuda_stream))
    if err != 0:
        log(f"hipGraphUpload returned {err}: the first replay also uploads")


def replay_us(torch, stream, g, units, reps=10):
    """Mean microseconds per unit over `reps` replays of graph g (one warm
    replay first)."""
    with torch.cuda.stream(stream):
        g.replay()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * units)


def time_steps(torch, stream, layers, steps, warmup, spread_reps=None):
    """Exactly `steps` steps timed: layers[r] is the list of launch callables
    of layer copy r; step i runs copy i mod len(layers). The warmup steps and
    the timed steps are captured as two graphs (the rotation continues from
    one to the other) and uploaded, and the timed graph is launched once
    untimed (its first launch carries one-time costs); then the warmup graph
    runs and the timed graph is replayed once between two synchronizations. Returns (ms per step, [p10, p50, p90] us per step over
    further replays of the timed graph each between two synchronizations,
    i.e. measured exactly as the timed one, and the p50 of back-to-back
    replays, where each replay's launch overlaps the previous one's work)."""
    R = len(layers)
    fw = [f for i in range(warmup) for f in layers[i % R]]
    ft = [f for i in range(warmup, warmup + steps) for f in layers[i % R]]
    g_warm = capture_fns(torch, stream, fw) if fw else None
    g_timed = capture_fns(torch, stream, ft)
    for g in (g_warm, g_timed):
        upload_graph(g, stream)
    # The first launch of an instantiated graph carries one-time costs (about
    # 1 us per step at 20 steps, upload or not): the timed graph is launched
    # once, untimed, before the warmup steps. Set-up, like the eager pass that
    # loads the code objects; the warmup steps and the timed steps follow.
    with torch.cuda.stream(stream):
        g_timed.replay()
    torch.cuda.synchronize()

    def one(pre=None):
        with torch.cuda.stream(stream):
            if pre is not None:
                pre.replay()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            g_timed.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms_step = one(g_warm)
    n = spread_reps or max(8, min(64, 2000 // steps))
    # the spread repeats the timed measurement as it is: warmup graph, then
    # the timed graph between two synchronizations (replaying the timed graph
    # alone would let the Infinity Cache keep part of its own working set)
    per = np.array([one(g_warm) * 1e3 for _ in range(n)])
    spread = [round(float(np.percentile(per, q)), 3) for q in (10, 50, 90)]
    marks = []
    with torch.cuda.stream(stream):
        for _ in range(n):
            a0 = torch.cuda.Event(enable_timing=True)
            a1 = torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            g_timed.replay()
            a1.record(stream)
            marks.append((a0, a1))
    torch.cuda.synchronize()
    piped = np.array([x0.elapsed_time(x1) * 1e3 / steps for x0, x1 in marks])
    del g_warm, g_timed
    return ms_step, spread, round(float(np.percentile(piped, 50)), 3)


# ------------------------------------------------------------ decode layers

def to_dev(torch, a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def bf16_dev(torch, bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def packed_layer(torch, bl, W, dev, cfg, p_zero_override=None):
    """{proj: (packed, gamma)} of one layer: fp32 master weights are
    ternarized and packed by bl_pack_i2s (absmean gamma), drawn ternary
    weights packed with the configuration's gamma."""
    out = {}
    for proj in cfg.projs:
        inp = W.proj_inputs(cfg, proj, 1, with_acts=False, p_zero_override=p_zero_override)
        if inp.w_f32 is not None:
            out[proj.name] = bl.pack_i2s(to_dev(torch, inp.w_f32, dev))
        else:
            out[proj.name] = (bl.pack_i2s(to_dev(torch, inp.w_tern, dev)),
                              to_dev(torch, np.array([inp.gamma], np.float32), dev))
        del inp
    return out


def decode_layers(torch, bl, W, dev, cfg, M, R=ROTATE, p_zero_override=None):
    """R distinct copies of a layer's packed weights and, per copy, the fused
    decode launches of W.LAYER_GROUPS over seeded bf16 activations [M][K]
    (one input per projection). Returns (layers, outputs by projection)."""
    base = packed_layer(torch, bl, W, dev, cfg, p_zero_override)
    xs = {p.name: bf16_dev(torch, W.activations_bf16(W.seed_for(cfg.cid, p.index, 1), M, p.K,
                                                     cfg.outlier_frac, cfg.outlier_scale), dev)
          for p in cfg.projs}
    ys = {p.name: torch.empty((M, p.N), dtype=torch.bfloat16, device=dev) for p in cfg.projs}
    layers = []
    for r in range(R):
        launches = []
        for names in W.LAYER_GROUPS:
            probs = [dict(packed=base[n][0] if r == 0 else base[n][0].clone(), gamma=base[n][1],
                          x=xs[n], y=ys[n]) for n in names]
            launches.append(bl.DecodeGroup(probs))
        layers.append(launches)
    torch.cuda.synchronize()
    return layers, ys


def stream_floors(torch, dev, stream, R, groups):
    """Floors of a decode launch on this machine with the measurement aids of
    libblprobe.so, in the same setting as the decode step (graph replays over
    R cold buffer copies): an empty kernel, a streaming read of each group's
    packed bytes by as many 256-thread blocks as its decode launch has 16-row
    tiles, and a 1 GiB streaming read (practical HBM peak)."""
    import ctypes
    probe = ctypes.CDLL(os.path.join(ROOT, "mpgemm_token_absmax_amd", "libblprobe.so"))
    probe.blp_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                      ctypes.c_void_p, ctypes.c_void_p]
    probe.blp_empty.argtypes = [ctypes.c_int, ctypes.c_void_p]
    sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)

    def read(buf, nbytes, blocks):
        def f():
            rc = probe.blp_stream_read(buf.data_ptr(), nbytes, blocks, sink.data_ptr(),
                                       torch.cuda.current_stream().cuda_stream)
            if rc:
                raise RuntimeError(f"blp_stream_read failed ({rc})")
        return f

    def empty():
        if probe.blp_empty(160, torch.cuda.current_stream().cuda_stream):
            raise RuntimeError("blp_empty failed")

    out = {}
    g = capture_fns(torch, stream, [empty] * 128)
    out["empty_launch_us"] = round(replay_us(torch, stream, g, 128), 3)
    stream_us = {}
    for names, nbytes, blocks in groups:
        bufs = [torch.ones(nbytes, dtype=torch.uint8, device=dev) for _ in range(R)]
        g = capture_fns(torch, stream, [read(b, nbytes, blocks) for b in bufs])
        stream_us["+".join(names)] = round(replay_us(torch, stream, g, R), 3)
        del g, bufs
    out["stream_read_us"] = stream_us
    total = sum(nb for _, nb, _ in groups)
    out["layer_floor_us"] = round(sum(stream_us.values()), 3)
    out["layer_floor_gbs"] = round(total / (out["layer_floor_us"] * 1e-6) / 1e9, 1)
    big = 1 << 30
    bufs = [torch.ones(big, dtype=torch.uint8, device=dev) for _ in range(2)]
    g = capture_fns(torch, stream, [read(b, big, 2048) for b in bufs])
    out["practical_peak_gbs"] = round(big / (replay_us(torch, stream, g, 2, reps=5) * 1e-6) / 1e9,
                                      1)
    del g, bufs
    torch.cuda.empty_cache()
    return out


def decode_workload(torch, bl, W, dev, stream, cid, M, p_zero_override=None):
    """A decode stream over ROTATE layer copies (graph replays): microseconds
    per layer and packed GB/s."""
    cfg = W.LAYERS[cid]
    layers, _ = decode_layers(torch, bl, W, dev, cfg, M, p_zero_override=p_zero_override)
    for f in layers[0]:
        f()
    g = capture_fns(torch, stream, [f for layer in layers for f in layer])
    us = replay_us(torch, stream, g, len(layers), reps=10)
    del g, layers
    torch.cuda.empty_cache()
    return {"workload": cfg.name, "tokens": M, "us_per_layer": round(us, 3),
            "packed_bytes": cfg.packed_bytes,
            "gbs": round(cfg.packed_bytes / (us * 1e-6) / 1e9, 1),
            "hbm_frac": round(cfg.packed_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "launches_per_layer": len(W.LAYER_GROUPS), "layer_copies": ROTATE}


def single_gemv_workload(torch, bl, W, dev, stream):
    """The 1024 x 1024 BitLinear GEMV at batch 1 (fp32 N(0, 0.02) weights,
    absmean-ternarized), one fused decode launch per call, rotating over 2048
    weight copies (537 MB, twice the Infinity Cache) so every call reads from
    HBM; and the same launch on one copy (L2-resident weights)."""
    cfg = W.LAYERS[1]
    proj = cfg.projs[0]
    inp = W.proj_inputs(cfg, proj, 1)
    packed, gamma = bl.pack_i2s(to_dev(torch, inp.w_f32, dev))
    x = bf16_dev(torch, inp.x_bf16, dev)
    y = torch.empty((1, proj.N), dtype=torch.bfloat16, device=dev)
    R = 2048
    copies = [packed] + [packed.clone() for _ in range(R - 1)]
    fns = [bl.DecodeGroup([dict(packed=c, gamma=gamma, x=x, y=y)]) for c in copies]
    fns[0]()
    g = capture_fns(torch, stream, fns)
    us = replay_us(torch, stream, g, R, reps=5)
    del g
    g = capture_fns(torch, stream, [fns[0]] * 256)
    us_warm = replay_us(torch, stream, g, 256, reps=10)
    del g, fns, copies
    torch.cuda.empty_cache()
    nbytes = proj.N * proj.K // 4
    return {"workload": cfg.name, "tokens": 1, "us_per_call": round(us, 3),
            "packed_bytes": nbytes, "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "warm_us_per_call": round(us_warm, 3), "weight_copies": R}


def one_token_gemv_100b(torch, bl, dev, stream):
    """One-token GEMVs of the 100B-class shapes (one fused launch each,
    rotating copies), and next to each a streaming read of the same bytes
    (libblprobe.so) by as many threads, in the same setting."""
    import ctypes
    probe = ctypes.CDLL(os.path.join(ROOT, "mpgemm_token_absmax_amd", "libblprobe.so"))
    probe.blp_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                      ctypes.c_void_p, ctypes.c_void_p]
    sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)

    def stream_read(buf, nbytes, blocks):
        def f():
            rc = probe.blp_stream_read(buf.data_ptr(), nbytes, blocks, sink.data_ptr(),
                                       torch.cuda.current_stream().cuda_stream)
            if rc:
                raise RuntimeError(f"blp_stream_read failed ({rc})")
        return f

    out = {}
    gen = torch.Generator(device=dev).manual_seed(2048)
    for N, K in ((28672, 8192), (8192, 28672)):
        t = torch.randint(-1, 2, (N, K), dtype=torch.int8, device=dev, generator=gen)
        x = torch.randn(1, K, device=dev, generator=gen).to(torch.bfloat16)
        gam = torch.tensor([0.01], device=dev)
        R = 8
        launches = [bl.DecodeGroup([dict(packed=bl.pack_i2s(t), gamma=gam, x=x)]) for _ in range(R)]
        del t
        launches[0]()
        g = capture_fns(torch, stream, launches)
        us = replay_us(torch, stream, g, R, reps=10)
        del g
        nbytes = N * K // 4
        blocks = (N + 15) // 16 * (2 if K > 16384 else 1)
        bufs = [c.problems[0]["packed"] for c in launches]
        g = capture_fns(torch, stream, [stream_read(b, nbytes, blocks) for b in bufs])
        floor = replay_us(torch, stream, g, R, reps=10)
        out[f"N{N}_K{K}"] = {"us": round(us, 3), "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
                             "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                             "stream_floor_us": round(floor, 3),
                             "frac_of_floor": round(floor / us, 3)}
        del g, launches, bufs
        torch.cuda.empty_cache()
    return out


def norm_layer_bench(torch, bl, W, dev, stream):
    """The BitNet-2B-like decode layer (batch 1) with its two RMSNorms before
    {q,k,v} and {gate,up} (residual add included): fused, 4 launches (two
    bl_decode_norm_group, two bl_decode_group), against unfused, 9 launches
    (bl_rmsnorm_quant, then one bl_gemv per projection of the normed input).
    32 rotating layer copies, graph replays; us per layer and packed GB/s."""
    cfg = W.LAYERS[2]
    by = {p.name: p for p in cfg.projs}
    K = 2560
    t = lambda a: bf16_dev(torch, a, dev)
    x1, r1, g1 = W.norm_inputs(2001, 1, K, cfg.outlier_frac, cfg.outlier_scale)
    x2, r2, g2 = W.norm_inputs(2002, 1, K, cfg.outlier_frac, cfg.outlier_scale)
    xo = W.activations_bf16(2003, 1, K, cfg.outlier_frac, cfg.outlier_scale)
    xd = W.activations_bf16(2004, 1, 6912, cfg.outlier_frac, cfg.outlier_scale)
    X1, R1, G1, X2, R2, G2, XO, XD = (t(a) for a in (x1, r1, g1, x2, r2, g2, xo, xd))
    H1, H2 = torch.empty_like(X1), torch.empty_like(X2)
    gam = torch.tensor([W.GAMMA_DRAWN], dtype=torch.float32, device=dev)
    base = {n: bl.pack_i2s(to_dev(torch, W.proj_inputs(cfg, by[n], 1, with_acts=False).w_tern, dev))
            for n in by}
    R = ROTATE
    copies = [{n: (p if r == 0 else p.clone()) for n, p in base.items()} for r in range(R)]
    fused, unfused = [], []
    q1 = torch.empty((1, K), dtype=torch.int8, device=dev)
    d1 = torch.empty((1,), dtype=torch.float32, device=dev)
    q2, d2 = torch.empty_like(q1), torch.empty_like(d1)
    for c in copies:
        prob = lambda n: dict(packed=c[n], gamma=gam)
        fused += [bl.NormDecodeGroup([prob("q"), prob("k"), prob("v")], X1, G1, 1e-5, residual=R1, h_out=H1),
                  bl.DecodeGroup([dict(prob("o"), x=XO)]),
                  bl.NormDecodeGroup([prob("gate"), prob("up")], X2, G2, 1e-5, residual=R2, h_out=H2),
                  bl.DecodeGroup([dict(prob("down"), x=XD)])]
        ys = {n: torch.empty((1, by[n].N), dtype=torch.bfloat16, device=dev) for n in by}
        unfused += [(lambda: bl.rmsnorm_quant(X1, G1, 1e-5, residual=R1, h_out=H1, q=q1, d=d1))]
        unfused += [(lambda c=c, n=n, ys=ys: bl.gemv(c[n], gam, q1, d1, out=ys[n])) for n in ("q", "k", "v")]
        unfused += [bl.DecodeGroup([dict(prob("o"), x=XO)])]
        unfused += [(lambda: bl.rmsnorm_quant(X2, G2, 1e-5, residual=R2, h_out=H2, q=q2, d=d2))]
        unfused += [(lambda c=c, n=n, ys=ys: bl.gemv(c[n], gam, q2, d2, out=ys[n])) for n in ("gate", "up")]
        unfused += [bl.DecodeGroup([dict(prob("down"), x=XD)])]
    out = {"layer": cfg.name, "packed_bytes": cfg.packed_bytes}
    for name, fns in (("fused_4_launches", fused), ("unfused_9_launches", unfused)):
        for f in fns[:9]:
            f()
        g = capture_fns(torch, stream, fns)
        us = replay_us(torch, stream, g, R, reps=10)
        out[name] = {"us_per_layer": round(us, 3), "gbs": round(cfg.packed_bytes / (us * 1e-6) / 1e9, 1)}
        del g
    del copies, fused, unfused
    torch.cuda.empty_cache()
    return out


def t3_bench(torch, bl, W, dev, stream):
    """Base-3 weights (five per byte, 1.6 bits per weight) against I2_S (2 bits
    per weight), one token, through the fused one-token decode (bf16 x in,
    quantize in the kernel): bl_decode_group_t3 against bl_decode_group, graph
    replays over copies of the packed weights (>= 700 MB), microseconds per
    call, GB/s of packed bytes and billions of weights per second."""
    out = {}
    for N, K in ((2560, 2560), (6912, 2560), (28672, 8192), (8192, 28672)):
        t = to_dev(torch, W.ternary_drawn(7 + N + K, N, K, 1.0 / 3.0), dev)
        p2, p3 = bl.pack_i2s(t), bl.pack_t3(t)
        del t
        xb = bf16_dev(torch, W.activations_bf16(9 + K, 1, K, 0.005, 50.0), dev)
        gam = torch.tensor([W.GAMMA_DRAWN], dtype=torch.float32, device=dev)
        R = max(2, -(-700_000_000 // p3.numel()))
        y = torch.empty((1, N), dtype=torch.bfloat16, device=dev)
        rec = {}
        for name, p, fn in (("i2s_fused", p2, bl.DecodeGroup), ("t3_fused", p3, bl.DecodeGroupT3)):
            copies = [p] + [p.clone() for _ in range(R - 1)]
            fns = [fn([dict(packed=c, gamma=gam, x=xb, y=y)]) for c in copies]
            fns[0]()
            g = capture_fns(torch, stream, fns)
            us = replay_us(torch, stream, g, R, reps=10)
            rec[name] = {"us": round(us, 3), "packed_bytes": p.numel(),
                         "gbs": round(p.numel() / (us * 1e-6) / 1e9, 1),
                         "gweights_s": round(N * K / (us * 1e-6) / 1e9, 1)}
            del g, copies, fns
        out[f"N{N}_K{K}"] = rec
        del p2, p3
        torch.cuda.empty_cache()
    return out


def norm_bench(torch, bl, W, dev, stream):
    """Fused residual add + RMSNorm + per-token quantize (bl_rmsnorm_quant)
    on the prefill and decode shapes, against the same step done unfused
    (torch bf16 add, torch rms_norm, bl_quantize_act). Each figure is a graph
    replay over R copies of the buffers (about 600 MB in all, so the data come
    from HBM). Algorithmic bytes per token: x, r and h (2K each) plus q (K)
    plus d (4); g once (2K)."""
    out = {}
    for name, cid, M in (("100b-prefill-2048", 5, 2048), ("2b-prefill-512", 3, 512),
                         ("100b-decode-1", 5, 1), ("2b-decode-1", 3, 1)):
        cfg = W.LAYERS[cid]
        K = cfg.projs[0].K
        xb, rb, gb = W.norm_inputs(4242 + cid, M, K, cfg.outlier_frac, cfg.outlier_scale)
        g = bf16_dev(torch, gb, dev)
        nbytes = M * (7 * K + 4) + 2 * K
        R = max(1, min(64, -(-600_000_000 // nbytes)))
        bufs = [dict(x=bf16_dev(torch, xb, dev), r=bf16_dev(torch, rb, dev),
                     h=torch.empty((M, K), dtype=torch.bfloat16, device=dev),
                     q=torch.empty((M, K), dtype=torch.int8, device=dev),
                     d=torch.empty((M,), dtype=torch.float32, device=dev)) for _ in range(R)]

        def fused(b):
            return lambda: bl.rmsnorm_quant(b["x"], g, 1e-5, residual=b["r"], h_out=b["h"],
                                            q=b["q"], d=b["d"])

        def unfused(b):
            def f():
                hh = b["x"] + b["r"]
                y = torch.nn.functional.rms_norm(hh, (K,), weight=g, eps=1e-5)
                bl.quantize_act(y, b["q"], b["d"])
            return f

        gr = capture_fns(torch, stream, [fused(b) for b in bufs])
        us = replay_us(torch, stream, gr, R)
        del gr
        gr = capture_fns(torch, stream, [unfused(b) for b in bufs])
        us_unf = replay_us(torch, stream, gr, R)
        del gr, bufs
        half = nbytes // 2
        cbufs = [(torch.empty(half, dtype=torch.uint8, device=dev),
                  torch.ones(half, dtype=torch.uint8, device=dev)) for _ in range(R)]
        gr = capture_fns(torch, stream, [(lambda a=a, b=b: a.copy_(b)) for a, b in cbufs])
        us_copy = replay_us(torch, stream, gr, R)
        del gr, cbufs
        torch.cuda.empty_cache()
        gbs = nbytes / (us * 1e-6) / 1e9
        out[name] = {"M": M, "K": K, "us": round(us, 3), "gbs": round(gbs, 1),
                     "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "bytes": nbytes,
                     "unfused_us": round(us_unf, 3), "copy_floor_us": round(us_copy, 3),
                     "copies": R}
    return out


# ------------------------------------------------------------------ prefill

def build_prefill(torch, bl, W, dev, cid=5, M=2048, groups=None):
    """A prefill layer (by default the 100B-class layer at 2048 tokens): one
    bf16 input per group of W.LAYER_GROUPS (or of `groups`); each group's
    GEMMs run through one bl_gemm_group call on its quantized codes. The
    quantizer also writes the token sums and `group` takes them (offset
    weights); `plain` is the same group without them."""
    cfg = W.LAYERS[cid]
    log(f"setup prefill: {cfg.name}")
    by = {proj.name: proj for proj in cfg.projs}
    G = []
    for names in (groups or W.LAYER_GROUPS):
        inps = [W.proj_inputs(cfg, by[n], M) for n in names]
        K = by[names[0]].K
        x = bf16_dev(torch, inps[0].x_bf16, dev)
        q = torch.empty((M, K), dtype=torch.int8, device=dev)
        d = torch.empty((M,), dtype=torch.float32, device=dev)
        qs = torch.empty((M,), dtype=torch.int32, device=dev)
        probs = [dict(packed=bl.pack_i2s(to_dev(torch, inp.w_tern, dev)),
                      gamma=to_dev(torch, np.array([inp.gamma], np.float32), dev),
                      y=torch.empty((M, by[n].N), dtype=torch.bfloat16, device=dev))
                 for n, inp in zip(names, inps)]
        G.append(dict(names=names, x=x, q=q, d=d, qs=qs,
                      group=bl.GemmGroup(probs, q, d, qsum=qs),
                      plain=bl.GemmGroup(probs, q, d),
                      ops=sum(2 * M * by[n].N * by[n].K for n in names)))
        del inps
    torch.cuda.synchronize()
    return cfg, M, G


def prefill_100b(torch, bl, W, dev, gemm_steps):
    """The 100B-class layer at 2048 tokens: per input one bl_quantize_act
    (codes, scales, token sums), then one bl_gemm_group per group (offset
    weights). TOPS with and without the quantize launches, without the token
    sums (interleaved rounds), per group, and with one scale per tensor."""
    cfg5, M5, G = build_prefill(torch, bl, W, dev)

    def layer(gemm_only=False, plain=False):
        for e in G:
            if not gemm_only:
                bl.quantize_act(e["x"], e["q"], e["d"], qsum=e["qs"])
            e["plain" if plain else "group"]()

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(n):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / n

    layer()
    ms_layer = timed(layer, gemm_steps)
    ops = cfg5.ops(M5)
    # GEMMs only, with and without the token sums, interleaved (the clock
    # drifts with the power state): medians over 3 rounds
    ms_by = {False: [], True: []}
    for rnd in range(3):
        for plain in ((False, True) if rnd % 2 == 0 else (True, False)):
            ms_by[plain].append(timed(lambda: layer(gemm_only=True, plain=plain), gemm_steps))
    ms_gemm = float(np.median(ms_by[False]))
    ws_t = torch.empty((max(16, int(bl.lib().bl_quantize_act_tensor_workspace(M5))),),
                       dtype=torch.uint8, device=dev)

    def layer_pt():
        for e in G:
            bl.quantize_act_tensor(e["x"], e["q"], e["d"], workspace=ws_t, qsum=e["qs"])
            e["group"]()

    ms_layer_pt = timed(layer_pt, gemm_steps)
    per_group = {}
    for e in G:
        ms = timed(e["group"], 3)
        per_group["+".join(e["names"])] = {"us": round(ms * 1e3, 2),
                                           "tops": round(e["ops"] / (ms * 1e-3) / 1e12, 1)}
    del G
    torch.cuda.empty_cache()
    return {"workload": cfg5.name, "tokens": M5, "ops_per_layer": ops,
            "ms_per_layer": round(ms_layer, 4), "tops": round(ops / (ms_layer * 1e-3) / 1e12, 1),
            "gemm_only_ms": round(ms_gemm, 4),
            "gemm_only_tops": round(ops / (ms_gemm * 1e-3) / 1e12, 1),
            "frac": round(ops / (ms_gemm * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
            "gemm_only_tops_without_token_sums":
                round(ops / (float(np.median(ms_by[True])) * 1e-3) / 1e12, 1),
            "step": "per input: bl_quantize_act (codes, scales, token sums), then one "
                    "bl_gemm_group for {q,k,v}, {o}, {gate,up}, {down} (offset weights)",
            "per_group": per_group,
            "tops_per_tensor_scale": round(ops / (ms_layer_pt * 1e-3) / 1e12, 1)}


def prefill_2b(torch, bl, W, dev, stream):
    """The BitNet-2B-like layer at 512 tokens (small matrices on the int8
    MFMA path): per input one bl_quantize_act, then one bl_gemm_group per
    group, as graph replays over 32 layer copies (17.4 MB of packed weights
    each, so the weights come from HBM). TOPS of the GEMMs alone and of the
    layer with its quantize launches."""
    cfg, M, G = build_prefill(torch, bl, W, dev, cid=3, M=512)
    R = ROTATE
    copies = []
    for r in range(R):
        copies.append([e["group"] if r == 0 else
                       bl.GemmGroup([dict(p, packed=p["packed"].clone()) for p in e["group"].problems],
                                    e["q"], e["d"], qsum=e["qs"], workspace=e["group"].workspace)
                       for e in G])
    quant = [(lambda e=e: bl.quantize_act(e["x"], e["q"], e["d"], qsum=e["qs"])) for e in G]
    gemm_only = [grp for layer in copies for grp in layer]
    with_q = [f for layer in copies for pair in zip(quant, layer) for f in pair]
    for f in with_q[:2 * len(G)]:
        f()
    out = {"workload": cfg.name, "tokens": M, "ops_per_layer": cfg.ops(M)}
    for name, fns in (("gemm_only", gemm_only), ("with_quantize", with_q)):
        g = capture_fns(torch, stream, fns)
        us = replay_us(torch, stream, g, R, reps=10)
        out[name] = {"us_per_layer": round(us, 2), "tops": round(cfg.ops(M) / (us * 1e-6) / 1e12, 1),
                     "frac": round(cfg.ops(M) / (us * 1e-6) / 1e12 / INT8_PEAK_TOPS, 4)}
        del g
    del copies, G
    torch.cuda.empty_cache()
    return out


# --------------------------------------------------------------- CPU oracle

# Each workload's oracle step: per projection, the bf16 input quantized per
# token, the packed rows unpacked, the int64 dot and the dequant to bf16; the
# packing itself is the offline conversion and is not timed. The oracle's
# speed does not depend on the weight values (a dense integer matmul), so the
# packed rows are drawn ternary at the workload's zero fraction.
CPU_PLAN = {
    # cid: (tokens, workload name, row fraction on one core, row fraction on all cores)
    1: (1, "single-1024x1024-decode", 1, 1),
    2: (1, "bitnet-2b-layer-decode", 1, 1),
    3: (512, "bitnet-2b-layer-prefill-512", 16, 1),
    4: (1, "7b-layer-decode", 1, 1),
    5: (2048, "100b-layer-prefill-2048", 512, 16),
}


def _cpu_inputs(cid, rows_div, shard, nshard):
    """Seeded inputs of one shard of a workload's row sample: per projection
    (x bf16 [M][K], packed rows, gamma, K). The sample is N/rows_div output
    rows of every projection; shard s of n takes its s-th part."""
    import oracle
    import workloads as W
    cfg = W.LAYERS[cid]
    M = CPU_PLAN[cid][0]
    p0 = 0.31 if cfg.weights == "f32_normal" else cfg.p_zero
    out = []
    for proj in cfg.projs:
        n_rows = max(1, proj.N // rows_div)
        lo, hi = n_rows * shard // nshard, n_rows * (shard + 1) // nshard
        if hi <= lo:
            continue
        x = W.activations_bf16(W.seed_for(cid, proj.index, 1), M, proj.K,
                               cfg.outlier_frac, cfg.outlier_scale)
        w = W.ternary_drawn(W.seed_for(cid, proj.index, 0) + 7 * shard + 1, hi - lo, proj.K, p0)
        out.append((x, oracle.pack_i2s(w), np.float32(W.GAMMA_DRAWN), proj.K))
    return out


def _cpu_step(data):
    """One oracle step over the given inputs; returns the seconds it took."""
    import oracle
    t0 = time.perf_counter()
    for x, packed, gamma, K in data:
        q, d = oracle.quantize_act_absmax(x)
        t = oracle.unpack_i2s(packed, K)
        acc = oracle.mpgemm_acc(q, t)
        oracle.round_f64_to_bf16_bits(oracle.dequant_f64(acc, gamma, d))
    return time.perf_counter() - t0


def _cpu_worker(cid, rows_div, shard, nshard, ready, go, results):
    """One worker process: builds its shard's inputs, waits until every worker
    has, runs one oracle step when the parent says go, reports its time."""
    data = _cpu_inputs(cid, rows_div, shard, nshard)
    if data:
        _cpu_step(data[:1])                              # warm the code paths
    ready.wait()
    go.wait()
    results.put((shard, _cpu_step(data)))


def cpu_baseline(gpu_us, headline_cid=4):
    """The oracle timed per workload on this host: on one core (this process)
    over a row sample, and on all cores (one spawned worker process per core,
    each a contiguous shard of a row sample, all started together) as the wall
    time until the last worker finishes; both extrapolated to the whole
    workload by the row fraction. gpu_us: the GPU time of each workload's step
    in microseconds."""
    import multiprocessing as mp
    import workloads as W
    ncores = min(16, len(os.sched_getaffinity(0)))
    out = {"host_cores": len(os.sched_getaffinity(0)), "worker_processes": ncores, "per_config": {}}
    ctx = mp.get_context("spawn")
    for cid, (M, name, div1, divn) in CPU_PLAN.items():
        data = _cpu_inputs(cid, div1, 0, 1)
        _cpu_step(data[:1])
        t1 = _cpu_step(data) * div1
        del data
        ready, go, results = ctx.Barrier(ncores + 1), ctx.Event(), ctx.Queue()
        procs = [ctx.Process(target=_cpu_worker, args=(cid, divn, s, ncores, ready, go, results))
                 for s in range(ncores)]
        for pr in procs:
            pr.start()
        ready.wait(timeout=600)
        t0 = time.perf_counter()
        go.set()
        shards = [results.get(timeout=600) for _ in range(ncores)]
        tn = (time.perf_counter() - t0) * divn
        for pr in procs:
            pr.join(timeout=60)
        if sorted(s for s, _ in shards) != list(range(ncores)):
            raise RuntimeError("cpu baseline: missing worker results")
        cfg = W.LAYERS[cid]
        rec = {"workload": name, "tokens": M,
               "one_core_s": round(t1, 4), "one_core_row_fraction": f"1/{div1}",
               "all_cores_s": round(tn, 4), "all_cores_row_fraction": f"1/{divn}",
               "extrapolated": div1 > 1 or divn > 1,
               "slowest_worker_s": round(max(t for _, t in shards) * divn, 4)}
        if M == 1:
            rec["one_core_gbs"] = round(cfg.packed_bytes / t1 / 1e9, 4)
            rec["all_cores_gbs"] = round(cfg.packed_bytes / tn / 1e9, 4)
        else:
            rec["one_core_tops"] = round(cfg.ops(M) / t1 / 1e12, 6)
            rec["all_cores_tops"] = round(cfg.ops(M) / tn / 1e12, 6)
        if gpu_us.get(cid):
            rec["gpu_us"] = round(gpu_us[cid], 3)
            rec["gpu_speedup_vs_all_cores"] = round(tn / (gpu_us[cid] * 1e-6), 1)
            rec["gpu_speedup_vs_one_core"] = round(t1 / (gpu_us[cid] * 1e-6), 1)
        out["per_config"][str(cid)] = rec
        log(f"cpu oracle config {cid}: one core {t1:.3f} s, {ncores} cores {tn:.3f} s")
    h = out["per_config"][str(headline_cid)]
    out.update({"value": h["all_cores_gbs"], "unit": "GB/s", "cores": ncores, "kind": "oracle",
                "sample": f"the 7B-class decode layer at batch 1 (7 projections, 50.6 MB "
                          f"packed): quantize, unpack, int64 dot, dequant, bf16 (numpy), row "
                          f"shards in {ncores} worker processes on a {out['host_cores']}-core "
                          f"host; one core: {h['one_core_gbs']} GB/s; every workload in "
                          f"per_config (configs 3 and 5 on row samples, extrapolated)"})
    return out


# --------------------------------------------------------------------- main

def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=640)
    p.add_argument("--warmup", type=int, default=64)
    p.add_argument("--gemm-steps", type=int, default=5)
    p.add_argument("--no-gemm", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extras", action="store_true",
                   help="only the headline stream (and the prefill unless --no-gemm)")
    p.add_argument("--mfma-counters", action="store_true",
                   help="counter-collection mode: only the prefill GEMM layers (eager) of the "
                        "100B-class layer at 2048 tokens and the 2B-class layer at 512; no JSON line")
    p.add_argument("--traffic", action="store_true",
                   help="counter-collection mode: a 256 MiB plain copy (calibration), "
                        "eager decode launches of the headline stream, 4 fused norm launches "
                        "on the 100B-class prefill shape and 4 one-token GEMVs of 28672 x 8192; "
                        "no JSON line")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)
    import torch

    import mpgemm_token_absmax_amd as bl
    import workloads as W

    bl.lib()
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)

    if args.mfma_counters:
        # the 100B-class layer at 2048 tokens, then the 2B-class layer at 512
        for cid, M in ((5, 2048), (3, 512)):
            _, _, G = build_prefill(torch, bl, W, dev, cid=cid, M=M)
            for _ in range(args.gemm_steps):
                for e in G:
                    bl.quantize_act(e["x"], e["q"], e["d"], qsum=e["qs"])
                    e["group"]()
            torch.cuda.synchronize()
            log(f"mfma-counters mode: config {cid}, {args.gemm_steps} prefill layers "
                f"({len(G)} groups each)")
            del G
            torch.cuda.empty_cache()
        return

    # ----------------------------------------------- headline: 7B decode stream
    cfg = W.LAYERS[4]
    log(f"setup decode stream: {cfg.name}, {ROTATE} layer copies")
    layers, _ = decode_layers(torch, bl, W, dev, cfg, 1)
    step_bytes = cfg.packed_bytes
    if args.traffic:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src).fill_(0)
        torch.cuda.synchronize()
        torch.bitwise_not(src, out=dst)       # calibration kernel: 256 MiB read, 256 MiB written
        torch.cuda.synchronize()
        for layer in layers:                  # each launch reads weights no earlier launch read
            for f in layer:
                f()
        torch.cuda.synchronize()
        # the fused norm on the 100B-class prefill shape, 4 launches on fresh buffers
        cfg5 = W.LAYERS[5]
        K5 = cfg5.projs[0].K
        xb, rb, gb = W.norm_inputs(4242 + 5, 2048, K5, cfg5.outlier_frac, cfg5.outlier_scale)
        g5 = bf16_dev(torch, gb, dev)
        for _ in range(4):
            bl.rmsnorm_quant(bf16_dev(torch, xb, dev), g5, 1e-5, residual=bf16_dev(torch, rb, dev),
                             h_out=torch.empty((2048, K5), dtype=torch.bfloat16, device=dev),
                             q=torch.empty((2048, K5), dtype=torch.int8, device=dev),
                             d=torch.empty((2048,), dtype=torch.float32, device=dev))
        torch.cuda.synchronize()
        # the one-token GEMV of the 100B-class 28672 x 8192 shape, 4 launches on fresh weights
        gen = torch.Generator(device=dev).manual_seed(2048)
        t = torch.randint(-1, 2, (28672, 8192), dtype=torch.int8, device=dev, generator=gen)
        x1 = torch.randn(1, 8192, device=dev, generator=gen).to(torch.bfloat16)
        gam = torch.tensor([0.01], device=dev)
        gemvs = [bl.DecodeGroup([dict(packed=bl.pack_i2s(t), gamma=gam, x=x1)]) for _ in range(4)]
        del t
        torch.cuda.synchronize()
        for f in gemvs:
            f()
        torch.cuda.synchronize()
        log(f"traffic mode: 1 calibration kernel over {src.numel()} B, "
            f"{len(layers) * len(W.LAYER_GROUPS)} decode launches "
            f"({step_bytes // len(W.LAYER_GROUPS)} packed bytes per launch on average), "
            f"4 bl_rmsnorm_quant launches of 2048 x {K5}, 4 one-token GEMVs of 28672 x 8192")
        return
    for layer in layers:                      # eager pass: loads the code objects
        for f in layer:
            f()
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    log(f"timing {args.steps} steps after {args.warmup} warmup steps")
    ms_step, spread, piped_p50 = time_steps(torch, stream, layers, args.steps, args.warmup)
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    launches = len(W.LAYER_GROUPS)
    us_launch = ms_step * 1e3 / launches
    log(f"7B decode stream: {ms_step * 1e3:.2f} us/step, {gbs:.1f} GB/s packed; p10/p50/p90 {spread}")
    # warm: every step reuses layer copy 0 (weights resident in the Infinity Cache)
    g_warm = capture_fns(torch, stream, [f for _ in range(ROTATE) for f in layers[0]])
    us_warm = replay_us(torch, stream, g_warm, ROTATE)
    del g_warm
    blocks16 = lambda names: sum((next(p.N for p in cfg.projs if p.name == n) + 15) // 16 for n in names)
    floors = stream_floors(torch, dev, stream, ROTATE,
                           [(names, sum(p.N * p.K // 4 for p in cfg.projs if p.name in names),
                             blocks16(names)) for names in W.LAYER_GROUPS])
    log(f"floors {floors}")
    del layers
    torch.cuda.empty_cache()

    result = {
        "metric": "ternary GEMV packed-weight GB/s (% HBM peak); prefill GEMM int8 TOPS (% peak)",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": "7b-layer-decode-stream", "tokens": 1, "hidden": 4096,
                   "ffn": 11008, "heads": 32, "layer_copies": ROTATE,
                   "packed_bytes_per_step": step_bytes,
                   "step": "one layer: 4 fused launches {q,k,v},{o},{gate,up},{down}, each "
                           "per-token absmax int8 quantize + I2_S GEMV + bf16 dequant; step i "
                           "on layer copy i mod 32",
                   "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                   "us_per_step_p10_p50_p90": spread,
                   "us_per_step_back_to_back_p50": piped_p50,
                   "warm_us_per_step": round(us_warm, 3),
                   "floors": floors,
                   "frac_of_layer_floor": round(floors["layer_floor_us"] / (ms_step * 1e3), 4)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(),
                     "kernel": "k_decode1 / k_decode1w (one-token fused decode launches)",
                     "us_per_launch": round(us_launch, 3),
                     "bytes_per_launch": step_bytes / launches},
    }
    gpu_us = {4: ms_step * 1e3}
    configs = {"4": {"M1": {"us_per_layer": round(ms_step * 1e3, 3), "gbs": round(gbs, 1),
                            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}}}

    if not args.no_extras:
        for M in (4, 16):
            configs["4"][f"M{M}"] = decode_workload(torch, bl, W, dev, stream, 4, M)
            log(f"7B decode M={M}: {configs['4'][f'M{M}']}")
        configs["4"]["M1_p_zero_0.65"] = decode_workload(torch, bl, W, dev, stream, 4, 1,
                                                         p_zero_override=0.65)
        log(f"7B decode, 65% zeros: {configs['4']['M1_p_zero_0.65']}")
        configs["2"] = decode_workload(torch, bl, W, dev, stream, 2, 1)
        gpu_us[2] = configs["2"]["us_per_layer"]
        log(f"2B decode: {configs['2']}")
        configs["1"] = single_gemv_workload(torch, bl, W, dev, stream)
        gpu_us[1] = configs["1"]["us_per_call"]
        log(f"1024x1024 GEMV: {configs['1']}")
        result["one_token_gemv_100b"] = one_token_gemv_100b(torch, bl, dev, stream)
        log(f"100B one-token GEMVs: {result['one_token_gemv_100b']}")

    if not args.no_gemm:
        g5 = prefill_100b(torch, bl, W, dev, args.gemm_steps)
        configs["5"] = g5
        gpu_us[5] = g5["ms_per_layer"] * 1e3
        log(f"prefill 100B: {g5}")
        tops = g5["gemm_only_tops"]
        result["roofline_gemm"] = {"bound": "mfma", "achieved": tops, "peak": INT8_PEAK_TOPS,
                                   "unit": "TOP/s", "frac": round(tops / INT8_PEAK_TOPS, 4),
                                   "kernel": "k_gemm_i2s", "workload": g5["workload"],
                                   "us_per_layer": round(g5["gemm_only_ms"] * 1e3, 2)}
        if not args.no_extras:
            configs["3"] = prefill_2b(torch, bl, W, dev, stream)
            gpu_us[3] = configs["3"]["with_quantize"]["us_per_layer"]
            log(f"prefill 2B: {configs['3']}")
    result["configs"] = configs

    if not args.no_extras:
        result["rmsnorm_quant"] = norm_bench(torch, bl, W, dev, stream)
        log(f"rmsnorm_quant: {result['rmsnorm_quant']}")
        result["decode_layer_with_norms"] = norm_layer_bench(torch, bl, W, dev, stream)
        log(f"decode layer with norms: {result['decode_layer_with_norms']}")
        result["t3_gemv"] = t3_bench(torch, bl, W, dev, stream)
        log(f"t3_gemv: {result['t3_gemv']}")

    if not args.no_cpu_baseline:
        log("cpu baseline: oracle per workload")
        result["cpu_baseline"] = cpu_baseline(gpu_us)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
