"""Benchmark of the ternary BitLinear hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

Headline (the JSON `value`): decode GEMV packed-weight GB/s on the
BitNet-2B-like layer at batch 1 (hidden 2560, k/v 640, FFN 6912). One step =
one pass of the per-token hot path over that layer: for each of the 7
projections (q, k, v, o, gate, up, down) the per-token absmax int8
quantization of its bf16 input and the I2_S GEMV with the bf16 dequant fused
into the store, issued as one fused launch per group of projections that do
not depend on each other in a decoder layer: {q,k,v}, {o}, {gate,up}, {down}.
Weight packing is the offline conversion and is done once before timing. Steps rotate over R distinct copies of the layer's packed
weights (R * 17.4 MB > the 256 MB Infinity Cache), so every step streams its
weights from HBM. Steps are replayed from HIP graphs (captured through
torch.cuda.CUDAGraph) so host launch cost is not timed.

Also reported on the same JSON line:
  roofline      the fused decode kernel: algorithmic packed bytes per launch
                over its average launch duration (HIP events around graph
                replays on the replay stream), against 8 TB/s;
  gemm          prefill on the 100B-class layer (2048 tokens, hidden 8192,
                FFN 28672, k/v 1024): 2*M*N*K int8 ops per second over the 7
                projections (quantize + GEMM), against 5.0 POP/s dense int8;
  cpu_baseline  the CPU oracle on a bounded sample of the decode workload.
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

PREFILL_GROUPS = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))
HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode1_traffic.json")
DECODE_SOURCES = ("mpgemm_token_absmax_amd/csrc/gemv_i2s.hip",
                  "mpgemm_token_absmax_amd/csrc/common.hpp",
                  "mpgemm_token_absmax_amd/csrc/launch.hpp")


def measured_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by a plain-kernel calibration), or
    None when the decode kernel's sources changed since the counters were taken."""
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


def capture_fns(torch, stream, fns):
    """HIP graph of the given launch callables, captured on `stream`."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for f in fns:
            f()
    return g


def replay_us(torch, stream, g, launches, reps=20):
    """Mean microseconds per launch over `reps` replays of graph g."""
    with torch.cuda.stream(stream):
        g.replay()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * launches)


def measure_floors(torch, dev, stream, capture_fn, R, groups):
    """Floors of a decode launch on this machine, with the measurement aids of
    libblprobe.so in the same setting as the decode step (graph replays over R
    cold buffer copies): an empty kernel, a streaming read of each group's
    packed bytes by as many 256-thread blocks as its decode launch has, and a
    1 GiB streaming read (practical HBM peak)."""
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
    g = capture_fn(torch, stream, [empty] * 128)
    out["empty_launch_us"] = round(replay_us(torch, stream, g, 128), 3)
    stream_us = {}
    for names, nbytes, blocks in groups:
        bufs = [torch.ones(nbytes, dtype=torch.uint8, device=dev) for _ in range(R)]
        g = capture_fn(torch, stream, [read(b, nbytes, blocks) for b in bufs])
        stream_us["+".join(names)] = round(replay_us(torch, stream, g, R), 3)
        del g, bufs
    out["stream_read_us"] = stream_us
    total = sum(nb for _, nb, _ in groups)
    out["layer_floor_us"] = round(sum(stream_us.values()), 3)
    out["layer_floor_gbs"] = round(total / (out["layer_floor_us"] * 1e-6) / 1e9, 1)
    big = 1 << 30
    bufs = [torch.ones(big, dtype=torch.uint8, device=dev) for _ in range(2)]
    g = capture_fn(torch, stream, [read(b, big, 2048) for b in bufs])
    out["practical_peak_gbs"] = round(big / (replay_us(torch, stream, g, 2, reps=5) * 1e-6) / 1e9,
                                      1)
    del g, bufs
    torch.cuda.empty_cache()
    return out


def decode_more(torch, bl, W, dev, stream):
    """The 7B-class layer at 1, 4 and 16 tokens (4 group launches per layer,
    a stream over 32 distinct layer copies = 1.62 GB) and one-token GEMVs of
    the 100B-class shapes (one launch, rotating copies), in GB/s of packed
    weights; next to each 100B-class GEMV, a streaming read of the same bytes
    (libblprobe.so) in the same setting."""
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
    cfg = W.LAYERS[4]
    layer_groups = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))
    packed = {}
    for proj in cfg.projs:
        inp = W.proj_inputs(cfg, proj, 1, with_acts=False)
        packed[proj.name] = bl.pack_i2s(torch.from_numpy(inp.w_f32).to(dev))
        del inp
    R = 32
    copies = [{n: (pg[0] if r == 0 else pg[0].clone(), pg[1]) for n, pg in packed.items()}
              for r in range(R)]
    for M in (1, 4, 16):
        xs = {}
        for proj in cfg.projs:
            bits = W.activations_bf16(W.seed_for(cfg.cid, proj.index, 1), M, proj.K,
                                      cfg.outlier_frac, cfg.outlier_scale)
            xs[proj.name] = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
        launches = [bl.DecodeGroup([dict(packed=copies[r][n][0], gamma=copies[r][n][1], x=xs[n])
                                    for n in names]) for r in range(R) for names in layer_groups]
        for f in launches[:len(layer_groups)]:
            f()
        g = capture_fns(torch, stream, launches)
        us = replay_us(torch, stream, g, 1, reps=10) / R
        out[f"7b_layer_M{M}"] = {"us_per_layer": round(us, 3),
                                 "gbs": round(cfg.packed_bytes / (us * 1e-6) / 1e9, 1)}
        del g, launches
    del copies, packed
    torch.cuda.empty_cache()
    for N, K in ((28672, 8192), (8192, 28672)):
        t = torch.randint(-1, 2, (N, K), dtype=torch.int8, device=dev)
        x = torch.randn(1, K, device=dev).to(torch.bfloat16)
        gam = torch.tensor([0.01], device=dev)
        R = 8
        launches = [bl.DecodeGroup([dict(packed=bl.pack_i2s(t), gamma=gam, x=x)]) for _ in range(R)]
        del t
        launches[0]()
        g = capture_fns(torch, stream, launches)
        us = replay_us(torch, stream, g, R, reps=10)
        del g
        # floor: a streaming read of the same bytes by as many threads as the
        # decode launch has (16 rows per block, 256 or 512 threads), R copies
        nbytes = N * K // 4
        blocks = (N + 15) // 16 * (2 if K > 16384 else 1)
        bufs = [c.problems[0]["packed"] for c in launches]
        g = capture_fns(torch, stream, [stream_read(b, nbytes, blocks) for b in bufs])
        floor = replay_us(torch, stream, g, R, reps=10)
        out[f"one_token_gemv_N{N}_K{K}"] = {"us": round(us, 3),
                                           "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
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
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    x1, r1, g1 = W.norm_inputs(2001, 1, K, cfg.outlier_frac, cfg.outlier_scale)
    x2, r2, g2 = W.norm_inputs(2002, 1, K, cfg.outlier_frac, cfg.outlier_scale)
    xo = W.activations_bf16(2003, 1, K, cfg.outlier_frac, cfg.outlier_scale)
    xd = W.activations_bf16(2004, 1, 6912, cfg.outlier_frac, cfg.outlier_scale)
    X1, R1, G1, X2, R2, G2, XO, XD = (t(a) for a in (x1, r1, g1, x2, r2, g2, xo, xd))
    H1, H2 = torch.empty_like(X1), torch.empty_like(X2)
    gam = torch.tensor([W.GAMMA_DRAWN], dtype=torch.float32, device=dev)
    base = {n: bl.pack_i2s(torch.from_numpy(W.proj_inputs(cfg, by[n], 1, with_acts=False).w_tern).to(dev))
            for n in by}
    R = 32
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
        us = replay_us(torch, stream, g, 1, reps=10) / R
        out[name] = {"us_per_layer": round(us, 3), "gbs": round(cfg.packed_bytes / (us * 1e-6) / 1e9, 1)}
        del g
    del copies, fused, unfused
    torch.cuda.empty_cache()
    return out


def t3_bench(torch, bl, W, dev, stream):
    """Base-3 weights (five per byte, 1.6 bits per weight) against I2_S (2 bits
    per weight), one token:
      - through the GEMV kernels of the same structure (int8 codes in):
        bl_gemv_t3 and bl_gemv ("t3", "i2s");
      - through the fused one-token decode (bf16 x in, quantize in the
        kernel): bl_decode_group_t3 and bl_decode_group ("t3_fused",
        "i2s_fused");
    graph replays over copies of the packed weights (>= 700 MB), microseconds
    per call, GB/s of packed bytes and billions of weights per second; and the
    BitNet-2B-like decode layer (4 fused launches, 32 rotating layer copies)
    in both formats."""
    out = {}
    for N, K in ((2560, 2560), (6912, 2560), (2560, 6912), (28672, 8192), (8192, 28672)):
        t = torch.from_numpy(W.ternary_drawn(7 + N + K, N, K, 1.0 / 3.0)).to(dev)
        p2, p3 = bl.pack_i2s(t), bl.pack_t3(t)
        del t
        x = torch.from_numpy(W.activations_bf16(9 + K, 1, K, 0.005, 50.0).view(np.int16)).to(dev)
        xb = x.view(torch.bfloat16)
        q, d = bl.quantize_act(xb)
        gam = torch.tensor([W.GAMMA_DRAWN], dtype=torch.float32, device=dev)
        R = max(2, -(-700_000_000 // p3.numel()))
        y = torch.empty((1, N), dtype=torch.bfloat16, device=dev)
        rec = {}
        for name, p, fn in (("i2s", p2, bl.gemv), ("t3", p3, bl.gemv_t3),
                            ("i2s_fused", p2, bl.DecodeGroup), ("t3_fused", p3, bl.DecodeGroupT3)):
            copies = [p] + [p.clone() for _ in range(R - 1)]
            if name.endswith("_fused"):
                fns = [fn([dict(packed=c, gamma=gam, x=xb, y=y)]) for c in copies]
                fns[0]()
            else:
                fns = [(lambda c=c: fn(c, gam, q, d, out=y)) for c in copies]
            g = capture_fns(torch, stream, fns)
            us = replay_us(torch, stream, g, R, reps=10)
            rec[name] = {"us": round(us, 3), "packed_bytes": p.numel(),
                         "gbs": round(p.numel() / (us * 1e-6) / 1e9, 1),
                         "gweights_s": round(N * K / (us * 1e-6) / 1e9, 1)}
            del g, copies, fns
        out[f"N{N}_K{K}"] = rec
        del p2, p3
        torch.cuda.empty_cache()
    # the 2B decode layer, both formats
    cfg = W.LAYERS[2]
    layer_groups = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))
    gam = torch.tensor([W.GAMMA_DRAWN], dtype=torch.float32, device=dev)
    xs, tern = {}, {}
    for proj in cfg.projs:
        inp = W.proj_inputs(cfg, proj, 1)
        tern[proj.name] = torch.from_numpy(inp.w_tern).to(dev)
        xs[proj.name] = torch.from_numpy(inp.x_bf16.view(np.int16)).to(dev).view(torch.bfloat16)
    R = 32
    layer = {}
    for name, pack, Grp in (("i2s_fused", bl.pack_i2s, bl.DecodeGroup),
                            ("t3_fused", bl.pack_t3, bl.DecodeGroupT3)):
        base = {n: pack(t) for n, t in tern.items()}
        nbytes = sum(p.numel() for p in base.values())
        copies = [{n: (p if r == 0 else p.clone()) for n, p in base.items()} for r in range(R)]
        ys = {n: torch.empty((1, t.shape[0]), dtype=torch.bfloat16, device=dev) for n, t in tern.items()}
        fns = [Grp([dict(packed=c[n], gamma=gam, x=xs[n], y=ys[n]) for n in names])
               for c in copies for names in layer_groups]
        for f in fns[:4]:
            f()
        g = capture_fns(torch, stream, fns)
        us = replay_us(torch, stream, g, 1, reps=10) / R
        layer[name] = {"us_per_layer": round(us, 3), "packed_bytes": nbytes,
                       "gbs": round(nbytes / (us * 1e-6) / 1e9, 1)}
        del g, fns, copies, base
    out["bitnet2b_decode_layer"] = layer
    del tern, xs
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
        t = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        g = t(gb)
        nbytes = M * (7 * K + 4) + 2 * K
        R = max(1, min(64, -(-600_000_000 // nbytes)))
        bufs = [dict(x=t(xb), r=t(rb), h=torch.empty((M, K), dtype=torch.bfloat16, device=dev),
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
        # floor: a plain device copy moving the same bytes (half read, half written)
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


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=640)
    p.add_argument("--warmup", type=int, default=64)
    p.add_argument("--rotate", type=int, default=32, help="distinct layer copies")
    p.add_argument("--gemm-steps", type=int, default=5)
    p.add_argument("--no-gemm", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the 7B-layer and 100B-shape decode measurements")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--mfma-counters", action="store_true",
                   help="counter-collection mode: only the prefill GEMM layers (eager), no JSON line")
    p.add_argument("--traffic", action="store_true",
                   help="counter-collection mode: a 256 MiB plain copy (calibration) and "
                        "eager decode launches over distinct weight copies; no JSON line")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_prefill(torch, bl, W, dev, cid=5, M5=2048):
    """A prefill layer (by default the 100B-class layer at 2048 tokens): one
    bf16 input per group of projections that read it; each group's GEMMs run
    through one bl_gemm_group call on its quantized codes. The quantizer also
    writes the token sums and `group` takes them (offset weights); `plain` is
    the same group without them."""
    cfg5 = W.LAYERS[cid]
    log(f"setup prefill: {cfg5.name}")
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    by = {proj.name: proj for proj in cfg5.projs}
    G = []
    for names in PREFILL_GROUPS:
        inps = [W.proj_inputs(cfg5, by[n], M5) for n in names]
        K = by[names[0]].K
        x = to_dev(inps[0].x_bf16.view(np.int16)).view(torch.bfloat16)
        q = torch.empty((M5, K), dtype=torch.int8, device=dev)
        d = torch.empty((M5,), dtype=torch.float32, device=dev)
        qs = torch.empty((M5,), dtype=torch.int32, device=dev)
        probs = [dict(packed=bl.pack_i2s(to_dev(inp.w_tern)),
                      gamma=to_dev(np.array([inp.gamma], np.float32)),
                      y=torch.empty((M5, by[n].N), dtype=torch.bfloat16, device=dev))
                 for n, inp in zip(names, inps)]
        G.append(dict(names=names, x=x, q=q, d=d, qs=qs,
                      group=bl.GemmGroup(probs, q, d, qsum=qs),
                      plain=bl.GemmGroup(probs, q, d),
                      ops=sum(2 * M5 * by[n].N * by[n].K for n in names)))
        del inps
    torch.cuda.synchronize()
    return cfg5, M5, G


def prefill_2b(torch, bl, W, dev, stream):
    """The BitNet-2B-like layer at 512 tokens (small matrices on the int8
    MFMA path): per input one bl_quantize_act, then one bl_gemm_group per
    {q,k,v}, {o}, {gate,up}, {down}, as graph replays over 32 layer copies
    (17.4 MB of packed weights each, so the weights come from HBM). TOPS of
    the GEMMs alone and of the layer with its quantize launches."""
    cfg, M, G = build_prefill(torch, bl, W, dev, cid=3, M5=512)
    R = 32
    copies = []
    for r in range(R):
        copies.append([e["group"] if r == 0 else
                       bl.GemmGroup([dict(p, packed=p["packed"].clone()) for p in e["group"].problems],
                                    e["q"], e["d"], qsum=e["qs"]) for e in G])
    quant = [(lambda e=e: bl.quantize_act(e["x"], e["q"], e["d"], qsum=e["qs"])) for e in G]
    gemm_only = [grp for layer in copies for grp in layer]
    with_q = [f for layer in copies for pair in zip(quant, layer) for f in pair]
    for f in with_q[:2 * len(G)]:
        f()
    out = {"workload": cfg.name, "tokens": M, "ops_per_layer": cfg.ops(M)}
    for name, fns in (("gemm_only", gemm_only), ("with_quantize", with_q)):
        g = capture_fns(torch, stream, fns)
        us = replay_us(torch, stream, g, 1, reps=10) / R
        out[name] = {"us_per_layer": round(us, 2), "tops": round(cfg.ops(M) / (us * 1e-6) / 1e12, 1)}
        del g
    del copies, G
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    import mpgemm_token_absmax_amd as bl
    import workloads as W

    bl.lib()
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    if args.mfma_counters:
        # counter-collection mode for the prefill GEMMs: quantize (with token
        # sums) and bl_gemm_group per input, --gemm-steps layers, eager
        _, _, G = build_prefill(torch, bl, W, dev)
        for _ in range(args.gemm_steps):
            for e in G:
                bl.quantize_act(e["x"], e["q"], e["d"], qsum=e["qs"])
                e["group"]()
        torch.cuda.synchronize()
        log(f"mfma-counters mode: {args.gemm_steps} prefill layers ({len(G)} groups each)")
        return


    # ----------------------------------------------------------------- decode
    cfg = W.LAYERS[2]
    M = 1
    R = max(1, args.rotate)
    log(f"setup decode: {cfg.name}, {R} layer copies")
    inputs = {}
    for proj in cfg.projs:
        inp = W.proj_inputs(cfg, proj, M)
        inputs[proj.name] = dict(
            packed=bl.pack_i2s(to_dev(inp.w_tern)),
            gamma=to_dev(np.array([inp.gamma], np.float32)),
            x=to_dev(inp.x_bf16.view(np.int16)).view(torch.bfloat16),
            y=torch.empty((M, proj.N), dtype=torch.bfloat16, device=dev),
            q=torch.empty((M, proj.K), dtype=torch.int8, device=dev),
            d=torch.empty((M,), dtype=torch.float32, device=dev))
    torch.cuda.synchronize()
    step_bytes = cfg.packed_bytes
    # the projections of a decoder layer that do not depend on each other
    GROUPS = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))
    layers = []            # layers[r] = fused decode launches of layer copy r
    for r in range(R):
        launches = []
        for names in GROUPS:
            probs = []
            for nm in names:
                e = inputs[nm]
                packed = e["packed"] if r == 0 else e["packed"].clone()
                probs.append(dict(packed=packed, gamma=e["gamma"], x=e["x"], y=e["y"], name=nm))
            launches.append(bl.DecodeGroup(probs))
        layers.append(launches)
    torch.cuda.synchronize()

    def step(r):
        for launch in layers[r]:
            launch()

    if args.traffic:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src).fill_(0)
        torch.cuda.synchronize()
        torch.bitwise_not(src, out=dst)       # calibration kernel: 256 MiB read, 256 MiB written
        torch.cuda.synchronize()
        for r in range(R):                    # each launch reads weights no earlier launch read
            step(r)
        torch.cuda.synchronize()
        if not args.no_extras:                # 4 fused norm launches, 100B prefill shape
            cfg5 = W.LAYERS[5]
            K5 = cfg5.projs[0].K
            xb, rb, gb = W.norm_inputs(4247, 2048, K5, cfg5.outlier_frac, cfg5.outlier_scale)
            t = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
            gn = t(gb)
            for _ in range(4):
                xn, rn = t(xb), t(rb)
                bl.rmsnorm_quant(xn, gn, 1e-5, residual=rn, h_out=rn)
            torch.cuda.synchronize()
        log(f"traffic mode: 1 calibration kernel over {src.numel()} B, {R * len(GROUPS)} decode launches "
            f"({step_bytes // len(GROUPS)} packed bytes per launch on average)")
        return

    def step_unfused(r):        # 7 x (bl_quantize_act + bl_gemv), for comparison
        for launch in layers[r]:
            for p in launch.problems:
                e = inputs[p["name"]]
                bl.quantize_act(p["x"], e["q"], e["d"])
                bl.gemv(p["packed"], p["gamma"], e["q"], e["d"], out_dtype="bf16", out=p["y"])

    for r in range(R):          # eager warm-up (loads the code objects) before capture
        step(r)
        step_unfused(r)
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()

    def capture(fn, rs):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for r in rs:
                fn(r)
        return g

    g_all = capture(step, range(R))
    g_one = [capture(step, [r]) for r in range(R)]
    g_unfused = capture(step_unfused, range(R))
    torch.cuda.synchronize()

    def run_steps(n):
        full, rem = divmod(n, R)
        for _ in range(full):
            g_all.replay()
        for r in range(rem):
            g_one[r].replay()

    log(f"warmup {args.warmup} steps")
    run_steps(args.warmup)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    run_steps(args.steps)
    e1.record()
    torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    ms_step = ms_total / args.steps
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    log(f"decode: {ms_step * 1e3:.2f} us/step, {gbs:.1f} GB/s packed")

    # The dominant kernel is the fused decode kernel itself (the step is made of
    # its launches): average launch duration from events on the replay stream.
    reps = max(4, args.steps // R)
    with torch.cuda.stream(stream):
        g_all.replay()
        k0 = torch.cuda.Event(enable_timing=True)
        k1 = torch.cuda.Event(enable_timing=True)
        k0.record(stream)
        for _ in range(reps):
            g_all.replay()
        k1.record(stream)
        u0 = torch.cuda.Event(enable_timing=True)
        u1 = torch.cuda.Event(enable_timing=True)
        g_unfused.replay()
        u0.record(stream)
        for _ in range(reps):
            g_unfused.replay()
        u1.record(stream)
    torch.cuda.synchronize()
    launches = reps * R * len(GROUPS)
    us_launch = k0.elapsed_time(k1) * 1e3 / launches
    bytes_launch = step_bytes / len(GROUPS)
    gemv_gbs = bytes_launch / (us_launch * 1e-6) / 1e9
    us_unfused = u0.elapsed_time(u1) * 1e3 / (reps * R)
    log(f"fused decode kernel: {us_launch:.2f} us/launch avg, {gemv_gbs:.1f} GB/s; "
        f"unfused 7x(quantize+gemv): {us_unfused:.2f} us/step")

    # per-replay spread: each replay of g_all is R steps
    marks = []
    with torch.cuda.stream(stream):
        for _ in range(max(8, min(64, args.steps // R))):
            a0 = torch.cuda.Event(enable_timing=True)
            a1 = torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            g_all.replay()
            a1.record(stream)
            marks.append((a0, a1))
    torch.cuda.synchronize()
    per_step = np.array([x0.elapsed_time(x1) * 1e3 / R for x0, x1 in marks])
    spread = [round(float(np.percentile(per_step, q)), 3) for q in (10, 50, 90)]

    # warm mode: every step reuses layer copy 0 (weights stay in the Infinity Cache)
    g_warm = capture(step, [0] * R)
    with torch.cuda.stream(stream):
        g_warm.replay()
        w0 = torch.cuda.Event(enable_timing=True)
        w1 = torch.cuda.Event(enable_timing=True)
        w0.record(stream)
        for _ in range(reps):
            g_warm.replay()
        w1.record(stream)
    torch.cuda.synchronize()
    us_warm = w0.elapsed_time(w1) * 1e3 / (reps * R)

    floors = measure_floors(torch, dev, stream, capture_fn=capture_fns, R=R,
                            groups=[(names, sum(inputs[n]["packed"].numel() for n in names),
                                     sum((inputs[n]["packed"].shape[0] + 15) // 16 for n in names))
                                    for names in GROUPS])
    log(f"decode spread p10/p50/p90 {spread} us/step; warm (cache-resident weights) "
        f"{us_warm:.2f} us/step; floors {floors}")
    del g_warm

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
        "config": {"workload": cfg.name, "tokens": M, "hidden": 2560, "ffn": 6912, "kv": 640,
                   "layer_copies": R, "packed_bytes_per_step": step_bytes,
                   "step": "4 fused launches {q,k,v},{o},{gate,up},{down}: per-token absmax "
                           "int8 quantize + I2_S GEMV + bf16 dequant",
                   "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                   "unfused_us_per_step": round(us_unfused, 3),
                   "us_per_step_p10_p50_p90": spread,
                   "warm_us_per_step": round(us_warm, 3),
                   "floors": floors,
                   "frac_of_layer_floor": round(floors["layer_floor_us"] / (ms_step * 1e3), 4)},
        "roofline": {"bound": "hbm", "achieved": round(gemv_gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gemv_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(),
                     "kernel": "k_decode1 (one-token fused decode group)",
                     "us_per_launch": round(us_launch, 3), "bytes_per_launch": bytes_launch},
    }
    del layers, g_all, g_one, g_unfused
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    # ------------------------------------------------ more decode workloads
    if not args.no_extras:
        result["decode_more"] = decode_more(torch, bl, W, dev, stream)
        log(f"more decode: {result['decode_more']}")

    # ----------------------------------------------------------------- prefill
    if not args.no_gemm:
        cfg5, M5, G = build_prefill(torch, bl, W, dev)

        def layer(gemm_only=False, plain=False):
            for e in G:
                if not gemm_only:
                    bl.quantize_act(e["x"], e["q"], e["d"], qsum=e["qs"])
                e["plain" if plain else "group"]()

        layer()
        layer()
        torch.cuda.synchronize()
        a0 = torch.cuda.Event(enable_timing=True)
        a1 = torch.cuda.Event(enable_timing=True)
        a0.record()
        for _ in range(args.gemm_steps):
            layer()
        a1.record()
        torch.cuda.synchronize()
        ms_layer = a0.elapsed_time(a1) / args.gemm_steps
        ops = cfg5.ops(M5)
        tops = ops / (ms_layer * 1e-3) / 1e12
        # GEMMs only, with and without the token sums, interleaved (the clock
        # drifts with the power state, so back-to-back blocks would favour
        # whichever runs second): medians over 3 rounds of gemm_steps layers
        b0 = torch.cuda.Event(enable_timing=True)
        b1 = torch.cuda.Event(enable_timing=True)
        ms_by = {False: [], True: []}
        for rnd in range(3):
            for plain in ((False, True) if rnd % 2 == 0 else (True, False)):
                b0.record()
                for _ in range(args.gemm_steps):
                    layer(gemm_only=True, plain=plain)
                b1.record()
                torch.cuda.synchronize()
                ms_by[plain].append(b0.elapsed_time(b1) / args.gemm_steps)
        ms_gemm = float(np.median(ms_by[False]))
        gemm_tops = ops / (ms_gemm * 1e-3) / 1e12
        gemm_tops_plain = ops / (float(np.median(ms_by[True])) * 1e-3) / 1e12
        # one activation scale per layer input (per tensor) instead of per token
        ws_t = torch.empty((max(16, int(bl.lib().bl_quantize_act_tensor_workspace(M5))),),
                           dtype=torch.uint8, device=dev)

        def quantize_all(per_tensor):
            for e in G:
                if per_tensor:
                    bl.quantize_act_tensor(e["x"], e["q"], e["d"], workspace=ws_t, qsum=e["qs"])
                else:
                    bl.quantize_act(e["x"], e["q"], e["d"], qsum=e["qs"])

        def layer_pt():
            for e in G:
                bl.quantize_act_tensor(e["x"], e["q"], e["d"], workspace=ws_t, qsum=e["qs"])
                e["group"]()

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

        ms_layer_pt = timed(layer_pt, args.gemm_steps)
        tops_pt = ops / (ms_layer_pt * 1e-3) / 1e12
        us_q_tok = timed(lambda: quantize_all(False), 10) * 1e3
        us_q_ten = timed(lambda: quantize_all(True), 10) * 1e3
        per_group = {}
        for e in G:
            c0 = torch.cuda.Event(enable_timing=True)
            c1 = torch.cuda.Event(enable_timing=True)
            c0.record()
            for _ in range(3):
                e["group"]()
            c1.record()
            torch.cuda.synchronize()
            ms = c0.elapsed_time(c1) / 3
            per_group["+".join(e["names"])] = round(e["ops"] / (ms * 1e-3) / 1e12, 1)
        log(f"prefill: {ms_layer:.3f} ms/layer ({tops:.1f} TOPS incl. quantize), "
            f"GEMM only {gemm_tops:.1f} TOPS ({gemm_tops_plain:.1f} without token sums); "
            f"per group {per_group}; per-tensor scale "
            f"{tops_pt:.1f} TOPS; quantize per layer {us_q_tok:.1f} us per token, "
            f"{us_q_ten:.1f} us per tensor")
        result["gemm"] = {"workload": cfg5.name, "tokens": M5, "ops_per_layer": ops,
                          "ms_per_layer": round(ms_layer, 4), "tops": round(tops, 1),
                          "gemm_only_tops": round(gemm_tops, 1), "peak_tops": INT8_PEAK_TOPS,
                          "frac": round(gemm_tops / INT8_PEAK_TOPS, 4),
                          "gemm_only_tops_without_token_sums": round(gemm_tops_plain, 1),
                          "step": "per input: bl_quantize_act (codes, scales and token sums), "
                                  "then one bl_gemm_group for {q,k,v}, {o}, {gate,up}, {down} "
                                  "(offset weights)",
                          "tops_per_group": per_group,
                          "tops_per_tensor_scale": round(tops_pt, 1),
                          "quantize_us_per_layer": {"per_token": round(us_q_tok, 1),
                                                    "per_tensor": round(us_q_ten, 1)}}
        del G
        torch.cuda.empty_cache()

    # ------------------------------------- residual add + RMSNorm + quantize
    if not args.no_extras:
        result["rmsnorm_quant"] = norm_bench(torch, bl, W, dev, stream)
        log(f"rmsnorm_quant: {result['rmsnorm_quant']}")
        result["decode_layer_with_norms"] = norm_layer_bench(torch, bl, W, dev, stream)
        log(f"decode layer with norms: {result['decode_layer_with_norms']}")
        result["t3_gemv"] = t3_bench(torch, bl, W, dev, stream)
        log(f"t3_gemv: {result['t3_gemv']}")
        result["gemm_2b_prefill_512"] = prefill_2b(torch, bl, W, dev, stream)
        log(f"gemm_2b_prefill_512: {result['gemm_2b_prefill_512']}")

    # ------------------------------------------------------------ CPU oracle
    if not args.no_cpu_baseline:
        import oracle
        log("cpu baseline: oracle on the decode layer")
        host_inputs = []
        for proj in cfg.projs:
            inp = W.proj_inputs(cfg, proj, M)
            host_inputs.append((inp, oracle.pack_i2s(inp.w_tern)))

        def oracle_step():
            for inp, packed in host_inputs:
                q, d = oracle.quantize_act_absmax(inp.x_bf16)
                t = oracle.unpack_i2s(packed, inp.proj.K)
                acc = oracle.mpgemm_acc(q, t)
                oracle.round_f64_to_bf16_bits(oracle.dequant_f64(acc, inp.gamma, d))

        n = 0
        t0 = time.perf_counter()
        while True:
            oracle_step()
            n += 1
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        dt = time.perf_counter() - t0
        cpu_gbs = step_bytes * n / dt / 1e9
        result["cpu_baseline"] = {
            "value": round(cpu_gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} decode steps of the same layer (7 projections: quantize, unpack, "
                      f"int64 dot, dequant, bf16) in {dt:.1f} s; numpy, single thread; "
                      f"host has {len(os.sched_getaffinity(0))} cores"}
        log(f"cpu oracle: {cpu_gbs:.4f} GB/s ({n} steps in {dt:.1f} s)")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
