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


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=640)
    p.add_argument("--warmup", type=int, default=64)
    p.add_argument("--rotate", type=int, default=32, help="distinct layer copies")
    p.add_argument("--gemm-steps", type=int, default=5)
    p.add_argument("--no-gemm", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--traffic", action="store_true",
                   help="counter-collection mode: a 256 MiB plain copy (calibration) and "
                        "eager decode launches over distinct weight copies; no JSON line")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    import mpgemm_token_absmax_amd as bl
    import workloads as W

    bl.lib()
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # ----------------------------------------------------------------- decode
    cfg = W.CONFIGS[2]
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
                   "unfused_us_per_step": round(us_unfused, 3)},
        "roofline": {"bound": "hbm", "achieved": round(gemv_gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gemv_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(),
                     "kernel": "k_decode1 (one-token fused decode group)",
                     "us_per_launch": round(us_launch, 3), "bytes_per_launch": bytes_launch},
    }
    del layers, g_all, g_one, g_unfused
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    # ----------------------------------------------------------------- prefill
    if not args.no_gemm:
        cfg5 = W.CONFIGS[5]
        M5 = 2048
        log(f"setup prefill: {cfg5.name}")
        # one bf16 input per group of projections that read it; the group's
        # GEMMs run through one bl_gemm_group call on its quantized codes
        by = {proj.name: proj for proj in cfg5.projs}
        G = []
        for names in PREFILL_GROUPS:
            inps = [W.proj_inputs(cfg5, by[n], M5) for n in names]
            K = by[names[0]].K
            x = to_dev(inps[0].x_bf16.view(np.int16)).view(torch.bfloat16)
            q = torch.empty((M5, K), dtype=torch.int8, device=dev)
            d = torch.empty((M5,), dtype=torch.float32, device=dev)
            probs = [dict(packed=bl.pack_i2s(to_dev(inp.w_tern)),
                          gamma=to_dev(np.array([inp.gamma], np.float32)),
                          y=torch.empty((M5, by[n].N), dtype=torch.bfloat16, device=dev))
                     for n, inp in zip(names, inps)]
            G.append(dict(names=names, x=x, q=q, d=d, group=bl.GemmGroup(probs, q, d),
                          ops=sum(2 * M5 * by[n].N * by[n].K for n in names)))
            del inps
        torch.cuda.synchronize()

        def layer(gemm_only=False):
            for e in G:
                if not gemm_only:
                    bl.quantize_act(e["x"], e["q"], e["d"])
                e["group"]()

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
        b0 = torch.cuda.Event(enable_timing=True)
        b1 = torch.cuda.Event(enable_timing=True)
        b0.record()
        for _ in range(args.gemm_steps):
            layer(gemm_only=True)
        b1.record()
        torch.cuda.synchronize()
        ms_gemm = b0.elapsed_time(b1) / args.gemm_steps
        gemm_tops = ops / (ms_gemm * 1e-3) / 1e12
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
            f"GEMM only {gemm_tops:.1f} TOPS; per group {per_group}")
        result["gemm"] = {"workload": cfg5.name, "tokens": M5, "ops_per_layer": ops,
                          "ms_per_layer": round(ms_layer, 4), "tops": round(tops, 1),
                          "gemm_only_tops": round(gemm_tops, 1), "peak_tops": INT8_PEAK_TOPS,
                          "frac": round(gemm_tops / INT8_PEAK_TOPS, 4),
                          "step": "per input: bl_quantize_act, then one bl_gemm_group for "
                                  "{q,k,v}, {o}, {gate,up}, {down}",
                          "tops_per_group": per_group}
        del G
        torch.cuda.empty_cache()

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
