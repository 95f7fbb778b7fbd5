"""Benchmark of the block-quantized decode matmuls on one MI355X.

Timed step: one decode token of a Qwen2.5-0.5B-shaped stack at M=1 with
Q8_0 weights and fp32 activations: 24 layers of qkv 896->1152, wo 896->896,
gate and up 896->4864, down 4864->896, then the LM head 896->151936.  Every
layer has its own weights, and steps alternate between two copies of the
whole stack (about 1.05 GB), so each step streams its 525 MB of weights from
HBM rather than from the 256 MB Infinity Cache.  The 121 launches of a step
are captured in one HIP graph per copy.  value = weight bytes per step /
wall time per step (GB/s).

The other parts of the path are timed alongside (kernel time from HIP events
on the launch stream, cold weights by rotation) and reported under "legs":
the Q8 x Q8 path at M=1 and M=32, the fused gate/up SwiGLU at M=8,
N=17408, K=5120, and the M=1024 Q4 x Q8 prefill matmul (plain and fused).
The reference oracle is timed on a bounded sample on the host cores.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-legs]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Q-GEMV weight-stream GB/s (% HBM peak) M=1 Q8_0; M=1024 int8 TOPS"
HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0
FP32_VALU_PEAK_TFLOPS = 78.6   # 256 CU x 4 SIMD x 16 lanes x 2 flop x 2.4 GHz, no packed FP32
N_LAYERS = 24
N_COPIES = 2


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def q8_bytes(n, k):
    return n * k + n * (k // 32) * 2


def q4_bytes(n, k):
    return n * (k // 2) + n * (k // 32) * 2


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-legs", action="store_true")
    ap.add_argument("--leg-iters", type=int, default=30)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    return ap.parse_args()


def event_times(torch, fn, iters, warm=3):
    """Per-call kernel time (ms) from HIP events on torch's current stream."""
    for i in range(warm):
        fn(i)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(iters)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(iters)]
    for i in range(iters):
        starts[i].record()
        fn(warm + i)
        ends[i].record()
    torch.cuda.synchronize()
    return np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU mode in this build)", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_quantized_decode_amd as qbd
    from block_quantized_decode_amd import datagen

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    log("device", props.name, getattr(props, "gcnArchName", ""))

    def gpu(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # ---------------------------------------------------------------- inputs
    t0 = time.time()
    layers = []   # [copy][layer] -> {name: (wq, wd)}
    heads = []
    for c in range(N_COPIES):
        layers.append([{k: (gpu(w), gpu(d)) for k, (w, d) in
                        datagen.decode_layer_weights(c * N_LAYERS + l).items()}
                       for l in range(N_LAYERS)])
        heads.append(tuple(gpu(a) for a in datagen.lm_head_weights(c)))
        log(f"weights copy {c} ready ({time.time() - t0:.1f}s)")
    acts = {k: gpu(v) for k, v in datagen.decode_activations(1).items()}
    outs = {name: torch.empty((1, n), dtype=torch.float32, device=dev)
            for name, n, _ in datagen.DECODE_LAYER}
    _, n_head, k_head = datagen.LM_HEAD
    logits = torch.empty((1, n_head), dtype=torch.float32, device=dev)

    layer_bytes = sum(q8_bytes(n, k) for _, n, k in datagen.DECODE_LAYER)
    head_bytes = q8_bytes(n_head, k_head)
    step_bytes = N_LAYERS * layer_bytes + head_bytes

    def step(c):
        for lw in layers[c]:
            for name, n, k in datagen.DECODE_LAYER:
                wq, wd = lw[name]
                qbd.qmv_q8_0_f32(wq, wd, acts[k], out=outs[name])
        qbd.qmv_q8_0_f32(heads[c][0], heads[c][1], acts[k_head], out=logits)

    # eager warm-up, then one graph per weight copy
    for i in range(3):
        step(i % N_COPIES)
    torch.cuda.synchronize()
    graphs = []
    for c in range(N_COPIES):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(c)
        graphs.append(g)
    torch.cuda.synchronize()
    log("graphs captured")

    for i in range(args.warmup):
        graphs[i % N_COPIES].replay()
    torch.cuda.synchronize()

    # ------------------------------------------------------------ timed steps
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        graphs[i % N_COPIES].replay()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = wall * 1e3 / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"step: {ms_per_step * 1e3:.1f} us wall, {gpu_ms * 1e3 / args.steps:.1f} us gpu, "
        f"{value:.0f} GB/s")

    # ------------------------------------------- per-kernel time, cold weights
    shape_stats = {}
    for name, n, k in datagen.DECODE_LAYER:
        def call(i, name=name, k=k):
            c, l = divmod(i % (N_COPIES * N_LAYERS), N_LAYERS)
            wq, wd = layers[c][l][name]
            qbd.qmv_q8_0_f32(wq, wd, acts[k], out=outs[name])
        t = event_times(torch, call, 96)
        shape_stats[name] = dict(N=n, K=k, bytes=q8_bytes(n, k), us=float(np.median(t) * 1e3))

    def call_head(i):
        c = i % N_COPIES
        qbd.qmv_q8_0_f32(heads[c][0], heads[c][1], acts[k_head], out=logits)
    t = event_times(torch, call_head, 40)
    shape_stats["lm_head"] = dict(N=n_head, K=k_head, bytes=head_bytes, us=float(np.median(t) * 1e3))
    for s in shape_stats.values():
        s["GBs"] = s["bytes"] / (s["us"] * 1e-6) / 1e9
    per_layer_kernel_us = sum(shape_stats[nm]["us"] for nm, _, _ in datagen.DECODE_LAYER)
    log("per-shape:", {k: round(v["GBs"]) for k, v in shape_stats.items()})

    # dominant kernel: the LM head launch (largest single stream, its own
    # kernel instantiation: rows-per-wave 4 is used only for N >= 32768)
    hs = shape_stats["lm_head"]
    roofline = {"bound": "hbm", "achieved": round(hs["GBs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(hs["GBs"] / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": "qmv_f32_m1<Q8_0,Plain,J=1,R=4> (LM head 896->151936)",
                "bytes_per_launch": head_bytes, "avg_launch_us": round(hs["us"], 3)}

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; Q8_0 codes U[-127,127], fp16 scales U[0.001,0.02], x ~ N(0,1))",
        "config": {"workload": "decode token, Qwen2.5-0.5B-shaped: 24 x (qkv 896->1152, wo 896->896, "
                               "gate 896->4864, up 896->4864, down 4864->896) + lm_head 896->151936, "
                               "M=1, Q8_0 weights x fp32 activations",
                   "M": 1, "layers": N_LAYERS, "weight_bytes_per_step": step_bytes,
                   "weight_copies": N_COPIES, "launches_per_step": N_LAYERS * 5 + 1,
                   "hip_graph": True},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(1e3 / ms_per_step, 2),
        "gpu_us_per_step": round(gpu_ms * 1e3 / args.steps, 2),
        "per_layer_kernel_us": round(per_layer_kernel_us, 3),
        "per_shape": shape_stats,
        "roofline": roofline,
    }

    if not args.no_legs:
        result["legs"] = run_legs(torch, qbd, datagen, gpu, dev, args.leg_iters)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(datagen, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def run_legs(torch, qbd, datagen, gpu, dev, iters):
    legs = {}

    # Q8 x Q8 path: quantize + qmm over the decode-layer shapes at M=1 and M=32
    n_rot = 8
    wsets = [{k: (gpu(w), gpu(d)) for k, (w, d) in datagen.decode_layer_weights(100 + r).items()}
             for r in range(n_rot)]
    layer_bytes = sum(q8_bytes(n, k) for _, n, k in datagen.DECODE_LAYER)
    for m in (1, datagen.PP32_M):
        xs = {k: gpu(datagen.activations(np.random.default_rng(m * 10 + k), m, k, outliers=True))
              for k in (896, 4864)}
        xqs = {k: qbd.quantize_act_q8_0(v) for k, v in xs.items()}
        outs = {name: torch.empty((m, n), dtype=torch.float32, device=dev)
                for name, n, _ in datagen.DECODE_LAYER}

        def layer(i):
            ws = wsets[i % n_rot]
            for name, n, k in datagen.DECODE_LAYER:
                qbd.quantize_act_q8_0(xs[k], *xqs[k])
                xq, xd = xqs[k]
                qbd.qmm_q8_0_q8act(ws[name][0], ws[name][1], xq, xd, out=outs[name])
        t = event_times(torch, layer, iters) * 1e3
        us = float(np.median(t))
        legs[f"q8q8_layer_M{m}"] = {"us_per_layer": round(us, 3),
                                    "weight_GBs": round(layer_bytes / (us * 1e-6) / 1e9, 1),
                                    "int8_TOPS": round(2 * m * sum(n * k for _, n, k in datagen.DECODE_LAYER)
                                                       / (us * 1e-6) / 1e12, 3),
                                    "includes": "5 x (quantize_act_q8_0 + qmm_q8_0_q8act)"}
    log("q8q8 legs done")
    del wsets

    # fused gate/up SwiGLU, M=8, N=17408, K=5120 (Q4 x fp32)
    n_rot = 6
    sets = []
    for r in range(n_rot):
        gq, gd, uq, ud, x = datagen.gate_up_inputs() if r == 0 else (None,) * 5
        if r > 0:
            rr = datagen.streams(30 + r, 4)
            gq, gd = datagen.q4_weights(rr[0], rr[1], datagen.GATE_UP["N"], datagen.GATE_UP["K"])
            uq, ud = datagen.q4_weights(rr[2], rr[3], datagen.GATE_UP["N"], datagen.GATE_UP["K"])
        sets.append(tuple(gpu(a) for a in (gq, gd, uq, ud)))
        if r == 0:
            xg = gpu(x)
    M4, N4, K4 = datagen.GATE_UP["M"], datagen.GATE_UP["N"], datagen.GATE_UP["K"]
    out4 = torch.empty((M4, N4), dtype=torch.float32, device=dev)
    g4 = torch.empty_like(out4)
    u4 = torch.empty_like(out4)
    t_fused = event_times(torch, lambda i: qbd.gate_up_swiglu_q4(*sets[i % n_rot], xg, out=out4), iters)

    def unfused(i):
        s = sets[i % n_rot]
        qbd.qmv_q4_0_f32(s[0], s[1], xg, out=g4)
        qbd.qmv_q4_0_f32(s[2], s[3], xg, out=u4)
        qbd.swiglu_f32(g4, u4, out=out4)
    t_unf = event_times(torch, unfused, iters)
    wbytes = 2 * q4_bytes(N4, K4)
    us_f = float(np.median(t_fused) * 1e3)
    us_u = float(np.median(t_unf) * 1e3)
    flops = 2 * 2 * M4 * N4 * K4
    legs["gate_up_swiglu_M8"] = {"us": round(us_f, 3), "unfused_us": round(us_u, 3),
                                 "fused_vs_unfused_time": round(us_f / us_u - 1, 4),
                                 "weight_GBs": round(wbytes / (us_f * 1e-6) / 1e9, 1),
                                 "pct_hbm": round(100 * wbytes / (us_f * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
                                 "TFLOPs": round(flops / (us_f * 1e-6) / 1e12, 2),
                                 "pct_fp32_valu": round(100 * flops / (us_f * 1e-6) / 1e12
                                                        / FP32_VALU_PEAK_TFLOPS, 2)}
    log("gate/up leg done")
    del sets

    # prefill M=1024, N=17408, K=5120, Q4 x Q8 activations
    gq, gd, uq, ud, x = datagen.prefill_inputs()
    P = [gpu(a) for a in (gq, gd, uq, ud)]
    xp = gpu(x)
    M5, N5, K5 = datagen.PREFILL["M"], datagen.PREFILL["N"], datagen.PREFILL["K"]
    xq, xd = qbd.quantize_act_q8_0(xp)
    y5 = torch.empty((M5, N5), dtype=torch.float32, device=dev)
    it5 = max(5, iters // 3)
    t_q = event_times(torch, lambda i: qbd.quantize_act_q8_0(xp, xq, xd), it5)
    t_p = event_times(torch, lambda i: qbd.qmm_q4_0_q8act(P[0], P[1], xq, xd, out=y5), it5)
    t_f = event_times(torch, lambda i: qbd.gate_up_swiglu_q4_q8act(*P, xq, xd, out=y5), it5)
    ops = 2 * M5 * N5 * K5
    us_p = float(np.median(t_p) * 1e3)
    us_f = float(np.median(t_f) * 1e3)
    legs["prefill_M1024"] = {"quantize_us": round(float(np.median(t_q) * 1e3), 3),
                             "plain_us": round(us_p, 3),
                             "plain_int8_TOPS": round(ops / (us_p * 1e-6) / 1e12, 2),
                             "plain_pct_int8_peak": round(100 * ops / (us_p * 1e-6) / 1e12 / INT8_PEAK_TOPS, 2),
                             "fused_us": round(us_f, 3),
                             "fused_int8_TOPS": round(2 * ops / (us_f * 1e-6) / 1e12, 2),
                             "fused_pct_int8_peak": round(100 * 2 * ops / (us_f * 1e-6) / 1e12
                                                          / INT8_PEAK_TOPS, 2)}
    log("prefill leg done")
    return legs


def cpu_baseline(datagen, seconds):
    """The oracle on the host cores, on a bounded sample of the decode step:
    whole decode layers (all five shapes) and LM-head row slices, repeated
    until about `seconds` of CPU time; reported as weight GB/s."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = 1
    mats = datagen.decode_layer_weights(0)
    acts = datagen.decode_activations(1)
    wq_h, wd_h = datagen.lm_head_weights(0)
    rows = 151936 // 16
    head = (wq_h[:rows], wd_h[:rows])
    done_bytes = 0
    layers = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for name, n, k in datagen.DECODE_LAYER:
            wq, wd = mats[name]
            oracle.qmv_q8_0_f32(wq, wd, acts[k])
            done_bytes += q8_bytes(n, k)
        oracle.qmv_q8_0_f32(head[0], head[1], acts[896])
        done_bytes += q8_bytes(rows, 896)
        layers += 1
    el = time.perf_counter() - t0
    return {"value": round(done_bytes / el / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{layers} x (one decode layer: qkv, wo, gate, up, down + 1/16 of the LM head rows), "
                      f"M=1, float64 numpy oracle, {el:.1f} s"}


if __name__ == "__main__":
    main()
