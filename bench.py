"""Benchmark of the block-quantized decode matmuls on one MI355X.

Timed step (the decode-layer workload): one Qwen2.5-0.5B-shaped decode
layer plus the LM head at M=1, Q8_0 weights x fp32 activations - qkv
896->1152, wo 896->896, gate and up 896->4864 as one fused SwiGLU launch
whose output feeds down 4864->896, then lm_head 896->151936 - launched in
dependency order on one stream and captured in one HIP graph per weight
copy (the same step with gate and up as two plain launches is reported
beside it).  Steps rotate over 6 copies of
all weights (about 963 MB), so every step streams its 160.5 MB from HBM
rather than from the 256 MB Infinity Cache.  value = weight bytes per step
/ wall time per step (GB/s).

roofline: the LM-head launch, the largest weight stream of the step and a
kernel instantiation of its own (the grid-capped looping GEMV), timed live
with HIP events over back-to-back launches on the launch stream (cold
copies).  Its HBM traffic comes from the committed PMC profile of that
kernel and is reported only while the kernel source is unchanged.
read_ceiling: a plain streaming read of the same number of bytes
(libqbd_ceiling.so), timed the same way, beside the nominal 8 TB/s: one
launch's launch, ramp and drain cost a few microseconds that no kernel
streaming that many bytes in one launch avoids.

legs (timed alongside, kernel time from HIP events on the launch stream,
cold weights by rotation): a 24-layer decode token, the Q8 x Q8 path at
M=1 and M=32 (quantize + matmul per projection, graphed), the fused gate/up
SwiGLU at M=8, N=17408, K=5120 (and its unfused composition), the 4-bit
FFN of the 27B-class target at M=1 (fused gate/up + down) and its down
projection at M=8, and the M=1024 Q4 x Q8 prefill product (plain and
fused).  A/B comparisons (fused against unfused, a shared activation
producer against one per consumer, fp32 against Q8 x Q8 activations at
M=1) are timed in 20 paired rounds whose order alternates, and reported as
p10 / median / p90 with the median of the per-round ratios.  Every long
launch (the LM head, the 4-bit and M=8 legs, the prefill) first runs back to
back for about 30 ms of GPU time, untimed, so that it is timed at the
sustained clock.  cpu_baseline: the reference oracle on a bounded sample of
the step, on the host cores.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-legs] [--no-cpu-baseline]
"""
import argparse
import hashlib
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
FP32_VALU_PEAK_TFLOPS = 78.6   # 256 CU x 64 FMA lanes x 2 flop x 2.4 GHz (no packed FP32)
N_COPIES = 6
N_LAYERS_TOKEN = 24
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "lm_head_gemv_traffic.txt")
GEMV_SOURCE = os.path.join(ROOT, "block_quantized_decode_amd", "csrc", "qmv_f32.hip")


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
    ap.add_argument("--legs", default="",
                    help="comma-separated leg names to run (default: all), e.g. prefill_M1024 for a profiler")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run device copies of this size (a known-size kernel for PMC calibration)")
    return ap.parse_args()


def source_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profile(kernel_bytes):
    """HBM bytes per LM-head launch from the committed PMC profile, or None
    if there is none or the GEMV source changed since it was taken."""
    try:
        kv = {}
        with open(TRAFFIC_PROFILE) as f:
            for ln in f:
                if "=" in ln and not ln.startswith("#"):
                    k, v = ln.split("=", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_source_sha256_16") != source_sha(GEMV_SOURCE):
            return None
        return int(round(float(kv["hbm_bytes_per_launch"])))
    except (OSError, KeyError, ValueError):
        return None


def event_ms(torch, fn, iters, warm=2):
    """Per-call time (ms): HIP events around each call on the current stream."""
    for i in range(warm):
        fn(i)
    s = [torch.cuda.Event(enable_timing=True) for _ in range(iters)]
    e = [torch.cuda.Event(enable_timing=True) for _ in range(iters)]
    for i in range(iters):
        s[i].record()
        fn(warm + i)
        e[i].record()
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in zip(s, e)])


SETTLE_MS = 30.0


def settle(torch, fn, ms=SETTLE_MS):
    """Run fn back to back for about `ms` of GPU time, untimed.  From idle
    the GPU clocks take about 20 ms of continuous work to reach their
    sustained level: the LM-head GEMV runs 25.1 us per launch at first and
    23.6 us once settled, the M=1024 prefill product 348 and 272 us.  Each
    long launch is therefore settled before its timed batches."""
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(4):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    per_call = max(a.elapsed_time(b) / 4, 1e-3)
    for i in range(int(ms / per_call) + 1):
        fn(i)
    torch.cuda.synchronize()


def batch_stats(torch, fn, calls, reps=5, warm=3):
    """Time per call (ms) of `calls` back-to-back calls between two HIP
    events on the current stream, for each of `reps` batches."""
    for i in range(warm):
        fn(i)
    out = []
    k = 0
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(calls):
            fn(k)
            k += 1
        b.record()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) / calls)
    return np.array(out)


def batch_ms(torch, fn, calls, reps=5, warm=3):
    """Median over `reps` batches of batch_stats."""
    return float(np.median(batch_stats(torch, fn, calls, reps, warm)))


def paired_ms(torch, fa, fb, rounds=20, calls=6, warm=3):
    """A/B comparison in paired rounds.  Each round times `calls` back-to-back
    calls of fa and then of fb (the order alternates from round to round),
    HIP events around each batch, so that slow drifts of clock and
    temperature hit both arms alike.  Returns per-call times (ms) of both
    arms per round and the per-round ratios a / b."""
    for i in range(warm):
        fa(i)
        fb(i)
    torch.cuda.synchronize()
    ta, tb = [], []
    k = 0
    for r in range(rounds):
        res = {}
        for arm in (("a", "b") if r % 2 == 0 else ("b", "a")):
            f = fa if arm == "a" else fb
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(calls):
                f(k)
                k += 1
            e1.record()
            torch.cuda.synchronize()
            res[arm] = e0.elapsed_time(e1) / calls
        ta.append(res["a"])
        tb.append(res["b"])
    ta, tb = np.array(ta), np.array(tb)
    return ta, tb, ta / tb


def pct_us(t_ms):
    """p10, median and p90 of per-call times (ms), in us."""
    p = np.percentile(np.asarray(t_ms) * 1e3, [10, 50, 90])
    return [round(float(v), 3) for v in p]


def ab_summary(ta, tb, ratio):
    """The paired comparison as reported: medians, spreads and ratio."""
    return {"rounds": int(len(ratio)), "a_us_p10_p50_p90": pct_us(ta), "b_us_p10_p50_p90": pct_us(tb),
            "ratio_a_over_b_p10_p50_p90": [round(float(v), 4) for v in np.percentile(ratio, [10, 50, 90])]}


def graph_ms(torch, graphs, reps):
    """Average replay time (ms) of HIP graphs replayed round-robin."""
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(reps):
        graphs[i % len(graphs)].replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def capture(torch, fn):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


CEILING_LIB = os.path.join(ROOT, "block_quantized_decode_amd", "libqbd_ceiling.so")


class ReadCeiling:
    """The streaming-read reference kernel (include/qbd_ceiling.h) over
    N_COPIES buffers of a given size, called like a product launch (call(i)
    reads copy i % N_COPIES), so that it can be timed exactly as the product
    it is compared with: its time for the product's weight bytes is the most
    that one launch streaming those bytes can reach here."""

    def __init__(self, torch, dev, nbytes):
        import ctypes
        lib = ctypes.CDLL(CEILING_LIB)
        lib.qbd_read_ceiling.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        lib.qbd_read_ceiling.restype = ctypes.c_int
        lib.qbd_read_ceiling_sink_words.restype = ctypes.c_int64
        self.lib, self.torch, self.ctypes = lib, torch, ctypes
        self.nbytes = (int(nbytes) + 15) // 16 * 16
        self.bufs = [torch.full((self.nbytes,), c + 1, dtype=torch.uint8, device=dev) for c in range(N_COPIES)]
        self.sink = torch.empty(int(lib.qbd_read_ceiling_sink_words()), dtype=torch.int32, device=dev)

    def __call__(self, i):
        st = self.lib.qbd_read_ceiling(self.bufs[i % N_COPIES].data_ptr(), self.nbytes, self.sink.data_ptr(),
                                       self.ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise RuntimeError(f"qbd_read_ceiling returned {st}")

    def report(self, ms, product_ms):
        gbs = self.nbytes / (ms * 1e-3) / 1e9
        return {"us": round(ms * 1e3, 3), "GBs": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                "product_frac_of_ceiling": round(ms / product_ms, 4),
                "kernel": "qbd_read_ceiling: a plain streaming read of the same bytes, timed the same way"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the decode matmuls "
              "run on one GPU (each GPU of a sharded deployment would run these kernels on its own "
              "slice of the weight rows)",
              file=sys.stderr)
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

    # ------------------------------------------------------------ inputs
    t0 = time.time()
    copies = []
    for c in range(N_COPIES):
        layer = {k: (gpu(w), gpu(d)) for k, (w, d) in datagen.decode_layer_weights(c).items()}
        head = tuple(gpu(a) for a in datagen.lm_head_weights(c))
        copies.append((layer, head))
    log(f"{N_COPIES} weight copies ready ({time.time() - t0:.1f}s)")
    acts = {k: gpu(v) for k, v in datagen.decode_activations(1).items()}
    outs = {name: torch.empty((1, n), dtype=torch.float32, device=dev)
            for name, n, _ in datagen.DECODE_LAYER}
    _, n_head, k_head = datagen.LM_HEAD
    logits = torch.empty((1, n_head), dtype=torch.float32, device=dev)

    layer_bytes = sum(q8_bytes(n, k) for _, n, k in datagen.DECODE_LAYER)
    head_bytes = q8_bytes(n_head, k_head)
    step_bytes = layer_bytes + head_bytes

    h = torch.empty((1, dict((nm, n) for nm, n, _ in datagen.DECODE_LAYER)["gate"]),
                    dtype=torch.float32, device=dev)

    def run_layer(layer):
        # qkv, wo, then gate and up in one fused SwiGLU launch whose output
        # feeds the down projection
        qbd.qmv_q8_0_f32(*layer["qkv"], acts[896], out=outs["qkv"])
        qbd.qmv_q8_0_f32(*layer["wo"], acts[896], out=outs["wo"])
        qbd.gate_up_swiglu_q8_0(*layer["gate"], *layer["up"], acts[896], out=h)
        qbd.qmv_q8_0_f32(*layer["down"], h, out=outs["down"])

    def run_layer_unfused(layer):
        for name, n, k in datagen.DECODE_LAYER:
            wq, wd = layer[name]
            qbd.qmv_q8_0_f32(wq, wd, acts[k], out=outs[name])

    def step(c):
        layer, head = copies[c]
        run_layer(layer)
        qbd.qmv_q8_0_f32(head[0], head[1], acts[k_head], out=logits)

    def step_unfused(c):
        layer, head = copies[c]
        run_layer_unfused(layer)
        qbd.qmv_q8_0_f32(head[0], head[1], acts[k_head], out=logits)

    if args.copy_probe_mib > 0:
        nb = args.copy_probe_mib << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: 3 x {args.copy_probe_mib} MiB device copies")

    for i in range(2 * N_COPIES):
        step(i % N_COPIES)
    torch.cuda.synchronize()
    # One HIP graph holds a whole sequence of steps (copies in rotation), so
    # a step's launches follow each other on the device with no host work
    # between steps, as the layers of a token do.  One graph per step adds
    # a host graph launch (about 6 us) to every step; that figure is
    # reported beside the headline.
    rotation = capture(torch, lambda: [step(c) for c in range(N_COPIES)])
    timed = capture(torch, lambda: [step(i % N_COPIES) for i in range(args.steps)])
    warm = capture(torch, lambda: [step(i % N_COPIES) for i in range(args.warmup)]) if args.warmup else None
    torch.cuda.synchronize()
    # clocks: replay steps back to back for about 30 ms first (untimed, like
    # every leg below), so that K steps are timed at the sustained clock
    # whatever W and K are; then the W warmup steps
    settle(torch, lambda i: rotation.replay())
    if warm is not None:
        warm.replay()
    torch.cuda.synchronize()

    # ----------------------------------------------------------- timed steps
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record()
    timed.replay()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = wall * 1e3 / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"step: {ms_per_step * 1e3:.2f} us wall, {gpu_ms * 1e3 / args.steps:.2f} us gpu, {value:.0f} GB/s")
    del timed, warm
    # spread over rotations (outside the timed region): each replay of the
    # rotation graph between two HIP events, per step
    step_t = event_ms(torch, lambda i: rotation.replay(), 40, warm=2) / N_COPIES
    # one graph launch per step (host launch overhead between steps)
    graphs = [capture(torch, lambda c=c: step(c)) for c in range(N_COPIES)]
    settle(torch, lambda i: graphs[i % N_COPIES].replay())
    one_per_step_ms = batch_ms(torch, lambda i: graphs[i % N_COPIES].replay(), 4 * N_COPIES, reps=5)
    del graphs

    # the same step with gate and up as two plain launches (six launches)
    for i in range(N_COPIES):
        step_unfused(i)
    torch.cuda.synchronize()
    rotation_u = capture(torch, lambda: [step_unfused(c) for c in range(N_COPIES)])
    ta, tb, ratio = paired_ms(torch, lambda k: rotation.replay(), lambda k: rotation_u.replay(), rounds=20, calls=2)
    ta, tb = ta / N_COPIES, tb / N_COPIES
    unfused_us = float(np.median(tb)) * 1e3
    step_ab = ab_summary(ta, tb, ratio)
    del rotation_u

    # -------------------------------------- per-launch time, cold weights
    # (the layer's launches are shorter than their host-side launch cost,
    # so each is timed in one HIP graph of four calls per weight copy)
    def graph_call_ms(call):
        for i in range(N_COPIES):
            call(i)
        torch.cuda.synchronize()
        g = capture(torch, lambda: [call(i) for i in range(4 * N_COPIES)])
        ms = graph_ms(torch, [g], 20) / (4 * N_COPIES)
        del g
        return ms

    per_shape = {}
    for name, n, k in datagen.DECODE_LAYER:
        def call(i, name=name, k=k):
            wq, wd = copies[i % N_COPIES][0][name]
            qbd.qmv_q8_0_f32(wq, wd, acts[k], out=outs[name])
        ms = graph_call_ms(call)
        per_shape[name] = {"N": n, "K": k, "bytes": q8_bytes(n, k), "us": round(ms * 1e3, 3),
                           "GBs": round(q8_bytes(n, k) / (ms * 1e-3) / 1e9, 1)}

    def call_gate_up(i):
        layer = copies[i % N_COPIES][0]
        qbd.gate_up_swiglu_q8_0(*layer["gate"], *layer["up"], acts[896], out=h)
    ms = graph_call_ms(call_gate_up)
    gu_bytes = per_shape["gate"]["bytes"] + per_shape["up"]["bytes"]
    per_shape["gate_up_swiglu"] = {"N": h.shape[1], "K": 896, "bytes": gu_bytes, "us": round(ms * 1e3, 3),
                                   "GBs": round(gu_bytes / (ms * 1e-3) / 1e9, 1)}

    def call_head(i):
        head = copies[i % N_COPIES][1]
        qbd.qmv_q8_0_f32(head[0], head[1], acts[k_head], out=logits)
    settle(torch, call_head)
    head_t = batch_stats(torch, call_head, 24, reps=7)
    head_ms = float(np.median(head_t))
    per_shape["lm_head"] = {"N": n_head, "K": k_head, "bytes": head_bytes, "us": round(head_ms * 1e3, 3),
                            "GBs": round(head_bytes / (head_ms * 1e-3) / 1e9, 1)}
    log("per-launch GB/s:", {k: v["GBs"] for k, v in per_shape.items()})

    ceil = ReadCeiling(torch, dev, head_bytes)
    settle(torch, ceil)
    head_ceiling = ceil.report(float(np.median(batch_stats(torch, ceil, 24, reps=7))), head_ms)
    del ceil

    achieved = head_bytes / (head_ms * 1e-3) / 1e9
    traffic = traffic_from_profile(head_bytes)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "qmv_f32_m1_pipe<Q8_0, Plain, J=1, R=4> (LM head 896->151936, M=1)",
                "algorithmic_bytes_per_launch": head_bytes, "avg_launch_us": round(head_ms * 1e3, 3),
                "launch_us_p10_p50_p90": pct_us(head_t), "read_ceiling": head_ceiling}

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
        "data": "synthetic, seeded: Q8_0 codes U[-127,127], fp16 scales U[0.001,0.02], x ~ N(0,1)",
        "config": {"workload": "Qwen2.5-0.5B-shaped decode layer + LM head at M=1, Q8_0 x fp32: "
                               "qkv 896->1152, wo 896->896, gate+up 896->2x4864 as one fused SwiGLU "
                               "launch, down 4864->896 on its output, lm_head 896->151936",
                   "M": 1, "weight_bytes_per_step": step_bytes, "launches_per_step": 5,
                   "weight_copies": N_COPIES, "hip_graph": f"{args.steps} steps per graph"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "gpu_us_per_step": round(gpu_ms * 1e3 / args.steps, 3),
        "step_us_p10_p50_p90": pct_us(step_t),
        "timing": f"{args.steps} steps captured in one HIP graph (weight copies in rotation), one replay timed",
        "one_graph_per_step_us": round(one_per_step_ms * 1e3, 3),
        "unfused_gate_up_step_us": round(unfused_us, 3),
        "fused_vs_unfused_step": dict(step_ab, a="fused gate/up (5 launches)", b="gate and up unfused (6 launches)"),
        "layer_us": round(sum(per_shape[nm]["us"] for nm in ("qkv", "wo", "gate_up_swiglu", "down")), 3),
        "per_launch": per_shape,
        "roofline": roofline,
    }

    if not args.no_legs:
        legs = {}
        only = set(args.legs.split(",")) if args.legs else None
        if only is None or "decode_token_24_layers" in only:
            legs["decode_token_24_layers"] = leg_token(torch, qbd, datagen, gpu, dev, copies, acts, outs, logits)
        legs.update(run_legs(torch, qbd, datagen, gpu, dev, args.leg_iters, only))
        result["legs"] = legs
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(datagen, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def leg_token(torch, qbd, datagen, gpu, dev, copies, acts, outs, logits):
    """24 distinct layers + the LM head, one HIP graph (one token)."""
    layers = [{k: (gpu(w), gpu(d)) for k, (w, d) in datagen.decode_layer_weights(100 + l).items()}
              for l in range(N_LAYERS_TOKEN)]
    _, n_head, k_head = datagen.LM_HEAD
    head = copies[0][1]

    h = torch.empty((1, dict((nm, n) for nm, n, _ in datagen.DECODE_LAYER)["gate"]),
                    dtype=torch.float32, device=dev)

    def token():
        for layer in layers:
            qbd.qmv_q8_0_f32(*layer["qkv"], acts[896], out=outs["qkv"])
            qbd.qmv_q8_0_f32(*layer["wo"], acts[896], out=outs["wo"])
            qbd.gate_up_swiglu_q8_0(*layer["gate"], *layer["up"], acts[896], out=h)
            qbd.qmv_q8_0_f32(*layer["down"], h, out=outs["down"])
        qbd.qmv_q8_0_f32(head[0], head[1], acts[k_head], out=logits)

    token()
    torch.cuda.synchronize()
    g = capture(torch, token)
    ms = graph_ms(torch, [g], 30)
    nbytes = N_LAYERS_TOKEN * sum(q8_bytes(n, k) for _, n, k in datagen.DECODE_LAYER) + q8_bytes(n_head, k_head)
    del layers
    log(f"24-layer token: {ms * 1e3:.1f} us")
    return {"us_per_token": round(ms * 1e3, 2), "tokens_per_s": round(1e3 / ms, 1),
            "weight_GBs": round(nbytes / (ms * 1e-3) / 1e9, 1), "weight_bytes": nbytes,
            "launches": N_LAYERS_TOKEN * 4 + 1}


def run_legs(torch, qbd, datagen, gpu, dev, iters, only=None):
    """The extra legs; `only` (a set of leg names) runs a subset of them."""
    legs = {}

    def want(name):
        return only is None or name in only

    if want("q8q8_layer") or want("m1_per_shape_choice"):
        # Q8 x Q8: per projection, quantize its input then the int-dot matmul
        n_rot = N_COPIES
        wsets = [{k: (gpu(w), gpu(d)) for k, (w, d) in datagen.decode_layer_weights(200 + r).items()}
                 for r in range(n_rot)]
        layer_bytes = sum(q8_bytes(n, k) for _, n, k in datagen.DECODE_LAYER)
        layer_macs = sum(n * k for _, n, k in datagen.DECODE_LAYER)
        for m in (1, datagen.PP32_M):
            xs = {k: gpu(datagen.activations(np.random.default_rng(m * 10 + k), m, k, outliers=True))
                  for k in (896, 4864)}
            xqs = {k: qbd.quantize_act_q8_0(v) for k, v in xs.items()}
            outs = {name: torch.empty((m, n), dtype=torch.float32, device=dev)
                    for name, n, _ in datagen.DECODE_LAYER}

            def layer(ws):
                for name, n, k in datagen.DECODE_LAYER:
                    qbd.quantize_act_q8_0(xs[k], *xqs[k])
                    xq, xd = xqs[k]
                    qbd.qmm_q8_0_q8act(ws[name][0], ws[name][1], xq, xd, out=outs[name])

            # one activation producer shared by the gate and up consumers (they
            # read the same input): four quantizations per layer instead of five
            def layer_shared(ws):
                for name, n, k in datagen.DECODE_LAYER:
                    if name != "up":
                        qbd.quantize_act_q8_0(xs[k], *xqs[k])
                    xq, xd = xqs[k]
                    qbd.qmm_q8_0_q8act(ws[name][0], ws[name][1], xq, xd, out=outs[name])

            # one producer per distinct activation panel: in this layer's
            # wiring qkv, wo, gate and up read one 896-wide panel and down
            # the 4864-wide one, so two quantizations feed five consumers
            def layer_one_per_panel(ws):
                for k in (896, 4864):
                    qbd.quantize_act_q8_0(xs[k], *xqs[k])
                for name, n, k in datagen.DECODE_LAYER:
                    xq, xd = xqs[k]
                    qbd.qmm_q8_0_q8act(ws[name][0], ws[name][1], xq, xd, out=outs[name])
            # at M=1: each distinct panel comes from its first consumer's
            # quantize-and-multiply call (one launch each): the gate's call
            # produces the 896-wide panel that qkv, wo and up then read, and
            # down's call quantizes its own 4864-wide panel; 5 launches
            def layer_first_consumer_produces(ws):
                xq, xd = xqs[896]
                qbd.qmm_q8_0_q8act_from_f32(ws["gate"][0], ws["gate"][1], xs[896], xq, xd, out=outs["gate"])
                for name in ("qkv", "wo", "up"):
                    qbd.qmm_q8_0_q8act(ws[name][0], ws[name][1], xq, xd, out=outs[name])
                qbd.qmm_q8_0_q8act_from_f32(ws["down"][0], ws["down"][1], xs[4864], *xqs[4864], out=outs["down"])
            for ws in wsets:
                layer(ws)
                layer_shared(ws)
                layer_one_per_panel(ws)
                layer_first_consumer_produces(ws)
            torch.cuda.synchronize()
            # each arrangement: one graph over all weight sets (layers back to
            # back on the device), paired rounds, time per layer
            g5 = capture(torch, lambda: [layer(ws) for ws in wsets])
            g4 = capture(torch, lambda: [layer_shared(ws) for ws in wsets])
            g2 = capture(torch, lambda: [layer_one_per_panel(ws) for ws in wsets])
            settle(torch, lambda i: g5.replay())
            ta, tb, ratio = paired_ms(torch, lambda k: g5.replay(), lambda k: g4.replay(), rounds=20, calls=2)
            tc, td, ratio2 = paired_ms(torch, lambda k: g5.replay(), lambda k: g2.replay(), rounds=20, calls=2)
            ta, tb, tc, td = ta / n_rot, tb / n_rot, tc / n_rot, td / n_rot
            us, us_s, us_p = float(np.median(ta)) * 1e3, float(np.median(tb)) * 1e3, float(np.median(td)) * 1e3
            legs[f"q8q8_layer_M{m}"] = {"us_per_layer": round(us, 3),
                                        "weight_GBs": round(layer_bytes / (us * 1e-6) / 1e9, 1),
                                        "int8_TOPS": round(2 * m * layer_macs / (us * 1e-6) / 1e12, 3),
                                        "launches": "5 x (quantize_act_q8_0 + qmm_q8_0_q8act); the layers of "
                                                    f"{n_rot} weight sets in one HIP graph",
                                        "shared_gate_up_producer_us": round(us_s, 3),
                                        "separate_vs_shared_producer": dict(
                                            ab_summary(ta, tb, ratio), a="5 producers", b="4 producers (gate and up share)"),
                                        "one_producer_per_panel_us": round(us_p, 3),
                                        "separate_vs_one_per_panel": dict(
                                            ab_summary(tc, td, ratio2), a="5 producers",
                                            b="2 producers (one per distinct panel) for 5 consumers")}
            if m == 1:
                g1 = capture(torch, lambda: [layer_first_consumer_produces(ws) for ws in wsets])
                te, tf, ratio3 = paired_ms(torch, lambda k: g2.replay(), lambda k: g1.replay(), rounds=20, calls=2)
                te, tf = te / n_rot, tf / n_rot
                legs[f"q8q8_layer_M{m}"]["first_consumer_produces_us"] = round(float(np.median(tf)) * 1e3, 3)
                legs[f"q8q8_layer_M{m}"]["one_per_panel_vs_first_consumer_produces"] = dict(
                    ab_summary(te, tf, ratio3), a="2 producers (one per distinct panel)",
                    b="each panel produced by its first consumer's quantize-and-multiply call (5 launches)")
                del g1
            del g5, g4, g2
        log("q8q8 legs done")

        # per-shape choice at M=1 (Lumen's hybrid dispatch): Q8_0 x fp32 GEMV
        # against quantize + Q8 x Q8 product, per decode-layer shape, cold
        # weights, each variant captured in a HIP graph (per-launch GPU time)
        choice = {}
        xs1 = {k: gpu(datagen.activations(np.random.default_rng(11 + k), 1, k)) for k in (896, 4864)}
        xq1 = {k: qbd.quantize_act_q8_0(v) for k, v in xs1.items()}
        for name, n, k in datagen.DECODE_LAYER:
            out1 = torch.empty((1, n), dtype=torch.float32, device=dev)

            def f32(i, name=name, k=k, out1=out1):
                w = wsets[i % n_rot][name]
                qbd.qmv_q8_0_f32(w[0], w[1], xs1[k], out=out1)

            def q8q8(i, name=name, k=k, out1=out1):
                w = wsets[i % n_rot][name]
                qbd.quantize_act_q8_0(xs1[k], *xq1[k])
                qbd.qmm_q8_0_q8act(w[0], w[1], *xq1[k], out=out1)

            # the same in one call (one launch where the staged kernel
            # quantizes the panel itself: N >= 4096)
            def q8x(i, name=name, k=k, out1=out1):
                w = wsets[i % n_rot][name]
                qbd.qmm_q8_0_q8act_from_f32(w[0], w[1], xs1[k], *xq1[k], out=out1)
            for i in range(n_rot):
                f32(i)
                q8q8(i)
                q8x(i)
            torch.cuda.synchronize()
            g_f = capture(torch, lambda: [f32(i) for i in range(n_rot)])
            g_q = capture(torch, lambda: [q8q8(i) for i in range(n_rot)])
            g_x = capture(torch, lambda: [q8x(i) for i in range(n_rot)])
            ta, tb, ratio = paired_ms(torch, lambda k: g_f.replay(), lambda k: g_q.replay(), rounds=20,
                                      calls=4)
            tc, td, ratio_x = paired_ms(torch, lambda k: g_f.replay(), lambda k: g_x.replay(), rounds=20,
                                        calls=4)
            t_f, t_q = float(np.median(ta)) * 1e3 / n_rot, float(np.median(tb)) * 1e3 / n_rot
            t_x = float(np.median(td)) * 1e3 / n_rot
            times = {"q8_f32": t_f, "q8q8": t_q, "q8q8_from_f32": t_x}
            choice[name] = {"N": n, "K": k, "q8_f32_us": round(t_f, 3), "quantize_plus_q8q8_us": round(t_q, 3),
                            "q8q8_from_f32_us": round(t_x, 3), "faster": min(times, key=times.get),
                            "ratio_f32_over_q8q8_p10_p50_p90": [round(float(v), 4)
                                                                for v in np.percentile(ratio, [10, 50, 90])],
                            "ratio_f32_over_from_f32_p10_p50_p90": [round(float(v), 4)
                                                                    for v in np.percentile(ratio_x, [10, 50, 90])]}
            del g_f, g_q, g_x
        legs["m1_per_shape_choice"] = choice
        del wsets

    if want("gate_up_swiglu_M8"):
        # fused gate/up SwiGLU, M=8, N=17408, K=5120, Q4 x fp32
        M4, N4, K4 = datagen.GATE_UP["M"], datagen.GATE_UP["N"], datagen.GATE_UP["K"]
        gq, gd, uq, ud, x = datagen.gate_up_inputs()
        sets = [tuple(gpu(a) for a in (gq, gd, uq, ud))]
        for r in range(1, N_COPIES):
            rr = datagen.streams(30 + r, 4)
            g2 = datagen.q4_weights(rr[0], rr[1], N4, K4)
            u2 = datagen.q4_weights(rr[2], rr[3], N4, K4)
            sets.append(tuple(gpu(a) for a in (*g2, *u2)))
        xg = gpu(x)
        out4 = torch.empty((M4, N4), dtype=torch.float32, device=dev)
        g4 = torch.empty_like(out4)
        u4 = torch.empty_like(out4)
        def fused(i):
            qbd.gate_up_swiglu_q4(*sets[i % N_COPIES], xg, out=out4)

        def unfused(i):
            s = sets[i % N_COPIES]
            qbd.qmv_q4_0_f32(s[0], s[1], xg, out=g4)
            qbd.qmv_q4_0_f32(s[2], s[3], xg, out=u4)
            qbd.swiglu_f32(g4, u4, out=out4)
        settle(torch, lambda i: (fused(i), unfused(i)))
        t_f, t_u, ratio = paired_ms(torch, fused, unfused, rounds=20, calls=N_COPIES)
        wbytes = 2 * q4_bytes(N4, K4)
        us_f = float(np.median(t_f) * 1e3)
        us_u = float(np.median(t_u) * 1e3)
        flops = 2 * 2 * M4 * N4 * K4
        legs["gate_up_swiglu_M8"] = {
            "us": round(us_f, 3), "unfused_us": round(us_u, 3),
            "fused_vs_unfused_time": round(float(np.median(ratio)) - 1, 4),
            "fused_vs_unfused": dict(ab_summary(t_f, t_u, ratio), a="fused (one launch)",
                                     b="gate, up, then swiglu_f32 (three launches)"),
            "weight_GBs": round(wbytes / (us_f * 1e-6) / 1e9, 1),
            "pct_hbm": round(100 * wbytes / (us_f * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
            "TFLOPs": round(flops / (us_f * 1e-6) / 1e12, 2),
            # the products run on the bf16 matrix cores (activations split
            # exactly into three bf16 parts), whose work here is a few us: the
            # roof of the launch is its weight stream; the FMA-equivalent rate
            # against the unpacked fp32 VALU roof is kept as context
            "roofline": {"bound": "hbm", "achieved": round(wbytes / (us_f * 1e-6) / 1e9, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(wbytes / (us_f * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                         "kernel": "qmv_f32_mfma<Q4, SwiGLU, MT=8, NT=5> (v_mfma_f32_16x16x32_bf16)"},
            "fp32_fma_equivalent_frac_of_valu_roof": round(flops / (us_f * 1e-6) / 1e12 / FP32_VALU_PEAK_TFLOPS, 4)}
        # the same fused gate/up on Q8 activations: quantize + one launch
        xq4, xd4 = qbd.quantize_act_q8_0(xg)

        def fused_q8(i):
            qbd.quantize_act_q8_0(xg, xq4, xd4)
            qbd.gate_up_swiglu_q4_q8act(*sets[i % N_COPIES], xq4, xd4, out=out4)
        settle(torch, fused_q8)
        t_f2, t_q, ratio_q = paired_ms(torch, fused, fused_q8, rounds=20, calls=N_COPIES)
        us_q = float(np.median(t_q) * 1e3)
        legs["gate_up_swiglu_M8"]["q8act"] = {
            "us": round(us_q, 3), "weight_GBs": round(wbytes / (us_q * 1e-6) / 1e9, 1),
            "frac_of_hbm": round(wbytes / (us_q * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "fp32_vs_q8act": dict(ab_summary(t_f2, t_q, ratio_q), a="gate_up_swiglu_q4 (fp32 x)",
                                  b="quantize_act_q8_0 + gate_up_swiglu_q4_q8act"),
            "kernel": "qmm_q8_tile16<Q4, SwiGLU, Q=5, persistent> (16 x 16 int8 tiles, one workgroup per CU)"}
        log("gate/up leg done")
        del sets

    if want("q4_ffn_decode_M1") or want("q4_down_M8"):
        # 4-bit FFN of the 27B-class target at M=1 (decode): the fused gate/up
        # SwiGLU launch and the down projection, then the down projection at
        # M=8 (its verifier-block panel); cold weights by rotation over copies
        ffn = [{k: tuple(gpu(a) for a in v) for k, v in datagen.q4_ffn_weights(c).items()} for c in range(N_COPIES)]
        (_, NF, KF), (_, ND, KD) = datagen.Q4_FFN[0], datagen.Q4_FFN[2]
        x1, h1 = (gpu(a) for a in datagen.q4_ffn_activations(1))
        x8, h8 = (gpu(a) for a in datagen.q4_ffn_activations(datagen.DOWN_M8["M"]))
        gu1 = torch.empty((1, NF), dtype=torch.float32, device=dev)
        d1 = torch.empty((1, ND), dtype=torch.float32, device=dev)
        d8 = torch.empty((datagen.DOWN_M8["M"], ND), dtype=torch.float32, device=dev)

        def gate_up1(i):
            w = ffn[i % N_COPIES]
            qbd.gate_up_swiglu_q4(*w["gate"], *w["up"], x1, out=gu1)

        def down1(i):
            qbd.qmv_q4_0_f32(*ffn[i % N_COPIES]["down"], h1, out=d1)

        def down8(i):
            qbd.qmv_q4_0_f32(*ffn[i % N_COPIES]["down"], h8, out=d8)

        # the same FFN on Q8 activations: each input quantized per block
        # (quantize_act_q8_0), then the fused gate/up and the down product
        # with exact int32 block dots (activations staged in LDS per CU)
        x1q, x1d = qbd.quantize_act_q8_0(x1)
        h1q, h1d = qbd.quantize_act_q8_0(h1)

        def gate_up1_q8(i):
            w = ffn[i % N_COPIES]
            qbd.quantize_act_q8_0(x1, x1q, x1d)
            qbd.gate_up_swiglu_q4_q8act(*w["gate"], *w["up"], x1q, x1d, out=gu1)

        def down1_q8(i):
            qbd.quantize_act_q8_0(h1, h1q, h1d)
            qbd.qmm_q4_0_q8act(*ffn[i % N_COPIES]["down"], h1q, h1d, out=d1)

        def gate_up1_q8_product(i):
            w = ffn[i % N_COPIES]
            qbd.gate_up_swiglu_q4_q8act(*w["gate"], *w["up"], x1q, x1d, out=gu1)

        def down1_q8_product(i):
            qbd.qmm_q4_0_q8act(*ffn[i % N_COPIES]["down"], h1q, h1d, out=d1)

        def rot(fn):
            # one graph of two rotations over the weight copies; time per call
            for i in range(N_COPIES):
                fn(i)
            torch.cuda.synchronize()
            g = capture(torch, lambda: [fn(i) for i in range(2 * N_COPIES)])
            return lambda k: g.replay()

        # quantization and product in one call: the staged kernel quantizes
        # the panel in each workgroup, one launch per projection
        def gate_up1_qx(i):
            w = ffn[i % N_COPIES]
            qbd.gate_up_swiglu_q4_q8act_from_f32(*w["gate"], *w["up"], x1, x1q, x1d, out=gu1)

        def down1_qx(i):
            qbd.qmm_q4_0_q8act_from_f32(*ffn[i % N_COPIES]["down"], h1, h1q, h1d, out=d1)

        g_gu, g_gu8, g_gu8p = rot(gate_up1), rot(gate_up1_q8), rot(gate_up1_q8_product)
        g_dn, g_dn8, g_dn8p = rot(down1), rot(down1_q8), rot(down1_q8_product)
        g_gux, g_dnx = rot(gate_up1_qx), rot(down1_qx)
        settle(torch, g_gu)
        per = 2 * N_COPIES
        ta, tb, r_gu = paired_ms(torch, g_gu, g_gu8, rounds=20, calls=2)
        tc, td, r_dn = paired_ms(torch, g_dn, g_dn8, rounds=20, calls=2)
        te, tf, r_gux = paired_ms(torch, g_gu, g_gux, rounds=20, calls=2)
        tg, th, r_dnx = paired_ms(torch, g_dn, g_dnx, rounds=20, calls=2)
        gux_ms, dnx_ms = float(np.median(tf)) / per, float(np.median(th)) / per
        gu_ms, gu8_ms = float(np.median(ta)) / per, float(np.median(tb)) / per
        dn_ms, dn8_ms = float(np.median(tc)) / per, float(np.median(td)) / per
        gu8p_ms = batch_ms(torch, g_gu8p, 4, reps=5) / per
        dn8p_ms = batch_ms(torch, g_dn8p, 4, reps=5) / per
        settle(torch, down8)
        d8_ms = batch_ms(torch, down8, 2 * N_COPIES, reps=5)
        gu_bytes, dn_bytes = 2 * q4_bytes(NF, KF), q4_bytes(ND, KD)
        ceilings = {}
        for nm, nbytes, prod_ms in (("gate_up_product", gu_bytes, gu8p_ms), ("down_product", dn_bytes, dn8p_ms)):
            ceil = ReadCeiling(torch, dev, nbytes)
            ceilings[nm] = ceil.report(batch_ms(torch, rot(ceil), 4, reps=5) / per, prod_ms)
            del ceil

        def hbm(nbytes, ms):
            gbs = nbytes / (ms * 1e-3) / 1e9
            return {"GBs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}
        legs["q4_ffn_decode_M1"] = {
            "gate_up_swiglu_us": round(gu_ms * 1e3, 3), "gate_up_swiglu": hbm(gu_bytes, gu_ms),
            "down_us": round(dn_ms * 1e3, 3), "down": hbm(dn_bytes, dn_ms),
            "ffn_us": round((gu_ms + dn_ms) * 1e3, 3),
            "roofline": {"bound": "hbm", "achieved": hbm(gu_bytes + dn_bytes, gu_ms + dn_ms)["GBs"],
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": hbm(gu_bytes + dn_bytes, gu_ms + dn_ms)["frac"]},
            "shapes": "gate/up 5120->17408 (fused SwiGLU, one launch), down 17408->5120; Q4 x fp32",
            "q8act": {
                "gate_up_swiglu_us": round(gu8_ms * 1e3, 3), "gate_up_product_us": round(gu8p_ms * 1e3, 3),
                "gate_up_product": dict(hbm(gu_bytes, gu8p_ms), read_ceiling=ceilings["gate_up_product"]),
                "down_us": round(dn8_ms * 1e3, 3), "down_product_us": round(dn8p_ms * 1e3, 3),
                "down_product": dict(hbm(dn_bytes, dn8p_ms), read_ceiling=ceilings["down_product"]),
                "ffn_us": round((gu8_ms + dn8_ms) * 1e3, 3),
                "roofline": {"bound": "hbm", "achieved": hbm(gu_bytes + dn_bytes, gu8p_ms + dn8p_ms)["GBs"],
                             "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": hbm(gu_bytes + dn_bytes, gu8p_ms + dn8p_ms)["frac"],
                             "note": "the two products, without their activation quantization"},
                "gate_up_f32_vs_q8act": ab_summary(ta / per, tb / per, r_gu),
                "down_f32_vs_q8act": ab_summary(tc / per, td / per, r_dn),
                "shapes": "quantize_act_q8_0 + gate_up_swiglu_q4_q8act 5120->17408; quantize_act_q8_0 + "
                          "qmm_q4_0_q8act 17408->5120; graphs of 12 calls"},
            "q8act_from_f32": {
                "gate_up_swiglu_us": round(gux_ms * 1e3, 3), "gate_up": hbm(gu_bytes, gux_ms),
                "down_us": round(dnx_ms * 1e3, 3), "down": hbm(dn_bytes, dnx_ms),
                "ffn_us": round((gux_ms + dnx_ms) * 1e3, 3),
                "roofline": {"bound": "hbm", "achieved": hbm(gu_bytes + dn_bytes, gux_ms + dnx_ms)["GBs"],
                             "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": hbm(gu_bytes + dn_bytes, gux_ms + dnx_ms)["frac"],
                             "note": "the whole FFN from fp32 activations, quantization included"},
                "gate_up_f32_vs_from_f32": ab_summary(te / per, tf / per, r_gux),
                "down_f32_vs_from_f32": ab_summary(tg / per, th / per, r_dnx),
                "shapes": "gate_up_swiglu_q4_q8act_from_f32 5120->17408 and qmm_q4_0_q8act_from_f32 "
                          "17408->5120, one launch each (each workgroup quantizes the panel); graphs of 12 calls"}}
        m8 = datagen.DOWN_M8["M"]
        flops8 = 2 * m8 * ND * KD
        tf8 = flops8 / (d8_ms * 1e-3) / 1e12
        # the same M=8 down projection on Q8 activations: quantize + product
        h8q, h8d = qbd.quantize_act_q8_0(h8)
        d8q = torch.empty_like(d8)

        def down8_q8(i):
            qbd.quantize_act_q8_0(h8, h8q, h8d)
            qbd.qmm_q4_0_q8act(*ffn[i % N_COPIES]["down"], h8q, h8d, out=d8q)
        settle(torch, down8_q8)
        d8q_ms = batch_ms(torch, down8_q8, 2 * N_COPIES, reps=5)
        legs["q4_down_M8"] = {
            "us": round(d8_ms * 1e3, 3), "weight": hbm(dn_bytes, d8_ms), "TFLOPs": round(tf8, 2),
            "roofline": {"bound": "alu", "achieved": round(tf8, 2), "peak": FP32_VALU_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf8 / FP32_VALU_PEAK_TFLOPS, 4)},
            "shape": f"M={m8}, N={ND}, K={KD}, Q4 x fp32",
            "q8act": {"us": round(d8q_ms * 1e3, 3), "weight": hbm(dn_bytes, d8q_ms),
                      "shape": "quantize_act_q8_0 + qmm_q4_0_q8act at the same shape (back-to-back calls)"}}
        del ffn
        log("q4 ffn legs done")

    if want("prefill_M1024"):
        # prefill M=1024, N=17408, K=5120, Q4 x Q8 activations
        gq, gd, uq, ud, x = datagen.prefill_inputs()
        P = [gpu(a) for a in (gq, gd, uq, ud)]
        xp = gpu(x)
        M5, N5, K5 = datagen.PREFILL["M"], datagen.PREFILL["N"], datagen.PREFILL["K"]
        xq, xd = qbd.quantize_act_q8_0(xp)
        y5 = torch.empty((M5, N5), dtype=torch.float32, device=dev)
        # each long launch is settled (see settle) before it is timed
        it5 = max(20, iters // 3)
        # the quantization launch is short (a few microseconds): timed inside a
        # graph of 10 calls, so host call overhead stays out of it
        qbd.quantize_act_q8_0(xp, xq, xd)
        torch.cuda.synchronize()
        gq8 = capture(torch, lambda: [qbd.quantize_act_q8_0(xp, xq, xd) for _ in range(10)])
        t_q = np.array([graph_ms(torch, [gq8], 20) / 10])
        del gq8
        plain = lambda i: qbd.qmm_q4_0_q8act(P[0], P[1], xq, xd, out=y5)  # noqa: E731
        fused5 = lambda i: qbd.gate_up_swiglu_q4_q8act(*P, xq, xd, out=y5)  # noqa: E731
        settle(torch, plain)
        t_p = event_ms(torch, plain, it5, warm=2)
        settle(torch, fused5)
        t_s = event_ms(torch, fused5, it5, warm=2)
        ops = 2 * M5 * N5 * K5
        us_p = float(np.median(t_p) * 1e3)
        us_s = float(np.median(t_s) * 1e3)
        tops_p = ops / (us_p * 1e-6) / 1e12
        tops_s = 2 * ops / (us_s * 1e-6) / 1e12
        # the product with its activation quantization, as one graph of both
        # launches (the pages report activation preparation with the matmul)
        qp = capture(torch, lambda: (qbd.quantize_act_q8_0(xp, xq, xd),
                                     qbd.qmm_q4_0_q8act(P[0], P[1], xq, xd, out=y5)))
        us_qp = graph_ms(torch, [qp], 10) * 1e3
        del qp
        legs["prefill_M1024"] = {
            "quantize_us": round(float(np.median(t_q) * 1e3), 3),
            "plain_us": round(us_p, 3), "plain_int8_TOPS": round(tops_p, 2),
            "plain_us_p10_p50_p90": pct_us(t_p),
            "quantize_plus_plain_us": round(us_qp, 3),
            "fused_us": round(us_s, 3), "fused_int8_TOPS": round(tops_s, 2),
            "fused_us_p10_p50_p90": pct_us(t_s),
            "roofline": {"bound": "mfma", "achieved": round(tops_p, 2), "peak": INT8_PEAK_TOPS,
                         "unit": "TOPS", "frac": round(tops_p / INT8_PEAK_TOPS, 4),
                         "note": "plain product; int8 MFMA dense peak"}}
        log("prefill leg done")

    if want("dependent_step"):
        legs["dependent_step"] = leg_dependent_step(torch, dev)
        log("dependent-step leg done")
    return legs


def leg_dependent_step(torch, dev):
    """What one dependent step of a decode chain costs as a kernel launch
    replayed from a HIP graph (an empty kernel, 400 launches in one graph),
    and as a grid-wide handoff of a 4 KB vector inside one persistent
    cooperative grid of 256 workgroups (three arrival forms; the per-handoff
    figure is the time difference of 401 and 201 phases over 200).  Each
    handoff run must report no wait given up and no value read back
    wrong."""
    import ctypes
    lib = ctypes.CDLL(CEILING_LIB)
    lib.qbd_grid_handoff.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.qbd_grid_handoff.restype = ctypes.c_int
    lib.qbd_grid_handoff_work_words.restype = ctypes.c_int64
    lib.qbd_empty_launch.argtypes = [ctypes.c_void_p]
    lib.qbd_empty_launch.restype = ctypes.c_int

    def stream():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    n_launch = 400
    g = capture(torch, lambda: [lib.qbd_empty_launch(stream()) for _ in range(n_launch)])
    launch_us = [graph_ms(torch, [g], 3) * 1e3 / n_launch for _ in range(5)]
    del g

    words = int(lib.qbd_grid_handoff_work_words())
    work = torch.zeros(words + 64, dtype=torch.int32, device=dev)
    off = (-work.data_ptr()) % 256 // 4
    wp = work.data_ptr() + 4 * off

    def handoff_ms(mode, phases):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        st = lib.qbd_grid_handoff(mode, phases, wp, stream())
        b.record()
        torch.cuda.synchronize()
        if st != 0:
            raise RuntimeError(f"qbd_grid_handoff returned {st}")
        w = work[off:off + words].cpu().numpy().view(np.uint32)
        if w[words - 64] or w[words - 63]:
            raise RuntimeError(f"grid handoff mode {mode}: timeout word {w[words - 64]}, wrong values {w[words - 63]}")
        return a.elapsed_time(b)

    forms = {0: "one arrival counter", 1: "16 arrival counters on separate lines", 2: "one arrival word per workgroup"}
    handoff = {}
    for mode, name in forms.items():
        handoff_ms(mode, 1)
        per = sorted((handoff_ms(mode, 401) - handoff_ms(mode, 201)) * 1e3 / 200 for _ in range(5))
        handoff[name] = {"us_per_handoff": round(per[2], 3), "range_us": [round(per[0], 3), round(per[-1], 3)]}
    best = min(v["us_per_handoff"] for v in handoff.values())
    return {"graph_launch_us": round(float(np.median(launch_us)), 3),
            "graph_launch_range_us": [round(min(launch_us), 3), round(max(launch_us), 3)],
            "grid_handoff": handoff,
            "best_handoff_over_launch": round(best / float(np.median(launch_us)), 2),
            "note": "per dependent step: an empty kernel launched from a HIP graph against a 4 KB vector "
                    "handed to all 256 workgroups of a persistent grid (agent-scope atomics, no cache "
                    "write-back); values checked on every run"}


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(datagen, seconds):
    """The reference oracle on the host cores, on a bounded sample of the
    timed step (one decode layer + 1/16 of the LM-head rows, repeated for
    about `seconds` with numpy's BLAS threads as they are, then for about
    half that long on one thread); reported as weight GB/s like the step."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    mats = datagen.decode_layer_weights(0)
    acts = datagen.decode_activations(1)
    wq_h, wd_h = datagen.lm_head_weights(0)
    rows = 151936 // 16
    head = (wq_h[:rows], wd_h[:rows])
    per_rep = sum(q8_bytes(n, k) for _, n, k in datagen.DECODE_LAYER) + q8_bytes(rows, 896)

    def run(budget):
        reps = 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget:
            for name in ("qkv", "wo"):
                oracle.qmv_q8_0_f32(*mats[name], acts[896])
            gate_up = oracle.gate_up_swiglu_q8_0(*mats["gate"], *mats["up"], acts[896])
            oracle.qmv_q8_0_f32(*mats["down"], gate_up["out32"])
            oracle.qmv_q8_0_f32(head[0], head[1], acts[896])
            reps += 1
        return reps, time.perf_counter() - t0

    reps, el = run(seconds)
    with threadpool_limits(limits=1):
        reps1, el1 = run(seconds / 2)
    return {"value": round(reps * per_rep / el / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "value_1_thread": round(reps1 * per_rep / el1 / 1e9, 4),
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"one decode layer (qkv, wo, fused gate/up SwiGLU, down) plus 1/16 of the LM-head rows "
                      f"at M=1 through the float64 numpy oracle: {reps} repetitions in {el:.1f} s on "
                      f"{threads} BLAS threads, {reps1} in {el1:.1f} s on 1 thread"}


if __name__ == "__main__":
    main()
