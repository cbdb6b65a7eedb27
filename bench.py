"""Throughput of the FP4 routed-expert MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one pass of the whole layer -- route, permute, gate/up grouped GEMM
with SwiGLU, down grouped GEMM, combine -- over one batch of synthetic input
resident in HBM.  The headline workload is the decode shape (256 experts in 8
groups, keep 4 groups, top-8, hidden 4096, expert intermediate 2048, W4A16
MXFP4) at a batch of 64 tokens; decode timings rotate four independent layer
weight sets so the 256 MB Infinity Cache cannot serve repeated weight reads.
The headline step time comes from one captured HIP graph holding all K timed
steps (each the layer on the next weight set, as successive layers of a decode
step would be), replayed once; the eager step time is reported beside it, and
the dominant kernel's time comes from HIP events around its launch in the
eager steps.
The JSON line also carries the batch-1/8 decode lines, the prefill, W4A4 and
REAP-50 shapes, the roofline of the dominant kernel (the gate/up GEMM) and the
CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP4_PEAK_TFLOPS = 10100.0      # MI355X dense fp4 MFMA
MX_BYTES_PER_WEIGHT = 0.5 + 1.0 / 32.0

# HBM bytes per launch of the decode gate/up GEMM at 64 tokens, measured with
# rocprofv3 --pmc (FETCH_SIZE x 2.000 + WRITE_SIZE x 1.000, the factors a plain
# 1 GiB device copy gives), keyed by the hash of the kernel's sources at the
# time; a changed kernel has no entry and reports null.
MEASURED_TRAFFIC = {"67eb1b87dfbc9156": 2020959969}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in ("gemm_decode.h", "gemm_decode.hip", "gemm_decode_tiled.hip", "gemm_common.h", "common.h"):
        with open(os.path.join(ROOT, "block_scaled_fp4_group_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(bits):
    import torch
    return dev(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


TILED = True                   # weights prepared once in the kernels' tiled layout (--row-major: off)


def make_weights(W, tiled=None):
    import block_scaled_fp4_group_amd as moe
    tiled = TILED if tiled is None else tiled

    def one(name):
        p, s = W[name][0], W[name][1]
        w = moe.Weights(dev(p), dev(s))
        return moe.tile_weights(w) if tiled else w
    return moe.LayerWeights(one("gate"), one("up"), one("down"))


def layer_for(moe, lw, shape, T, act_mode="bf16"):
    return moe.MoELayer(lw, shape.num_experts, shape.n_group, shape.topk_group, shape.top_k,
                        shape.routed_scaling_factor, T, act_mode=act_mode)


def time_steps(layers, inputs, steps, warmup, algo=0, ev_name="gate_up"):
    """Run warmup + timed steps, rotating over (layer, input) pairs.  Returns
    (ms per step, mean gate/up launch ms over the timed steps)."""
    import torch
    n = len(layers)
    for i in range(warmup):
        x, l, b, r = inputs[i % len(inputs)]
        layers[i % n].forward(x, l, b, r, algo=algo)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        x, l, b, r = inputs[i % len(inputs)]
        layers[i % n].forward(x, l, b, r, algo=algo, events={ev_name: ev[i]})
    end.record()
    torch.cuda.synchronize()
    total = start.elapsed_time(end)
    k_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    return total / steps, k_ms


def graph_steps(layers, inputs, steps, warmup):
    """The same steps as time_steps captured in HIP graphs, as a decode engine
    captures a whole token step: one graph of the warmup steps and one of the
    timed steps, each step the layer forward of the next weight set in turn
    (the rotating sets stand for successive layers).  Returns ms per step."""
    import torch
    x, l, b, r = inputs[0]
    n = len(layers)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for ly in layers:
            ly.forward(x, l, b, r)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    def capture(count):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(count):
                layers[i % n].forward(x, l, b, r)
        return g
    warm, timed = capture(max(warmup, 1)), capture(steps)
    torch.cuda.synchronize()
    warm.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    timed.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def distinct_experts(layer, T):
    off = layer.offsets.cpu().numpy()
    return int(np.sum(np.diff(off) > 0))


def gate_up_bytes(D, T, shape):
    """Algorithmic HBM bytes of one gate/up launch: the routed experts' gate and
    up weights once, the token rows once, z written once."""
    H, I, k = shape.hidden, shape.inter, shape.top_k
    w = D * 2 * I * H * MX_BYTES_PER_WEIGHT
    return w + T * H * 2 + T * k * I * 2


def layer_bytes(D, T, shape):
    H, I, k, E = shape.hidden, shape.inter, shape.top_k, shape.num_experts
    return D * 3 * I * H * MX_BYTES_PER_WEIGHT + T * (2 * H + 4 * E + 64 + 2 * H)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(shape, W, x, l, bias, sample_tokens):
    """The oracle on a bounded sample, with NumPy's BLAS pool set to the cores
    this process may run on.  Returns (tokens/s, seconds, threads used, cores)."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limiter = threadpool_limits(limits=cores, user_api="blas")
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        limiter, threads = None, 1
    t0 = time.perf_counter()
    oracle.moe_layer(x, l, bias, W, shape.n_group, shape.topk_group, shape.top_k, shape.routed_scaling_factor,
                     tokens=sample_tokens)
    dt = time.perf_counter() - t0
    if limiter is not None:
        limiter.restore_original_limits()
    return len(sample_tokens) / dt, dt, threads, cores


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--rotate", type=int, default=4, help="independent decode weight sets")
    ap.add_argument("--no-extras", action="store_true", help="only the headline decode line")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--row-major", action="store_true",
                    help="keep the weights in their row-major layout (default: tiled once before timing)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times (the reference "
                         "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes) and exit")
    args = ap.parse_args()
    global TILED
    TILED = not args.row_major
    if args.copy_calibration:
        import torch
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 3}), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path (asked for {args.gpus}).",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    import block_scaled_fp4_group_amd as moe
    import synth

    torch.cuda.init()
    wd = synth.WORKLOADS["decode"]
    s = wd.shape
    log(f"[bench] generating {args.rotate} decode weight sets")
    Ws = [synth.expert_weights(wd, layer=i) for i in range(args.rotate)]
    lws = [make_weights(W) for W in Ws]
    torch.cuda.synchronize()

    def decode_line(T, steps, warmup, graph=False):
        x = synth.activations(wd, T)
        l = synth.logits(wd, T)
        inputs = [(dev_bf16(x), dev(l), None, None)]
        layers = [layer_for(moe, lw, s, T) for lw in lws]
        ms, k_ms = time_steps(layers, inputs, steps, warmup)
        g_ms = graph_steps(layers, inputs, steps, warmup) if graph else None
        Ds = []
        for ly in layers:
            ly.forward(*inputs[0])
            Ds.append(distinct_experts(ly, T))
        D = float(np.mean(Ds))
        return dict(T=T, ms=ms, gate_up_ms=k_ms, graph_ms=g_ms, D=D, x=x, l=l, layers=layers)

    log("[bench] decode T=64 (headline)")
    main_r = decode_line(64, args.steps, args.warmup, graph=True)
    T = 64
    step_ms = main_r["graph_ms"]            # the layer step replayed from a captured HIP graph
    tok_s = T / (step_ms / 1e3)
    gu_bytes = gate_up_bytes(main_r["D"], T, s)
    achieved = gu_bytes / (main_r["gate_up_ms"] / 1e3) / 1e9
    lb = layer_bytes(main_r["D"], T, s)
    src_hash = kernel_source_hash()   # of the decode kernel
    tr = MEASURED_TRAFFIC.get(src_hash)
    out = {
        "metric": "MoE-layer tokens/s at 1 MI355X (decode shape, HBM roofline)",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "ms_per_step_eager": round(main_r["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode W4A16 MXFP4: 256 experts (8 groups, keep 4, top-8, scale 2.827), "
                               "hidden 4096, expert intermediate 2048, 64 tokens, 4 rotated weight sets",
                   "tokens": T, "experts": 256, "hidden": 4096, "intermediate": 2048, "top_k": 8,
                   "weights": "MXFP4, " + ("tiled layout" if TILED else "row-major"), "activations": "bf16",
                   "distinct_experts": main_r["D"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if tr is None else tr,
                     "kernel": "gemm_decode_kernel (gate/up + SwiGLU" + (", tiled weights)" if TILED else ")"),
                     "kernel_ms": round(main_r["gate_up_ms"], 5),
                     "algorithmic_bytes": int(gu_bytes)},
        "layer_hbm_frac": round(lb / (step_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
    }
    extras = {}
    if not args.no_extras:
        for Tx in (1, 8):
            log(f"[bench] decode T={Tx}")
            r = decode_line(Tx, max(args.steps, 50), args.warmup, graph=True)
            b = layer_bytes(r["D"], Tx, s)
            extras[f"decode_T{Tx}"] = {"tokens_per_s": round(Tx / (r["ms"] / 1e3), 1), "ms_per_step": round(r["ms"], 4),
                                       "hip_graph_ms_per_step": round(r["graph_ms"], 4),
                                       "hip_graph_tokens_per_s": round(Tx / (r["graph_ms"] / 1e3), 1),
                                       "distinct_experts": r["D"],
                                       "layer_hbm_frac": round(b / (r["ms"] / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                                       "gate_up_hbm_frac": round(gate_up_bytes(r["D"], Tx, s) / (r["gate_up_ms"] / 1e3)
                                                                 / 1e9 / HBM_PEAK_GBS, 4)}
            del r
        extras.update(prefill_lines(moe, synth, Ws[0], args))
    out["extras"] = extras
    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        sample = list(range(12))          # about 10 s of float64 work on the host
        v, dt, threads, cores = cpu_baseline(s, Ws[0], main_r["x"], main_r["l"], None, sample)
        out["cpu_baseline"] = {"value": round(v, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
                               "cpu": cpu_model(), "cores_available": cores,
                               "sample": f"oracle.moe_layer on the decode T=64 batch: routing and permutation of all 64 "
                                         f"tokens, expert FFNs and combine of tokens {sample} (float64 NumPy, "
                                         f"BLAS threads {threads} of {cores} cores in the affinity mask), "
                                         f"{dt:.1f} s wall"}
    print(json.dumps(out), flush=True)


def prefill_lines(moe, synth, decode_W, args):
    """MFMA-bound shapes: prefill (T=8192, biased routing), W4A4 (T=4096 on the
    NVFP4 transcode of the decode weights) and REAP-50 (128 experts, 2 layers)."""
    import torch
    res = {}
    steps = max(5, min(args.steps, 20))
    warm = 3

    def mfma_frac(T, ms, layers=1):
        flops = T * 402653184.0 * layers
        return flops / (ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS

    wp = synth.WORKLOADS["prefill"]
    log("[bench] prefill T=8192")
    Wp = synth.expert_weights(wp)
    lwp = make_weights(Wp)
    del Wp
    T = 8192
    x = dev_bf16(synth.activations(wp, T))
    l = dev(synth.logits(wp, T))
    b = dev(synth.correction_bias(wp))
    ly = layer_for(moe, lwp, wp.shape, T)
    ms, k_ms = time_steps([ly], [(x, l, b, None)], steps, warm)
    res["prefill_T8192"] = {"tokens_per_s": round(T / (ms / 1e3), 1), "ms_per_step": round(ms, 4),
                            "mfma_frac_bf16": round(mfma_frac(T, ms), 4), "gate_up_ms": round(k_ms, 4)}
    del ly, lwp
    torch.cuda.empty_cache()

    log("[bench] W4A4 T=4096")
    ww = synth.WORKLOADS["w4a4"]
    src = make_weights(decode_W, tiled=False)    # the transcode reads the row-major MXFP4 tensors
    nvw = {}
    tc_ms = []
    for name in ("gate", "up", "down"):
        t = getattr(src, name)
        M, n, kb = t.scale.shape
        sc = torch.empty((M, n, kb * 2), dtype=torch.uint8, device="cuda")
        g = torch.empty(M, dtype=torch.float32, device="cuda")
        cnt = torch.empty(4, dtype=torch.int64, device="cuda")
        moe.transcode_mx_to_nv(t.scale, t.packed, sc, g, cnt)          # warm-up (outputs preallocated)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        moe.transcode_mx_to_nv(t.scale, t.packed, sc, g, cnt)
        e1.record()
        torch.cuda.synchronize()
        tc_ms.append(e0.elapsed_time(e1))
        assert int(cnt[2].item()) == 0
        nvw[name] = moe.Weights(t.packed, sc, g, scales_pow2=True)    # the transcode's scales are powers of two
        if TILED:
            nvw[name] = moe.tile_weights(nvw[name])
    E = ww.shape.num_experts
    tc_bytes = 3 * E * 2048 * 4096 * (1 / 32 + 2 / 16)      # read E8M0, write 2x E4M3
    T = 4096
    lw4 = moe.LayerWeights(nvw["gate"], nvw["up"], nvw["down"])
    ly = layer_for(moe, lw4, ww.shape, T, act_mode="nvfp4")
    x = dev_bf16(synth.activations(ww, T))
    l = dev(synth.logits(ww, T))
    ms, k_ms = time_steps([ly], [(x, l, None, None)], steps, warm)
    res["w4a4_T4096"] = {"tokens_per_s": round(T / (ms / 1e3), 1), "ms_per_step": round(ms, 4),
                         "mfma_frac_bf16": round(mfma_frac(T, ms), 4),
                         "fp4_peak_frac": round(mfma_frac(T, ms) * BF16_PEAK_TFLOPS / FP4_PEAK_TFLOPS, 4),
                         "transcode_GBs": round(tc_bytes / (sum(tc_ms) / 1e3) / 1e9, 1)}
    del ly, lw4, nvw, src
    torch.cuda.empty_cache()

    log("[bench] REAP-50 T=16384, 2 layers")
    wr = synth.WORKLOADS["reap50"]
    T = 16384
    lws = [make_weights(synth.expert_weights(wr, i)) for i in range(2)]
    lys = [layer_for(moe, lw, wr.shape, T) for lw in lws]
    h0 = dev_bf16(synth.activations(wr, T, 0))
    ls = [dev(synth.logits(wr, T, i)) for i in range(2)]
    for _ in range(warm):
        h1 = lys[0].forward(h0, ls[0], None, h0)
        lys[1].forward(h1, ls[1], None, h1)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        h1 = lys[0].forward(h0, ls[0], None, h0)
        lys[1].forward(h1, ls[1], None, h1)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    off = lys[0].offsets.cpu().numpy()
    loads = np.diff(off)
    res["reap50_T16384_2layers"] = {"tokens_per_s_per_layer": round(2 * T / (ms / 1e3), 1),
                                    "ms_per_step_2layers": round(ms, 4),
                                    "mfma_frac_bf16": round(mfma_frac(T, ms, 2), 4),
                                    "expert_load_max": int(loads.max()), "expert_load_median": float(np.median(loads))}
    return res


if __name__ == "__main__":
    main()
