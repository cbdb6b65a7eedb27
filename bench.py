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
HOST_LEAD_CYCLES = 40_000_000  # GPU spin before a timed eager loop: ~20 ms at 2 GHz, time to queue its steps
MXC_BYTES_PER_WEIGHT = 0.5 + 0.5 / 32.0       # compact MXFP4: a 4-bit exponent code per 32 weights

# HBM bytes per launch of the decode gate/up GEMM at 64 tokens, measured with
# rocprofv3 --pmc (FETCH_SIZE x 2.000 + WRITE_SIZE x 1.000, the factors a plain
# 1 GiB device copy gives), keyed by the hash of the kernel's sources at the
# time and the token count; a changed kernel or another batch has no entry and
# reports null.
MEASURED_TRAFFIC = {("6c07dd1792f9b8b4", 64): 2019543159}


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


def time_steps(layers, inputs, steps, warmup, algo=0, ev_names=("gate_up", "down")):
    """Run warmup + timed steps, rotating over (layer, input) pairs.  Returns
    (ms per step, {kernel: mean launch ms over the timed steps}); the launch
    times come from HIP events recorded on the launching stream around the
    gate/up and down GEMM launches.  The timed steps start behind a short GPU
    spin, so the host has queued them before the GPU reaches them and the
    events time the kernels, not the host's launch gaps (which dominate a
    1-token step)."""
    import torch
    n = len(layers)
    for i in range(warmup):
        x, l, b, r = inputs[i % len(inputs)]
        layers[i % n].forward(x, l, b, r, algo=algo)
    torch.cuda.synchronize()
    ev = {k: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
          for k in ev_names}
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(HOST_LEAD_CYCLES)
    start.record()
    for i in range(steps):
        x, l, b, r = inputs[i % len(inputs)]
        layers[i % n].forward(x, l, b, r, algo=algo, events={k: ev[k][i] for k in ev_names})
    end.record()
    torch.cuda.synchronize()
    total = start.elapsed_time(end)
    k_ms = {k: float(np.mean([a.elapsed_time(b) for a, b in ev[k]])) for k in ev_names}
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


def gate_up_bytes(D, T, shape, bpw=MX_BYTES_PER_WEIGHT):
    """Algorithmic HBM bytes of one gate/up launch: the routed experts' gate and
    up weights once, the token rows once, z written once."""
    H, I, k = shape.hidden, shape.inter, shape.top_k
    w = D * 2 * I * H * bpw
    return w + T * H * 2 + T * k * I * 2


def layer_bytes(D, T, shape, bpw=MX_BYTES_PER_WEIGHT):
    H, I, k, E = shape.hidden, shape.inter, shape.top_k, shape.num_experts
    return D * 3 * I * H * bpw + T * (2 * H + 4 * E + 64 + 2 * H)


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
    ap.add_argument("--decode-tokens", type=int, default=64,
                    help="batch of the decode line (64 is the headline; other values only for profiling)")
    ap.add_argument("--workload", default="all", choices=["all"] + list(WORKLOAD_RUNNERS) + list(SWEEPS),
                    help="run one extra workload alone and print its figures (for profiling)")
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
    if args.workload != "all":
        r = {**WORKLOAD_RUNNERS, **SWEEPS}[args.workload](moe, synth, args)
        print(json.dumps({"workload_only": EXTRA_KEYS[args.workload], "result": r}), flush=True)
        return
    wd = synth.WORKLOADS["decode"]
    s = wd.shape
    log(f"[bench] generating {args.rotate} decode weight sets")
    Ws = [host_weights(synth, "decode", i) for i in range(args.rotate)]
    lws = [make_weights(W) for W in Ws]
    torch.cuda.synchronize()

    def decode_line(T, steps, warmup, graph=False):
        x = synth.activations(wd, T)
        l = synth.logits(wd, T)
        inputs = [(dev_bf16(x), dev(l), None, None)]
        layers = [layer_for(moe, lw, s, T) for lw in lws]
        ms, k_ms = time_steps(layers, inputs, steps, warmup)
        k_ms = k_ms["gate_up"]
        g_ms = graph_steps(layers, inputs, steps, warmup) if graph else None
        Ds = []
        for ly in layers:
            ly.forward(*inputs[0])
            Ds.append(distinct_experts(ly, T))
        D = float(np.mean(Ds))
        return dict(T=T, ms=ms, gate_up_ms=k_ms, graph_ms=g_ms, D=D, x=x, l=l, layers=layers)

    T = args.decode_tokens
    log(f"[bench] decode T={T} (headline)")
    main_r = decode_line(T, args.steps, args.warmup, graph=True)
    step_ms = main_r["graph_ms"]            # the layer step replayed from a captured HIP graph
    tok_s = T / (step_ms / 1e3)
    gu_bytes = gate_up_bytes(main_r["D"], T, s)
    achieved = gu_bytes / (main_r["gate_up_ms"] / 1e3) / 1e9
    lb = layer_bytes(main_r["D"], T, s)
    src_hash = kernel_source_hash()   # of the decode kernel
    tr = MEASURED_TRAFFIC.get((src_hash, T))
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
                               f"hidden 4096, expert intermediate 2048, {T} tokens, 4 rotated weight sets",
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
                                       "layer_hbm_frac": round(b / (r["graph_ms"] / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                                       "gate_up_hbm_frac": round(gate_up_bytes(r["D"], Tx, s) / (r["gate_up_ms"] / 1e3)
                                                                 / 1e9 / HBM_PEAK_GBS, 4)}
            del r
        for name, fn in WORKLOAD_RUNNERS.items():
            extras[EXTRA_KEYS[name]] = fn(moe, synth, args)
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


_HOST_WEIGHTS = {}


def host_weights(synth, name, layer=0):
    """Seeded host weights of a workload, generated once per run."""
    key = (name, layer)
    if key not in _HOST_WEIGHTS:
        _HOST_WEIGHTS[key] = synth.expert_weights(synth.WORKLOADS[name], layer)
    return _HOST_WEIGHTS[key]


FP8_PEAK_TFLOPS = 5000.0      # MI355X dense fp8 MFMA (an FP8 x FP4 block-scaled MFMA runs at this rate)
FLOPS_PER_TOKEN = 402653184.0  # 8 experts x 6 x 4096 x 2048 per token and layer


def _frac(T, ms, peak, layers=1):
    return T * FLOPS_PER_TOKEN * layers / (ms / 1e3) / 1e12 / peak


def _kernel_fracs(T, k_ms, peak):
    """Algorithmic MFMA fraction of the gate/up (2/3 of the FLOPs) and down (1/3) launches."""
    f = T * FLOPS_PER_TOKEN
    return {"gate_up_ms": round(k_ms["gate_up"], 4), "down_ms": round(k_ms["down"], 4),
            "gate_up_frac": round(f * 2 / 3 / (k_ms["gate_up"] / 1e3) / 1e12 / peak, 4),
            "down_frac": round(f / 3 / (k_ms["down"] / 1e3) / 1e12 / peak, 4)}


def run_prefill(moe, synth, args, act_mode="bf16"):
    """Prefill shape, 8192 tokens, biased routing; W4A16 (bf16 MFMA) or W4A8
    (MXFP8 activations, block-scaled FP8 x FP4 MFMA)."""
    import torch
    steps, warm = max(5, min(args.steps, 20)), 3
    wp = synth.WORKLOADS["prefill"]
    log(f"[bench] prefill T=8192 act={act_mode}")
    lw = make_weights(host_weights(synth, "prefill"))
    T = 8192
    x, l, b = dev_bf16(synth.activations(wp, T)), dev(synth.logits(wp, T)), dev(synth.correction_bias(wp))
    ly = layer_for(moe, lw, wp.shape, T, act_mode=act_mode)
    ms, k_ms = time_steps([ly], [(x, l, b, None)], steps, warm)
    peak = BF16_PEAK_TFLOPS if act_mode == "bf16" else FP8_PEAK_TFLOPS
    r = {"tokens_per_s": round(T / (ms / 1e3), 1), "ms_per_step": round(ms, 4),
         "mfma_frac_bf16": round(_frac(T, ms, BF16_PEAK_TFLOPS), 4)}
    if act_mode != "bf16":
        r["mfma_frac_fp8"] = round(_frac(T, ms, FP8_PEAK_TFLOPS), 4)
    r.update(_kernel_fracs(T, k_ms, peak))
    del ly, lw
    torch.cuda.empty_cache()
    return r


def run_w4a4(moe, synth, args, a_mode="dequant"):
    """NVFP4 W4A4, 4096 tokens on the exact NVFP4 transcode of the decode
    weights; a_mode "dequant" (bf16 MFMA on the exact NVFP4 values) or
    "planes" (block-scaled MFMA, FP4 weights native)."""
    import torch
    steps, warm = max(5, min(args.steps, 20)), 3
    ww = synth.WORKLOADS["w4a4"]
    log(f"[bench] W4A4 T=4096 a_mode={a_mode}")
    src = make_weights(host_weights(synth, "w4a4"), tiled=False)    # the transcode reads the row-major tensors
    nvw, tc_ms = {}, []
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
        nvw[name] = moe.Weights(t.packed, sc, g, scales_pow2=True, mx_exact=True)   # an exact MX transcode
        if TILED:
            nvw[name] = moe.tile_weights(nvw[name])
    E = ww.shape.num_experts
    tc_bytes = 3 * E * 2048 * 4096 * (1 / 32 + 2 / 16)      # read E8M0, write 2x E4M3
    T = 4096
    lw4 = moe.LayerWeights(nvw["gate"], nvw["up"], nvw["down"])
    ly = moe.MoELayer(lw4, E, ww.shape.n_group, ww.shape.topk_group, ww.shape.top_k, ww.shape.routed_scaling_factor,
                      T, act_mode="nvfp4", a_mode=a_mode)
    x, l = dev_bf16(synth.activations(ww, T)), dev(synth.logits(ww, T))
    ms, k_ms = time_steps([ly], [(x, l, None, None)], steps, warm)
    r = {"tokens_per_s": round(T / (ms / 1e3), 1), "ms_per_step": round(ms, 4),
         "mfma_frac_bf16": round(_frac(T, ms, BF16_PEAK_TFLOPS), 4),
         "fp4_peak_frac": round(_frac(T, ms, FP4_PEAK_TFLOPS), 4),
         "transcode_GBs": round(tc_bytes / (sum(tc_ms) / 1e3) / 1e9, 1)}
    r.update(_kernel_fracs(T, k_ms, BF16_PEAK_TFLOPS))
    del ly, lw4, nvw, src
    torch.cuda.empty_cache()
    return r


def run_outliers(moe, synth, args):
    """Down projection alone on bf16 z [32768, 2048] N(0,1) with 0.1% outliers
    of amax 2960 / 18560 / 311296, quantised to NVFP4 (saturating at 2688) and
    multiplied on the exact NVFP4 values (bf16 MFMA)."""
    import torch
    ww = synth.WORKLOADS["w4a4"]
    s = ww.shape
    rows, E = 32768, s.num_experts
    log("[bench] down projection with outliers")
    Wd = synth.mx_matrix(2, 0, synth.T_DOWN_CODES, synth.T_DOWN_EXP, E, s.hidden, s.inter)
    w = moe.Weights(dev(Wd[0]), dev(Wd[1]))
    wt = moe.tile_weights(w) if TILED else w
    offsets = dev(np.asarray(np.arange(E + 1) * (rows // E), dtype=np.int32))
    out = torch.empty((rows, s.hidden), dtype=torch.bfloat16, device="cuda")
    zc = torch.empty((rows, s.inter // 2), dtype=torch.uint8, device="cuda")
    zs = torch.empty((rows, s.inter // 16), dtype=torch.uint8, device="cuda")
    zdq = torch.empty((rows, s.inter), dtype=torch.bfloat16, device="cuda")
    res = {}
    for amax in synth.OUTLIER_AMAX:
        z = dev_bf16(synth.down_inputs_with_outliers(rows, s.inter, amax))

        def step():
            moe.quantize_nvfp4(z, 1.0, zc, zs, dequant=zdq)
            moe.grouped_gemm(zdq, wt, None, offsets, rows, out=out)
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = 10
        e0.record()
        for _ in range(n):
            step()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / n
        flops = 2.0 * rows * s.hidden * s.inter
        byts = E * s.hidden * s.inter * MX_BYTES_PER_WEIGHT + rows * s.inter * 2 * 2 + rows * s.hidden * 2
        res[f"amax_{int(amax)}"] = {"ms": round(ms, 4), "TFLOPs": round(flops / (ms / 1e3) / 1e12, 1),
                                    "mfma_frac_bf16": round(flops / (ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                                    "GBs": round(byts / (ms / 1e3) / 1e9, 1),
                                    "saturated_max": float(zdq.float().abs().max().item())}
        del z
    return res


def run_reap50(moe, synth, args):
    import torch
    steps, warm = max(5, min(args.steps, 20)), 3
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
    ev = {k: [] for k in ("gate_up", "down")}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        evs = [{k: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for k in ev}
               for _ in range(2)]
        h1 = lys[0].forward(h0, ls[0], None, h0, events=evs[0])
        lys[1].forward(h1, ls[1], None, h1, events=evs[1])
        for k in ev:
            ev[k] += [evs[0][k], evs[1][k]]
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    k_ms = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in ev.items()}
    loads = np.diff(lys[0].offsets.cpu().numpy())
    r = {"tokens_per_s_per_layer": round(2 * T / (ms / 1e3), 1), "ms_per_step_2layers": round(ms, 4),
         "mfma_frac_bf16": round(_frac(T, ms, BF16_PEAK_TFLOPS, 2), 4),
         "expert_load_max": int(loads.max()), "expert_load_median": float(np.median(loads))}
    r.update(_kernel_fracs(T, k_ms, BF16_PEAK_TFLOPS))
    del lys, lws
    torch.cuda.empty_cache()
    return r


def run_compact(moe, synth, args):
    """The decode line (T = 1, 8, 64; 4 rotated weight sets, HIP-graph replay)
    on the same weights in compact MXFP4 storage (4.125 bits per weight)."""
    import torch
    wd = synth.WORKLOADS["decode"]
    s = wd.shape
    log("[bench] compact MXFP4 decode")
    lws = []
    for i in range(args.rotate):
        src = make_weights(host_weights(synth, "decode", i), tiled=False)
        ws = []
        for name in ("gate", "up", "down"):
            w, cnt = moe.compact_weights(getattr(src, name))
            assert int(cnt[2].item()) == 0 and int(cnt[3].item()) == 0     # lossless
            ws.append(moe.tile_weights(w) if TILED else w)
        lws.append(moe.LayerWeights(*ws))
        del src
    torch.cuda.synchronize()
    res = {}
    for T in (1, 8, 64):
        x, l = dev_bf16(synth.activations(wd, T)), dev(synth.logits(wd, T))
        inputs = [(x, l, None, None)]
        layers = [layer_for(moe, lw, s, T) for lw in lws]
        steps = max(args.steps, 50)
        ms, k_ms = time_steps(layers, inputs, steps, args.warmup)
        g_ms = graph_steps(layers, inputs, steps, args.warmup)
        D = float(np.mean([distinct_experts(ly, T) for ly in layers]))
        res[f"T{T}"] = {"hip_graph_ms_per_step": round(g_ms, 4), "hip_graph_tokens_per_s": round(T / (g_ms / 1e3), 1),
                        "ms_per_step_eager": round(ms, 4), "distinct_experts": D,
                        "layer_hbm_frac": round(layer_bytes(D, T, s, MXC_BYTES_PER_WEIGHT) / (g_ms / 1e3) / 1e9
                                                / HBM_PEAK_GBS, 4),
                        "gate_up_ms": round(k_ms["gate_up"], 5),
                        "gate_up_hbm_frac": round(gate_up_bytes(D, T, s, MXC_BYTES_PER_WEIGHT) / (k_ms["gate_up"] / 1e3)
                                                  / 1e9 / HBM_PEAK_GBS, 4)}
        del layers
    del lws
    torch.cuda.empty_cache()
    return res


def run_tsweep(moe, synth, args):
    """Both GEMM kernels forced at each batch (decode weights, tiled): the
    token counts where the MFMA-tiled kernel overtakes the weight-streaming one
    (MOE_ALGO_AUTO switches at rows >= 4 E, i.e. 128 tokens at 256 experts and top-8)."""
    import torch
    wd = synth.WORKLOADS["decode"]
    s = wd.shape
    lw = make_weights(host_weights(synth, "decode", 0))
    res = {}
    for T in (64, 128, 192, 256, 384, 512, 1024, 2048, 4096):
        x, l = dev_bf16(synth.activations(wd, T)), dev(synth.logits(wd, T))
        ly = layer_for(moe, lw, s, T)
        row = {}
        for name, algo in (("decode", moe.MOE_ALGO_DECODE), ("prefill", moe.MOE_ALGO_PREFILL)):
            ms, k_ms = time_steps([ly], [(x, l, None, None)], 10, 3, algo=algo)
            row[name] = {"layer_ms": round(ms, 4), "gate_up_ms": round(k_ms["gate_up"], 4),
                         "down_ms": round(k_ms["down"], 4)}
        log(f"[bench] T-sweep T={T}: decode {row['decode']['layer_ms']} ms, prefill {row['prefill']['layer_ms']} ms")
        res[f"T{T}"] = row
        del ly
    del lw
    torch.cuda.empty_cache()
    return res


def run_router(moe, synth, args):
    """Router matmul fused with the group top-k (moe_route_gemv) at decode
    batches, against the top-k alone on given logits (moe_route) and a torch
    FP32 matmul (the router matmul done by a library GEMM)."""
    import torch
    w = synth.WORKLOADS["decode"]
    RW = dev(synth.router_weight(w))
    res = {}
    for T in (1, 8, 64):
        log(f"[bench] router matmul + top-k T={T}")
        x, l = dev_bf16(synth.activations(w, T)), dev(synth.logits(w, T))
        ws = torch.zeros(moe.route_gemv_workspace_bytes(T, 256), dtype=torch.uint8, device="cuda")
        ids = torch.empty((T, 8), dtype=torch.int32, device="cuda")
        wt = torch.empty((T, 8), dtype=torch.float32, device="cuda")

        def us(f, n=100):
            for _ in range(10):
                f()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(n):
                f()
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) / n * 1000
        res[f"T{T}"] = {
            "route_gemv_us": round(us(lambda: moe.route_gemv(x, RW, None, 256, 8, 4, 8, 2.827, ws, ids=ids,
                                                             weights=wt)), 2),
            "route_only_us": round(us(lambda: moe.route(l, None, 256, 8, 4, 8, 2.827, ids=ids, weights=wt)), 2),
            "torch_fp32_matmul_us": round(us(lambda: torch.matmul(x.float(), RW.t())), 2)}
    return res


WORKLOAD_RUNNERS = {
    "prefill": lambda moe, synth, a: run_prefill(moe, synth, a, "bf16"),
    "w4a8": lambda moe, synth, a: run_prefill(moe, synth, a, "mxfp8"),
    "w4a4": lambda moe, synth, a: run_w4a4(moe, synth, a, "dequant"),
    "w4a4_planes": lambda moe, synth, a: run_w4a4(moe, synth, a, "planes"),
    "reap50": run_reap50,
    "outliers": run_outliers,
    "router": run_router,
    "compact": run_compact,
}
# run only when asked for (--workload tsweep): a sweep for the kernel choice, not a bench line
SWEEPS = {"tsweep": run_tsweep}
EXTRA_KEYS = {"prefill": "prefill_T8192", "w4a8": "prefill_T8192_w4a8_mxfp8", "w4a4": "w4a4_T4096",
              "w4a4_planes": "w4a4_T4096_planes", "reap50": "reap50_T16384_2layers",
              "outliers": "down_proj_outliers_32768x2048", "router": "fused_router_decode",
              "compact": "decode_compact_mxfp4_4p125", "tsweep": "gemm_kernel_choice_T_sweep"}


if __name__ == "__main__":
    main()
