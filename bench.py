"""Benchmark of the latent-MoE block forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_bf16]
                    [--also prefill_bf16,mxfp4,mxfp4_decode] [--no-cpu-baseline] [--no-convert]

A step is one lmoe_forward over one batch of synthetic tokens already resident
in HBM: routing, permutation, pooler, experts, combine, unpooler. The timed
steps are lmoe_forward calls back to back; the same steps as replays of one
forward captured into a HIP graph are timed beside them (no faster: the host
enqueues far enough ahead that launches leave no gaps). The headline
workload is decode-sized (T=128 tokens; D=8192, Dp=4096, F=4096, E=256, k=8,
bf16), which streams the touched experts' weights and is bound by HBM; the
prefill chunk (T=16384) is reported beside it against the bf16 MFMA peak, and
the same chunk with MXFP4 experts (MXFP8 expert inputs) against the fp8 peak,
the decode batch with MXFP4 experts against HBM, and the load-time NVFP4 ->
MXFP4 re-encoding of a layer's experts against HBM.
Prints one JSON line. Weights are random-initialized (seed 0) with the model's
shapes; inputs are synthetic (see synth/).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "latent-MoE layer tokens/sec + % bf16 MFMA peak (T=16K) / % HBM BW (T=128)"
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense fp8 MFMA (the MXFP4 experts' fp8 x fp4 products)


def expert_bytes_per_weight(w):
    """Bytes per expert weight element: bf16, or MXFP4 (half a byte + 1/32 scale)."""
    return 0.5 + 1 / 32 if w.mx_act else 2


def act_bytes(w):
    """Bytes per expert-input activation element: bf16, or MXFP8 (1 + 1/32)."""
    return 1 + 1 / 32 if w.mx_act else 2


def algorithmic(w, n_active: int, kernel: str):
    """Algorithmic bytes and flops of one launch of a kernel (every touched weight
    read once, every activation it consumes read once and its output written once)."""
    wb, ab = expert_bytes_per_weight(w), act_bytes(w)
    T, D, Dp, F, E, k = w.T, w.D, w.Dp, w.F, w.E, w.k
    A = T * k
    if kernel == "gate_up":
        return int(n_active * 2 * F * Dp * wb + T * Dp * ab + A * F * ab), 2.0 * A * Dp * 2 * F
    if kernel == "down":
        return int(n_active * Dp * F * wb + A * F * ab + A * Dp * 2), 2.0 * A * F * Dp
    raise ValueError(kernel)


def step_work(w, n_active: int):
    """Algorithmic bytes and flops of one whole step."""
    es = 2
    T, D, Dp, F, E, k = w.T, w.D, w.Dp, w.F, w.E, w.k
    byts = int(n_active * 3 * F * Dp * expert_bytes_per_weight(w) + (E + 2 * Dp) * D * es
               + T * D * es + T * D * 4 + (Dp + E * Dp) * 4)
    flops = 2.0 * T * (E * D + Dp * D + k * 3 * Dp * F + D * Dp)
    return byts, flops


def run_workload(lmoe, torch, synth, sdev, block, w, steps, warmup, dev, graph=True):
    """Warmup, per-stage HIP-event times over `steps` forwards, then the timed
    region: `steps` forwards back to back, bracketed by synchronizations (no
    stage events inside). With `graph`, the same is timed again as replays of
    one forward captured into a HIP graph (reported beside the eager time)."""
    x = sdev.upload_x(w, dev)
    out = torch.empty((w.T, w.D), dtype=torch.float32, device=dev)
    _, aux = block.forward(x, out=out, aux=True)
    torch.cuda.synchronize()
    counts = (aux["expert_offsets"][1:] - aux["expert_offsets"][:-1]).cpu()
    n_active = int((counts > 0).sum())
    for _ in range(warmup):
        block.forward(x, out=out)
    torch.cuda.synchronize()
    block.set_timing(True)
    for _ in range(steps):
        block.forward(x, out=out)
    torch.cuda.synchronize()
    block.set_timing(False)
    stage_ms, n = block.get_timing()
    stage_ms = {s: v / n for s, v in stage_ms.items()}

    def timed(step):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    ms = timed(lambda: block.forward(x, out=out))
    graph_ms = None
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            block.forward(x, out=out)
        for _ in range(warmup):
            g.replay()
        graph_ms = timed(g.replay)
        del g
    return ms, stage_ms, n_active, counts, graph_ms


def cold_steps(torch, block, w, sdev, dev, n=10):
    """Per-step times (HIP events on the launching stream) with the Infinity
    Cache (256 MiB) flushed before each step by writing a 512 MiB buffer
    outside the timed events. Median and minimum, ms."""
    x = sdev.upload_x(w, dev)
    out = torch.empty((w.T, w.D), dtype=torch.float32, device=dev)
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    s = torch.cuda.current_stream()
    times = []
    for i in range(n + 1):
        scratch.fill_(i & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        block.forward(x, out=out, stream=s)
        e1.record(s)
        torch.cuda.synchronize()
        if i:
            times.append(e0.elapsed_time(e1))
    del scratch
    times.sort()
    return round(times[len(times) // 2], 4), round(times[0], 4)


# The gate/up kernel of each regime and the sources that define it: the
# weight-streaming kernels for decode-sized batches, the tiled grouped GEMMs
# for prefill-sized ones (bf16 or MXFP4 experts).
CSRC = os.path.join(ROOT, "latent_moe_layer_router_amd", "csrc")
GATE_UP_KERNEL = {"hbm": ("stream_kernel<EPI_SWIGLU>", ("stream.hip", "common.h")),
                  "hbm_mx": ("stream_mx_kernel<EPI_SWIGLU>", ("stream_mx.hip", "mx.h", "common.h")),
                  "mfma": ("gemm_grouped_kernel<EPI_SWIGLU>", ("gemm_grouped.hip", "common.h")),
                  "mfma_mx": ("gemm_grouped_mx_kernel<EPI_SWIGLU>", ("gemm_grouped_mx.hip", "mx.h", "common.h")),
                  "convert": ("nvfp4_to_mxfp4_kernel", ("convert.hip", "common.h"))}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gate_up_traffic.txt")


def kernel_digest(bound):
    h = hashlib.sha256()
    for f in GATE_UP_KERNEL[bound][1]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, bound):
    """Memory-side bytes per launch of the workload's dominant kernel, from the
    profiles: reads from the L2's 32-, 64- and 128-byte read requests to memory
    (TCC_EA0_RDREQ_32B/64B/128B; a 1 GiB device copy reads 1.00 GiB this way),
    writes from WRITE_SIZE (the copy writes 1.00 GiB). None unless they were
    taken on the kernel source as it is now."""
    try:
        with open(TRAFFIC_FILE) as fh:
            lines = fh.read().splitlines()
    except OSError:
        return None
    digest = kernel_digest(bound)
    for ln in lines:
        f = ln.split()
        if len(f) == 4 and not ln.startswith("#") and f[0] == workload and f[1] == digest:
            return int(f[2]) + int(f[3])
    return None


def roofline(w, stage_ms, n_active, bound):
    byts, flops = algorithmic(w, n_active, "gate_up")
    t = stage_ms["gate_up"] * 1e-3
    traffic = measured_traffic(w.name, bound)
    common = {"kernel": GATE_UP_KERNEL[bound][0] + " (gate/up grouped GEMM + SwiGLU)",
              "traffic": traffic, "algorithmic_bytes": byts,
              "traffic_over_algorithmic": None if traffic is None else round(traffic / byts, 3),
              "avg_ms": round(stage_ms["gate_up"], 4)}
    if bound in ("hbm", "hbm_mx"):
        ach = byts / t / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), **common}
    ach = flops / t / 1e12
    peak = PEAK_FP8_TFLOPS if bound == "mfma_mx" else PEAK_BF16_TFLOPS
    return {"bound": "mfma", "achieved": round(ach, 1), "peak": peak, "unit": "TFLOP/s",
            "frac": round(ach / peak, 4), "algorithmic_flops": flops, **common}


def regime(w):
    """The gate/up kernel a workload runs on: weight streaming when every expert
    gets a few rows (decode batches: T * k / E = 4 here), else the tiles."""
    decode = w.T * w.k <= 4 * w.E
    if w.mx_act:
        return "hbm_mx" if decode else "mfma_mx"
    return "hbm" if decode else "mfma"


def cpu_baseline(synth, w):
    """The CPU oracle on the whole decode batch (its T tokens, four times over),
    timed on this host's cores; expert weights are generated before the clock
    starts."""
    import numpy as np

    import oracle
    x = synth.x(w)
    wts = {"w_router": synth.w_router(w), "b_router": synth.router_bias(w),
           "w_pool": synth.w_pool(w), "g_pool": synth.g_pool(w), "g_expert": synth.g_expert(w),
           "w_unpool": synth.w_unpool(w)}
    O = oracle.default()
    ids, _ = O.topk_softmax(O.router(x, wts["w_router"], wts["b_router"]), w.k)
    experts = {int(e): (synth.w_gate_up(w, int(e)), synth.w_down(w, int(e))) for e in np.unique(ids)}
    reps = 4
    t0 = time.perf_counter()
    for _ in range(reps):
        O.forward(x, wts, w.k, w.eps_pool, w.eps_expert, get_expert=experts.__getitem__,
                  rnd=w.act == synth.BF16)
    dt = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count())
    return {"value": round(reps * w.T / dt, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"all {w.T} tokens of the {w.name} batch (one full step) run {reps} times, "
                      f"{dt:.1f} s in total"}


def nvfp4_convert(lmoe, torch, dev, E=256, Dp=4096, F=4096, reps=5):
    """Load-time re-encoding of a layer's NVFP4 expert weights as MXFP4: both
    matrices of all E experts (gate/up [E][2F][Dp], down [E][Dp][F]) from seeded
    random NVFP4 codes and scales, timed with HIP events on the launching stream.
    Algorithmic bytes per element: 1/2 (codes) + 1/16 (UE4M3 scales) read,
    1/2 (codes) + 1/32 (E8M0 scales) written."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    s = torch.cuda.current_stream()
    shapes = [(E, 2 * F, Dp), (E, Dp, F)]
    bufs = []
    for m, r, c in shapes:
        codes = torch.randint(0, 256, (m, r, c // 2), dtype=torch.uint8, device=dev, generator=gen)
        s16 = torch.randint(0x18, 0x60, (m, r, c // 16), dtype=torch.uint8, device=dev, generator=gen)
        g = torch.full((m,), 2.0 ** -7, dtype=torch.float32, device=dev)
        bufs.append((codes, s16, g, torch.empty_like(codes),
                     torch.empty((m, r, c // 32), dtype=torch.uint8, device=dev), m, r, c))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    times = []
    for rep in range(reps + 1):
        ev[0].record(s)
        for i, (codes, s16, g, oc, os_, m, r, c) in enumerate(bufs):
            lmoe.lmoe_nvfp4_to_mxfp4(codes.data_ptr(), s16.data_ptr(), g.data_ptr(), m, r, c,
                                     oc.data_ptr(), os_.data_ptr(), s.cuda_stream)
            ev[i + 1].record(s)
        torch.cuda.synchronize()
        if rep:
            times.append(ev[0].elapsed_time(ev[2]))
    n = sum(m * r * c for m, r, c in shapes)
    byts = n * (1 / 2 + 1 / 16 + 1 / 2 + 1 / 32)
    ms = sorted(times)[len(times) // 2]
    gbs = byts / (ms * 1e-3) / 1e9
    del bufs
    torch.cuda.empty_cache()
    traffic = measured_traffic("nvfp4_to_mxfp4", "convert")   # both launches
    return {"workload": "nvfp4_to_mxfp4", "what": f"all {E} experts' gate/up and down weights, "
            "NVFP4 -> MXFP4 (load time, two launches)", "elements": n, "ms": round(ms, 4),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                         "traffic_over_algorithmic": None if traffic is None else round(traffic / byts, 3),
                         "kernel": "nvfp4_to_mxfp4_kernel", "algorithmic_bytes": int(byts)}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_bf16")
    ap.add_argument("--also", default="prefill_bf16,mxfp4,mxfp4_decode",
                    help="comma-separated extra workloads, or ''")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the extra timing of HIP graph replays")
    ap.add_argument("--no-convert", action="store_true",
                    help="skip timing the load-time NVFP4 -> MXFP4 weight re-encoding")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run one plain device-to-device copy of this many MiB (a kernel of "
                         "known traffic, to calibrate hardware byte counters against)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the block is built and "
              "measured on a single MI355X", file=sys.stderr)
        sys.exit(2)

    import torch

    import latent_moe_layer_router_amd as lmoe
    import synth
    from synth import device as sdev

    dev = torch.device("cuda:0")
    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    w = synth.WORKLOADS[args.workload]
    extra = [synth.WORKLOADS[n] for n in args.also.split(",") if n]
    max_tokens = max([w.T] + [e.T for e in extra])
    t0 = time.perf_counter()
    tw = sdev.upload_weights(w, dev)
    print(f"[bench] weights uploaded in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    block = lmoe.LatentMoE(tw, w.k, max_tokens, w.eps_pool, w.eps_expert, out_dtype=torch.float32)

    ms, stage_ms, n_active, _, graph_ms = run_workload(lmoe, torch, synth, sdev, block, w, args.steps,
                                                       args.warmup, dev, graph=not args.no_graph)
    print(f"[bench] {w.name}: {ms:.3f} ms/step (graph replay {graph_ms}), stages {stage_ms}", file=sys.stderr,
          flush=True)
    cold_med, cold_min = cold_steps(torch, block, w, sdev, dev)
    print(f"[bench] {w.name} with the Infinity Cache flushed before each step: median {cold_med:.3f} ms, "
          f"min {cold_min:.3f} ms", file=sys.stderr, flush=True)
    byts, flops = step_work(w, n_active)
    res = {
        "metric": METRIC, "value": round(w.T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "graph_replay_ms_per_step": None if graph_ms is None else round(graph_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) tokens, N(0,1/fan_in) random-init weights)",
        "config": {"workload": w.name, "T": w.T, "D": w.D, "Dp": w.Dp, "F": w.F, "E": w.E, "k": w.k,
                   "out_dtype": "f32", "active_experts": n_active},
        "step_hbm_frac": round(byts / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "roofline": roofline(w, stage_ms, n_active, regime(w)),
        "stages_ms": {s: round(v, 4) for s, v in stage_ms.items()},
        "cold_cache_ms": {"median": cold_med, "min": cold_min,
                          "what": "per-step HIP-event time, 512 MiB written between steps"},
    }
    also = []
    for e in extra:
        if e.expert_w != w.expert_w:
            # another expert format (MXFP4): its own weights and handle, after
            # the bf16 ones are released
            block.close()
            del tw
            torch.cuda.empty_cache()
            t0 = time.perf_counter()
            tw = sdev.upload_weights(e, dev)
            print(f"[bench] {e.name} weights uploaded in {time.perf_counter() - t0:.1f} s",
                  file=sys.stderr, flush=True)
            w = e
            block = lmoe.LatentMoE(tw, e.k, max_tokens, e.eps_pool, e.eps_expert,
                                   out_dtype=torch.float32)
        ems, est, ena, _, gms = run_workload(lmoe, torch, synth, sdev, block, e, args.steps, args.warmup, dev,
                                             graph=not args.no_graph)
        print(f"[bench] {e.name}: {ems:.3f} ms/step (graph replay {gms}), stages {est}", file=sys.stderr,
              flush=True)
        eb, ef = step_work(e, ena)
        entry = {"workload": e.name, "T": e.T, "expert_weights": e.expert_w,
                 "value": round(e.T / (ems * 1e-3), 1), "unit": "tokens/s",
                 "ms_per_step": round(ems, 4),
                 "graph_replay_ms_per_step": None if gms is None else round(gms, 4),
                 "step_tflops": round(ef / (ems * 1e-3) / 1e12, 1),
                 "roofline": roofline(e, est, ena, regime(e)),
                 "stages_ms": {s: round(v, 4) for s, v in est.items()}}
        if not e.mx_act:
            entry["step_mfma_frac"] = round(ef / (ems * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
        also.append(entry)
    block.close()
    del tw
    torch.cuda.empty_cache()
    if not args.no_convert:
        conv = nvfp4_convert(lmoe, torch, dev)
        print(f"[bench] nvfp4_to_mxfp4: {conv['ms']:.3f} ms, {conv['roofline']['achieved']} GB/s",
              file=sys.stderr, flush=True)
        also.append(conv)
    res["also"] = also
    w = synth.WORKLOADS[args.workload]
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(synth, w)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
