"""Benchmark of the latent-MoE block forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_bf16]
                    [--also prefill_bf16,skewed_bf16,mxfp4,mxfp4_decode] [--no-cpu-baseline]
                    [--no-convert]

A step is one lmoe_forward over one batch of synthetic tokens already resident
in HBM: routing, permutation, pooler, experts, combine, unpooler. The timed
steps are lmoe_forward calls back to back (the Infinity Cache stays warm
between them; the cold-cache figure beside them flushes it before each step),
and the same steps as replays of one forward captured into a HIP graph are
timed beside them. The headline workload is decode-sized (T=128 tokens;
D=8192, Dp=4096, F=4096, E=256, k=8, bf16), which streams the touched experts'
weights and is bound by HBM. Reported beside it: the prefill chunk (T=16384)
against the bf16 MFMA peak, the skewed-routing batch (T=4096, Zipf expert
load) against max(bytes / HBM, flops / MFMA), the prefill chunk with MXFP4
experts (MXFP8 expert inputs) against the fp8 and fp4 peaks, the decode batch
with MXFP4 experts against HBM, and the load-time NVFP4 -> MXFP4 re-encoding
of a layer's experts against HBM. Each workload lists every kernel stage with
its own roofline. Prints one JSON line. Weights are random-initialized
(seed 0) with the model's shapes; inputs are synthetic (see synth/).
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
PEAK_FP4_TFLOPS = 10100.0    # MI355X dense fp4 / fp6 MFMA
STREAM_MAX_ROWS = 64         # experts with at most this many rows are streamed (bf16)
ALL_STREAMED_T = 128         # batches of at most this many tokens stream every expert


def expert_bytes_per_weight(w):
    """Bytes per expert weight element: bf16, or MXFP4 (half a byte + 1/32 scale)."""
    return 0.5 + 1 / 32 if w.mx_act else 2


def act_bytes(w):
    """Bytes per expert-input activation element: bf16, or MXFP8 (1 + 1/32)."""
    return 1 + 1 / 32 if w.mx_act else 2


def algorithmic(w, n_active: int, kernel: str):
    """Algorithmic bytes and flops of one stage (every touched weight read once,
    every activation it consumes read once and its output written once)."""
    wb, ab = expert_bytes_per_weight(w), act_bytes(w)
    T, D, Dp, F, E, k = w.T, w.D, w.Dp, w.F, w.E, w.k
    A = T * k
    if kernel == "gate_up":
        return int(n_active * 2 * F * Dp * wb + T * Dp * ab + A * F * ab), 2.0 * A * Dp * 2 * F
    if kernel == "down":
        return int(n_active * Dp * F * wb + A * F * ab + A * Dp * 2), 2.0 * A * F * Dp
    if kernel == "experts":
        b0, f0 = algorithmic(w, n_active, "gate_up")
        b1, f1 = algorithmic(w, n_active, "down")
        return b0 + b1, f0 + f1
    if kernel == "proj_in":      # router + pooler: weights, x in, P and logits out (fp32)
        return int((E + Dp) * D * 2 + T * D * 2 + T * (Dp + E) * 4), 2.0 * T * (E + Dp) * D
    if kernel == "unpool":       # weights, u in (bf16), out (fp32)
        return int(D * Dp * 2 + T * Dp * 2 + T * D * 4), 2.0 * T * D * Dp
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


# Kernels and the sources that define them (a profile's counters are used
# only while these sources are unchanged).
CSRC = os.path.join(ROOT, "latent_moe_layer_router_amd", "csrc")
KERNEL_SOURCES = {"fused_stream_kernel": ("stream.hip", "common.h"),
                  "stream_kernel": ("stream.hip", "common.h"),
                  "dense_stream_kernel": ("stream.hip", "norm.hip", "common.h"),
                  "splitk_pool_norm_kernel": ("norm.hip", "mx.h", "route.h", "common.h"),
                  "splitk_reduce_kernel": ("stream.hip", "common.h"),
                  "stream_mx_kernel": ("stream_mx.hip", "mx.h", "common.h"),
                  "gemm_grouped_kernel": ("gemm_grouped.hip", "common.h"),
                  "gemm_grouped_mx_kernel": ("gemm_grouped_mx.hip", "mx.h", "common.h"),
                  "nvfp4_to_mxfp4_kernel": ("convert.hip", "common.h")}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kernel_traffic.txt")


def kernel_digest(kernel):
    srcs = KERNEL_SOURCES.get(kernel.split(":")[0].split("<")[0])
    if srcs is None:
        return None
    h = hashlib.sha256()
    for f in srcs:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, stages, launches=1):
    """Memory-side bytes of the given stages of a workload, from the profiles:
    the sum over every kernel those stages launch of its reads (the L2's 32-,
    64- and 128-byte read requests to memory, TCC_EA0_RDREQ_32B/64B/128B; a
    1 GiB device copy reads 1.00 GiB this way) and writes (WRITE_SIZE; the copy
    writes 1.00 GiB), per launch, times `launches`. None unless every such
    kernel was profiled on its sources as they are now."""
    try:
        with open(TRAFFIC_FILE) as fh:
            lines = fh.read().splitlines()
    except OSError:
        return None
    total, seen = 0, False
    for ln in lines:
        f = ln.split()
        if ln.startswith("#") or len(f) != 6 or f[0] != workload or f[1] not in stages:
            continue
        if kernel_digest(f[2]) != f[3]:
            return None
        total += int(f[4]) + int(f[5])
        seen = True
    return total * launches if seen else None


def roofline_entry(w, kernel, what, work, stages, ms, mfma_peak):
    """Roofline of one stage: its algorithmic bytes and flops over its HIP-event
    time, against the larger of bytes / HBM peak and flops / MFMA peak."""
    byts, flops = work
    t = ms * 1e-3
    t_hbm, t_mfma = byts / (PEAK_HBM_GBS * 1e9), flops / (mfma_peak * 1e12)
    traffic = measured_traffic(w.name, stages)
    e = {"kernel": kernel, "what": what, "stages": stages, "avg_ms": round(ms, 4),
         "algorithmic_bytes": byts, "algorithmic_flops": flops, "traffic": traffic,
         "traffic_over_algorithmic": None if traffic is None else round(traffic / byts, 3)}
    if t_hbm >= t_mfma:
        ach = byts / t / 1e9
        e.update({"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                  "frac": round(ach / PEAK_HBM_GBS, 4)})
    else:
        ach = flops / t / 1e12
        e.update({"bound": "mfma", "achieved": round(ach, 1), "peak": mfma_peak, "unit": "TFLOP/s",
                  "frac": round(ach / mfma_peak, 4)})
        if w.mx_act and mfma_peak == PEAK_FP8_TFLOPS:
            e.update({"peak_fp4": PEAK_FP4_TFLOPS, "frac_fp4": round(ach / PEAK_FP4_TFLOPS, 4)})
    return e


def stream_limit(w):
    """The largest expert the weight-streaming kernels take in this workload."""
    if w.T <= ALL_STREAMED_T:
        return ALL_STREAMED_T
    return 32 if w.mx_act else STREAM_MAX_ROWS


def kernel_rooflines(w, stage_ms, counts, n_cu):
    """Every compute stage of a workload with its roofline. Expert stages name
    the kernel that carries their work, decided from the routing the way the
    library decides it: the fused expert kernel when at least 3/4 as many
    experts as CUs are streamed (at most 64 rows each, bf16), else the
    weight-streaming kernels (MXFP4: at most 32 rows) and the tiled GEMMs. A
    batch of at most 128 tokens streams every expert (in passes)."""
    n_active = int((counts > 0).sum())
    mx = w.mx_act
    small = stream_limit(w)
    n_stream = int(((counts > 0) & (counts <= small)).sum())
    n_tiled = int((counts > small).sum())
    peak = PEAK_FP8_TFLOPS if mx else PEAK_BF16_TFLOPS
    dense = "dense_stream_kernel" if w.T <= 128 else "gemm_grouped_kernel<EPI_F32>"
    out = [roofline_entry(w, dense, "router + pooler GEMM (+ pooled RMSNorm at T <= 128)",
                          algorithmic(w, n_active, "proj_in"), ["proj_in"], stage_ms["proj_in"],
                          PEAK_BF16_TFLOPS)]
    fused = (not mx and n_stream >= (3 * n_cu + 3) // 4 and w.T * w.k >= (3 * n_cu + 3) // 4)
    sfx = "mx_kernel" if mx else "kernel"
    if fused and n_tiled == 0:
        out.append(roofline_entry(w, "fused_stream_kernel", "both expert GEMMs, SwiGLU and the "
                                  "sums of squares, one launch", algorithmic(w, n_active, "experts"),
                                  ["gate_up", "down"], stage_ms["gate_up"] + stage_ms["down"], peak))
    else:
        if n_tiled == 0:
            ku, kd = f"stream_{sfx}<EPI_SWIGLU>", f"stream_{sfx}<EPI_DOWN>"
        elif n_stream == 0:
            ku, kd = f"gemm_grouped_{sfx}<EPI_SWIGLU>", f"gemm_grouped_{sfx}<EPI_DOWN>"
        else:
            ku = kd = None
        out.append(roofline_entry(w, ku or "gate/up stage (streamed and tiled experts)",
                                  "gate/up grouped GEMM + SwiGLU", algorithmic(w, n_active, "gate_up"),
                                  ["gate_up"], stage_ms["gate_up"], peak))
        out.append(roofline_entry(w, kd or "down stage (streamed and tiled experts)",
                                  "down grouped GEMM + sums of squares", algorithmic(w, n_active, "down"),
                                  ["down"], stage_ms["down"], peak))
    out.append(roofline_entry(w, dense, "unpooler GEMM", algorithmic(w, n_active, "unpool"), ["unpool"],
                              stage_ms["unpool"], PEAK_BF16_TFLOPS))
    return out


def load_histogram(counts, small):
    c = counts[counts > 0]
    return {"active_experts": int(c.size), "empty_experts": int((counts == 0).sum()),
            "max_rows": int(c.max()), "mean_rows": round(float(c.mean()), 1),
            "max_over_mean": round(float(c.max() / c.mean()), 2),
            "streamed_experts": int((c <= small).sum()), "tiled_experts": int((c > small).sum()),
            "one_row_experts": int((c == 1).sum())}


def workload_entry(w, ms, stage_ms, counts, n_cu, graph_ms=None):
    """The measured figures of one workload."""
    n_active = int((counts > 0).sum())
    byts, flops = step_work(w, n_active)
    peak = PEAK_FP8_TFLOPS if w.mx_act else PEAK_BF16_TFLOPS
    ks = kernel_rooflines(w, stage_ms, counts, n_cu)
    experts = [k for k in ks if k["stages"] != ["proj_in"] and k["stages"] != ["unpool"]]
    dom = max(experts, key=lambda k: k["avg_ms"])
    t = ms * 1e-3
    e = {"workload": w.name, "T": w.T, "expert_weights": w.expert_w,
         "value": round(w.T / t, 1), "unit": "tokens/s", "ms_per_step": round(ms, 4),
         "graph_replay_ms_per_step": None if graph_ms is None else round(graph_ms, 4),
         "step_tflops": round(flops / t / 1e12, 1),
         "step_hbm_frac": round(byts / t / 1e9 / PEAK_HBM_GBS, 4),
         "step_mfma_frac": round(flops / t / 1e12 / peak, 4),
         "step_bound": "hbm" if byts / (PEAK_HBM_GBS * 1e9) >= flops / (peak * 1e12) else "mfma",
         "roofline": dom, "kernels": ks,
         "stages_ms": {s: round(v, 4) for s, v in stage_ms.items()},
         "load": load_histogram(counts, stream_limit(w))}
    if w.mx_act:
        e["step_mfma_frac_fp4"] = round(flops / t / 1e12 / PEAK_FP4_TFLOPS, 4)
    return e


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_tokens_per_s(synth, w, rows, reps=1):
    """The CPU oracle on the given token rows of workload w, timed; its expert
    weights are generated before the clock starts. Returns (tokens/s, seconds)."""
    import numpy as np

    import oracle
    x = synth.x(w, rows=rows)
    wts = {"w_router": synth.w_router(w), "b_router": synth.router_bias(w),
           "w_pool": synth.w_pool(w), "g_pool": synth.g_pool(w), "g_expert": synth.g_expert(w),
           "w_unpool": synth.w_unpool(w)}
    O = oracle.default()
    ids, _ = O.topk_softmax(O.router(x, wts["w_router"], wts["b_router"]), w.k)
    experts = {}
    for e in np.unique(ids):
        gu, dn = synth.w_gate_up(w, int(e)), synth.w_down(w, int(e))
        experts[int(e)] = (gu[0], gu[1], dn[0], dn[1]) if w.expert_w == synth.MXFP4 else (gu, dn)
    t0 = time.perf_counter()
    for _ in range(reps):
        O.forward(x, wts, w.k, w.eps_pool, w.eps_expert, mx_act=w.mx_act, get_expert=experts.__getitem__,
                  rnd=w.act == synth.BF16)
    dt = time.perf_counter() - t0
    del experts
    return reps * len(x) / dt, dt


def cpu_baseline(synth, w, subsets=("prefill_bf16", "skewed_bf16", "mxfp4")):
    """The CPU oracle (plain C, double accumulation, OpenMP over tokens) timed
    on this host: the whole decode batch on every core, 16 of its tokens on one
    thread, and seeded subsets of the larger workloads (64 tokens; 16 with
    MXFP4 experts, whose weights take longer to generate) on every core."""
    import numpy as np

    import oracle
    O = oracle.default()
    cores = O.threads()
    tps, dt = oracle_tokens_per_s(synth, w, np.arange(w.T), reps=2)
    total = dt
    O.set_threads(1)
    tps1, dt1 = oracle_tokens_per_s(synth, w, np.arange(16))
    O.set_threads(cores)
    total += dt1
    subs = []
    for name in subsets:
        sw = synth.WORKLOADS[name]
        n = 16 if sw.mx_act else 64
        r, d = oracle_tokens_per_s(synth, sw, synth.subset(sw, n, seed=1))
        total += d
        subs.append({"workload": name, "tokens": n, "value": round(r, 3), "unit": "tokens/s",
                     "cores": cores, "seconds": round(d, 2)})
    return {"value": round(tps, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"all {w.T} tokens of the {w.name} batch (one full step) run twice on {cores} "
                      f"threads, {dt:.1f} s; oracle runs here total {total:.1f} s",
            "single_thread": {"value": round(tps1, 3), "unit": "tokens/s", "cores": 1,
                              "sample": f"16 tokens of the {w.name} batch, {dt1:.1f} s"},
            "subsets": subs}


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
    traffic = measured_traffic("nvfp4_to_mxfp4", ["convert"], launches=2)   # profiled per launch
    return {"workload": "nvfp4_to_mxfp4", "what": f"all {E} experts' gate/up and down weights, "
            "NVFP4 -> MXFP4 (load time, two launches)", "elements": n, "ms": round(ms, 4),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                         "traffic_over_algorithmic": None if traffic is None else round(traffic / byts, 3),
                         "kernel": "nvfp4_to_mxfp4_kernel", "algorithmic_bytes": int(byts)}}


def pack_experts(lmoe, torch, tw):
    """The bf16 expert weights re-laid out in place by lmoe_pack_experts (each
    matrix through a one-matrix staging copy), timed with HIP events on the
    stream it runs on. Nothing large is allocated or freed: releasing a second
    25.8 GB copy slows HBM-bound kernels by a few percent for the next one to
    three seconds on MI355X, which would land in the timed steps."""
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    tw = lmoe.pack_expert_weights(tw, s, in_place=True)
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    byts = 4 * sum(tw[n].numel() * tw[n].element_size() for n in ("w_gate_up", "w_down"))
    return tw, {"ms": round(ms, 2), "GB/s": round(byts / (ms * 1e-3) / 1e9, 1),
                "what": "load-time re-layout of the bf16 expert weights in place (staging copy + pack: "
                        "each byte read twice and written twice), not in a step"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_bf16")
    ap.add_argument("--also", default="prefill_bf16,skewed_bf16,mxfp4,mxfp4_decode",
                    help="comma-separated extra workloads, or ''")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the extra timing of HIP graph replays")
    ap.add_argument("--no-convert", action="store_true",
                    help="skip timing the load-time NVFP4 -> MXFP4 weight re-encoding")
    ap.add_argument("--row-major-experts", action="store_true",
                    help="keep the bf16 expert weights row-major instead of packing them at load")
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
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    t0 = time.perf_counter()
    tw = sdev.upload_weights(w, dev)
    print(f"[bench] weights uploaded in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    packed = w.expert_w == synth.BF16 and not args.row_major_experts
    pack = None
    if packed:
        # load-time re-layout of the expert weights into 64 x 64 blocks, in
        # place (not part of a step)
        tw, pack = pack_experts(lmoe, torch, tw)
        print(f"[bench] expert weights packed in {pack['ms']:.1f} ms ({pack['GB/s']} GB/s)", file=sys.stderr,
              flush=True)
    block = lmoe.LatentMoE(tw, w.k, max_tokens, w.eps_pool, w.eps_expert, out_dtype=torch.float32,
                           packed=packed)

    ms, stage_ms, n_active, counts, graph_ms = run_workload(lmoe, torch, synth, sdev, block, w, args.steps,
                                                            args.warmup, dev, graph=not args.no_graph)
    print(f"[bench] {w.name}: {ms:.3f} ms/step (graph replay {graph_ms}), stages {stage_ms}", file=sys.stderr,
          flush=True)
    cold_med, cold_min = cold_steps(torch, block, w, sdev, dev)
    print(f"[bench] {w.name} with the Infinity Cache flushed before each step: median {cold_med:.3f} ms, "
          f"min {cold_min:.3f} ms", file=sys.stderr, flush=True)
    head = workload_entry(w, ms, stage_ms, counts.numpy(), n_cu, graph_ms)
    res = {
        "metric": METRIC, "value": head["value"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "graph_replay_ms_per_step": head["graph_replay_ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) tokens, N(0,1/fan_in) random-init weights)",
        "config": {"workload": w.name, "T": w.T, "D": w.D, "Dp": w.Dp, "F": w.F, "E": w.E, "k": w.k,
                   "out_dtype": "f32", "active_experts": n_active,
                   "expert_layout": "packed 64x64 blocks" if packed else "row-major"},
        "pack_experts": pack,
        "cache": "warm: steps back to back, so the 132 MiB of dense weights can stay in the 256 MiB "
                 "Infinity Cache (the 25 GB of expert weights cannot); cold_cache_ms flushes it",
        "step_hbm_frac": head["step_hbm_frac"],
        "roofline": head["roofline"],
        "kernels": head["kernels"],
        "stages_ms": head["stages_ms"],
        "cold_cache_ms": {"median": cold_med, "min": cold_min,
                          "step_hbm_frac_median": round(step_work(w, n_active)[0] / (cold_med * 1e-3) / 1e9
                                                        / PEAK_HBM_GBS, 4),
                          "what": "per-step HIP-event time, 512 MiB written between steps"},
        "load": head["load"],
    }
    also = []
    held = []            # handles kept open until the end (see below)
    for e in extra:
        if e.expert_w != w.expert_w:
            # another expert format (MXFP4): its own weights and handle, after
            # the bf16 ones are released (the upload that follows takes longer
            # than the clearing of the freed memory that slows kernels)
            for b_ in held + [block]:
                b_.close()
            held = []
            del tw
            torch.cuda.empty_cache()
            t0 = time.perf_counter()
            tw = sdev.upload_weights(e, dev)
            print(f"[bench] {e.name} weights uploaded in {time.perf_counter() - t0:.1f} s",
                  file=sys.stderr, flush=True)
            w = e
            block = lmoe.LatentMoE(tw, e.k, max_tokens, e.eps_pool, e.eps_expert,
                                   out_dtype=torch.float32)
        elif e.skew != w.skew:
            # the skewed workload: the same model plus a router bias (its own
            # handle; the previous one stays open, since a freed workspace is
            # cleared under the next timed steps)
            b = synth.router_bias(e)
            tw = dict(tw, b_router=None if b is None else sdev.to_device(b, dev))
            w = e
            held.append(block)
            block = lmoe.LatentMoE(tw, e.k, max_tokens, e.eps_pool, e.eps_expert,
                                   out_dtype=torch.float32, packed=packed)
        ems, est, _, ecounts, gms = run_workload(lmoe, torch, synth, sdev, block, e, args.steps, args.warmup,
                                                 dev, graph=not args.no_graph)
        print(f"[bench] {e.name}: {ems:.3f} ms/step (graph replay {gms}), stages {est}", file=sys.stderr,
              flush=True)
        also.append(workload_entry(e, ems, est, ecounts.numpy(), n_cu, gms))
    if not args.no_convert:
        # timed before anything is released, for the same reason
        conv = nvfp4_convert(lmoe, torch, dev)
        print(f"[bench] nvfp4_to_mxfp4: {conv['ms']:.3f} ms, {conv['roofline']['achieved']} GB/s",
              file=sys.stderr, flush=True)
        also.append(conv)
    for b_ in held + [block]:
        b_.close()
    del tw
    torch.cuda.empty_cache()
    res["also"] = also
    w = synth.WORKLOADS[args.workload]
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(synth, w)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
