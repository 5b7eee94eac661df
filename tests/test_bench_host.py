"""Host logic of bench.py (CPU): the algorithmic work formulas, the choice of
the kernel each expert stage is priced on, and the digest-checked lookup of
profiled memory traffic."""
import numpy as np
import pytest

import bench
import synth


def test_step_work_of_the_decode_batch():
    """25.62 GB for the decode batch with 253 of 256 experts touched: the
    touched experts' three matrices, the router, pooler and unpooler, x in, out
    (fp32) and the fp32 logits and pooled rows."""
    w = synth.WORKLOADS["decode_bf16"]
    byts, flops = bench.step_work(w, 253)
    expert = 253 * 3 * 4096 * 4096 * 2
    dense = (256 + 2 * 4096) * 8192 * 2
    io = 128 * 8192 * 2 + 128 * 8192 * 4 + (4096 + 256 * 4096) * 4
    assert byts == expert + dense + io
    assert abs(byts / 1e9 - 25.62) < 0.01
    # 943.7 MFLOP per token
    assert abs(flops / w.T / 1e6 - 943.7) < 0.1


def test_stage_work_adds_up_to_the_expert_gemms():
    w = synth.WORKLOADS["prefill_bf16"]
    gu_b, gu_f = bench.algorithmic(w, 256, "gate_up")
    dn_b, dn_f = bench.algorithmic(w, 256, "down")
    ex_b, ex_f = bench.algorithmic(w, 256, "experts")
    assert (ex_b, ex_f) == (gu_b + dn_b, gu_f + dn_f)
    A = w.T * w.k
    assert gu_f == 2.0 * A * w.Dp * 2 * w.F and dn_f == 2.0 * A * w.F * w.Dp
    # weights dominate: 256 experts x 2F x Dp bf16
    assert gu_b >= 256 * 2 * w.F * w.Dp * 2
    # MXFP4 weights: half a byte plus one scale byte per 32
    mw = synth.WORKLOADS["mxfp4"]
    mb, _ = bench.algorithmic(mw, 256, "gate_up")
    assert mb == int(256 * 2 * mw.F * mw.Dp * (0.5 + 1 / 32) + mw.T * mw.Dp * (1 + 1 / 32)
                     + A * mw.F * (1 + 1 / 32))
    with pytest.raises(ValueError):
        bench.algorithmic(w, 1, "nope")


def stage_kernels(w, counts, n_cu=256):
    stage_ms = {s: 1.0 for s in ("proj_in", "gate_up", "down", "unpool")}
    return [(k["kernel"], k["stages"]) for k in bench.kernel_rooflines(w, stage_ms, np.asarray(counts), n_cu)]


def test_expert_stages_are_priced_on_the_kernel_that_runs():
    d = synth.WORKLOADS["decode_bf16"]
    # decode: 253 streamed experts (>= 3/4 of the CUs): the fused kernel
    ks = stage_kernels(d, [4] * 253 + [0] * 3)
    assert ks[0][0] == "dense_stream_kernel" and ks[-1][0] == "dense_stream_kernel"
    assert ("fused_stream_kernel", ["gate_up", "down"]) in ks
    # few streamed experts: the single-wave streaming kernels
    ks = stage_kernels(d, [64] * 16 + [0] * 240)
    assert ("stream_kernel<EPI_SWIGLU>", ["gate_up"]) in ks and ("stream_kernel<EPI_DOWN>", ["down"]) in ks
    # prefill: every expert on the tiled GEMM; dense projections on the tiled kernel
    p = synth.WORKLOADS["prefill_bf16"]
    ks = stage_kernels(p, [512] * 256)
    assert ("gemm_grouped_kernel<EPI_SWIGLU>", ["gate_up"]) in ks
    assert ks[0] == ("gemm_grouped_kernel<EPI_F32>", ["proj_in"])
    # mixed: both kinds in one stage
    ks = stage_kernels(synth.WORKLOADS["skewed_bf16"], [4000] + [30] * 255)
    assert any(k.startswith("gate/up stage") for k, _ in ks)
    # MXFP4: streamed up to 32 rows, never fused
    m = synth.WORKLOADS["mxfp4_decode"]
    ks = stage_kernels(m, [4] * 256)
    assert ("stream_mx_kernel<EPI_SWIGLU>", ["gate_up"]) in ks
    # at most 128 tokens every expert is streamed (in passes), whatever its rows
    ks = stage_kernels(m, [100] + [4] * 7 + [0] * 248)
    assert ("stream_mx_kernel<EPI_DOWN>", ["down"]) in ks
    ks = stage_kernels(d, [100] * 2 + [0] * 254)
    assert ("stream_kernel<EPI_SWIGLU>", ["gate_up"]) in ks
    assert bench.stream_limit(d) == 128 and bench.stream_limit(p) == 64
    assert bench.stream_limit(synth.WORKLOADS["mxfp4"]) == 32


def test_profiled_traffic_is_used_only_for_the_current_sources(tmp_path, monkeypatch):
    f = tmp_path / "traffic.txt"
    good = bench.kernel_digest("stream_kernel<EPI_SWIGLU>")
    assert good is not None and len(good) == 16
    # digests follow the sources: the fused and single-wave kernels share stream.hip
    assert bench.kernel_digest("fused_stream_kernel") == good
    assert bench.kernel_digest("gemm_grouped_kernel<EPI_DOWN>") != good
    assert bench.kernel_digest("no_such_kernel") is None
    f.write_text("# comment line\n"
                 f"w gate_up stream_kernel<EPI_SWIGLU> {good} 1000 10\n"
                 f"w gate_up fused_stream_kernel {good} 5 5\n"
                 f"w down stream_kernel<EPI_DOWN> {good} 7 3\n"
                 f"w2 gate_up stream_kernel<EPI_SWIGLU> 0123456789abcdef 1 1\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("w", ["gate_up"]) == 1020
    assert bench.measured_traffic("w", ["gate_up", "down"]) == 1030
    assert bench.measured_traffic("w", ["down"], launches=2) == 20
    # a line taken on other sources voids the figure; no line gives none
    assert bench.measured_traffic("w2", ["gate_up"]) is None
    assert bench.measured_traffic("w", ["unpool"]) is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.measured_traffic("w", ["gate_up"]) is None


def test_roofline_entry_picks_the_binding_resource():
    w = synth.WORKLOADS["decode_bf16"]
    e = bench.roofline_entry(w, "k", "x", (8e9, 1e9), ["gate_up"], 1.0, bench.PEAK_BF16_TFLOPS)
    assert e["bound"] == "hbm" and e["achieved"] == 8000.0 and e["frac"] == 1.0
    e = bench.roofline_entry(w, "k", "x", (1e6, 2.5e12), ["gate_up"], 2.0, bench.PEAK_BF16_TFLOPS)
    assert e["bound"] == "mfma" and abs(e["frac"] - 0.5) < 1e-9
    m = synth.WORKLOADS["mxfp4"]
    e = bench.roofline_entry(m, "k", "x", (1e6, 5e12), ["gate_up"], 2.0, bench.PEAK_FP8_TFLOPS)
    assert e["peak"] == bench.PEAK_FP8_TFLOPS and e["peak_fp4"] == bench.PEAK_FP4_TFLOPS
    assert abs(e["frac_fp4"] - 2500 / 10100) < 1e-4
