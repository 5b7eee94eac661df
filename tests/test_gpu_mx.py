"""GPU parity of the MXFP4-expert path (MXFP4 expert weights, MXFP8 E4M3 expert
inputs on the block-scaled MFMA) against the CPU oracle.

* The activation quantizer (lmoe_mx_quantize_e4m3, the rule the path applies to
  xp and h) is compared bit for bit with the oracle's MXFP8 codec on the same
  fp32 values: codes and scales are integers decided from identical inputs.
* The block output is compared with the oracle in MX mode (it dequantizes the
  MXFP4 weights and quantizes xp and h to MXFP8 at the same points) within
  max|err|/RMS(out) <= 6e-2, at small multi-tile shapes and at the full size on
  a seeded 64-token subset of the 16K prefill chunk.
* Experts with at most 32 rows take the MX weight-streaming kernel, the rest
  the tiled grouped GEMM (row tiles of up to 320): row counts at the boundaries (0, 1, 16, 17, 32, 33), both
  GEMMs at K = 1024, 2048 and 4096, and the full-size decode batch (T=128).
"""
import numpy as np
import pytest
import torch

import latent_moe_layer_router_amd as lmoe
import oracle
import synth
from synth import device as sdev
from tests import harness as H
from tests.pins import tiny
from tests.test_gpu_parity import run_case, run_crafted, upload

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def quant_inputs(seed=7):
    """fp32 blocks of 32 covering the codec's cases: normal data at scales from
    2^-30 to 2^30, an all-zero block, exact ties of the E4M3 grid, values that
    saturate at 448, values in the E4M3 subnormal range, extreme blocks
    (largest finite floats, fp32 subnormals), and signed zeros and NaNs."""
    rng = np.random.default_rng(seed)
    blocks = []
    for e in range(-30, 31, 3):
        blocks.append(rng.standard_normal((8, 32)) * 2.0 ** e)
    blocks.append(np.zeros((1, 32)))
    # ties: amax fixes X = 0 (amax = 256); other values at midpoints of the grid
    mant = np.arange(8) / 8.0
    for _ in range(8):
        ex = rng.integers(-6, 8, 31)
        m = rng.integers(0, 8, 31)
        mid = (1.0 + mant[m] + 1 / 16.0) * 2.0 ** ex
        sign = rng.choice([-1.0, 1.0], 31)
        blocks.append(np.concatenate([[256.0], sign * mid])[None, :])
    # saturation: amax in [464, 512) * 2^X rounds to 512, stored as 448
    for a in (464.0, 480.0, 500.0, 511.0):
        b = rng.standard_normal(32) * 100
        b[5] = a
        blocks.append(b[None, :] * 2.0 ** 3)
    # E4M3 subnormals: tiny values next to a large one
    b = rng.uniform(-1, 1, 32) * 2.0 ** -8
    b[0] = 300.0
    blocks.append(b[None, :])
    # extremes
    blocks.append(rng.uniform(-3.4e38, 3.4e38, (1, 32)))
    blocks.append(rng.uniform(-1e-40, 1e-40, (1, 32)))
    # signed zeros and NaNs: -0 codes as +0, a NaN codes as +0 and is left out
    # of the block maximum
    b = rng.standard_normal(32) * 4.0
    b[[1, 7, 20]] = -0.0
    b[[3, 11]] = np.nan
    blocks.append(b[None, :])
    v = np.concatenate(blocks).astype(np.float32).ravel()
    return v


def test_mx_quantize_bitexact():
    v = quant_inputs()
    n = v.size
    H.say(f"[gpu] mx quantize: {n // 32} blocks")
    x = torch.from_numpy(v).to(DEV)
    codes = torch.empty(n, dtype=torch.uint8, device=DEV)
    scales = torch.empty(n // 32, dtype=torch.uint8, device=DEV)
    lmoe.lmoe_mx_quantize_e4m3(x.data_ptr(), n, codes.data_ptr(), scales.data_ptr(),
                               torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    rc, rs, _ = oracle.default().mx_quant_e4m3(v.astype(np.float64))
    gc, gs = codes.cpu().numpy(), scales.cpu().numpy()
    bad_s = np.nonzero(gs != rs)[0]
    assert bad_s.size == 0, f"{bad_s.size} scales differ, first block {bad_s[:4]}"
    bad = np.nonzero(gc != rc)[0]
    assert bad.size == 0, (f"{bad.size} codes differ, first at {bad[:4]}: "
                           f"v={v[bad[:4]]} gpu={gc[bad[:4]]} oracle={rc[bad[:4]]}")


def mx_tiny(**kw):
    return tiny(act=synth.BF16, expert_w=synth.MXFP4, **kw)


@pytest.mark.parametrize("T,E,k", [(100, 8, 2), (600, 4, 2), (37, 16, 3)])
def test_mx_small(T, E, k):
    """Dp = F = 1024 (the path needs multiples of 1024). T=600, E=4, k=2 puts
    about 300 rows on each expert: one tile of up to 320 rows split between
    two wave rows with a ragged tail; the others leave each expert a few rows."""
    run_case(mx_tiny(T=T, D=256, Dp=1024, F_=1024, E=E, k=k, seed=200 + T))


@pytest.mark.parametrize("T", [136, 40])
def test_mx_wide_pooled_rows(T):
    """Dp = 9216: the MXFP8 pooled norm of T > 128 (256 threads) reads the row a
    second time instead of keeping it in registers; at T = 40 the small-batch
    kernel (1024 threads) keeps it, with a partial third chunk on some
    threads, each MXFP8 block still the chunks of 8 consecutive lanes."""
    run_case(mx_tiny(T=T, D=256, Dp=9216, F_=1024, E=4, k=1, seed=250 + T))


def test_mx_all_tokens_same_experts():
    """Every token on the same two experts (300 rows each: one full tile and a
    44-row tail), every other expert empty."""
    w = mx_tiny(T=300, D=256, Dp=1024, F_=1024, E=8, k=2, seed=210)
    wts = synth.dense_weights(w)
    b = np.zeros(w.E, np.float32)
    b[[2, 6]] = [60.0, 50.0]
    wts["b_router"] = b
    _, a = run_case(w, wts=wts)
    assert np.all(a["topk_ids"] == np.array([2, 6]))


def test_mx_full_size_prefill_subset():
    """Full shapes (D=8192, Dp=F=4096, E=256, k=8), T=16384, MXFP4 experts:
    selection and permutation on every token, the output on a seeded 64-token
    subset, in the benchmark's launch configuration (max_tokens = 16384)."""
    w = synth.WORKLOADS["mxfp4"]
    H.say("[gpu] mxfp4 full size: uploading weights (6.9 GB of MXFP4 experts)")
    tw = sdev.upload_weights(w, DEV)
    hw = H.host_weights(w, with_experts=False)
    block = lmoe.LatentMoE(tw, w.k, w.T, w.eps_pool, w.eps_expert, out_dtype=torch.float32)
    x = synth.x(w)
    out, aux = block.forward(sdev.to_device(x, DEV), aux=True)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    a = {n: t.cpu().numpy() for n, t in aux.items()}
    block.close()
    O = oracle.default()
    logits = O.router(x, hw["w_router"], hw.get("b_router"))
    ids, wts = O.topk_softmax(logits, w.k)
    near = H.check_routing(a["topk_ids"], a["topk_w"], a["logits"], logits, ids, wts, w.k)
    H.check_permutation(a["topk_ids"], a["expert_offsets"], a["sorted_assign"], w.E)
    rows = synth.subset(w)
    ref, _ = H.oracle_ref(w, x[rows], hw)
    keep = ~near[rows]
    err = H.out_error(got[rows][keep], ref[keep])
    H.say(f"[gpu]   mxfp4: max|err|/rms = {err:.3e} on {int(keep.sum())} tokens")
    assert err <= H.tol(w), err
    del tw
    torch.cuda.empty_cache()


def test_mx_stream_row_boundaries():
    """Experts with 32 rows (the MX weight-streaming kernel's limit: two token
    tiles), 33 and 40 (the tiled GEMM), 17 and 16 (two and one token tiles), 1
    and 0 rows in one call (139 tokens: above 128 the tiled GEMM takes the
    experts with more than 32 rows)."""
    counts = [32, 33, 17, 16, 1, 40, 0]
    assign = np.repeat(np.arange(len(counts)), counts)
    w = mx_tiny(T=len(assign), D=256, Dp=1024, F_=1024, E=len(counts), k=1, seed=220)
    a = run_crafted(w, assign)
    assert np.diff(a["expert_offsets"]).tolist() == counts


@pytest.mark.parametrize("counts", [[90, 33, 4, 1, 0], [128, 0, 0, 0, 0]])
def test_mx_small_batch_experts_in_passes(counts):
    """At most 128 tokens: the MX weight-streaming kernel takes every expert,
    those above 32 rows in passes of 32 rows (90 = 32 + 32 + 26, 33 = 32 + 1,
    128 = 4 x 32), and the tiled GEMM is not launched."""
    assign = np.repeat(np.arange(len(counts)), counts)
    w = mx_tiny(T=len(assign), D=256, Dp=1024, F_=1024, E=len(counts), k=1, seed=221 + counts[0])
    a = run_crafted(w, assign)
    assert np.diff(a["expert_offsets"]).tolist() == counts


@pytest.mark.parametrize("Dp,F_", [(2048, 1024), (1024, 4096), (4096, 2048)])
def test_mx_stream_k_sizes(Dp, F_):
    """A few rows per expert (all streamed), gate/up over K = Dp and down over
    K = F of different sizes."""
    w = mx_tiny(T=24, D=256, Dp=Dp, F_=F_, E=16, k=4, seed=230 + Dp // 1024 + F_ // 512)
    _, a = run_case(w)
    assert np.diff(a["expert_offsets"]).max() <= 32


def test_mx_full_size_decode_subset():
    """Full shapes (D=8192, Dp=F=4096, E=256, k=8) at the decode batch T=128,
    MXFP4 experts: every expert gets a few rows, so both expert GEMMs stream
    their weights. Selection and permutation on every token, the output on a
    seeded 64-token subset."""
    w = synth.WORKLOADS["mxfp4_decode"]
    H.say("[gpu] mxfp4 full size, T=128: uploading weights")
    tw = sdev.upload_weights(w, DEV)
    hw = H.host_weights(w, with_experts=False)
    block = lmoe.LatentMoE(tw, w.k, w.T, w.eps_pool, w.eps_expert, out_dtype=torch.float32)
    x = synth.x(w)
    out, aux = block.forward(sdev.to_device(x, DEV), aux=True)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    a = {n: t.cpu().numpy() for n, t in aux.items()}
    block.close()
    counts = np.diff(a["expert_offsets"])
    assert counts.max() <= 32, counts.max()
    O = oracle.default()
    logits = O.router(x, hw["w_router"], hw.get("b_router"))
    ids, wts = O.topk_softmax(logits, w.k)
    near = H.check_routing(a["topk_ids"], a["topk_w"], a["logits"], logits, ids, wts, w.k)
    H.check_permutation(a["topk_ids"], a["expert_offsets"], a["sorted_assign"], w.E)
    rows = synth.subset(w)
    ref, _ = H.oracle_ref(w, x[rows], hw)
    keep = ~near[rows]
    err = H.out_error(got[rows][keep], ref[keep])
    H.say(f"[gpu]   mxfp4 decode: max|err|/rms = {err:.3e} on {int(keep.sum())} tokens")
    assert err <= H.tol(w), err
    del tw
    torch.cuda.empty_cache()


def test_mx_deterministic_and_token_permutation_invariant():
    """MXFP4 experts: two runs give identical bits, and permuting the tokens
    permutes the output rows bit-exactly. E = 24, k = 3 gives experts of about
    42 rows, so both the streamed (<= 32 rows) and the tiled kernel run."""
    w = mx_tiny(T=333, D=256, Dp=1024, F_=1024, E=24, k=3, seed=240)
    block = lmoe.LatentMoE(upload(synth.dense_weights(w)), w.k, w.T)
    x = sdev.to_device(synth.x(w), DEV)
    H.say("[gpu] mxfp4 determinism: two runs, then permuted tokens")
    o1, a1 = block.forward(x, aux=True)
    o2, a2 = block.forward(x, aux=True)
    perm = torch.from_numpy(np.random.default_rng(5).permutation(w.T)).to(DEV)
    o3 = block.forward(x[perm].contiguous())
    torch.cuda.synchronize()
    counts = np.diff(a1["expert_offsets"].cpu().numpy())
    assert counts.min() <= 32 < counts.max(), counts
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    for n in a1:
        assert torch.equal(a1[n], a2[n])
    assert torch.equal(o1[perm].view(torch.int16), o3.view(torch.int16))
    block.close()
