"""GPU parity of the HIP path against the CPU oracle, small and mid-size shapes.

Every case calls the library through its C ABI (via the ctypes binding), on
seeded synthetic inputs, and compares element by element with the oracle:
expert selection and the permutation bit-exactly (outside near-tie tokens),
routing weights to the bound their logits imply, and the output within
max|err|/RMS(out) of 1e-4 (fp32) or 2e-2 (bf16; the oracle rounds at the same bf16
boundaries). The output is compared in fp32 (out_dtype = fp32); a bf16 output is
checked to be exactly the nearest-even rounding of the fp32 one.
"""
import numpy as np
import pytest
import torch

import latent_moe_layer_router_amd as lmoe
import synth
from synth import device as sdev
from tests import harness as H
from tests.pins import tiny

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def upload(wts: dict) -> dict:
    return {n: (sdev.to_device(a, DEV) if a is not None else None) for n, a in wts.items()}


def run_case(w, T=None, wts=None, max_tokens=None, check_out=True):
    T = w.T if T is None else T
    H.say(f"[gpu] case {w.name} T={T} D={w.D} Dp={w.Dp} F={w.F} E={w.E} k={w.k} act={w.act}")
    wts = synth.dense_weights(w) if wts is None else wts
    block = lmoe.LatentMoE(upload(wts), w.k, max_tokens or max(T, 1), w.eps_pool, w.eps_expert,
                           out_dtype=torch.float32)
    x = synth.x(w, T=T)
    out, aux = block.forward(sdev.to_device(x, DEV), aux=True)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    a = {n: t.cpu().numpy() for n, t in aux.items()}
    ref, raux = H.oracle_ref(w, x, wts)
    near = H.check_routing(a["topk_ids"], a["topk_w"], a["logits"], raux["logits"], raux["ids"],
                           raux["w"], w.k)
    H.check_permutation(a["topk_ids"], a["expert_offsets"], a["sorted_assign"], w.E)
    err = H.out_error(got[~near], ref[~near]) if check_out else 0.0
    H.say(f"[gpu]   max|err|/rms = {err:.3e}, near-ties = {int(near.sum())}")
    assert err <= H.tol(w), err
    block.close()
    return got, a


def test_tiny_fp32_config():
    """The tiny fp32 configuration: T=64, D=256, Dp=128, F=128, E=8, k=2."""
    run_case(synth.WORKLOADS["tiny_fp32"])


@pytest.mark.parametrize("T", [1, 63, 65, 200])
def test_small_bf16_ragged_T(T):
    run_case(tiny(T=T, D=256, Dp=128, F_=192, E=8, k=2, seed=101, act=synth.BF16), T=T)


@pytest.mark.parametrize("T", [128, 129, 1024, 1025])
def test_regime_boundaries(T):
    """Batch sizes at the host's switches: up to 128 tokens the split-K dense
    projections with the top-k inside the pooled-norm kernel and every expert
    streamed, from 129 the tiled projections, the top-k kernel and the tiled
    expert GEMM; up to 1024 tokens (16 chunks of 64) the sort's scan workgroup
    also places the assignments, from 1025 a second launch does."""
    run_case(tiny(T=T, D=512, Dp=256, F_=256, E=16, k=2, seed=140 + T % 7, act=synth.BF16), T=T)


@pytest.mark.parametrize("T", [641, 1000])
def test_dense_tiled_ragged_T(T):
    """T > 128 with Dp a multiple of 256: the router + pooler and the unpooler run
    on the tiled kernel's dense mode, M split evenly over the row-tile count the
    host picks (641 rows: 6 tiles of 106-107; 1000 rows: 8 tiles of 125)."""
    run_case(tiny(T=T, D=512, Dp=256, F_=256, E=8, k=2, seed=113, act=synth.BF16), T=T)


@pytest.mark.parametrize("E,k", [(1, 1), (3, 3), (37, 5), (64, 16)])
def test_small_bf16_expert_counts(E, k):
    run_case(tiny(T=77, D=128, Dp=64, F_=128, E=E, k=k, seed=102 + E, act=synth.BF16))


def test_multi_tile_bf16():
    """Several 128-row tiles per expert with ragged tails, several N and K tiles."""
    run_case(tiny(T=517, D=1024, Dp=512, F_=768, E=16, k=4, seed=103, act=synth.BF16))


def test_multi_tile_fp32():
    run_case(tiny(T=300, D=512, Dp=256, F_=384, E=12, k=3, seed=104, act=synth.F32))


@pytest.mark.parametrize("T,Dp", [(200, 8192), (200, 8448), (64, 8448)])
def test_wide_pooled_rows(T, Dp):
    """The pooled RMSNorm keeps a row in registers between its sum of squares
    and its scaling when the row fits (8192 values for the 256 threads of the
    T > 128 kernel, 32768 for the 1024 of the small-batch one). T = 200 with
    Dp = 8192 fills those registers exactly; with Dp = 8448 the row is read a
    second time; T = 64 with Dp = 8448 leaves some threads a partial third
    chunk in the small-batch kernel."""
    run_case(tiny(T=T, D=256, Dp=Dp, F_=256, E=4, k=2, seed=131 + T + Dp // 256, act=synth.BF16), T=T)


@pytest.mark.parametrize("Dp,F", [(128, 128), (256, 256)])
def test_all_tokens_same_experts(Dp, F):
    """A router bias forces every token onto the same k experts: three full
    experts of 300 rows and every other expert empty. With Dp = F = 128 they
    run as three 128-row tiles each; with Dp = F = 256 on the tiled grouped
    GEMM, one tile of 300 rows each (160 + 140 between the wave rows)."""
    w = tiny(T=300, D=256, Dp=Dp, F_=F, E=16, k=3, seed=105, act=synth.BF16)
    wts = synth.dense_weights(w)
    b = np.zeros(w.E, np.float32)
    b[[3, 5, 7]] = [60.0, 50.0, 40.0]
    wts["b_router"] = b
    _, a = run_case(w, wts=wts)
    assert np.all(a["topk_ids"] == np.array([3, 5, 7]))
    counts = np.diff(a["expert_offsets"])
    assert counts[3] == counts[5] == counts[7] == 300 and counts.sum() == 900


def test_experts_with_zero_and_one_rows():
    w = tiny(T=65, D=128, Dp=64, F_=64, E=70, k=1, seed=106, act=synth.BF16)
    _, a = run_case(w)
    counts = np.diff(a["expert_offsets"])
    assert (counts == 0).any() and (counts == 1).any()


def crafted_routing(w, assign, margin=8.0):
    """Weights and tokens of workload w where token t is routed to expert
    assign[t] (k = 1): router rows are the first E unit vectors and token t gets
    `margin` added at coordinate assign[t], so its logit leads by about margin."""
    wts = synth.dense_weights(w)
    wr = np.zeros((w.E, w.D), np.float32)
    wr[np.arange(w.E), np.arange(w.E)] = 1.0
    x = synth.as_f32(synth.x(w)).copy()
    x[np.arange(w.T), assign] += margin
    if w.act == synth.BF16:
        wr = synth.lib_round_bf16(wr)
        x = synth.lib_round_bf16(x)
    wts["w_router"] = wr
    return wts, x


def run_crafted(w, assign):
    wts, x = crafted_routing(w, assign)
    H.say(f"[gpu] crafted routing T={w.T} E={w.E} counts={np.bincount(assign, minlength=w.E).tolist()}")
    block = lmoe.LatentMoE(upload(wts), w.k, w.T, out_dtype=torch.float32)
    out, aux = block.forward(sdev.to_device(x, DEV), aux=True)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    a = {n: t.cpu().numpy() for n, t in aux.items()}
    ref, raux = H.oracle_ref(w, x, wts)
    H.check_routing(a["topk_ids"], a["topk_w"], a["logits"], raux["logits"], raux["ids"], raux["w"], w.k)
    H.check_permutation(a["topk_ids"], a["expert_offsets"], a["sorted_assign"], w.E)
    err = H.out_error(got, ref)
    H.say(f"[gpu]   max|err|/rms = {err:.3e}")
    assert err <= H.tol(w), err
    block.close()
    return a


def test_stream_path_row_boundaries():
    """Experts with 64 rows (the weight-streaming kernel's limit), 65 rows (the
    tiled GEMM), 1 row and 0 rows in one call (130 tokens: above 128 the
    tiled GEMM takes the experts with more than 64 rows)."""
    assign = np.array([0] * 64 + [1] * 65 + [2], np.int64)
    w = tiny(T=len(assign), D=256, Dp=128, F_=256, E=4, k=1, seed=110, act=synth.BF16)
    a = run_crafted(w, assign)
    assert np.diff(a["expert_offsets"]).tolist() == [64, 65, 1, 0]


@pytest.mark.parametrize("counts", [[100, 27, 1, 0], [128, 0, 0, 0], [64, 64, 0, 0], [65, 63, 0, 0]])
@pytest.mark.parametrize("fused", ["0", "1"])
def test_small_batch_experts_in_passes(monkeypatch, counts, fused):
    """At most 128 tokens: the weight-streaming kernels take every expert, those
    above 64 rows in passes of 64 rows (100 = 64 + 36, 128 = 64 + 64, 65 =
    64 + 1), and the tiled GEMM is not launched; through the single-wave
    kernels and through the fused kernel (forced by LMOE_FUSED_EXPERTS)."""
    monkeypatch.setenv("LMOE_FUSED_EXPERTS", fused)
    assign = np.repeat(np.arange(len(counts)), counts)
    w = tiny(T=len(assign), D=256, Dp=256, F_=256, E=len(counts), k=1, seed=114 + counts[0], act=synth.BF16)
    a = run_crafted(w, assign)
    assert np.diff(a["expert_offsets"]).tolist() == counts


def test_grouped_tile_boundaries():
    """Experts at the grouped GEMM's row-tile boundaries (tiles of up to 320
    rows, split in whole units of 64 rows; each split again between two wave
    rows): 65 rows (the smallest tiled expert), 320 (one full tile), 321 (192 +
    129) and 640 (two tiles of 320), 641 (192 + 256 + 193) and 1000 (four
    tiles, the last 232 rows), 64 (streamed) and 0."""
    counts = [65, 320, 321, 640, 641, 1000, 64, 0]
    assign = np.repeat(np.arange(len(counts)), counts)
    w = tiny(T=len(assign), D=256, Dp=256, F_=256, E=len(counts), k=1, seed=112, act=synth.BF16)
    a = run_crafted(w, assign)
    assert np.diff(a["expert_offsets"]).tolist() == counts


def test_stream_and_tiled_mixed():
    """Uneven routing over 16 experts: some experts above 64 rows (tiled GEMM),
    the rest streamed, several token tiles per streamed expert."""
    rng = np.random.default_rng(11)
    p = np.array([10, 8, 6, 1, 1, 1, 1, 1, 0.5, 0.5, 0.5, 0.5, 0.3, 0.3, 0.2, 0.2])
    assign = rng.choice(16, size=700, p=p / p.sum())
    w = tiny(T=700, D=512, Dp=256, F_=384, E=16, k=1, seed=111, act=synth.BF16)
    a = run_crafted(w, assign)
    counts = np.diff(a["expert_offsets"])
    assert (counts > 64).any() and ((counts > 16) & (counts <= 64)).any()


def test_deterministic_and_token_permutation_invariant():
    """Two runs give identical bits; permuting the tokens permutes the output
    rows bit-exactly (every row's arithmetic is independent of the batch)."""
    w = tiny(T=333, D=512, Dp=256, F_=256, E=16, k=4, seed=107, act=synth.BF16)
    wts = synth.dense_weights(w)
    block = lmoe.LatentMoE(upload(wts), w.k, w.T)
    x = sdev.to_device(synth.x(w), DEV)
    H.say("[gpu] determinism: two runs")
    o1, a1 = block.forward(x, aux=True)
    o2, a2 = block.forward(x, aux=True)
    perm = torch.from_numpy(np.random.default_rng(3).permutation(w.T)).to(DEV)
    H.say("[gpu] determinism: permuted tokens")
    o3 = block.forward(x[perm].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    for n in a1:
        assert torch.equal(a1[n], a2[n])
    assert torch.equal(o1[perm].view(torch.int16), o3.view(torch.int16))
    block.close()


def test_bf16_output_is_rounded_fp32_output():
    """out_dtype = bf16 gives exactly the nearest-even rounding of the fp32 output."""
    w = tiny(T=301, D=512, Dp=256, F_=256, E=16, k=4, seed=109, act=synth.BF16)
    wts = upload(synth.dense_weights(w))
    x = sdev.to_device(synth.x(w), DEV)
    b32 = lmoe.LatentMoE(wts, w.k, w.T, out_dtype=torch.float32)
    b16 = lmoe.LatentMoE(wts, w.k, w.T)
    H.say("[gpu] bf16 output vs rounded fp32 output")
    o32 = b32.forward(x)
    o16 = b16.forward(x)
    torch.cuda.synchronize()
    assert o16.dtype == torch.bfloat16 and o32.dtype == torch.float32
    assert torch.equal(o16.view(torch.int16), o32.to(torch.bfloat16).view(torch.int16))
    b32.close()
    b16.close()


def test_argument_errors():
    """Errors are reported before anything is enqueued."""
    w = tiny(T=16, D=128, Dp=64, F_=64, E=4, k=2, seed=108, act=synth.BF16)
    wts = upload(synth.dense_weights(w))
    block = lmoe.LatentMoE(wts, w.k, 16)
    x = sdev.to_device(synth.x(w), DEV)
    out = torch.empty_like(x)
    h = block.handle
    H.say("[gpu] argument errors")
    lmoe.lmoe_forward(h, x.data_ptr(), out.data_ptr(), 0, 0)           # T = 0: no-op
    with pytest.raises(lmoe.LmoeError) as e:
        lmoe.lmoe_forward(h, x.data_ptr(), out.data_ptr(), 17, 0)      # T > max_tokens
    assert e.value.status == lmoe.LMOE_E_INVAL
    with pytest.raises(lmoe.LmoeError) as e:
        lmoe.lmoe_forward(h, x.data_ptr() + 2, out.data_ptr(), 4, 0)   # misaligned
    assert e.value.status == lmoe.LMOE_E_INVAL
    with pytest.raises(lmoe.LmoeError) as e:
        lmoe.lmoe_forward(h, x.data_ptr(), x.data_ptr() + 64, 4, 0)    # out overlaps x
    assert e.value.status == lmoe.LMOE_E_INVAL
    with pytest.raises(lmoe.LmoeError) as e:
        lmoe.lmoe_forward(h, 0, out.data_ptr(), 4, 0)                 # NULL x
    assert e.value.status == lmoe.LMOE_E_INVAL
    # create-time checks
    cw = block.cw
    bad = lmoe.make_config(w.D, w.Dp, w.F, w.E, w.k, 16)
    bad.top_k = 17
    with pytest.raises(lmoe.LmoeError) as e:
        lmoe.lmoe_create(bad, cw)
    assert e.value.status == lmoe.LMOE_E_UNSUPPORTED
    good = lmoe.make_config(w.D, w.Dp, w.F, w.E, w.k, 16)
    nul = lmoe.lmoe_weights.from_buffer_copy(cw)
    nul.w_down = None
    with pytest.raises(lmoe.LmoeError) as e:
        lmoe.lmoe_create(good, nul)
    assert e.value.status == lmoe.LMOE_E_INVAL
    block.close()
