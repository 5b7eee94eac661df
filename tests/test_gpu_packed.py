"""GPU checks of the packed expert layout (LMOE_FLAG_PACKED_EXPERTS).

lmoe_pack_experts only reorders a matrix's values into 8 KiB blocks of 64 rows
x 64 columns, and the kernels that read that layout (the weight-streaming ones,
single-wave and fused, and the tiled grouped GEMM) do the same arithmetic in
the same order on the same values. A forward over packed weights must therefore
give the bits of the forward over the row-major ones: checked for each of those
kernels and for streamed and tiled experts in one batch (the full sizes are
checked beside the other full-size cases); one case is also compared with the
oracle. The
packing itself is checked element by element against a numpy re-layout.
"""
import numpy as np
import pytest
import torch

import latent_moe_layer_router_amd as lmoe
import synth
from synth import device as sdev
from tests import harness as H
from tests.pins import tiny
from tests.test_gpu_parity import crafted_routing, upload

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def numpy_packed(a: np.ndarray) -> np.ndarray:
    """[n][R][C] -> the packed layout, flat per matrix: blocks (g, s) in g-major
    order, each 64 x 64 row-major."""
    n, R, C = a.shape
    return a.reshape(n, R // 64, 64, C // 64, 64).transpose(0, 1, 3, 2, 4).reshape(n, R * C)


@pytest.mark.parametrize("n,R,C", [(3, 192, 320), (1, 64, 64), (2, 128, 4096)])
def test_pack_layout(n, R, C):
    H.say(f"[gpu] pack n={n} R={R} C={C}")
    bits = torch.randint(-32768, 32768, (n, R, C), dtype=torch.int32,
                         generator=torch.Generator().manual_seed(R + C)).to(torch.int16)
    src = bits.to(DEV).view(torch.bfloat16)
    dst = torch.empty_like(src)
    lmoe.lmoe_pack_experts(src.data_ptr(), dst.data_ptr(), n, R, C, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = dst.view(torch.int16).cpu().numpy().reshape(n, R * C)
    assert np.array_equal(got, numpy_packed(bits.numpy()))


def test_pack_in_place_matches_packed_copy():
    """pack_expert_weights(in_place=True) (one staging matrix, packed back into
    the same storage) gives the packed copy's bits and leaves the other tensors
    alone."""
    H.say("[gpu] pack in place")
    g = torch.Generator().manual_seed(5)
    mk = lambda *sh: torch.randint(-32768, 32768, sh, dtype=torch.int32, generator=g).to(torch.int16).to(DEV).view(torch.bfloat16)
    wts = {"w_gate_up": mk(5, 256, 192), "w_down": mk(5, 192, 128), "w_pool": mk(64, 64)}
    copy = lmoe.pack_expert_weights(wts)
    keep = {n: t.clone() for n, t in wts.items()}
    inpl = lmoe.pack_expert_weights(wts, in_place=True)
    torch.cuda.synchronize()
    for n in ("w_gate_up", "w_down"):
        assert inpl[n] is wts[n]
        assert torch.equal(inpl[n].view(torch.int16), copy[n].view(torch.int16)), n
        assert not torch.equal(inpl[n].view(torch.int16), keep[n].view(torch.int16)), n
    assert inpl["w_pool"] is wts["w_pool"]
    assert torch.equal(wts["w_pool"].view(torch.int16), keep["w_pool"].view(torch.int16))


def plain_and_packed(w, wts, x, max_tokens=None):
    """The forward over row-major and over packed expert weights; outputs and
    routing must be identical. Returns the output and routing (numpy)."""
    tw = upload(wts)
    pw = lmoe.pack_expert_weights(tw)
    xd = sdev.to_device(x, DEV)
    res = []
    for weights, packed in ((tw, False), (pw, True)):
        H.say(f"[gpu] packed={packed}: T={x.shape[0]} E={w.E} k={w.k} D={w.D} Dp={w.Dp} F={w.F}")
        b = lmoe.LatentMoE(weights, w.k, max_tokens or x.shape[0], w.eps_pool, w.eps_expert,
                           out_dtype=torch.float32, packed=packed)
        out, aux = b.forward(xd, aux=True)
        torch.cuda.synchronize()
        res.append((out, aux))
        b.close()
    (o0, a0), (o1, a1) = res
    assert torch.equal(o0.view(torch.int32), o1.view(torch.int32)), "packed and row-major outputs differ"
    for n in a0:
        assert torch.equal(a0[n], a1[n]), n
    return o0.cpu().numpy(), {n: t.cpu().numpy() for n, t in a0.items()}


def test_packed_streamed_experts_against_oracle():
    """Few rows per expert (the single-wave weight-streaming kernels), and the
    oracle on the packed run's output."""
    w = tiny(T=64, D=256, Dp=256, F_=256, E=8, k=2, seed=301, act=synth.BF16)
    wts = synth.dense_weights(w)
    x = synth.x(w)
    got, a = plain_and_packed(w, wts, x)
    ref, raux = H.oracle_ref(w, x, wts)
    near = H.check_routing(a["topk_ids"], a["topk_w"], a["logits"], raux["logits"], raux["ids"], raux["w"], w.k)
    err = H.out_error(got[~near], ref[~near])
    H.say(f"[gpu]   max|err|/rms = {err:.3e}")
    assert err <= H.tol(w), err


def test_packed_tiled_experts():
    """About 150 rows per expert: the tiled grouped GEMM (gate and up rows F
    apart in both layouts)."""
    w = tiny(T=300, D=512, Dp=512, F_=384, E=4, k=2, seed=302, act=synth.BF16)
    plain_and_packed(w, synth.dense_weights(w), synth.x(w))


def test_packed_streamed_and_tiled_mixed():
    """Experts above 64 rows and streamed ones (several token tiles) in one call."""
    rng = np.random.default_rng(12)
    p = np.array([10, 8, 6, 1, 1, 1, 1, 1, 0.5, 0.5, 0.5, 0.5, 0.3, 0.3, 0.2, 0.2])
    assign = rng.choice(16, size=700, p=p / p.sum())
    w = tiny(T=700, D=512, Dp=256, F_=384, E=16, k=1, seed=303, act=synth.BF16)
    wts, x = crafted_routing(w, assign)
    _, a = plain_and_packed(w, wts, x)
    counts = np.diff(a["expert_offsets"])
    assert (counts > 64).any() and ((counts > 16) & (counts <= 64)).any()


@pytest.mark.parametrize("fused", ["1", "0"])
def test_packed_fused_and_per_wave(monkeypatch, fused):
    """The fused expert kernel (whole experts per workgroup) and its per-wave
    form, forced by LMOE_FUSED_EXPERTS."""
    monkeypatch.setenv("LMOE_FUSED_EXPERTS", fused)
    w = tiny(T=96, D=256, Dp=512, F_=256, E=16, k=4, seed=304, act=synth.BF16)
    plain_and_packed(w, synth.dense_weights(w), synth.x(w))

