"""GPU parity of the fused expert kernel (the streamed experts' GEMMs in one
persistent launch over a device-side queue).

The kernel runs whole experts per workgroup (both GEMMs) when enough experts
are streamed, else per-wave gate/up items followed by the down launch; the
per-(expert, 64 weight rows) arithmetic and its K order are the same either
way, so the two modes must give identical bits; both are also compared with
the oracle. The environment variable LMOE_FUSED_EXPERTS forces the mode (1:
whole experts, 0: per-wave items), read by the library at every forward call;
unset, the count of streamed experts decides. Cases: every token-tile count of a
streamed expert (1..64 rows, across the 16-row tile boundaries, beside a
65-row tiled expert and an empty one), more streamed experts than workgroups
(each workgroup takes several tickets), streamed and tiled experts mixed,
determinism and token-permutation invariance, and the decode routing shape
(E = 256, k = 8).
"""
import numpy as np
import pytest
import torch

import latent_moe_layer_router_amd as lmoe
import synth
from synth import device as sdev
from tests import harness as H
from tests.pins import tiny
from tests.test_gpu_parity import crafted_routing, run_case, upload

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture
def fused(monkeypatch):
    monkeypatch.setenv("LMOE_FUSED_EXPERTS", "1")
    yield
    monkeypatch.delenv("LMOE_FUSED_EXPERTS", raising=False)


def both_paths(monkeypatch, w, wts, x):
    """The forward in both modes on the same inputs; outputs and routing must
    be identical."""
    block = lmoe.LatentMoE(upload(wts), w.k, x.shape[0], w.eps_pool, w.eps_expert, out_dtype=torch.float32)
    xd = sdev.to_device(x, DEV)
    res = {}
    for flag in ("1", "0"):
        monkeypatch.setenv("LMOE_FUSED_EXPERTS", flag)
        H.say(f"[gpu] fused={flag}: T={x.shape[0]} E={w.E} k={w.k} D={w.D} Dp={w.Dp} F={w.F}")
        out, aux = block.forward(xd, aux=True)
        torch.cuda.synchronize()
        res[flag] = (out, aux)
    monkeypatch.delenv("LMOE_FUSED_EXPERTS", raising=False)
    (o1, a1), (o0, a0) = res["1"], res["0"]
    assert torch.equal(o1.view(torch.int32), o0.view(torch.int32)), "the two modes' outputs differ"
    for n in a1:
        assert torch.equal(a1[n], a0[n]), n
    block.close()
    return o1.cpu().numpy(), {n: t.cpu().numpy() for n, t in a1.items()}


def check_oracle(w, wts, x, got, a):
    ref, raux = H.oracle_ref(w, x, wts)
    near = H.check_routing(a["topk_ids"], a["topk_w"], a["logits"], raux["logits"], raux["ids"], raux["w"], w.k)
    H.check_permutation(a["topk_ids"], a["expert_offsets"], a["sorted_assign"], w.E)
    err = H.out_error(got[~near], ref[~near])
    H.say(f"[gpu]   max|err|/rms = {err:.3e}, near-ties = {int(near.sum())}")
    assert err <= H.tol(w), err


def test_fused_row_counts_across_token_tiles(monkeypatch):
    """Streamed experts of 1, 16, 17, 32, 33, 48, 49 and 64 rows (one to four
    16-row token tiles), a 65-row expert on the tiled GEMM and an empty one."""
    counts = [64, 65, 1, 0, 16, 17, 32, 33, 48, 49]
    assign = np.repeat(np.arange(len(counts)), counts)
    w = tiny(T=len(assign), D=256, Dp=256, F_=256, E=len(counts), k=1, seed=151, act=synth.BF16)
    wts, x = crafted_routing(w, assign)
    got, a = both_paths(monkeypatch, w, wts, x)
    assert np.diff(a["expert_offsets"]).tolist() == counts
    check_oracle(w, wts, x, got, a)


def test_fused_more_experts_than_workgroups(monkeypatch):
    """1000 experts with about 4 rows each: far more streamed experts than the
    persistent grid's workgroups, so each takes several tickets."""
    w = tiny(T=1000, D=256, Dp=256, F_=128, E=1000, k=4, seed=152, act=synth.BF16)
    wts = synth.dense_weights(w)
    x = synth.x(w)
    got, a = both_paths(monkeypatch, w, wts, x)
    assert (np.diff(a["expert_offsets"]) > 0).sum() > 900
    check_oracle(w, wts, x, got, a)


def test_fused_stream_and_tiled_mixed(monkeypatch):
    """Uneven routing over 16 experts: some above 64 rows (tiled GEMM), the
    rest streamed with several token tiles."""
    rng = np.random.default_rng(12)
    p = np.array([10, 8, 6, 1, 1, 1, 1, 1, 0.5, 0.5, 0.5, 0.5, 0.3, 0.3, 0.2, 0.2])
    assign = rng.choice(16, size=700, p=p / p.sum())
    w = tiny(T=700, D=512, Dp=256, F_=384, E=16, k=1, seed=153, act=synth.BF16)
    wts, x = crafted_routing(w, assign)
    got, a = both_paths(monkeypatch, w, wts, x)
    counts = np.diff(a["expert_offsets"])
    assert (counts > 64).any() and ((counts > 16) & (counts <= 64)).any()
    check_oracle(w, wts, x, got, a)


@pytest.mark.parametrize("T", [16, 128])
def test_fused_decode_routing_shape(monkeypatch, T):
    """E = 256, k = 8 (the decode routing shape) at reduced widths."""
    w = tiny(T=T, D=512, Dp=512, F_=512, E=256, k=8, seed=154, act=synth.BF16)
    wts = synth.dense_weights(w)
    x = synth.x(w)
    got, a = both_paths(monkeypatch, w, wts, x)
    check_oracle(w, wts, x, got, a)


def test_fused_deterministic_and_token_permutation_invariant(fused):
    w = tiny(T=333, D=512, Dp=256, F_=256, E=64, k=4, seed=155, act=synth.BF16)
    block = lmoe.LatentMoE(upload(synth.dense_weights(w)), w.k, w.T)
    x = sdev.to_device(synth.x(w), DEV)
    H.say("[gpu] fused determinism: two runs, then permuted tokens")
    o1 = block.forward(x)
    o2 = block.forward(x)
    perm = torch.from_numpy(np.random.default_rng(4).permutation(w.T)).to(DEV)
    o3 = block.forward(x[perm].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(o1[perm].view(torch.int16), o3.view(torch.int16))
    block.close()


def test_fused_tiny_against_oracle(fused):
    """A small ragged case through run_case with the fused kernel forced."""
    run_case(tiny(T=65, D=256, Dp=256, F_=128, E=8, k=2, seed=156, act=synth.BF16))
