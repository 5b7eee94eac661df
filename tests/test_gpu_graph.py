"""lmoe_forward captured into a HIP graph (torch.cuda.graph over the library's
stream) and replayed: every replay gives the eager result bit for bit, with
eager work (a fill of the output, an eager forward) and synchronizations between
the replays. The forward is deterministic, so the comparison is exact.

Cases cover the kernels a forward launches: the small-batch dense projections
and the weight-streaming expert GEMMs (T <= 128; also the fused expert kernel on
packed weights), the tiled dense and grouped GEMMs (larger T, experts above the
streaming limit), and the MXFP4 path.
"""
import pytest
import torch

import latent_moe_layer_router_amd as lmoe
import synth
from synth import device as sdev
from tests import harness as H
from tests.pins import tiny
from tests.test_gpu_parity import upload

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def replay_case(w, replays=4, packed=False):
    H.say(f"[gpu] graph replay: T={w.T} D={w.D} Dp={w.Dp} F={w.F} E={w.E} k={w.k} experts={w.expert_w} "
          f"packed={packed}")
    tw = upload(synth.dense_weights(w))
    if packed:
        tw = lmoe.pack_expert_weights(tw)
    block = lmoe.LatentMoE(tw, w.k, w.T, w.eps_pool, w.eps_expert, out_dtype=torch.float32, packed=packed)
    x = sdev.to_device(synth.x(w), DEV)
    ref = block.forward(x).clone()
    torch.cuda.synchronize()
    out = torch.empty_like(ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        block.forward(x, out=out)
    torch.cuda.synchronize()
    for r in range(replays):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        bad = int((out != ref).sum())
        assert bad == 0, f"replay {r}: {bad} outputs differ from the eager forward"
        eager = block.forward(x)
        torch.cuda.synchronize()
        assert torch.equal(eager, ref), f"eager forward after replay {r} differs"
    del g
    block.close()


def test_graph_small_batch_bf16():
    """T = 100: dense projections by split-K streaming, all experts streamed."""
    replay_case(tiny(T=100, D=256, Dp=128, F_=192, E=8, k=2, seed=301, act=synth.BF16))


def test_graph_fused_packed(monkeypatch):
    """The fused expert kernel (forced by LMOE_FUSED_EXPERTS) on weights in the
    packed expert layout, after the top-k inside the small-batch pooled-norm
    kernel and the sort's one-launch placement."""
    monkeypatch.setenv("LMOE_FUSED_EXPERTS", "1")
    replay_case(tiny(T=96, D=256, Dp=512, F_=256, E=16, k=4, seed=303, act=synth.BF16), packed=True)


def test_graph_tiled_bf16():
    """T = 600 over 4 experts: tiled dense projections and grouped GEMMs."""
    replay_case(tiny(T=600, D=512, Dp=256, F_=256, E=4, k=2, seed=302, act=synth.BF16))


def test_graph_fp32():
    replay_case(tiny(T=70, D=256, Dp=128, F_=128, E=8, k=2, seed=303, act=synth.F32))


def test_graph_mxfp4():
    """MXFP4 experts, a mix of streamed (<= 32 rows) and tiled experts."""
    replay_case(tiny(T=100, D=256, Dp=1024, F_=1024, E=8, k=3, seed=304, act=synth.BF16,
                     expert_w=synth.MXFP4))
