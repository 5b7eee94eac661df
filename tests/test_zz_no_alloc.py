"""The no-allocation forward (lmoe_forward_noalloc) against lmoe_forward, on the GPU.

lmoe_forward_noalloc runs the same kernels in the same order as lmoe_forward,
on the library's static per-device scratch instead of a handle's workspace, so
its results must equal lmoe_forward's bit for bit: output, logits, ids,
weights, offsets and sorted order. Each case makes two calls in a row on one
device, the second with fewer tokens (the scratch keeps the first call's
contents and is laid out differently for the second). Cases cover both batch
regimes (split-K dense projections and weight-streaming experts at small T,
tiled ones at larger T), fp32, MXFP4 experts, and the full decode shape; a T
whose workspace exceeds the scratch is refused with nothing enqueued.
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
AUX = ("logits", "topk_ids", "topk_w", "expert_offsets", "sorted_assign")


def upload(wts: dict) -> dict:
    return {n: (sdev.to_device(a, DEV) if a is not None else None) for n, a in wts.items()}


def noalloc_forward(block, x):
    T = x.shape[0]
    out = torch.empty(x.shape, dtype=block.out_dtype, device=x.device)
    res = {"logits": torch.empty(T, block.E, dtype=torch.float32, device=x.device),
           "topk_ids": torch.empty(T, block.k, dtype=torch.int32, device=x.device),
           "topk_w": torch.empty(T, block.k, dtype=torch.float32, device=x.device),
           "expert_offsets": torch.empty(block.E + 1, dtype=torch.int32, device=x.device),
           "sorted_assign": torch.empty(T * block.k, dtype=torch.int32, device=x.device)}
    a = lmoe.lmoe_aux(*(res[n].data_ptr() for n in AUX))
    lmoe.lmoe_forward_noalloc(block.cfg, block.cw, x.data_ptr(), out.data_ptr(), T,
                              torch.cuda.current_stream(x.device).cuda_stream, a)
    return out, res


def compare(block, w, Ts):
    for T in Ts:
        H.say(f"[gpu] no-alloc forward: {w.name} T={T} D={w.D} Dp={w.Dp} F={w.F} E={w.E} k={w.k} "
              f"experts={w.expert_w}")
        x = sdev.to_device(synth.x(w, T=T), DEV)
        ref, raux = block.forward(x, aux=True)
        got, gaux = noalloc_forward(block, x)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int32) if got.dtype == torch.float32 else got.view(torch.int16),
                           ref.view(torch.int32) if ref.dtype == torch.float32 else ref.view(torch.int16))
        for n in AUX:
            assert torch.equal(gaux[n], raux[n]), n
        H.say(f"[gpu]   identical to lmoe_forward (output, {', '.join(AUX)})")


@pytest.mark.parametrize("case", ["bf16_tiled_then_streamed", "fp32", "mxfp4"])
def test_noalloc_matches_forward_small(case):
    if case == "bf16_tiled_then_streamed":
        w, Ts = tiny(T=300, D=512, Dp=256, F_=256, E=16, k=4, seed=141, act=synth.BF16), (300, 77)
    elif case == "fp32":
        w, Ts = tiny(T=200, D=256, Dp=128, F_=192, E=8, k=2, seed=142, act=synth.F32), (200, 64)
    else:
        w, Ts = tiny(T=150, D=1024, Dp=1024, F_=1024, E=8, k=2, seed=143, act=synth.BF16,
                     expert_w=synth.MXFP4), (150, 40)
    block = lmoe.LatentMoE(upload(synth.dense_weights(w)), w.k, max(Ts), w.eps_pool, w.eps_expert,
                           out_dtype=torch.float32)
    compare(block, w, Ts)
    block.close()


def test_noalloc_matches_forward_decode_full_size():
    """The full decode shape (D=8192, Dp=4096, F=4096, E=256, k=8, bf16): T=128
    then T=16; T=302 (the first T whose workspace exceeds 64 MiB at this shape)
    is refused."""
    w = synth.WORKLOADS["decode_bf16"]
    H.say("[gpu] no-alloc forward: uploading full-size weights (25.8 GB of experts)")
    tw = sdev.upload_weights(w, DEV)
    block = lmoe.LatentMoE(tw, w.k, 302, w.eps_pool, w.eps_expert, out_dtype=torch.float32)
    compare(block, w, (128, 16))
    x = sdev.to_device(synth.x(w, T=302), DEV)
    out = torch.full((302, w.D), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(lmoe.LmoeError) as e:
        lmoe.lmoe_forward_noalloc(block.cfg, block.cw, x.data_ptr(), out.data_ptr(), 302,
                                  torch.cuda.current_stream().cuda_stream, None)
    assert e.value.status == lmoe.LMOE_E_INVAL and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)                      # nothing was enqueued
    block.close()
    del tw
    torch.cuda.empty_cache()
