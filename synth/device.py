"""Upload a workload's synthetic tensors to a torch device.

Expert weights are generated one expert at a time into a pinned host buffer and
copied into one preallocated device tensor, so the host never holds the whole
expert set (25.8 GB for the full-size bf16 workloads).
"""
from __future__ import annotations

import numpy as np
import torch

import synth


def _tdtype(dtype: str):
    return torch.float32 if dtype == synth.F32 else torch.bfloat16


def to_device(a: np.ndarray, device) -> torch.Tensor:
    """A host array from synth (float32, or uint16 bfloat16 bits) as a device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.to(device)


def upload_weights(w: synth.Workload, device, experts=None) -> dict:
    """Every weight of workload w on `device` (expert tensors stacked [E, ...];
    MXFP4 experts as uint8 codes and scales)."""
    out = {
        "w_router": to_device(synth.w_router(w), device),
        "w_pool": to_device(synth.w_pool(w), device),
        "g_pool": to_device(synth.g_pool(w), device),
        "g_expert": to_device(synth.g_expert(w), device),
        "w_unpool": to_device(synth.w_unpool(w), device),
    }
    b = synth.router_bias(w)
    out["b_router"] = to_device(b, device) if b is not None else None
    if w.expert_w == synth.MXFP4:
        shapes = {"w_gate_up": (2 * w.F, w.Dp // 2), "s_gate_up": (2 * w.F, w.Dp // 32),
                  "w_down": (w.Dp, w.F // 2), "s_down": (w.Dp, w.F // 32)}
        for n, sh in shapes.items():
            out[n] = torch.empty((w.E,) + sh, dtype=torch.uint8, device=device)
        for e in range(w.E):
            (cg, sg), (cd, sd) = synth.w_gate_up(w, e), synth.w_down(w, e)
            for n, a in (("w_gate_up", cg), ("s_gate_up", sg), ("w_down", cd), ("s_down", sd)):
                out[n][e].copy_(torch.from_numpy(a))
        return out
    dt = _tdtype(w.expert_w)
    gu = torch.empty((w.E, 2 * w.F, w.Dp), dtype=dt, device=device)
    dn = torch.empty((w.E, w.Dp, w.F), dtype=dt, device=device)
    npdt = np.float32 if w.expert_w == synth.F32 else np.uint16
    hgu = torch.empty((2 * w.F, w.Dp), dtype=dt).pin_memory()
    hdn = torch.empty((w.Dp, w.F), dtype=dt).pin_memory()
    agu = hgu.view(torch.int16 if dt == torch.bfloat16 else torch.float32).numpy().view(npdt)
    adn = hdn.view(torch.int16 if dt == torch.bfloat16 else torch.float32).numpy().view(npdt)
    for e in range(w.E):
        synth.w_gate_up(w, e, out=agu)
        synth.w_down(w, e, out=adn)
        gu[e].copy_(hgu, non_blocking=True)
        dn[e].copy_(hdn, non_blocking=True)
        torch.cuda.current_stream(device).synchronize()   # the pinned buffers are reused
    out["w_gate_up"] = gu
    out["w_down"] = dn
    return out


def upload_x(w: synth.Workload, device, T: int | None = None) -> torch.Tensor:
    return to_device(synth.x(w, T=T), device)
