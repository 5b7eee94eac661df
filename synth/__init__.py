"""Seeded synthetic inputs for the latent-MoE block.

This module only draws random numbers and lays them out; it holds none of the
block's arithmetic. The HIP path and the CPU oracle both consume what it returns,
so both always see identical bits.

Every tensor is a counter-based stream named by (seed, tensor id, expert), so any
slice -- one expert's weights, one token's row -- can be regenerated on its own.
Weights follow N(0, 1/fan_in), activations N(0, 1), RMSNorm gammas 1 + N(0, 0.1).

Workloads (shapes from the pages: pooler 8192 -> 4096, 256 experts per layer,
expert width 4096 -- vLLM day-0 summary, "Model architecture" weight budget and
"Latent MoE"; a 16K-token prefill chunk -- LMSYS blog, "Sequence parallelism";
up to 128 concurrent decode requests -- LMSYS blog, highlights):

  tiny_fp32     T=64,    D=256,  Dp=128,  F=128,  E=8,   k=2, fp32
  decode_bf16   T=128,   D=8192, Dp=4096, F=4096, E=256, k=8, bf16
  prefill_bf16  T=16384, same shapes, bf16
  skewed_bf16   T=4096,  same shapes, bf16, router bias giving Zipf(1.2) load
                with 16 experts forced empty
  mxfp4         T=16384, same shapes, MXFP4 expert weights, MXFP8 activations
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")

# Tensor ids of the streams.
T_X, T_WR, T_BIAS, T_WP, T_GP, T_WGU, T_WD, T_GE, T_WUN, T_SUBSET = range(1, 11)

F32, BF16, MXFP4 = "f32", "bf16", "mxfp4"


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    D: int
    Dp: int
    F: int
    E: int
    k: int
    act: str            # F32 or BF16: x, out, router, pooler, unpooler
    expert_w: str       # F32, BF16 or MXFP4
    seed: int = 0       # weight seed (the "model")
    x_seed: int = 0     # activation seed
    skew: bool = False  # Zipf router bias
    eps_pool: float = 1e-6
    eps_expert: float = 1e-6
    extra: dict = field(default_factory=dict)

    @property
    def mx_act(self) -> bool:
        return self.expert_w == MXFP4


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 64, 256, 128, 128, 8, 2, F32, F32),
    "decode_bf16": Workload("decode_bf16", 128, 8192, 4096, 4096, 256, 8, BF16, BF16, x_seed=1),
    "prefill_bf16": Workload("prefill_bf16", 16384, 8192, 4096, 4096, 256, 8, BF16, BF16, x_seed=2),
    "skewed_bf16": Workload("skewed_bf16", 4096, 8192, 4096, 4096, 256, 8, BF16, BF16, x_seed=3,
                            skew=True),
    "mxfp4": Workload("mxfp4", 16384, 8192, 4096, 4096, 256, 8, BF16, MXFP4, x_seed=2),
    "mxfp4_decode": Workload("mxfp4_decode", 128, 8192, 4096, 4096, 256, 8, BF16, MXFP4, x_seed=1),
}


def _lib():
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    u64 = ctypes.c_uint64
    lib.synth_normal.argtypes = [u64, u64, u64, ctypes.c_size_t, ctypes.c_float, ctypes.c_float,
                                 ctypes.c_int, ctypes.c_void_p]
    lib.synth_normal.restype = None
    lib.synth_uniform.argtypes = [u64, u64, u64, ctypes.c_size_t, ctypes.c_void_p]
    lib.synth_uniform.restype = None
    lib.synth_bits.argtypes = [u64, u64, u64]
    lib.synth_bits.restype = u64
    lib.synth_mxfp4_normal.argtypes = [u64, u64, ctypes.c_size_t, ctypes.c_float,
                                       ctypes.c_void_p, ctypes.c_void_p]
    lib.synth_mxfp4_normal.restype = None
    lib.synth_f32_to_bf16.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.synth_f32_to_bf16.restype = None
    return lib


_LIB = None


def lib():
    global _LIB
    if _LIB is None:
        _LIB = _lib()
    return _LIB


def stream_id(tensor: int, index: int = 0) -> int:
    return (tensor << 32) | index


def normal(seed: int, stream: int, shape, scale: float = 1.0, shift: float = 0.0,
           dtype: str = F32, out: np.ndarray | None = None, first: int = 0) -> np.ndarray:
    """Elements [first, first + prod(shape)) of the N(shift, scale^2) stream.
    dtype F32 -> float32 array; BF16 -> uint16 array of bfloat16 bits."""
    n = int(np.prod(shape))
    npdt = np.float32 if dtype == F32 else np.uint16
    if out is None:
        out = np.empty(shape, npdt)
    assert out.dtype == npdt and out.size == n and out.flags.c_contiguous
    lib().synth_normal(seed, stream, first, n, scale, shift, 0 if dtype == F32 else 1,
                       out.ctypes.data)
    return out


def uniform(seed: int, stream: int, n: int, first: int = 0) -> np.ndarray:
    out = np.empty(n, np.float64)
    lib().synth_uniform(seed, stream, first, n, out.ctypes.data)
    return out


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """bfloat16 bits (uint16) -> float32, exactly."""
    return (a.astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_f32(a: np.ndarray) -> np.ndarray:
    return bf16_to_f32(a) if a.dtype == np.uint16 else a


def lib_round_bf16(a: np.ndarray) -> np.ndarray:
    """float32 array -> bfloat16 bits (uint16), nearest even (for hand-made inputs)."""
    a = np.ascontiguousarray(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    lib().synth_f32_to_bf16(a.ctypes.data, a.size, out.ctypes.data)
    return out


# ---------------------------------------------------------------------------
# Tensors of a workload. Every function returns host arrays: float32 for F32
# tensors, uint16 (bfloat16 bits) for BF16 tensors; gammas and biases are float32.
# ---------------------------------------------------------------------------

def x(w: Workload, rows=None, T: int | None = None) -> np.ndarray:
    """Activations [T, D]; `rows` selects token rows (regenerated independently)."""
    T = w.T if T is None else T
    s = stream_id(T_X, w.x_seed)
    if rows is None:
        return normal(w.seed, s, (T, w.D), 1.0, 0.0, w.act)
    out = np.empty((len(rows), w.D), np.float32 if w.act == F32 else np.uint16)
    for i, r in enumerate(rows):
        normal(w.seed, s, (w.D,), 1.0, 0.0, w.act, out=out[i], first=int(r) * w.D)
    return out


def w_router(w: Workload) -> np.ndarray:
    return normal(w.seed, stream_id(T_WR), (w.E, w.D), w.D ** -0.5, 0.0, w.act)


def w_pool(w: Workload) -> np.ndarray:
    return normal(w.seed, stream_id(T_WP), (w.Dp, w.D), w.D ** -0.5, 0.0, w.act)


def g_pool(w: Workload) -> np.ndarray:
    return normal(w.seed, stream_id(T_GP), (w.Dp,), 0.1, 1.0, F32)


def w_unpool(w: Workload) -> np.ndarray:
    return normal(w.seed, stream_id(T_WUN), (w.D, w.Dp), w.Dp ** -0.5, 0.0, w.act)


def g_expert(w: Workload) -> np.ndarray:
    return normal(w.seed, stream_id(T_GE), (w.E, w.Dp), 0.1, 1.0, F32)


def w_gate_up(w: Workload, e: int, out: np.ndarray | None = None):
    """Expert e's packed gate/up weight [2F, Dp] (rows [0, F) gate, [F, 2F) up).
    MXFP4 workloads return (codes [2F, Dp/2] uint8, scales [2F, Dp/32] uint8)."""
    s = stream_id(T_WGU, e)
    if w.expert_w == MXFP4:
        return mxfp4_normal(w.seed, s, 2 * w.F, w.Dp, w.Dp ** -0.5)
    return normal(w.seed, s, (2 * w.F, w.Dp), w.Dp ** -0.5, 0.0, w.expert_w, out=out)


def w_down(w: Workload, e: int, out: np.ndarray | None = None):
    """Expert e's down weight [Dp, F] (MXFP4: codes [Dp, F/2], scales [Dp, F/32])."""
    s = stream_id(T_WD, e)
    if w.expert_w == MXFP4:
        return mxfp4_normal(w.seed, s, w.Dp, w.F, w.F ** -0.5)
    return normal(w.seed, s, (w.Dp, w.F), w.F ** -0.5, 0.0, w.expert_w, out=out)


def mxfp4_normal(seed: int, stream: int, rows: int, K: int, scale: float):
    """An MXFP4 matrix [rows, K] holding N(0, scale^2) draws in MX form (E2M1
    codes, one E8M0 scale per 32 along K), as the checkpoint format stores them."""
    codes = np.empty((rows, K // 2), np.uint8)
    scales = np.empty((rows, K // 32), np.uint8)
    lib().synth_mxfp4_normal(seed, stream, rows * K, scale, codes.ctypes.data,
                             scales.ctypes.data)
    return codes, scales


def router_bias(w: Workload) -> np.ndarray | None:
    """Per-expert router bias, or None. For the skewed workload: expert load
    follows Zipf(1.2) over a seeded ranking of 240 experts, and the last 16 ranks
    are forced empty. Calibrated by fixed-point iteration on a seeded Monte-Carlo
    model of the router logits (iid N(0, 1) per token and expert, which is the
    distribution x . W_router^T has for x ~ N(0, 1), W_router ~ N(0, 1/D))."""
    if not w.skew:
        return None
    E, k = w.E, w.k
    n_live = 240
    rank_u = uniform(w.seed, stream_id(T_BIAS, 0), E)
    order = np.argsort(rank_u, kind="stable")          # order[r] = expert at rank r
    q = np.zeros(E)
    q[order[:n_live]] = np.arange(1, n_live + 1, dtype=np.float64) ** -1.2
    q /= q.sum()
    cap = 1.0 / k                                       # an expert appears once per token
    for _ in range(64):                                 # water-filling of the cap
        over = q > cap
        if not over.any():
            break
        excess = (q[over] - cap).sum()
        q[over] = cap
        free = (~over) & (q > 0)
        q[free] += excess * q[free] / q[free].sum()
    live = q > 0
    b = np.full(E, -1.0e4)
    b[live] = np.log(q[live])
    Tc = 4096
    logits = normal(w.seed, stream_id(T_BIAS, 1), (Tc, E), 1.0, 0.0, F32).astype(np.float64)
    for _ in range(30):
        sel = np.argpartition(-(logits + b), k - 1, axis=1)[:, :k]
        s = np.bincount(sel.ravel(), minlength=E) / (Tc * k)
        b[live] += 0.5 * (np.log(q[live]) - np.log(np.maximum(s[live], 1.0 / (2 * Tc * k))))
    return b.astype(np.float32)


def subset(w: Workload, n: int = 64, seed: int = 1) -> np.ndarray:
    """A seeded sample of n distinct token indices of [0, T), sorted."""
    if n >= w.T:
        return np.arange(w.T)
    u = uniform(seed, stream_id(T_SUBSET, w.x_seed), w.T)
    return np.sort(np.argsort(u, kind="stable")[:n])


def dense_weights(w: Workload) -> dict:
    """Every weight of a workload as host arrays (for small shapes). Expert
    weights are stacked [E, ...] (MXFP4: codes and scales stacked separately)."""
    d = {
        "w_router": w_router(w),
        "b_router": router_bias(w),
        "w_pool": w_pool(w),
        "g_pool": g_pool(w),
        "g_expert": g_expert(w),
        "w_unpool": w_unpool(w),
    }
    if w.expert_w == MXFP4:
        gu = [w_gate_up(w, e) for e in range(w.E)]
        dn = [w_down(w, e) for e in range(w.E)]
        d["w_gate_up"] = np.stack([c for c, _ in gu])
        d["s_gate_up"] = np.stack([s for _, s in gu])
        d["w_down"] = np.stack([c for c, _ in dn])
        d["s_down"] = np.stack([s for _, s in dn])
    else:
        d["w_gate_up"] = np.stack([w_gate_up(w, e) for e in range(w.E)])
        d["w_down"] = np.stack([w_down(w, e) for e in range(w.E)])
    return d


def shrink(w: Workload, **kw) -> Workload:
    """A copy of a workload with some fields replaced (e.g. smaller shapes)."""
    d = {f: getattr(w, f) for f in w.__dataclass_fields__}
    d.update(kw)
    return Workload(**d)
