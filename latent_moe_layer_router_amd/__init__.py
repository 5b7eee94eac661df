"""Python binding of liblmoe.so, the HIP latent-MoE block forward for MI355X.

Argument marshalling only: every step of the block runs in the library's HIP
kernels. The functions mirror the C ABI in include/lmoe.h one to one
(lmoe_create, lmoe_forward, lmoe_destroy, lmoe_workspace_bytes,
lmoe_set_timing, lmoe_get_timing, lmoe_status_str, lmoe_last_error,
lmoe_mx_quantize_e4m3, lmoe_nvfp4_to_mxfp4, lmoe_forward_noalloc) and take raw
device pointers; LatentMoE wraps them for torch tensors, which serve only as
device memory and streams. Importing works without a GPU; loading the library
raises if it has not been built (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblmoe.so")

LMOE_ABI_VERSION = 1
LMOE_OK, LMOE_E_INVAL, LMOE_E_UNSUPPORTED, LMOE_E_NOMEM, LMOE_E_HIP = 0, -1, -2, -3, -4
LMOE_F32, LMOE_BF16, LMOE_MXFP4, LMOE_MXFP8_E4M3 = 0, 1, 2, 3
LMOE_FLAG_ROUTER_BIAS = 1
LMOE_FLAG_PACKED_EXPERTS = 2
STAGES = ["proj_in", "topk", "sort", "pool_norm", "gate_up", "down", "combine", "unpool"]
LMOE_NUM_STAGES = len(STAGES)

LMOE_NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTS = ["lmoe_create", "lmoe_forward", "lmoe_forward_noalloc", "lmoe_destroy", "lmoe_workspace_bytes",
           "lmoe_set_timing", "lmoe_get_timing", "lmoe_status_str", "lmoe_last_error",
           "lmoe_mx_quantize_e4m3", "lmoe_nvfp4_to_mxfp4", "lmoe_pack_experts"]


class lmoe_config(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("d_pooled", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("eps_pool", ctypes.c_float), ("eps_expert", ctypes.c_float),
                ("act_dtype", ctypes.c_int32), ("expert_wdtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]


class lmoe_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_router", "b_router", "w_pool", "g_pool", "w_gate_up", "s_gate_up",
                 "w_down", "s_down", "g_expert", "w_unpool")]


class lmoe_aux(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("logits", "topk_ids", "topk_w", "expert_offsets", "sorted_assign")]


class LmoeError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {lmoe_status_str(status)} ({detail})")
        self.status = status


_LIB = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load liblmoe.so; raises if it is missing (build it with __graft_entry__.build())."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    P, I32 = ctypes.c_void_p, ctypes.c_int32
    lib.lmoe_create.argtypes = [ctypes.POINTER(lmoe_config), ctypes.POINTER(lmoe_weights),
                                ctypes.POINTER(P)]
    lib.lmoe_forward.argtypes = [P, P, P, I32, P, ctypes.POINTER(lmoe_aux)]
    lib.lmoe_forward_noalloc.argtypes = [ctypes.POINTER(lmoe_config), ctypes.POINTER(lmoe_weights), P, P, I32,
                                         P, ctypes.POINTER(lmoe_aux)]
    lib.lmoe_destroy.argtypes = [P]
    lib.lmoe_workspace_bytes.argtypes = [ctypes.POINTER(lmoe_config), ctypes.POINTER(ctypes.c_size_t)]
    lib.lmoe_set_timing.argtypes = [P, ctypes.c_int]
    lib.lmoe_get_timing.argtypes = [P, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(I32)]
    lib.lmoe_mx_quantize_e4m3.argtypes = [P, ctypes.c_int64, P, P, P]
    lib.lmoe_nvfp4_to_mxfp4.argtypes = [P, P, P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, P, P, P]
    lib.lmoe_pack_experts.argtypes = [P, P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, P]
    for f in ("lmoe_create", "lmoe_forward", "lmoe_forward_noalloc", "lmoe_destroy", "lmoe_workspace_bytes",
              "lmoe_set_timing", "lmoe_get_timing", "lmoe_mx_quantize_e4m3", "lmoe_nvfp4_to_mxfp4",
              "lmoe_pack_experts"):
        getattr(lib, f).restype = ctypes.c_int
    lib.lmoe_status_str.argtypes = [ctypes.c_int]
    lib.lmoe_status_str.restype = ctypes.c_char_p
    lib.lmoe_last_error.argtypes = []
    lib.lmoe_last_error.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def lmoe_status_str(status: int) -> str:
    return load().lmoe_status_str(status).decode()


def lmoe_last_error() -> str:
    return load().lmoe_last_error().decode()


def _check(status: int, where: str):
    if status != LMOE_OK:
        raise LmoeError(status, where, lmoe_last_error())


def lmoe_workspace_bytes(cfg: lmoe_config) -> int:
    n = ctypes.c_size_t()
    _check(load().lmoe_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)), "lmoe_workspace_bytes")
    return n.value


def lmoe_create(cfg: lmoe_config, weights: lmoe_weights) -> int:
    h = ctypes.c_void_p()
    _check(load().lmoe_create(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(h)), "lmoe_create")
    return h.value


def lmoe_forward(h: int, x: int, out: int, T: int, stream: int = 0, aux: lmoe_aux | None = None):
    _check(load().lmoe_forward(h, x, out, T, stream, ctypes.byref(aux) if aux is not None else None),
           "lmoe_forward")


def lmoe_forward_noalloc(cfg: lmoe_config, weights: lmoe_weights, x: int, out: int, T: int, stream: int = 0,
                         aux: lmoe_aux | None = None):
    _check(load().lmoe_forward_noalloc(ctypes.byref(cfg), ctypes.byref(weights), x, out, T, stream,
                                       ctypes.byref(aux) if aux is not None else None),
           "lmoe_forward_noalloc")


def lmoe_destroy(h: int | None):
    _check(load().lmoe_destroy(h), "lmoe_destroy")


def lmoe_set_timing(h: int, enable: bool):
    _check(load().lmoe_set_timing(h, int(enable)), "lmoe_set_timing")


def lmoe_get_timing(h: int):
    """Accumulated ms per stage (dict) and the number of timed forward calls."""
    ms = (ctypes.c_float * LMOE_NUM_STAGES)()
    n = ctypes.c_int32()
    _check(load().lmoe_get_timing(h, ms, ctypes.byref(n)), "lmoe_get_timing")
    return dict(zip(STAGES, list(ms))), n.value


def lmoe_mx_quantize_e4m3(x: int, n: int, codes: int, scales: int, stream: int = 0):
    _check(load().lmoe_mx_quantize_e4m3(x, n, codes, scales, stream), "lmoe_mx_quantize_e4m3")


def lmoe_nvfp4_to_mxfp4(codes: int, scales16: int, global_scale: int, n_mats: int, rows: int, cols: int,
                        out_codes: int, out_scales: int, stream: int = 0):
    _check(load().lmoe_nvfp4_to_mxfp4(codes, scales16, global_scale, n_mats, rows, cols, out_codes,
                                      out_scales, stream), "lmoe_nvfp4_to_mxfp4")


def lmoe_pack_experts(src: int, dst: int, n_mats: int, rows: int, cols: int, stream: int = 0):
    _check(load().lmoe_pack_experts(src, dst, n_mats, rows, cols, stream), "lmoe_pack_experts")


def make_config(D, Dp, F, E, k, max_tokens, act="bf16", eps_pool=1e-6, eps_expert=1e-6,
                router_bias=False, out=None, experts=None, packed=False) -> lmoe_config:
    """act / out: "bf16" or "f32" (out defaults to act); experts: the expert
    weight format, act (default) or "mxfp4"; packed: the bf16 expert weights
    are in the packed expert layout (lmoe_pack_experts)."""
    dts = {"bf16": LMOE_BF16, "f32": LMOE_F32, "mxfp4": LMOE_MXFP4}
    dt = dts[act]
    return lmoe_config(LMOE_ABI_VERSION, D, Dp, F, E, k, eps_pool, eps_expert, dt,
                       dts[experts or act], dts[out or act], max_tokens,
                       (LMOE_FLAG_ROUTER_BIAS if router_bias else 0) |
                       (LMOE_FLAG_PACKED_EXPERTS if packed else 0))


def pack_expert_weights(weights: dict, stream=None, in_place: bool = False) -> dict:
    """A bf16 weight dict whose w_gate_up and w_down are in the packed expert
    layout, filled by lmoe_pack_experts on `stream` (default: the current one);
    the other tensors are shared. By default the packed tensors are new ones of
    the same shapes. in_place: each expert matrix is copied to a one-matrix
    staging buffer and packed back into its own storage, so no second copy of
    the experts is allocated (or later freed); the given tensors are modified."""
    import torch
    out = dict(weights)
    st = stream or torch.cuda.current_stream()
    for name in ("w_gate_up", "w_down"):
        w = weights[name]
        assert w.dtype == torch.bfloat16 and w.is_contiguous() and w.dim() == 3
        n, R, C = w.shape
        if not in_place:
            p = torch.empty_like(w)
            lmoe_pack_experts(w.data_ptr(), p.data_ptr(), n, R, C, st.cuda_stream)
            out[name] = p
            continue
        with torch.cuda.stream(st):
            stage = torch.empty_like(w[0])
            for e in range(n):
                stage.copy_(w[e])
                lmoe_pack_experts(stage.data_ptr(), w[e].data_ptr(), 1, R, C, st.cuda_stream)
            stage.record_stream(st)
    return out


class LatentMoE:
    """A created block over torch device tensors (kept referenced here, since the
    library borrows them). weights: w_router [E, D], b_router [E] or None,
    w_pool [Dp, D], g_pool [Dp], w_gate_up [E, 2F, Dp], w_down [E, Dp, F],
    g_expert [E, Dp], w_unpool [D, Dp]; activations and weights in one dtype
    (torch.bfloat16 or torch.float32), gammas and bias float32. MXFP4 experts:
    w_gate_up [E, 2F, Dp/2] and w_down [E, Dp, F/2] as uint8 E2M1 pairs plus
    s_gate_up [E, 2F, Dp/32] and s_down [E, Dp, F/32] uint8 E8M0 scales.
    out_dtype: torch.float32 or the activation dtype (the default). packed: the
    bf16 w_gate_up and w_down are in the packed expert layout
    (pack_expert_weights)."""

    def __init__(self, weights: dict, top_k: int, max_tokens: int, eps_pool=1e-6, eps_expert=1e-6,
                 out_dtype=None, packed: bool = False):
        import torch
        wp = weights["w_pool"]
        act = {torch.bfloat16: "bf16", torch.float32: "f32"}[wp.dtype]
        E, D = weights["w_router"].shape
        Dp = wp.shape[0]
        mx = weights.get("s_down") is not None
        F = weights["w_down"].shape[2] * (2 if mx else 1)
        self.weights = weights
        self.dtype = wp.dtype
        self.out_dtype = out_dtype or wp.dtype
        out = {torch.bfloat16: "bf16", torch.float32: "f32"}[self.out_dtype]
        self.D, self.Dp, self.F, self.E, self.k = D, Dp, F, E, top_k
        self.max_tokens = max_tokens
        self.cfg = make_config(D, Dp, F, E, top_k, max_tokens, act, eps_pool, eps_expert,
                               weights.get("b_router") is not None, out,
                               "mxfp4" if mx else None, packed)
        ptr = lambda name: weights[name].data_ptr() if weights.get(name) is not None else None
        self.cw = lmoe_weights(ptr("w_router"), ptr("b_router"), ptr("w_pool"), ptr("g_pool"),
                               ptr("w_gate_up"), ptr("s_gate_up"), ptr("w_down"), ptr("s_down"),
                               ptr("g_expert"),
                               ptr("w_unpool"))
        self.handle = lmoe_create(self.cfg, self.cw)

    def forward(self, x, out=None, aux: bool = False, stream=None):
        import torch
        T = x.shape[0]
        assert x.dtype == self.dtype and x.is_contiguous() and x.shape[1] == self.D
        if out is None:
            out = torch.empty(x.shape, dtype=self.out_dtype, device=x.device)
        assert out.dtype == self.out_dtype and out.is_contiguous() and out.shape == x.shape
        a = None
        res = {}
        if aux:
            dev = x.device
            res = {"logits": torch.empty(T, self.E, dtype=torch.float32, device=dev),
                   "topk_ids": torch.empty(T, self.k, dtype=torch.int32, device=dev),
                   "topk_w": torch.empty(T, self.k, dtype=torch.float32, device=dev),
                   "expert_offsets": torch.empty(self.E + 1, dtype=torch.int32, device=dev),
                   "sorted_assign": torch.empty(T * self.k, dtype=torch.int32, device=dev)}
            a = lmoe_aux(*(res[n].data_ptr() for n in
                           ("logits", "topk_ids", "topk_w", "expert_offsets", "sorted_assign")))
        s = (stream or torch.cuda.current_stream(x.device)).cuda_stream
        lmoe_forward(self.handle, x.data_ptr(), out.data_ptr(), T, s, a)
        return (out, res) if aux else out

    def set_timing(self, enable: bool):
        lmoe_set_timing(self.handle, enable)

    def get_timing(self):
        return lmoe_get_timing(self.handle)

    def close(self):
        if self.handle:
            lmoe_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
