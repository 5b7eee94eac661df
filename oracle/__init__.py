"""CPU oracle of the latent-MoE block forward -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. The product path (the HIP library and its binding) never loads it
and shares no code with it.

This is a thin ctypes layer over liboracle.so (plain C, double accumulation, one
function per step of the block; the C source cites the passage each step
follows). Arrays are numpy: float32, uint16 (bfloat16 bits) or uint8 (MXFP4 codes
and E8M0 scales).

Every function here is pinned by the CPU tests (brute force, closed forms,
invariants and special cases); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

ORC_F32, ORC_BF16, ORC_MXFP4 = 0, 1, 2

_P = ctypes.c_void_p
_I = ctypes.c_int
_D = ctypes.c_double


def load(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    sig = {
        "orc_router": [_P, _P, _I, _P, _I, _I, _I, _P],
        "orc_topk_softmax": [_P, _I, _I, _I, _P, _P],
        "orc_permutation": [_P, _I, _I, _I, _P, _P, _P, _P],
        "orc_pool_norm": [_P, _P, _I, _P, _I, _I, _I, _D, _I, _I, _P],
        "orc_expert": [_P, _I, _I, _P, _P, _P, _P, _I, _P, _D, _I, _I, _P, _P],
        "orc_combine_unpool": [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P],
        "orc_expert_assign": [_P, _I, _P, _P, _I, _I, _P, _P, _P, _P, _I, _P, _D, _I, _I, _P, _P],
        "orc_mx_quant_e4m3": [_P, _I, _P, _P, _P],
        "orc_mx_quant_e2m1": [_P, _I, _P, _P, _P],
        "orc_nvfp4_to_mxfp4": [_P, _P, _P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _P, _P],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = None
    for name in ("orc_e8m0_value", "orc_e2m1_value", "orc_e4m3_value"):
        fn = getattr(lib, name)
        fn.argtypes = [ctypes.c_uint8]
        fn.restype = _D
    lib.orc_set_threads.argtypes = [ctypes.c_int]
    lib.orc_set_threads.restype = None
    lib.orc_get_threads.argtypes = []
    lib.orc_get_threads.restype = ctypes.c_int
    lib.orc_set_flush_modes.argtypes = [ctypes.c_int]
    lib.orc_set_flush_modes.restype = None
    lib.orc_round_bf16.argtypes = [_D]
    lib.orc_round_bf16.restype = _D
    return lib


class Oracle:
    """The oracle over one loaded liboracle.so (tests may load a variant build)."""

    def __init__(self, path: str = LIB_PATH):
        self.lib = load(path)

    # -- helpers ---------------------------------------------------------
    @staticmethod
    def _dt(a: np.ndarray) -> int:
        if a.dtype == np.float32:
            return ORC_F32
        if a.dtype == np.uint16:
            return ORC_BF16
        raise TypeError(f"unsupported dtype {a.dtype}")

    @staticmethod
    def _c(a, dtype=None):
        if a is None:
            return None
        a = np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))
        return a

    # -- steps -------------------------------------------------------------
    def router(self, x, wr, bias=None) -> np.ndarray:
        x, wr = self._c(x), self._c(wr)
        assert x.dtype == wr.dtype
        T, D = x.shape
        E = wr.shape[0]
        b = self._c(bias, np.float32)
        out = np.empty((T, E), np.float32)
        self.lib.orc_router(x.ctypes.data, wr.ctypes.data, self._dt(x),
                            None if b is None else b.ctypes.data, T, D, E, out.ctypes.data)
        return out

    def topk_softmax(self, logits, k):
        logits = self._c(logits, np.float32)
        T, E = logits.shape
        ids = np.empty((T, k), np.int32)
        w = np.empty((T, k), np.float64)
        self.lib.orc_topk_softmax(logits.ctypes.data, T, E, k, ids.ctypes.data, w.ctypes.data)
        return ids, w

    def permutation(self, ids, E):
        ids = self._c(ids, np.int32)
        T, k = ids.shape
        counts = np.empty(E, np.int32)
        offsets = np.empty(E + 1, np.int32)
        sa = np.empty(T * k, np.int32)
        inv = np.empty(T * k, np.int32)
        self.lib.orc_permutation(ids.ctypes.data, T, k, E, counts.ctypes.data, offsets.ctypes.data,
                                 sa.ctypes.data, inv.ctypes.data)
        return counts, offsets, sa, inv

    def pool_norm(self, x, wp, gp, eps, mx_act=False, rnd=False) -> np.ndarray:
        x, wp, gp = self._c(x), self._c(wp), self._c(gp, np.float32)
        T, D = x.shape
        Dp = wp.shape[0]
        xp = np.empty((T, Dp), np.float64)
        self.lib.orc_pool_norm(x.ctypes.data, wp.ctypes.data, self._dt(x), gp.ctypes.data, T, D, Dp,
                               eps, int(mx_act), int(rnd), xp.ctypes.data)
        return xp

    def combine_unpool(self, z, w, wun, rnd=False) -> np.ndarray:
        z, w, wun = self._c(z, np.float64), self._c(w, np.float64), self._c(wun)
        T, k, Dp = z.shape
        D = wun.shape[0]
        out = np.empty((T, D), np.float64)
        self.lib.orc_combine_unpool(z.ctypes.data, w.ctypes.data, wun.ctypes.data, self._dt(wun),
                                    T, k, Dp, D, int(rnd), out.ctypes.data)
        return out

    # -- MX codec ------------------------------------------------------------
    def mx_quant_e4m3(self, v):
        v = self._c(v, np.float64)
        n = v.size
        codes = np.empty(n, np.uint8)
        scales = np.empty(n // 32, np.uint8)
        deq = np.empty(n, np.float64)
        self.lib.orc_mx_quant_e4m3(v.ctypes.data, n, codes.ctypes.data, scales.ctypes.data,
                                   deq.ctypes.data)
        return codes, scales, deq

    def mx_quant_e2m1(self, v):
        v = self._c(v, np.float64)
        n = v.size
        packed = np.empty(n // 2, np.uint8)
        scales = np.empty(n // 32, np.uint8)
        deq = np.empty(n, np.float64)
        self.lib.orc_mx_quant_e2m1(v.ctypes.data, n, packed.ctypes.data, scales.ctypes.data,
                                   deq.ctypes.data)
        return packed, scales, deq

    def nvfp4_to_mxfp4(self, codes, scales16, g):
        """codes [M][R][C/2] u8, scales16 [M][R][C/16] u8, g [M] f32 ->
        (codes [M][R][C/2], scales [M][R][C/32]) of the MXFP4 re-encoding."""
        codes = self._c(codes, np.uint8)
        scales16 = self._c(scales16, np.uint8)
        g = self._c(g, np.float32)
        M, R, half = codes.shape
        C = 2 * half
        assert scales16.shape == (M, R, C // 16) and g.shape == (M,) and C % 32 == 0
        oc = np.empty_like(codes)
        os_ = np.empty((M, R, C // 32), np.uint8)
        self.lib.orc_nvfp4_to_mxfp4(codes.ctypes.data, scales16.ctypes.data, g.ctypes.data, M, R, C,
                                    oc.ctypes.data, os_.ctypes.data)
        return oc, os_

    def set_threads(self, n: int):
        """Threads of the parallel loops (timing only; results do not depend on it)."""
        self.lib.orc_set_threads(int(n))

    def threads(self) -> int:
        return self.lib.orc_get_threads()

    def round_bf16(self, v: float) -> float:
        return self.lib.orc_round_bf16(float(v))

    def e2m1_value(self, c):
        return self.lib.orc_e2m1_value(c)

    def e4m3_value(self, c):
        return self.lib.orc_e4m3_value(c)

    def e8m0_value(self, c):
        return self.lib.orc_e8m0_value(c)

    # -- the block -----------------------------------------------------------
    def forward(self, x, wts: dict, k: int, eps_pool=1e-6, eps_expert=1e-6, mx_act=False,
                get_expert=None, rnd=False):
        """The whole block on the rows of x, in the pages' order: router, top-k
        and weights, pooler + pooled RMSNorm, each selected expert with its own
        RMSNorm, weighted sum, unpooler.

        wts holds w_router, b_router (or None), w_pool, g_pool, g_expert [E, Dp],
        w_unpool, and either stacked expert weights (w_gate_up [E, 2F, Dp], w_down
        [E, Dp, F], plus s_gate_up / s_down for MXFP4) or get_expert(e) returning
        (w_gate_up_e, w_down_e) or (codes_gu, scales_gu, codes_d, scales_d).

        Returns (out [T, D] float64, aux) with aux: logits, ids, w, rms_unit [T, k].
        """
        logits = self.router(x, wts["w_router"], wts.get("b_router"))
        ids, w = self.topk_softmax(logits, k)
        xp = self.pool_norm(x, wts["w_pool"], wts["g_pool"], eps_pool, mx_act, rnd)
        T, Dp = xp.shape
        ge = self._c(wts["g_expert"], np.float32)
        E = ge.shape[0]
        keep = []                                   # keeps the expert arrays alive
        ptrs = [(ctypes.c_void_p * E)() for _ in range(4)]
        mx = "s_gate_up" in wts or (get_expert is not None and mx_act)
        F = None
        for e in np.unique(ids):
            e = int(e)
            if get_expert is not None:
                ew = tuple(self._c(a) for a in get_expert(e))
            elif "s_gate_up" in wts:
                ew = (wts["w_gate_up"][e], wts["s_gate_up"][e], wts["w_down"][e], wts["s_down"][e])
            else:
                ew = (wts["w_gate_up"][e], wts["w_down"][e])
            ew = tuple(self._c(a) for a in ew)
            keep.append(ew)
            if len(ew) == 4:
                mx = True
                ptrs[0][e], ptrs[1][e], ptrs[2][e], ptrs[3][e] = (a.ctypes.data for a in ew)
                F = ew[2].shape[1] * 2
                wdt = ORC_MXFP4
            else:
                ptrs[0][e], ptrs[2][e] = ew[0].ctypes.data, ew[1].ctypes.data
                F = ew[1].shape[1]
                wdt = self._dt(ew[0])
        n = T * k
        z = np.zeros((T, k, Dp), np.float64)
        rms = np.zeros((T, k), np.float64)
        if n:
            tok = np.ascontiguousarray(np.repeat(np.arange(T, dtype=np.int32), k))
            ex = np.ascontiguousarray(ids.ravel().astype(np.int32))
            self.lib.orc_expert_assign(xp.ctypes.data, n, tok.ctypes.data, ex.ctypes.data, Dp, F,
                                       ptrs[0], ptrs[1] if mx else None, ptrs[2],
                                       ptrs[3] if mx else None, wdt, ge.ctypes.data, eps_expert,
                                       int(mx_act), int(rnd), z.ctypes.data, rms.ctypes.data)
        out = self.combine_unpool(z, w, wts["w_unpool"], rnd)
        return out, {"logits": logits, "ids": ids, "w": w, "rms_unit": rms, "xp": xp}


_DEFAULT = None


def default() -> Oracle:
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT


def topk_gap(logits: np.ndarray, k: int) -> np.ndarray:
    """Per token, the gap between the k-th and (k+1)-th largest logit (inf if
    k == E). Tokens whose gap is at most 1e-5 have two valid selections."""
    l = np.sort(np.asarray(logits, np.float64), axis=1)[:, ::-1]
    if k >= l.shape[1]:
        return np.full(l.shape[0], np.inf)
    return l[:, k - 1] - l[:, k]
