"""Helpers shared by the GPU parity tests: oracle references and comparisons.

All expected values come from the CPU oracle on the same seeded inputs; nothing
here reads a GPU result back into an oracle input.
"""
from __future__ import annotations

import sys

import numpy as np

import oracle
import synth

GAP = 1e-5          # tokens whose k-th/(k+1)-th logit gap is at most this have two valid selections
TOL = {synth.F32: 1e-4, synth.BF16: 2e-2, synth.MXFP4: 6e-2}


def tol(w: synth.Workload) -> float:
    """Output tolerance of a workload: its activation dtype's, or MXFP4's."""
    return TOL[synth.MXFP4] if w.mx_act else TOL[w.act]


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def host_weights(w: synth.Workload, with_experts: bool) -> dict:
    d = {"w_router": synth.w_router(w), "b_router": synth.router_bias(w), "w_pool": synth.w_pool(w),
         "g_pool": synth.g_pool(w), "g_expert": synth.g_expert(w), "w_unpool": synth.w_unpool(w)}
    if with_experts:
        full = synth.dense_weights(w)
        for key in ("w_gate_up", "w_down", "s_gate_up", "s_down"):
            if key in full:
                d[key] = full[key]
    return d


def oracle_ref(w: synth.Workload, x_rows: np.ndarray, wts: dict | None = None):
    """The oracle on the given token rows. Experts are regenerated from their
    seeds when wts holds no expert weights."""
    if wts is None:
        wts = host_weights(w, with_experts=False)
    get = None
    if "w_gate_up" not in wts:
        def get(e):
            gu, dn = synth.w_gate_up(w, e), synth.w_down(w, e)
            return (gu[0], gu[1], dn[0], dn[1]) if w.expert_w == synth.MXFP4 else (gu, dn)
    rnd = w.act == synth.BF16
    return oracle.default().forward(x_rows, wts, w.k, w.eps_pool, w.eps_expert, mx_act=w.mx_act,
                                    get_expert=get, rnd=rnd)


def out_error(got: np.ndarray, ref: np.ndarray) -> float:
    """max |err| / RMS(ref)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.abs(got - ref).max() / np.sqrt((ref ** 2).mean()))


def check_routing(ids_gpu, w_gpu, logits_gpu, logits_ref, ids_ref, w_ref, k):
    """Routing checks. Logits: within 1e-4 + 4 ulp(|l|) of the oracle's (both
    are fp32 roundings of the same dot product plus bias; the GPU sums in fp32,
    and a large bias makes the final add round at a coarse ulp). Selection:
    bit-exact (same ids, same order) wherever the oracle's k-th/(k+1)-th gap
    exceeds GAP; elsewhere the GPU's choice must still be a valid top-k.
    Weights: the softmax of the GPU's own selected logits within 1e-6, and the
    oracle's weights within the first-order bound |dw_j| <= 2 w_j max_i|dl_i|
    that the logit difference implies (plus 1e-6). Returns the near-tie mask."""
    logits_gpu = np.asarray(logits_gpu, np.float64)
    logits_ref = np.asarray(logits_ref, np.float64)
    diff = np.abs(logits_gpu - logits_ref)
    lim = 1e-4 + 4 * 2.0 ** -24 * np.abs(logits_ref)
    assert np.all(diff <= lim), f"router logits differ by {(diff - lim).max() + 1e-4:.3e}"
    gap = oracle.topk_gap(logits_ref, k)
    near = gap <= GAP
    ok = ~near
    assert np.array_equal(ids_gpu[ok], ids_ref[ok]), \
        f"selection differs on {int((ids_gpu[ok] != ids_ref[ok]).any(1).sum())} tokens"
    sel = np.take_along_axis(logits_gpu, ids_gpu.astype(np.int64), 1)
    dl = np.take_along_axis(diff, ids_gpu.astype(np.int64), 1).max(axis=1)   # selected logits only
    own = np.exp(sel - sel.max(1, keepdims=True))
    own /= own.sum(1, keepdims=True)
    assert np.abs(w_gpu - own).max(initial=0.0) <= 1e-6
    bound = 2 * w_ref[ok] * dl[ok][:, None] + 1e-6
    assert np.all(np.abs(w_gpu[ok] - w_ref[ok]) <= bound)
    for t in np.nonzero(near)[0]:
        kth = np.sort(logits_ref[t])[::-1][k - 1]
        assert np.all(logits_ref[t][ids_gpu[t]] >= kth - GAP)
        assert len(set(ids_gpu[t].tolist())) == k
    return near


def check_permutation(ids_gpu, offsets_gpu, sorted_gpu, E):
    """The GPU permutation equals the oracle's permutation of the GPU's own
    selection, bit for bit."""
    _, offsets, sa, _ = oracle.default().permutation(ids_gpu, E)
    assert np.array_equal(offsets_gpu, offsets), "expert offsets differ"
    assert np.array_equal(sorted_gpu, sa), "sorted assignment order differs"
