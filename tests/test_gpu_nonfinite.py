"""GPU regression test: routing on non-finite logits.

A NaN anywhere in a token's x row makes all of its router logits NaN; a router
bias of -inf (or +inf) pins experts out of (or into) every selection. The
oracle's reading: NaN scores as -inf, ties (the -inf ones included) go to the
lower expert id, so every token still selects k distinct valid experts; the
weights are the softmax of the selected scores, or equal shares among the
slots holding the largest score when it is infinite. These cases check the
GPU's ids, expert offsets and sorted order bit for bit against the oracle's,
its weights against the oracle's, and that a NaN token leaves every other
token's output within the bf16 tolerance (its own output is NaN, as the
oracle's is). Cases run on both batch regimes (at T <= 128 split-K streaming
dense projections, the top-k inside the pooled-norm kernel and every expert on
the weight-streaming kernels; above, the tiled dense projections, the top-k
kernel, and the tiled expert GEMM when the bias sends every token to the same
experts).
"""
import numpy as np
import pytest
import torch

import latent_moe_layer_router_amd as lmoe
import oracle
import synth
from synth import device as sdev
from tests import harness as H
from tests.pins import tiny

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF16_NAN = np.uint16(0x7FC0)


def upload(wts: dict) -> dict:
    return {n: (sdev.to_device(a, DEV) if a is not None else None) for n, a in wts.items()}


def run(w, wts, x):
    T = x.shape[0]
    H.say(f"[gpu] non-finite routing: T={T} E={w.E} k={w.k} D={w.D} Dp={w.Dp} F={w.F}")
    block = lmoe.LatentMoE(upload(wts), w.k, T, w.eps_pool, w.eps_expert, out_dtype=torch.float32)
    out, aux = block.forward(sdev.to_device(x, DEV), aux=True)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    a = {n: t.cpu().numpy() for n, t in aux.items()}
    block.close()
    ref, raux = oracle.default().forward(x, wts, w.k, w.eps_pool, w.eps_expert, rnd=True)
    return got, a, ref, raux


def check(w, got, a, ref, raux, bad_rows=()):
    lg, lr = a["logits"].astype(np.float64), raux["logits"].astype(np.float64)
    # logits: the same non-finite pattern, finite ones within 1e-4 + 4 ulp
    assert np.array_equal(np.isnan(lg), np.isnan(lr))
    assert np.array_equal(np.isposinf(lg), np.isposinf(lr)) and np.array_equal(np.isneginf(lg), np.isneginf(lr))
    fin = np.isfinite(lr)
    assert np.all(np.abs(lg[fin] - lr[fin]) <= 1e-4 + 4 * 2.0 ** -24 * np.abs(lr[fin]))
    ids = a["topk_ids"]
    assert np.all((ids >= 0) & (ids < w.E))
    assert all(len(set(r)) == w.k for r in ids.tolist())
    # selection: bit-exact, except tokens whose finite k-th/(k+1)-th gap is a near-tie
    with np.errstate(invalid="ignore"):
        near = oracle.topk_gap(np.where(np.isnan(lr), -np.inf, lr), w.k) <= H.GAP
    assert np.array_equal(ids[~near], raux["ids"][~near])
    H.check_permutation(ids, a["expert_offsets"], a["sorted_assign"], w.E)
    if not near.any():
        _, offsets, sa, _ = oracle.default().permutation(raux["ids"], w.E)
        assert np.array_equal(a["expert_offsets"], offsets) and np.array_equal(a["sorted_assign"], sa)
    # weights: exact shares where the largest selected score is infinite, else
    # the first-order bound of the logit difference
    wg, wr = a["topk_w"].astype(np.float64), raux["w"]
    assert np.all(np.isfinite(wg))
    sel = np.take_along_axis(np.where(np.isnan(lg), -np.inf, lg), ids.astype(np.int64), 1)
    sel_ref = np.take_along_axis(np.where(np.isnan(lr), -np.inf, lr), ids.astype(np.int64), 1)
    fin_sel = np.isfinite(sel)
    dl = np.zeros_like(sel)
    dl[fin_sel] = np.abs(sel[fin_sel] - sel_ref[fin_sel])
    bound = 2 * wr * np.nan_to_num(dl).max(1, keepdims=True) + 1e-6
    assert np.all(np.abs(wg[~near] - wr[~near]) <= bound[~near])
    assert np.abs(wg.sum(1) - 1).max() <= 1e-5
    # outputs: NaN tokens are NaN on both sides; every other token within tolerance
    bad = np.zeros(got.shape[0], bool)
    bad[list(bad_rows)] = True
    assert np.all(np.isnan(ref[bad])) and np.all(np.isnan(got[bad]))
    ok = ~bad & ~near
    assert np.all(np.isfinite(got[ok]))
    err = H.out_error(got[ok], ref[ok])
    H.say(f"[gpu]   max|err|/rms = {err:.3e} over {int(ok.sum())} tokens, near-ties = {int(near.sum())}")
    assert err <= H.TOL[synth.BF16], err


def workload(T):
    return tiny(T=T, D=512, Dp=256, F_=256, E=256, k=8, seed=131, act=synth.BF16)


@pytest.mark.parametrize("T", [100, 200])
def test_nan_token_rows(T):
    """NaN in two tokens' x rows (in different 64-token chunks when T > 64)."""
    w = workload(T)
    wts = synth.dense_weights(w)
    x = synth.x(w, T=T).copy()
    bad = (5, T - 3)
    x[bad[0], 17] = BF16_NAN
    x[bad[1], :] = BF16_NAN
    check(w, *run(w, wts, x), bad_rows=bad)


@pytest.mark.parametrize("T", [100, 200])
def test_minus_inf_bias_leaves_k_minus_1_experts(T):
    """-inf bias on E - k + 1 experts: each token selects the k - 1 finite ones and
    then the lowest-id -inf expert, with weight 0; one token also has a NaN row."""
    w = workload(T)
    wts = synth.dense_weights(w)
    rng = np.random.default_rng(17)
    b = (rng.standard_normal(w.E) * 0.5).astype(np.float32)
    b[rng.choice(w.E, w.E - w.k + 1, replace=False)] = -np.inf
    wts["b_router"] = b
    x = synth.x(w, T=T).copy()
    x[7, :] = BF16_NAN
    check(w, *run(w, wts, x), bad_rows=(7,))


@pytest.mark.parametrize("T", [100, 200])
def test_all_minus_inf_bias(T):
    """-inf bias on every expert: experts 0..k-1 with equal weights for every
    token, so each of them gets all T rows (the tiled expert GEMMs at 200
    tokens; at 100 the streaming kernels in two passes, after the top-k that
    runs inside the small-batch pooled-norm kernel)."""
    w = workload(T)
    wts = synth.dense_weights(w)
    wts["b_router"] = np.full(w.E, -np.inf, np.float32)
    got, a, ref, raux = run(w, wts, synth.x(w, T=T))
    assert np.all(a["topk_ids"] == np.arange(w.k)) and np.all(a["topk_w"] == np.float32(1 / w.k))
    check(w, got, a, ref, raux)


@pytest.mark.parametrize("T", [100, 200])
def test_plus_inf_bias(T):
    """+inf bias on two experts: both are selected first by every token and share
    the weight equally; the other slots get 0."""
    w = workload(T)
    wts = synth.dense_weights(w)
    b = np.zeros(w.E, np.float32)
    b[[200, 9]] = np.inf
    wts["b_router"] = b
    got, a, ref, raux = run(w, wts, synth.x(w, T=T))
    assert np.all(a["topk_ids"][:, :2] == [9, 200])
    assert np.all(a["topk_w"][:, :2] == 0.5) and np.all(a["topk_w"][:, 2:] == 0)
    check(w, got, a, ref, raux)
