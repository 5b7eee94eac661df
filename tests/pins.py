"""Pins of the CPU oracle: checks against facts that do not come from the oracle.

Each pin is a function of an Oracle instance and raises AssertionError when the
oracle disagrees with what the pages and the mathematics fix:
  - brute force on tiny shapes: every expert computed densely for every token
    with library routines (torch float64 linear / silu / rms_norm / softmax) and
    weighted by a mask built from an independent full sort (numpy lexsort);
  - special cases that reduce to a dense network (E = 1, k = 1; identical experts);
  - closed forms and invariants (routing weights sum to 1, per-expert RMS before
    gamma is sqrt(ms / (ms + eps)) <= 1, scale invariance of both RMSNorms,
    token-permutation invariance);
  - library sorts for top-k and the permutation;
  - the OCP MX element and scale tables, hand-worked blocks, and an independent
    MXFP4 encoder (the input generator's);
  - torch's float32 -> bfloat16 conversion for the bfloat16 rounding.
test_oracle_pins.py runs them on the built oracle; test_oracle_mutants.py plants
mistakes in copies of the oracle source and checks that some pin catches each.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F

import synth

E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])   # OCP MX v1.0, FP4 E2M1


def tiny(T=24, D=64, Dp=32, F_=64, E=6, k=3, seed=11, act=synth.F32, expert_w=None, skew=False):
    """A tiny workload (Dp != F and D != Dp so that a transposed operand shows)."""
    return synth.shrink(synth.WORKLOADS["tiny_fp32"], name="pin", T=T, D=D, Dp=Dp, F=F_, E=E, k=k,
                        seed=seed, x_seed=seed, act=act,
                        expert_w=act if expert_w is None else expert_w, skew=skew)


def weights(w, with_bias=False):
    d = synth.dense_weights(w)
    if with_bias:
        d["b_router"] = synth.normal(w.seed, synth.stream_id(99), (w.E,), 0.5, 0.0, synth.F32)
    return d


def f64(a):
    return synth.as_f32(np.asarray(a)).astype(np.float64)


def t64(a):
    return torch.from_numpy(np.ascontiguousarray(f64(a)))


def bf16_lib(t: torch.Tensor) -> torch.Tensor:
    """Round float64 values to bfloat16 (nearest, ties to even), kept as float64.

    torch converts float64 -> bfloat16 through float32, and that double rounding
    flips about one tie in 2^16, so this uses a different exact route: adding
    and subtracting C = 1.5 * 2^(s + 52) rounds a double to a multiple of 2^s with
    the FPU's own ties-to-even, where 2^s is the bfloat16 spacing at that value."""
    a = t.numpy()
    _, e = np.frexp(a)
    C = np.ldexp(1.5, e - 8 + 52)
    r = np.where(a == 0, a, (a + C) - C)
    return torch.from_numpy(r)


def mxfp4_dequant(codes, scales):
    """Dequantize an MXFP4 matrix with the OCP tables (E2M1 grid, E8M0 = 2^(c-127))."""
    c = np.asarray(codes)
    lo, hi = c & 0xF, c >> 4
    el = np.empty(c.shape[:-1] + (c.shape[-1] * 2,), np.uint8)
    el[..., 0::2], el[..., 1::2] = lo, hi
    mag = E2M1_GRID[el & 7]
    val = np.where(el & 8, -mag, mag)
    sc = np.ldexp(1.0, np.asarray(scales, np.int64) - 127)
    return val * np.repeat(sc, 32, axis=-1)


def brute_force(O, x, wts, k, eps_p, eps_e, rnd=False, mx_act=False):
    """Dense reference: all experts for every token, weighted by a 0/w mask."""
    X = t64(x)
    T = X.shape[0]
    Wr = t64(wts["w_router"])
    logits = F.linear(X, Wr)
    if wts.get("b_router") is not None:
        logits = logits + t64(wts["b_router"])
    logits = logits.to(torch.float32)                     # selection is decided on FP32 logits
    E = logits.shape[1]
    l64 = logits.to(torch.float64).numpy()
    order = np.lexsort((np.broadcast_to(np.arange(E), l64.shape), -l64), axis=-1)
    sel = order[:, :k]
    wsel = torch.softmax(torch.from_numpy(np.take_along_axis(l64, sel, 1)), dim=1).numpy()
    mask = np.zeros((T, E))
    np.put_along_axis(mask, sel, wsel, 1)

    P = F.linear(X, t64(wts["w_pool"]))
    xp = F.rms_norm(P, (P.shape[1],), weight=t64(wts["g_pool"]), eps=eps_p)
    if mx_act:
        xp = torch.from_numpy(O.mx_quant_e4m3(xp.numpy().ravel())[2].reshape(xp.shape))
    elif rnd:
        xp = bf16_lib(xp)
    Dp = xp.shape[1]
    acc = torch.zeros(T, Dp, dtype=torch.float64)
    ge = t64(wts["g_expert"])
    for e in range(E):
        if "s_gate_up" in wts:
            Wgu = torch.from_numpy(mxfp4_dequant(wts["w_gate_up"][e], wts["s_gate_up"][e]))
            Wd = torch.from_numpy(mxfp4_dequant(wts["w_down"][e], wts["s_down"][e]))
        else:
            Wgu, Wd = t64(wts["w_gate_up"][e]), t64(wts["w_down"][e])
        Fh = Wgu.shape[0] // 2
        H = F.silu(F.linear(xp, Wgu[:Fh])) * F.linear(xp, Wgu[Fh:])
        if mx_act:
            H = torch.from_numpy(O.mx_quant_e4m3(H.numpy().ravel())[2].reshape(H.shape))
        elif rnd:
            H = bf16_lib(H)
        Y = F.linear(H, Wd)
        if rnd:
            Y = bf16_lib(Y)
        Z = F.rms_norm(Y, (Dp,), weight=ge[e], eps=eps_e)
        acc += torch.from_numpy(mask[:, e:e + 1]) * Z
    if rnd:
        acc = bf16_lib(acc)
    out = F.linear(acc, t64(wts["w_unpool"]))
    return out.numpy(), sel, wsel


def rel_max(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return np.abs(a - b).max() / np.sqrt((b ** 2).mean())


# ---------------------------------------------------------------------------
# Pins
# ---------------------------------------------------------------------------

def pin_bruteforce(O):
    """P1: the oracle equals the dense brute force (fp32 and bf16 inputs, with
    and without the bf16 boundaries, with a router bias, small and large eps)."""
    cases = [dict(act=synth.F32), dict(act=synth.BF16, seed=12),
             dict(act=synth.F32, seed=13, E=9, k=4, T=17)]
    for c in cases:
        w = tiny(**c)
        for bias in (False, True):
            wts = weights(w, with_bias=bias)
            x = synth.x(w)
            for rnd in (False, True):
                for eps_p, eps_e in ((1e-6, 1e-6), (0.5, 2.0)):
                    out, aux = O.forward(x, wts, w.k, eps_p, eps_e, rnd=rnd)
                    ref, sel, wsel = brute_force(O, x, wts, w.k, eps_p, eps_e, rnd=rnd)
                    assert np.array_equal(aux["ids"], sel), (c, bias, rnd)
                    assert np.abs(aux["w"] - wsel).max() < 1e-12, (c, bias, rnd)
                    assert rel_max(out, ref) < 1e-9, (c, bias, rnd, eps_p, rel_max(out, ref))


def pin_bruteforce_mx(O):
    """P1 for the MXFP4-expert mode: MXFP4 weights dequantized with the OCP
    tables, expert input and SwiGLU output through the (separately pinned) MXFP8
    codec, bf16 boundaries elsewhere."""
    w = tiny(seed=21, act=synth.BF16, expert_w=synth.MXFP4)
    wts = weights(w)
    x = synth.x(w)
    out, aux = O.forward(x, wts, w.k, 1e-6, 1e-6, mx_act=True, rnd=True)
    ref, sel, _ = brute_force(O, x, wts, w.k, 1e-6, 1e-6, rnd=True, mx_act=True)
    assert np.array_equal(aux["ids"], sel)
    assert rel_max(out, ref) < 1e-9, rel_max(out, ref)


def pin_dense_e1k1(O):
    """P2: with E = 1, k = 1 the block is the dense network
    unpool(RMSNorm_e(SwiGLU(RMSNorm_p(pool(x))))), built here from torch routines."""
    w = tiny(E=1, k=1, seed=31)
    wts = weights(w)
    x = synth.x(w)
    out, aux = O.forward(x, wts, 1, 1e-6, 1e-6)
    X = t64(x)
    xp = F.rms_norm(F.linear(X, t64(wts["w_pool"])), (w.Dp,), t64(wts["g_pool"]), 1e-6)
    Wgu = t64(wts["w_gate_up"][0])
    h = F.silu(F.linear(xp, Wgu[:w.F])) * F.linear(xp, Wgu[w.F:])
    z = F.rms_norm(F.linear(h, t64(wts["w_down"][0])), (w.Dp,), t64(wts["g_expert"][0]), 1e-6)
    ref = F.linear(z, t64(wts["w_unpool"])).numpy()
    assert np.all(aux["ids"] == 0) and np.all(aux["w"] == 1.0)
    assert rel_max(out, ref) < 1e-12


def pin_topk(O):
    """P9: top-k equals a full library sort by (logit desc, index asc), including
    exact ties; the weights are the library softmax of the selected logits.
    Non-finite logits: NaN sorts as -inf (so the ids are always k distinct valid
    experts, ties to the lower index), and when the largest selected logit is
    infinite the weights are equal shares among the slots holding it (the
    softmax's limit) -- checked on rows of NaN, -inf and +inf against the same
    library sort and these closed forms."""
    rng = np.random.default_rng(5)
    for E, k in ((8, 2), (16, 5), (256, 8), (5, 5), (1, 1)):
        l = rng.integers(-3, 4, size=(40, E)).astype(np.float32) * np.float32(0.25)   # many ties
        ids, w = O.topk_softmax(l, k)
        order = np.lexsort((np.broadcast_to(np.arange(E), l.shape), -l.astype(np.float64)), axis=-1)
        assert np.array_equal(ids, order[:, :k]), (E, k)
        ref = torch.softmax(torch.from_numpy(np.take_along_axis(l, ids, 1).astype(np.float64)), 1)
        assert np.abs(w - ref.numpy()).max() < 1e-14
    # non-finite logits
    nan, inf = np.float32(np.nan), np.float32(np.inf)
    for E, k in ((8, 2), (16, 5), (256, 8), (5, 5), (70, 16)):
        l = rng.standard_normal((12, E)).astype(np.float32)
        l[0] = nan                                           # a NaN input row: every logit NaN
        l[1] = -inf                                          # every expert biased to -inf
        l[2, : E - k + 1] = -inf                             # only k - 1 finite logits
        l[3, rng.choice(E, E // 2, replace=False)] = nan     # NaN mixed with numbers
        l[4, 3 % E] = inf                                    # one +inf
        l[5, [1 % E, (E - 1)]] = inf                         # two +inf (one if E == 1)
        l[6, ::2] = -inf
        l[6, 1::3] = nan                                     # NaN and -inf interleaved
        l[7, : E - 1] = nan                                  # one number among NaNs
        ids, w = O.topk_softmax(l, k)
        score = np.where(np.isnan(l), -np.inf, l.astype(np.float64))
        order = np.lexsort((np.broadcast_to(np.arange(E), l.shape), -score), axis=-1)
        assert np.array_equal(ids, order[:, :k]), (E, k)
        assert np.all((ids >= 0) & (ids < E))
        assert all(len(set(r)) == k for r in ids.tolist())
        sel = np.take_along_axis(score, ids, 1)
        m = sel.max(1, keepdims=True)
        fin = np.isfinite(m[:, 0])
        ref = np.where(sel == m, 1.0, 0.0)
        ref = ref / ref.sum(1, keepdims=True)                # equal shares (infinite maximum)
        ref[fin] = torch.softmax(torch.from_numpy(sel[fin]), 1).numpy()
        assert np.abs(w - ref).max() < 1e-14, (E, k)
        assert np.array_equal(ids[0], np.arange(k)) and np.all(w[0] == 1.0 / k)
        assert np.array_equal(ids[1], np.arange(k)) and np.all(w[1] == 1.0 / k)
        assert ids[2, -1] == 0 and w[2, -1] == 0.0           # the lowest-id -inf expert, weight 0
        assert ids[4, 0] == 3 % E and w[4, 0] == 1.0
        assert np.abs(w.sum(1) - 1).max() <= 1e-15 * k


def pin_weights(O):
    """P4: routing weights are positive, non-increasing, and sum to 1."""
    rng = np.random.default_rng(6)
    l = rng.standard_normal((200, 64)).astype(np.float32) * 3
    for k in (1, 2, 8):
        _, w = O.topk_softmax(l, k)
        assert np.all(w > 0)
        assert np.all(np.diff(w, axis=1) <= 0)
        assert np.abs(w.sum(1) - 1).max() <= k * 2.0 ** -52 * 4


def pin_permutation(O):
    """P10: the permutation equals a library stable sort by expert; counts and
    offsets are the histogram and its exclusive prefix sum; inv inverts it."""
    rng = np.random.default_rng(7)
    for T, E, k in ((50, 8, 3), (1, 4, 4), (0, 5, 2), (300, 64, 8), (33, 256, 8)):
        ids = np.zeros((T, k), np.int32)
        for t in range(T):
            ids[t] = rng.choice(E, size=k, replace=False)
        if T:
            ids[: T // 3] = ids[0]                              # some repeated rows
        counts, offsets, sa, inv = O.permutation(ids, E)
        order = np.argsort(ids.ravel(), kind="stable")
        assert np.array_equal(sa, order)
        assert np.array_equal(counts, np.bincount(ids.ravel(), minlength=E))
        assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
        assert offsets[-1] == T * k
        assert np.array_equal(sa[inv], np.arange(T * k))


def pin_rms_unit(O):
    """P3: every selected expert's normalized row has RMS sqrt(ms / (ms + eps))
    before gamma, which lies in [1 - eps / (2 ms), 1]; here ms > 1e-3."""
    w = tiny(seed=41)
    wts = weights(w)
    x = synth.x(w)
    _, aux = O.forward(x, wts, w.k, 1e-6, 1e-6)
    r = aux["rms_unit"]
    assert np.all(r <= 1.0 + 1e-15) and np.all(r >= 1.0 - 1e-6 / (2 * 1e-3))
    _, aux2 = O.forward(x, wts, w.k, 1e-6, 10.0)            # large eps: strictly below 1
    assert np.all(aux2["rms_unit"] < 0.99)


def pin_token_permutation(O):
    """P5: tokens are independent; permuting x's rows permutes out's rows bit-exactly."""
    w = tiny(seed=51, T=20)
    wts = weights(w, with_bias=True)
    x = synth.x(w)
    perm = np.random.default_rng(8).permutation(w.T)
    for rnd in (False, True):
        a, _ = O.forward(x, wts, w.k, rnd=rnd)
        b, _ = O.forward(x[perm], wts, w.k, rnd=rnd)
        assert np.array_equal(a[perm], b)


def pin_norm_before_combine(O):
    """P6: each expert's output is normalized before its routing weight, so
    scaling one expert's W_down by 4 (exact) leaves out unchanged up to eps;
    scaling its gamma by 4 does change out (positive control)."""
    w = tiny(seed=61)
    wts = weights(w)
    x = synth.x(w)
    base, aux = O.forward(x, wts, w.k)
    e = int(np.bincount(aux["ids"].ravel()).argmax())
    w2 = dict(wts)
    w2["w_down"] = wts["w_down"].copy()
    w2["w_down"][e] *= 4
    out, _ = O.forward(x, w2, w.k)
    assert rel_max(out, base) < 1e-5
    w3 = dict(wts)
    w3["g_expert"] = wts["g_expert"].copy()
    w3["g_expert"][e] *= 4
    out3, _ = O.forward(x, w3, w.k)
    assert rel_max(out3, base) > 1e-2


def pin_pool_norm_invariance(O):
    """P7: the pooled input is normalized, so scaling W_pool by 4 leaves out
    unchanged up to eps; scaling g_pool by 4 changes it (positive control)."""
    w = tiny(seed=71)
    wts = weights(w)
    x = synth.x(w)
    base, _ = O.forward(x, wts, w.k)
    w2 = dict(wts)
    w2["w_pool"] = wts["w_pool"] * np.float32(4)
    out, _ = O.forward(x, w2, w.k)
    assert rel_max(out, base) < 1e-5
    w3 = dict(wts)
    w3["g_pool"] = wts["g_pool"] * np.float32(4)
    out3, _ = O.forward(x, w3, w.k)
    assert rel_max(out3, base) > 1e-2


def pin_identical_experts(O):
    """P8: with all experts (and their gammas) identical, out equals the E = 1,
    k = 1 dense block for any routing, because the weights sum to 1."""
    w = tiny(seed=81)
    wts = weights(w, with_bias=True)
    x = synth.x(w)
    same = dict(wts)
    same["w_gate_up"] = np.repeat(wts["w_gate_up"][:1], w.E, 0)
    same["w_down"] = np.repeat(wts["w_down"][:1], w.E, 0)
    same["g_expert"] = np.repeat(wts["g_expert"][:1], w.E, 0)
    out, _ = O.forward(x, same, w.k)
    one = dict(same)
    one["w_router"] = wts["w_router"][:1]
    one["b_router"] = None
    for key in ("w_gate_up", "w_down", "g_expert"):
        one[key] = same[key][:1]
    ref, _ = O.forward(x, one, 1)
    assert rel_max(out, ref) < 1e-12


def pin_round_bf16(O):
    """bfloat16 rounding equals torch's float32 -> bfloat16 conversion (nearest,
    ties to even), including constructed ties."""
    rng = np.random.default_rng(9)
    v = rng.standard_normal(4000).astype(np.float32) * np.float32(3.0)
    u = v.view(np.uint32).copy()
    u[:1000] = (u[:1000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)       # exact ties
    u[1000:1100] = (u[1000:1100] & np.uint32(0xFFFF0000)) | np.uint32(0x7FFF)
    v = u.view(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([O.round_bf16(float(a)) for a in v])
    assert np.array_equal(got, ref)


def pin_mx_codec(O):
    """P11: OCP MX v1.0 element and scale values, hand-worked blocks (shared
    exponent, ties to even, saturation, subnormals, all-zero block), round trips
    of representable values, and agreement with the input generator's
    independent MXFP4 encoder."""
    assert [O.e2m1_value(c) for c in range(8)] == list(E2M1_GRID)
    assert [O.e2m1_value(8 + c) for c in range(8)] == list(-E2M1_GRID)
    assert O.e4m3_value(0x7E) == 448.0 and np.isnan(O.e4m3_value(0x7F))
    assert O.e4m3_value(0x08) == 2.0 ** -6 and O.e4m3_value(0x01) == 2.0 ** -9
    assert O.e4m3_value(0x38) == 1.0 and O.e4m3_value(0xB8) == -1.0
    assert O.e8m0_value(127) == 1.0 and O.e8m0_value(0) == 2.0 ** -127
    assert np.isnan(O.e8m0_value(255))

    # E2M1 block with amax 6: exponent floor(log2 6) - 2 = 0 -> scale code 127.
    blk = np.zeros(32)
    blk[:12] = [6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.3, 7.9 / 2, -1.5, 0.2]
    _, sc, deq = O.mx_quant_e2m1(blk)
    assert sc[0] == 127
    assert list(deq[:12]) == [6.0, 0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, -0.5, 4.0, -1.5, 0.0]
    # saturation: amax 7.9 keeps exponent 0, and 7.9 saturates to 6
    blk2 = np.zeros(32)
    blk2[0] = 7.9
    _, sc2, deq2 = O.mx_quant_e2m1(blk2)
    assert sc2[0] == 127 and deq2[0] == 6.0
    # E4M3 block with amax 448: exponent 8 - 8 = 0; ties to even; subnormals
    b3 = np.zeros(32)
    b3[:6] = [448.0, 1 + 1 / 16, 1 + 3 / 16, 2.0 ** -9, 3 * 2.0 ** -10, 500.0 / 2]
    codes, sc3, deq3 = O.mx_quant_e4m3(b3)
    assert sc3[0] == 127
    assert list(deq3[:6]) == [448.0, 1.0, 1.25, 2.0 ** -9, 2 * 2.0 ** -9, 256.0]
    assert codes[0] == 0x7E and codes[1] == 0x38
    # a block scaled by 2^-20 gets scale code 127 - 20 and the same elements
    _, sc4, deq4 = O.mx_quant_e4m3(b3 * 2.0 ** -20)
    assert sc4[0] == 107 and np.array_equal(deq4, deq3 * 2.0 ** -20)
    # E4M3 saturation: amax 470 keeps exponent 0 and saturates to 448 (not 480)
    b6 = np.zeros(32)
    b6[0], b6[1] = 470.0, -500.0
    _, sc6, deq6 = O.mx_quant_e4m3(b6)
    assert sc6[0] == 127 and deq6[0] == 448.0 and deq6[1] == -448.0
    # all-zero block
    _, sc5, deq5 = O.mx_quant_e4m3(np.zeros(32))
    assert sc5[0] == 0 and not deq5.any()
    # round trips of representable values (grid times a block scale)
    rng = np.random.default_rng(10)
    g = rng.choice(np.concatenate([E2M1_GRID, -E2M1_GRID]), size=32 * 50)
    g[::32] = 6.0
    v = g * np.repeat(np.ldexp(1.0, rng.integers(-20, 20, size=50)), 32)
    assert np.array_equal(O.mx_quant_e2m1(v)[2], v)
    # agreement with the generator's independent MXFP4 encoder on the same draws
    vals = synth.normal(3, 77, (64 * 32,), 0.05, 0.0, synth.F32)
    codes_s, scales_s = synth.mxfp4_normal(3, 77, 64, 32, 0.05)
    packed, scales = O.mx_quant_e2m1(vals.astype(np.float64))[:2]
    assert np.array_equal(packed, codes_s.ravel()) and np.array_equal(scales, scales_s.ravel())


def nvfp4_block(codes16x2, sc0, sc1):
    """One 32-element NVFP4 block: 32 E2M1 codes (element order) packed two per
    byte (low nibble first), and its two per-16 scale bytes."""
    c = np.asarray(codes16x2, np.uint8)
    return (c[0::2] | (c[1::2] << 4)).astype(np.uint8), np.array([sc0, sc1], np.uint8)


def unpack4(b):
    b = np.asarray(b, np.uint8).ravel()
    out = np.empty(2 * b.size, np.uint8)
    out[0::2], out[1::2] = b & 0xF, b >> 4
    return out


def pin_nvfp4_requant(O):
    """P13: NVFP4 -> MXFP4 re-encoding. (a) Power-of-two block scales: with both
    per-16 scales 2^a and the matrix scale 2^b, and a +-6 in the block, the MXFP4
    block is the same codes with E8M0 exponent a + b (nibble order, per-16 scale
    indexing and the shared-exponent rule all show). (b) Hand-worked blocks:
    halves at scales 2^a and 2^(a-1); a non-power-of-two scale 1.5; a value that
    the FP32 product puts exactly on a tie of the E2M1 grid; NaN and overflow
    blocks; an all-zero block."""
    rng = np.random.default_rng(13)
    # (a) identity for power-of-two scales, 3 matrices x 5 rows x 128 columns
    M, R, C = 3, 5, 128
    codes = rng.integers(0, 16, size=(M, R, C)).astype(np.uint8)
    codes[:, :, ::32] = 7                                  # a +6 in every block
    a = rng.integers(-6, 9, size=(M, R, C // 32))          # UE4M3 2^a: exponent field a + 7
    sc16 = np.repeat(((a + 7) << 3).astype(np.uint8), 2, axis=2)
    bexp = np.array([0, -20, 9])
    g = np.ldexp(1.0, bexp).astype(np.float32)
    packed = (codes[:, :, 0::2] | (codes[:, :, 1::2] << 4)).astype(np.uint8)
    oc, osc = O.nvfp4_to_mxfp4(packed, sc16, g)
    # negative zero (code 8) re-encodes as +0 (code 0); everything else is unchanged
    want = np.where(codes == 8, 0, codes)
    assert np.array_equal(unpack4(oc).reshape(M, R, C), want)
    assert np.array_equal(osc, (a + bexp[:, None, None] + 127).astype(np.uint8))

    def one(c32, s0, s1, gm=1.0):
        pk, s = nvfp4_block(c32, s0, s1)
        o, os_ = O.nvfp4_to_mxfp4(pk.reshape(1, 1, 16), s.reshape(1, 1, 2), np.array([gm], np.float32))
        return unpack4(o), int(os_.ravel()[0])

    # (b1) half 0 at 2^2 (code 0x48) holding 6 -> amax 24, X = 4 - 2 = 2; half 1 at
    # 2^1 (0x40): value c * 2 / 2^2 = c / 2, so 6 -> 3 (code 5), 4 -> 2 (4), 2 -> 1 (2),
    # 1 -> 0.5 (1), 0.5 -> 0.25 = tie -> 0 (even), -3 -> -1.5 (code 11)
    c = [7, 1, 2] + [0] * 13 + [7, 6, 4, 2, 1, 13] + [0] * 10
    got, sc = one(c, 0x48, 0x40)
    assert sc == 127 + 2
    assert list(got[:3]) == [7, 1, 2] and list(got[16:22]) == [5, 4, 2, 1, 0, 11]
    # (b2) scale 1.5 (0x3C) on both halves: amax 6 * 1.5 = 9, X = 3 - 2 = 1; elements
    # v / 2: 6 -> 4.5 -> 4 (code 6); 1.5 -> 1.125 -> 1 (2); 3 -> 2.25 -> 2 (4);
    # 4 -> 3 (5); 0.5 -> 0.375 -> 0.5 (1); 1 -> 0.75 = tie -> 1 (2, even); 2 -> 1.5 (3)
    c = [7, 3, 5, 6, 1, 2, 4] + [0] * 25
    got, sc = one(c, 0x3C, 0x3C)
    assert sc == 128 and list(got[:7]) == [6, 2, 4, 5, 1, 2, 3]
    # (b3) FP32 products on ties of the grid: g = the float just above 5/6
    # (0x1.aaaaacp-1, 5/6 + 2^-24 * 2/3), scale 1.0. Code 7 (6) gives 6g = 5 + 2.4e-7,
    # which FP32 rounds to 5.0: amax 5 -> X = 0, and 5 is a tie between 4 (code 6,
    # even) and 6 (code 7) -> 6. Code 5 (3) gives 3g = 2.5 + 1.2e-7 -> 2.5 in FP32, a
    # tie between 2 (code 4, even) and 3 (code 5) -> 4. (Formed in double both would
    # sit above their ties and give 7 and 5.)
    gm = np.float32(float.fromhex("0x1.aaaaacp-1"))
    c = [7, 5] + [0] * 30
    got, sc = one(c, 0x38, 0x38, gm)
    assert sc == 127 and got[0] == 6 and got[1] == 4
    # (b4) NaN scale (0x7F, also with the ignored top bit 0xFF), non-finite matrix
    # scale, FP32 overflow -> E8M0 NaN (0xFF) and zero codes
    for s0, s1, gmv in ((0x7F, 0x38, 1.0), (0x38, 0xFF, 1.0), (0x38, 0x38, np.inf),
                        (0x38, 0x38, np.nan), (0x7E, 0x7E, 3.0e38)):
        got, sc = one([7] * 32, s0, s1, gmv)
        assert sc == 255 and not got.any(), (s0, s1, gmv)
    # top bit of a finite scale byte is ignored: 0xB8 acts as 0x38
    g1, s1_ = one([7, 1] + [0] * 30, 0xB8, 0xB8)
    g2, s2_ = one([7, 1] + [0] * 30, 0x38, 0x38)
    assert s1_ == s2_ == 127 and np.array_equal(g1, g2)
    # (b5) all-zero block (+0 and -0 codes): smallest scale, zero codes
    got, sc = one([0, 8] * 16, 0x38, 0x38)
    assert sc == 0 and not got.any()
    # (b6) FP32 subnormals, also with flush-to-zero / denormals-are-zero switched on
    # in the calling thread (as a fast-math library loaded into the process does):
    # g = 2^-126, scale 1: 6 g = 6 * 2^-126 -> X = -126 + 2 - 2 = -126; 0.5 g = 2^-127
    # (a subnormal product) / 2^-126 = 0.5 -> code 1. g = 2^-130 (a subnormal input):
    # 6 g -> X = -130 clamped to -127, 6 * 2^-130 / 2^-127 = 0.75 -> 1.0 (code 2, tie
    # to even); 4 g / 2^-127 = 0.5 -> code 1.
    # (the matrix scales are made from their bit patterns, before the modes change)
    g126, g130 = np.array([0x00800000, 0x00080000], np.uint32).view(np.float32)
    assert float(g126) == 2.0 ** -126 and float(g130) == 2.0 ** -130
    for flush in (0, 1):
        O.lib.orc_set_flush_modes(flush)
        try:
            got, sc = one([7, 1] + [0] * 30, 0x38, 0x38, g126)
            assert sc == 1 and list(got[:2]) == [7, 1], (flush, sc, got[:2])
            got, sc = one([7, 6] + [0] * 30, 0x38, 0x38, g130)
            assert sc == 0 and list(got[:2]) == [2, 1], (flush, sc, got[:2])
        finally:
            O.lib.orc_set_flush_modes(0)


PINS = [pin_bruteforce, pin_bruteforce_mx, pin_dense_e1k1, pin_topk, pin_weights,
        pin_permutation, pin_rms_unit, pin_token_permutation, pin_norm_before_combine,
        pin_pool_norm_invariance, pin_identical_experts, pin_round_bf16, pin_mx_codec,
        pin_nvfp4_requant]
