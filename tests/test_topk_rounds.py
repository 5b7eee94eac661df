"""Host model of the top-k kernel's selection rounds, run on the CPU.

topk_kernel (csrc/route.hip) gives each token one wave of 64 lanes. Lane L
holds the scores of experts q*64 + L for q < 16 (NaN read as -inf; slots past
E marked taken). In each of k rounds every lane offers its best untaken slot,
the wave maximum of the offers is taken, a ballot finds the lanes whose offer
equals it, and the lowest expert index among them wins. This module replays
those rounds lane by lane with the kernel's candidate rule and checks, on rows
of NaN, -inf and +inf, that every round picks a valid untaken expert and that
ids and weights equal the oracle's (selection by score, NaN as -inf, ties to
the lower index; softmax weights, equal shares when the largest selected score
is infinite).

It also replays the rule the kernel had before: a lane offered a slot only if
its score was above -inf. On a row with fewer than k scores above -inf no lane
then has an offer, the ballot is empty, and the round's winner stays the
"none" index 0x7FFFFFFF, which the kernel would have stored as an expert id
and used to index the chunk masks. The test shows that failure on the model,
so the fixed rule is shown on the CPU before it runs on a GPU.
"""
import numpy as np
import pytest

import oracle

NONE = 0x7FFFFFFF
WAVE, MAX_PER_LANE = 64, 16


def emulate(row, k, offer_any_untaken=True):
    """ids [k] and float32 weights [k] as the kernel's rounds produce them; a
    round that finds no winner leaves NONE (and the rest of the row unset)."""
    E = len(row)
    per = (E + WAVE - 1) // WAVE
    v = np.full((MAX_PER_LANE, WAVE), -np.inf, np.float32)
    taken = np.zeros((MAX_PER_LANE, WAVE), bool)
    for q in range(MAX_PER_LANE):
        for lane in range(WAVE):
            e = q * WAVE + lane
            ok = q < per and e < E
            x = np.float32(row[min(e, E - 1)])
            v[q, lane] = -np.inf if (not ok or np.isnan(x)) else x
            taken[q, lane] = not ok
    ids = np.full(k, NONE, np.int64)
    sel = np.zeros(k, np.float32)
    top = np.float32(0)
    den = np.float32(0)
    n_top = 0
    for j in range(k):
        bv = np.full(WAVE, -np.inf, np.float32)
        bi = np.full(WAVE, NONE, np.int64)
        for lane in range(WAVE):
            for q in range(MAX_PER_LANE):         # ascending q: ties keep the lower index
                if taken[q, lane]:
                    continue
                first = offer_any_untaken and bi[lane] == NONE
                if first or v[q, lane] > bv[lane]:
                    bv[lane] = v[q, lane]
                    bi[lane] = q * WAVE + lane
        vmax = bv.max()                            # the DPP wave maximum
        tie = [l for l in range(WAVE) if bi[l] != NONE and bv[l] == vmax]   # the ballot
        win = min((bi[l] for l in tie), default=NONE)
        if win == NONE:
            return ids, None                       # the kernel would go on with an invalid id
        taken[win >> 6, win & 63] = True
        if j == 0:
            top = vmax
        with np.errstate(invalid="ignore"):
            den = np.float32(den + np.exp(np.float32(vmax - top)))
        n_top += int(vmax == top)
        ids[j] = win
        sel[j] = vmax
    if np.isinf(top):
        w = np.where(sel == top, np.float32(1) / np.float32(n_top), np.float32(0)).astype(np.float32)
    else:
        w = (np.exp(sel - top) / den).astype(np.float32)
    return ids, w


def rows(E, k, rng):
    nan, inf = np.float32(np.nan), np.float32(np.inf)
    l = rng.standard_normal((10, E)).astype(np.float32)
    l[0] = nan                                      # a NaN in the token's x row
    l[1] = -inf                                     # every expert biased to -inf
    l[2, : E - k + 1] = -inf                        # only k - 1 finite logits
    l[3, rng.choice(E, E // 2, replace=False)] = nan
    l[4, 3 % E] = inf
    l[5, [1 % E, E - 1]] = inf
    l[6, ::2] = -inf
    l[6, 1::3] = nan
    l[7, : E - 1] = nan
    l[8] = np.float32(0.5)                          # all tied
    return l


CASES = [(8, 2), (16, 5), (64, 8), (256, 8), (70, 16), (1000, 16), (5, 5), (1, 1)]


@pytest.mark.parametrize("E,k", CASES)
def test_fixed_rounds_match_oracle(E, k):
    rng = np.random.default_rng(E * 31 + k)
    l = rows(E, k, rng)
    ids_ref, w_ref = oracle.default().topk_softmax(l, k)
    for t in range(l.shape[0]):
        ids, w = emulate(l[t], k)
        assert w is not None, f"row {t}: a round found no winner"
        assert np.all((ids >= 0) & (ids < E)) and len(set(ids.tolist())) == k
        assert np.array_equal(ids, ids_ref[t]), (t, ids, ids_ref[t])
        assert np.abs(w.astype(np.float64) - w_ref[t]).max() <= 1e-6, (t, w, w_ref[t])


@pytest.mark.parametrize("E,k", [(8, 2), (256, 8), (70, 16)])
def test_previous_rule_fails_on_minus_inf_rows(E, k):
    """The rule before the fix: rows with fewer than k scores above -inf end a
    round with no winner (the invalid id); rows with at least k finite scores
    were unaffected."""
    rng = np.random.default_rng(7)
    l = rows(E, k, rng)
    for t in (0, 1, 2):                            # all NaN, all -inf, k - 1 finite
        ids, w = emulate(l[t], k, offer_any_untaken=False)
        assert w is None and NONE in ids.tolist()
    ids_ref, _ = oracle.default().topk_softmax(l[9:10], k)
    ids, w = emulate(l[9], k, offer_any_untaken=False)
    assert w is not None and np.array_equal(ids, ids_ref[0])
