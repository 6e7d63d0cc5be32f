"""Pins for the oracle's optional sampling settings: frequency and presence
penalties, top-p (nucleus) and synthetic acceptance.  Each is checked against
what the pages print (golden files), closed forms worked out by hand, brute
force on tiny inputs, or the output law over many seeded trials."""
import itertools
import json
import os

import numpy as np
import pytest
from scipy import stats

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
P_MIN = 1e-4


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Frequency and presence penalties
# ---------------------------------------------------------------------------
def test_frequency_penalty_page_example():
    g = golden("frequency_penalty.json")
    f = g["frequency_penalty"]
    z = np.array([2.25, 1.5], np.float32)  # token "the" and a token never sampled
    for step in g["steps"]:
        counts = np.array([step["count"], 0], np.int32)
        out = oracle.frequency_presence_penalty(z, counts, f, 0.0)
        assert out[0] == np.float32(2.25 + step["logit_change"])
        assert out[1] == z[1]


def test_presence_penalty_and_rounding_by_hand():
    z = np.array([1.0, 1.0, 1.0, -3.0], np.float32)
    counts = np.array([0, 1, 7, 3], np.int32)
    # presence alone: a constant for every seen token, whatever its count
    out = oracle.frequency_presence_penalty(z, counts, 0.0, 0.25)
    assert out.tolist() == [1.0, 0.75, 0.75, -3.25]
    # both: 1 - 0.5*7 - 0.25 = -2.75, -3 - 1.5 - 0.25 = -4.75
    out = oracle.frequency_presence_penalty(z, counts, 0.5, 0.25)
    assert out.tolist() == [1.0, 0.25, -2.75, -4.75]
    # fp32 rounding: 0.1f * 3 rounds to 0.3f (0.30000001192...), and 1 - 0.3f = 0.7f
    out = oracle.frequency_presence_penalty(np.array([1.0], np.float32), np.array([3], np.int32),
                                            np.float32(0.1), 0.0)
    assert out[0] == np.float32(0.7)
    # a negative penalty raises the logit
    out = oracle.frequency_presence_penalty(np.array([0.5], np.float32), np.array([2], np.int32), -1.0, -0.5)
    assert out[0] == np.float32(3.0)


def test_penalty_order_repetition_then_frequency_then_presence():
    # z = 2 with theta = 2 -> 1; frequency 0.5 * count 2 -> 0; presence 0.25 -> -0.25.
    # The other token (count 0) keeps z = 0, so p0 / p1 = exp(-0.25) at T = 1.
    rows = np.array([[2.0, 0.0]], np.float32)
    counts = np.array([2, 0], np.int32)
    P, amax, err = oracle.prepare_request(rows, 1.0, theta=2.0, counts=counts, freq=0.5, pres=0.25)
    assert err == 0
    assert P[0, 0] / P[0, 1] == pytest.approx(np.exp(-0.25), rel=1e-12)
    # greedy sees the processed logits too: 0 beats -0.25
    P, amax, err = oracle.prepare_request(rows, 0.0, theta=2.0, counts=counts, freq=0.5, pres=0.25)
    assert amax[0] == 1


def test_penalty_validation():
    rows = np.zeros((1, 4), np.float32)
    counts = np.ones(4, np.int32)
    for f, pr in [(np.nan, 0.0), (0.0, np.inf), (-np.inf, 0.0)]:
        _, _, err = oracle.prepare_request(rows, 1.0, counts=counts, freq=f, pres=pr)
        assert err == oracle.ERR_PENALTY


# ---------------------------------------------------------------------------
# Top-p
# ---------------------------------------------------------------------------
def nucleus_by_enumeration(p, P):
    """Brute force: among the sets 'every token with p >= v' (v over the distinct
    positive values), the smallest whose mass reaches P."""
    best = None
    for v in sorted(set(p[p > 0].tolist()), reverse=True):
        s = p >= v
        if p[s].sum() >= P - 1e-15:
            best = s
            break
    if best is None:
        best = p > 0
    return best


@pytest.mark.parametrize("seed", range(40))
def test_top_p_matches_enumeration_on_tiny_rows(seed):
    rng = np.random.default_rng(seed)
    V = int(rng.integers(1, 9))
    w = rng.integers(1, 6, V).astype(np.float64)  # small integers: ties are common
    w[rng.random(V) < 0.2] = 0.0
    if w.sum() == 0:
        w[0] = 1.0
    p = w / w.sum()
    for P in [1e-6, 0.1, 0.25, 0.5, 0.6, 0.75, 0.9, 0.999]:
        # exact sums of multiples of 1/sum(w): compare on grid points away from exact hits
        keep, margin, n = oracle.top_p_keep(p, P)
        want = nucleus_by_enumeration(p, P)
        if margin > 1e-12:
            assert np.array_equal(keep, want), (p, P, keep, want)
            assert n == want.sum()


def test_top_p_invariants_on_large_rows():
    rng = np.random.default_rng(7)
    p = np.exp(rng.normal(0, 2.0, 5000))
    p /= p.sum()
    order = np.sort(p)[::-1]
    prev_n = 0
    for P in [1e-6, 0.01, 0.3, 0.7, 0.9, 0.99, 1.0]:
        keep, margin, n = oracle.top_p_keep(p, P)
        kept = p[keep]
        assert kept.sum() >= P - 1e-12 or n == p.size
        # dropping the least probable kept token falls below P (no ties here)
        assert kept.sum() - kept.min() < P
        # kept tokens are exactly the n most probable
        assert kept.min() == order[n - 1] and (n == p.size or order[n] < kept.min())
        assert n >= prev_n
        prev_n = n
    assert oracle.top_p_keep(p, 1e-6)[2] == 1


def test_top_p_keeps_ties_at_the_boundary():
    p = np.array([0.4, 0.2, 0.2, 0.2])
    keep, _, n = oracle.top_p_keep(p, 0.5)  # mass above each 0.2 is 0.4 < 0.5: all kept
    assert keep.all() and n == 4
    keep, _, n = oracle.top_p_keep(p, 0.4)  # mass above 0.2 reaches 0.4: only the top
    assert keep.tolist() == [True, False, False, False]


def test_top_p_in_prepare_request_after_temperature():
    # p = (0.5, 0.3, 0.2) at T = 1; top_p = 0.7 keeps the first two, renormalised
    rows = np.log(np.array([[0.5, 0.3, 0.2]])).astype(np.float32)
    P, amax, err, tm = oracle.prepare_request_ex(rows, 1.0, top_p=0.7)
    assert err == 0
    assert P[0, 2] == 0.0 and P[0, 0] / P[0, 1] == pytest.approx(5 / 3, rel=1e-6)
    assert P[0].sum() == pytest.approx(1.0, abs=1e-15)
    # masses above the three values: 0, 0.5, 0.8; the closest to 0.7 is 0.8
    assert tm[0] == pytest.approx(0.1, abs=1e-6)
    # a very high temperature flattens p to thirds: every token's mass above is < 0.7
    P, amax, err, tm = oracle.prepare_request_ex(rows, 1e6, top_p=0.7)
    assert (P[0] > 0).all()
    # clamps: top_p <= 0 acts as 1e-6 (only the argmax), > 1 as no restriction
    P, _, _, _ = oracle.prepare_request_ex(rows, 1.0, top_p=0.0)
    assert P[0].tolist() == [1.0, 0.0, 0.0]
    P, _, _, _ = oracle.prepare_request_ex(rows, 1.0, top_p=3.0)
    assert (P[0] > 0).all()
    _, _, err, _ = oracle.prepare_request_ex(rows, 1.0, top_p=np.nan)
    assert err == oracle.ERR_TOP_P
    # greedy ignores top-p
    P, amax, err, _ = oracle.prepare_request_ex(rows, 0.0, top_p=0.1)
    assert err == 0 and amax[0] == 0


def test_top_p_with_top_k_counts_only_the_kept_tokens():
    # top_k = 2 leaves (0.5, 0.3) -> (0.625, 0.375); top_p = 0.6 then keeps one token
    rows = np.log(np.array([[0.5, 0.3, 0.2]])).astype(np.float32)
    P, _, err, _ = oracle.prepare_request_ex(rows, 1.0, top_k=2, top_p=0.6)
    assert err == 0 and P[0].tolist() == [1.0, 0.0, 0.0]
    P, _, err, _ = oracle.prepare_request_ex(rows, 1.0, top_k=2, top_p=0.7)
    assert P[0, 2] == 0.0 and P[0, 1] > 0.0


def test_sampling_law_with_top_p_two_level_race():
    rng = np.random.default_rng(3)
    V, B = 400, 100_000
    p = np.exp(rng.normal(0, 1.5, V))
    p /= p.sum()
    keep, _, _ = oracle.top_p_keep(p, 0.8)
    want = np.where(keep, p, 0.0)
    want /= want.sum()
    # one bonus-only request per trial; the race uses C = 64 (several chunks)
    logits = np.tile(np.log(p).astype(np.float32), (B, 1))
    cu = np.zeros(B + 1, np.int32)
    o = oracle.verify_batch(logits, cu, np.zeros(0, np.int32), np.ones(B, np.float32),
                            top_p=np.full(B, 0.8, np.float32), C=64, seed=11)
    assert o["err"] == 0
    toks = o["tokens"][:, 0]
    assert keep[toks].all()
    counts = np.bincount(toks, minlength=V)
    # merge small-expectation tokens into one bin for the chi-square
    big = want * B >= 20
    obs = np.append(counts[big], counts[~big].sum())
    exp = np.append(want[big], want[~big].sum()) * B
    keepbin = exp > 0
    assert stats.chisquare(obs[keepbin], exp[keepbin]).pvalue > P_MIN


# ---------------------------------------------------------------------------
# Synthetic acceptance
# ---------------------------------------------------------------------------
def variance_from_rates(a):
    a = np.asarray(a, float)
    i = np.arange(1, a.size + 1)
    mean = a.sum()
    return (2 * i - 1) @ a - mean * mean, mean


def test_synthetic_rates_from_length_closed_forms():
    K = 4
    assert oracle.synthetic_rates(1.0, K).tolist() == [0, 0, 0, 0]
    assert oracle.synthetic_rates(5.0, K).tolist() == [1, 1, 1, 1]
    assert oracle.synthetic_rates(2.5, K).tolist() == [1, 0.5, 0, 0]
    assert oracle.synthetic_rates(3.75, K).tolist() == [1, 1, 0.75, 0]
    for L in [0.99, 5.01, np.nan, np.inf]:
        with pytest.raises(ValueError):
            oracle.synthetic_rates(L, K)


def test_synthetic_rates_have_minimum_variance_by_brute_force():
    K, grid = 3, np.linspace(0, 1, 9)
    for L in [1.25, 1.5, 2.0, 2.75, 3.5, 4.0]:
        best = np.inf
        for a in itertools.product(grid, repeat=K):
            if all(a[i] >= a[i + 1] for i in range(K - 1)) and abs(sum(a) - (L - 1)) < 1e-12:
                best = min(best, variance_from_rates(a)[0])
        var, mean = variance_from_rates(oracle.synthetic_rates(L, K))
        assert mean == pytest.approx(L - 1, abs=1e-7)
        assert var == pytest.approx(best, abs=1e-7)


def synthetic_trials(rates, B=200_000, T=1.0, seed=5):
    K = len(rates)
    V = 50
    rng = np.random.default_rng(1)
    logits = np.tile(rng.normal(0, 1, (K + 1, V)).astype(np.float32), (B, 1))
    cu = (np.arange(B + 1) * K).astype(np.int32)
    d = np.tile(np.arange(K, dtype=np.int32) + 3, B)
    return oracle.verify_batch(logits, cu, d, np.full(B, T, np.float32), seed=seed,
                               synthetic_rates=np.asarray(rates, np.float32))


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_synthetic_acceptance_law(T):
    rates = [0.9, 0.6, 0.6, 0.2]
    B = 200_000
    o = synthetic_trials(rates, B, T)
    assert o["err"] == 0
    acc = o["num_sampled"] - 1
    a = np.array([1.0] + rates + [0.0])
    pmf = a[:-1] - a[1:]  # P(N = n) = a_n - a_{n+1}
    obs = np.bincount(acc, minlength=5)
    assert obs[pmf == 0].sum() == 0
    assert stats.chisquare(obs[pmf > 0], pmf[pmf > 0] * B).pvalue > P_MIN
    # accepted positions output the drafts themselves
    k = len(rates)
    for r in range(0, B, 997):
        n = acc[r]
        assert o["tokens"][r, :n].tolist() == list(range(3, 3 + n))


def test_synthetic_extremes_and_greedy_recovered_token():
    o = synthetic_trials([1.0, 1.0, 1.0], B=500)
    assert (o["num_sampled"] == 4).all() and (o["num_rejected"] == 0).all()
    o = synthetic_trials([0.0, 0.0, 0.0], B=500)
    assert (o["num_sampled"] == 1).all()
    # greedy: the token after the accepted drafts is the argmax of that row
    rng = np.random.default_rng(1)
    rows = rng.normal(0, 1, (4, 50)).astype(np.float32)
    o = synthetic_trials([0.5, 0.5, 0.5], B=300, T=0.0)
    for r in range(300):
        n = o["num_sampled"][r]
        assert o["tokens"][r, n - 1] == int(np.argmax(rows[n - 1]))
    # invalid draft ids are rejected even at rate 1
    P, amax, _ = oracle.prepare_request(rows, 1.0)
    toks, ns, nr, _, _ = oracle.decide_request(P, amax, 1.0, np.array([3, -1, 4]), synthetic_rates=[1, 1, 1])
    assert ns == 2 and toks[0] == 3
