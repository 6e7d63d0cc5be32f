"""Pins of the oracle's decision margins, the numbers that decide which
GPU/oracle differences the parity tests excuse.

- An accept test's margin is |p - u q| / max(p, u q).
- A race level's margin is 1 - s2 / s1 over its two best scores (1 when it
  has a single candidate).
- A request's margin is the smallest over the accept tests it ran and both
  levels of its race.

The inputs are built so that the expected margin is known by construction.
The accept uniform u and the race noise E are the oracle's own draws, and its
Philox stream and uniform grids are pinned separately (test_oracle_pins.py).
The probabilities and race weights are then exact multiples of those draws,
so that u q, or each score w / E, takes a chosen value.  A slip that reads the
wrong side of the max, the second score of the other level, the uniform of
another position, or that combines the levels with max instead of min,
changes the value and fails here.
"""
import math

import numpy as np
import pytest

import oracle

SEED = 0x5EED5EED12345
TAG_ACCEPT, TAG_CHUNK, TAG_TOKEN = oracle.TAG_ACCEPT, oracle.TAG_CHUNK, oracle.TAG_TOKEN


def u_acc(seed, offset, g):
    return oracle.uniform_accept(oracle.word(seed, offset, g, TAG_ACCEPT, 0))


def find_offset(pred, seed=SEED, start=0):
    """First call offset whose draws satisfy pred(offset) (the draws are fixed
    by the pinned stream, so the search is deterministic)."""
    for off in range(start, start + 100000):
        if pred(off):
            return off
    raise AssertionError("no offset found")


def test_exp_noise_is_minus_log_of_the_race_uniform():
    # S2 of the spec: E = -ln U on the race grid (library log of the pinned uniform).
    for g, tag, idx, off in [(0, 1, 0, 0), (3, 2, 77, 5), (1000, 1, 125, 9), (12, 2, 4095, 1)]:
        u = oracle.uniform_race(oracle.word(SEED, off, g, tag, idx))
        assert u > 0.0
        assert oracle.exp_noise(SEED, off, g, tag, idx) == -math.log(u)


# ---------------------------------------------------------------------------
# Accept margins (no-draft-probs mode: q = 1; draft-probs mode: q = q(d))
# ---------------------------------------------------------------------------
def test_accept_margins_by_construction_no_draft():
    # Request K = 2 at target rows g0, g0+1 (bonus g0+2), V = 4, drafts 1 and 2.
    # Row 0: p(d0) = 1.5 u0    -> accepted, margin |1.5u - u| / 1.5u = 1/3.
    # Row 1: p(d1) = 0.5 u1    -> rejected, margin |0.5u - u| / u   = 1/2.
    # The recovered race over row 1 without d1 has one candidate (token 3): 1.
    # Request margin: 1/3.  With the denominator min(p, u q) instead it would be 1/2.
    g0 = 10
    off = find_offset(lambda o: u_acc(SEED, o, g0) <= 0.6)
    u0, u1 = u_acc(SEED, off, g0), u_acc(SEED, off, g0 + 1)
    a, b = 1.5 * u0, 0.5 * u1
    P = np.array([[0.0, a, 1.0 - a, 0.0],
                  [0.0, 0.0, b, 1.0 - b],
                  [0.0, 0.0, 0.0, 1.0]])
    toks, ns, nr, mg, pd = oracle.decide_request(P, [1, 2, 3], 1.0, [1, 2], None, g0, SEED, off)
    assert (toks, ns, nr) == ([1, 3], 2, 1)
    assert mg == pytest.approx(1.0 / 3.0, rel=1e-14)
    assert pd.tolist() == [np.float32(a), np.float32(b)]


def test_accept_margin_uses_each_positions_own_uniform():
    # Same layout, row 1 accepted at p = 1.25 u1 (margin 0.2) while row 0 has
    # margin 1/3: the request margin 0.2 needs u1, not u0, at position 1.
    g0 = 40
    off = find_offset(lambda o: u_acc(SEED, o, g0) <= 0.6 and u_acc(SEED, o, g0 + 1) <= 0.7
                      and abs(u_acc(SEED, o, g0) - u_acc(SEED, o, g0 + 1)) > 0.05)
    u0, u1 = u_acc(SEED, off, g0), u_acc(SEED, off, g0 + 1)
    a, b = 1.5 * u0, 1.25 * u1
    P = np.array([[0.0, a, 1.0 - a, 0.0],
                  [0.0, 0.0, b, 1.0 - b],
                  [1.0, 0.0, 0.0, 0.0]])
    toks, ns, nr, mg, _ = oracle.decide_request(P, [1, 2, 0], 1.0, [1, 2], None, g0, SEED, off)
    assert (toks, ns, nr) == ([1, 2, 0], 3, 0)  # bonus row has one token: race margin 1
    assert mg == pytest.approx(0.2, rel=1e-14)


def test_accept_margin_exact_tie_is_zero_and_accepted():
    # p(d) = u exactly (q = 1): the boundary p >= u q accepts, margin 0.
    g0 = 3
    off = find_offset(lambda o: 0.1 < u_acc(SEED, o, g0) < 0.9)
    u0 = u_acc(SEED, off, g0)
    P = np.array([[0.0, u0, 1.0 - u0], [0.0, 0.0, 1.0]])
    toks, ns, nr, mg, _ = oracle.decide_request(P, [1, 2], 1.0, [1], None, g0, SEED, off)
    assert (toks, ns, nr) == ([1, 2], 2, 0)
    assert mg == 0.0
    # one ulp below: rejected, margin one ulp relative
    below = np.nextafter(u0, 0.0)
    P[0, 1], P[0, 2] = below, 1.0 - below
    toks, ns, nr, mg, _ = oracle.decide_request(P, [1, 2], 1.0, [1], None, g0, SEED, off)
    assert (toks, ns, nr) == ([2], 1, 1)
    assert mg == pytest.approx((u0 - below) / u0, rel=1e-12) and 0.0 < mg < 1e-15


def test_accept_margin_with_draft_probs():
    # Draft-probs mode: q(d) = 0.5, p(d) = 0.75 u q -> rejected, margin 0.25.
    # Residual max(0, p - q) has one positive token (1): race margin 1.
    g0 = 21
    off = find_offset(lambda o: u_acc(SEED, o, g0) > 0.2)
    u0 = u_acc(SEED, off, g0)
    pd = 0.75 * u0 * 0.5
    P = np.array([[pd, 1.0 - pd, 0.0], [0.0, 0.0, 1.0]])
    Q = np.array([[0.5, 0.25, 0.25]], dtype=np.float32)
    toks, ns, nr, mg, _ = oracle.decide_request(P, [1, 2], 1.0, [0], Q, g0, SEED, off)
    assert (toks, ns, nr) == ([1], 1, 1)
    assert mg == pytest.approx(0.25, rel=1e-14)
    # q(d) = 0 rejects before any comparison: no accept margin, only the race's.
    # Residual (0, 0.5, 0): one candidate.
    Q0 = np.array([[0.0, 0.5, 0.5]], dtype=np.float32)
    P0 = np.array([[0.0, 1.0, 0.0], [0.0, 0.0, 1.0]])
    toks, ns, nr, mg, _ = oracle.decide_request(P0, [1, 2], 1.0, [0], Q0, g0, SEED, off)
    assert (toks, ns, nr) == ([1], 1, 1) and mg == 1.0


# ---------------------------------------------------------------------------
# Race margins at both levels
# ---------------------------------------------------------------------------
def E(off, g, tag, idx):
    e = oracle.exp_noise(SEED, off, g, tag, idx)
    assert math.isfinite(e) and e > 0.0
    return e


@pytest.mark.parametrize("scores", [(3.0, 2.0, 1.0), (2.0, 3.0, 1.0), (1.0, 2.0, 3.0)])
def test_flat_race_margin_and_winner(scores):
    # One chunk (C >= V): the chunk level has one candidate (margin 1); token
    # scores 3, 2, 1 (in every position order) give margin 1 - 2/3.
    g, off, V = 5, 11, 8
    w = np.zeros(V)
    xs = (1, 3, 4)
    for x, s in zip(xs, scores):
        w[x] = s * E(off, g, TAG_TOKEN, x)
    x, mg = oracle.race(w, V, SEED, off, g)
    assert x == xs[scores.index(3.0)]
    assert mg == pytest.approx(1.0 / 3.0, rel=1e-14)


@pytest.mark.parametrize("rho,winner,margin", [(0.9, 1, 0.1), (0.5, 1, 0.2), (1.0 / 0.7, 6, 0.3),
                                               (0.97, 1, 0.03)])
def test_two_level_race_margin(rho, winner, margin):
    # C = 4, V = 12.  Chunk 0 holds tokens 1 and 2 with token scores 5 and 4
    # (token-level margin 0.2 if chunk 0 wins); chunk 1 holds token 6 alone,
    # weighted so its chunk score is rho times chunk 0's; chunk 2 is empty.
    # Request margin: min(chunk-level 1 - s2/s1, token-level margin of the
    # winning chunk).
    C, V, g, off = 4, 12, 7, 2
    w = np.zeros(V)
    w[1] = 5.0 * E(off, g, TAG_TOKEN, 1)
    w[2] = 4.0 * E(off, g, TAG_TOKEN, 2)
    S0 = (w[1] + w[2]) / E(off, g, TAG_CHUNK, 0)
    w[6] = rho * S0 * E(off, g, TAG_CHUNK, 1)
    x, mg = oracle.race(w, C, SEED, off, g)
    assert x == winner
    assert mg == pytest.approx(margin, rel=1e-12)


def test_race_margin_single_candidates_ties_and_empty():
    g, off = 9, 4
    # one chunk with weight, one token in it: margin 1 at both levels
    w = np.zeros(16)
    w[13] = 0.25
    assert oracle.race(w, 4, SEED, off, g) == (13, 1.0)
    # equal token scores: margin 0, the lower index wins
    w = np.zeros(4)
    w[1] = 2.0 * E(off, g, TAG_TOKEN, 1)
    w[3] = 2.0 * E(off, g, TAG_TOKEN, 3)
    assert oracle.race(w, 4, SEED, off, g) == (1, 0.0)
    # no weight anywhere: no winner
    assert oracle.race(np.zeros(8), 4, SEED, off, g)[0] == -1


def test_request_margin_takes_the_race_margin_of_the_sampled_row():
    # Bonus-only request (K = 0, row g0): its margin is the bonus race's,
    # built with token scores 3 and 2 (margin 1/3) inside the one chunk.
    g0, off, V = 17, 6, 6
    w = np.zeros(V)
    w[2] = 3.0 * E(off, g0, TAG_TOKEN, 2)
    w[5] = 2.0 * E(off, g0, TAG_TOKEN, 5)
    P = (w / w.sum())[None, :]
    toks, ns, nr, mg, _ = oracle.decide_request(P, [2], 1.0, [], None, g0, SEED, off)
    assert (toks, ns, nr) == ([2], 1, 0)
    assert mg == pytest.approx(1.0 / 3.0, rel=1e-13)
    # A rejected draft (no-draft mode) followed by the recovered race: the
    # request margin is the smaller of the accept margin (1/2) and the race's (1/3).
    u0 = u_acc(SEED, off, g0)
    P2 = np.zeros((2, V))
    P2[0, 0] = 0.5 * u0
    rest = (1.0 - P2[0, 0])
    w2 = np.zeros(V)
    w2[2] = 3.0 * E(off, g0, TAG_TOKEN, 2)
    w2[5] = 2.0 * E(off, g0, TAG_TOKEN, 5)
    P2[0] += w2 / w2.sum() * rest
    P2[1, 4] = 1.0
    toks, ns, nr, mg, _ = oracle.decide_request(P2, [2, 4], 1.0, [0], None, g0, SEED, off)
    assert (toks, ns, nr) == ([2], 1, 1)
    assert mg == pytest.approx(1.0 / 3.0, rel=1e-12)


def test_draft_sampler_margin_by_construction():
    # Draft-side race (tags 3 and 4) over q = softmax(z): z = ln(s_x E_x) on
    # two tokens (others -inf), so the token scores are s = 4 and 3 up to the
    # fp32 rounding of z: margin 1/4 within 1e-5.
    key, off, V = 33, 8, 10
    e = lambda x: oracle.exp_noise(SEED, off, key, oracle.TAG_DRAFT_TOKEN, x)
    z = np.full(V, -np.inf, dtype=np.float32)
    z[2] = np.float32(math.log(4.0 * e(2)))
    z[7] = np.float32(math.log(3.0 * e(7)))
    d, q, mg = oracle.draft_sample(z, 1.0, SEED, off, key, C=1024)
    assert d == 2
    assert mg == pytest.approx(0.25, abs=1e-5)
    w = np.exp(z.astype(np.float64) - np.max(z))
    assert q == pytest.approx(w[2] / w.sum(), rel=1e-12)
