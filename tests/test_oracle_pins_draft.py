"""Pins for the oracle's draft-side sampling: the law of the sampled draft
tokens, the greedy case, q(d), the separation of its noise from the
verifier's, and the end-to-end property that drafting with it and verifying
against the same draft distributions leaves the target law unchanged."""
import numpy as np
import pytest
from scipy import special, stats

import oracle

P_MIN = 1e-4


def chi2_p(counts, p):
    keep = p * counts.sum() >= 5
    obs = np.append(counts[keep], counts[~keep].sum())
    exp = np.append(p[keep], p[~keep].sum()) * counts.sum()
    m = exp > 0
    assert counts[p == 0].sum() == 0
    return stats.chisquare(obs[m], exp[m]).pvalue


def test_draft_tokens_follow_q():
    rng = np.random.default_rng(2)
    V, T, N = 300, 0.8, 60_000
    z = rng.normal(0, 1.5, V).astype(np.float32)
    q = special.softmax(z.astype(np.float64) / T)
    counts = np.zeros(V, np.int64)
    for key in range(N):
        d, qd, _ = oracle.draft_sample(z, T, seed=9, offset=3, key=key, C=64)
        counts[d] += 1
    assert chi2_p(counts, q) > P_MIN


def test_draft_q_token_and_greedy():
    rng = np.random.default_rng(3)
    z = rng.normal(0, 2.0, 1000).astype(np.float32)
    q = special.softmax(z.astype(np.float64) / float(np.float32(1.3)))  # T is passed as fp32
    for key in range(20):
        d, qd, mg = oracle.draft_sample(z, 1.3, seed=1, offset=0, key=key, C=128)
        assert qd == pytest.approx(q[d], rel=1e-12)
    d, qd, mg = oracle.draft_sample(z, 0.0, seed=1, offset=0, key=0)
    assert d == int(np.argmax(z)) and qd == 1.0 and mg == np.inf
    # bf16 rows are widened like the target rows
    bits = (np.arange(16, dtype=np.uint16) + 0x3F80)
    d, _, _ = oracle.draft_sample(bits, 0.0, 0, 0, 0)
    assert d == 15


def test_draft_noise_is_not_the_verifiers():
    # Same weights, same counter row: the draft race (tags 3, 4) and the
    # verifier's race (tags 1, 2) agree only as often as two independent draws.
    rng = np.random.default_rng(4)
    w = rng.random(64) ** 4
    q = w / w.sum()
    N = 20_000
    same = 0
    for key in range(N):
        a, _ = oracle.race(w, 16, 5, 0, key)
        b, _ = oracle.race_tags(w, 16, 5, 0, key, oracle.TAG_DRAFT_CHUNK, oracle.TAG_DRAFT_TOKEN)
        same += a == b
    assert stats.binomtest(same, N, float(q @ q)).pvalue > P_MIN
    # The draft sampler itself: its token for draft row `key` against the
    # verifier's race of target row `key` over the same q.
    z = np.log(w).astype(np.float32)
    qz = oracle.softmax(z, 1.0)
    N2 = 4000
    same = sum(oracle.draft_sample(z, 1.0, 5, 0, key, C=16)[0] == oracle.race(qz, 16, 5, 0, key)[0]
               for key in range(N2))
    assert stats.binomtest(int(same), N2, float(qz @ qz)).pvalue > P_MIN


def test_drafting_then_verifying_keeps_the_target_law():
    # Two draft positions drawn from q_0, q_1 with the draft sampler, verified
    # against the same q rows: the first output token follows p_0, and after an
    # accepted first draft the second output follows p_1 (speculative sampling).
    rng = np.random.default_rng(5)
    V, K, N = 12, 2, 40_000
    zp = rng.normal(0, 1.0, (K + 1, V)).astype(np.float32)
    zq = (zp[:K] + rng.normal(0, 0.8, (K, V))).astype(np.float32)
    P, amax, err = oracle.prepare_request(zp, 1.0)
    assert err == 0
    Q = oracle.draft_q_rows(zq, 1.0)
    first = np.zeros(V, np.int64)
    second = np.zeros(V, np.int64)
    for t in range(N):
        d = [oracle.draft_sample(zq[i], 1.0, seed=77, offset=t, key=i, C=4)[0] for i in range(K)]
        toks, ns, nr, mg, _ = oracle.decide_request(P, amax, 1.0, np.array(d, np.int32), g0=0, seed=77,
                                                    offset=t, C=4, draft_q64=Q)
        first[toks[0]] += 1
        if ns >= 2:
            second[toks[1]] += 1
    assert chi2_p(first, P[0]) > P_MIN
    # given the first output, the second position's output follows p_1
    assert chi2_p(second, P[1]) > P_MIN
