"""Pins for the CPU oracle: facts the pages and the mathematics fix, checked
against the oracle's own code paths (never against a retyped copy of them).

Each worked example is loaded from tests/golden/*.json, which carries the
citation of the page and section it comes from.
"""
import json
import os

import numpy as np
import pytest
from scipy import special, stats

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TRIALS = 1_000_000
P_MIN = 1e-4  # chi-square / binomial p-value floor (inputs are seeded: no flakiness)


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Random stream
# ---------------------------------------------------------------------------
def test_philox_known_answer_vectors():
    # Known-answer vectors published with the Philox reference implementation
    # (Salmon et al., SC'11, Random123 distribution, philox4x32 with 10 rounds).
    kat = [
        ([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
        ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
        ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
         [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
    ]
    for ctr, key, want in kat:
        assert oracle.philox4x32_10(ctr, key).tolist() == want


def test_counter_layout_selects_word():
    seed = 0x0123456789ABCDEF
    for g, tag, idx, off in [(0, 0, 0, 0), (7, 1, 5, 3), (123456, 2, 1023, 99), (5, 2, 4095, 0)]:
        block = oracle.philox4x32_10([idx >> 2, g, tag, off], [seed & 0xFFFFFFFF, seed >> 32])
        assert oracle.word(seed, off, g, tag, idx) == int(block[idx & 3])


def test_uniform_grid_endpoints():
    assert oracle.uniform_accept(0) == 2.0 ** -24
    assert oracle.uniform_accept(0xFF) == 2.0 ** -24
    assert oracle.uniform_accept(0xFFFFFFFF) == 1.0
    assert oracle.uniform_race(0xFF) == 0.0
    assert oracle.uniform_race(0x100) == 2.0 ** -24
    assert oracle.uniform_race(0xFFFFFFFF) == 1.0 - 2.0 ** -24


def test_uniforms_are_uniform():
    # 2^16 words: the top-24-bit uniforms pass a 64-bin chi-square and a KS test.
    w = np.array([oracle.word(7, 0, g, 0, 0) for g in range(1 << 14)], dtype=np.uint64)
    u = np.array([oracle.uniform_race(int(x)) for x in w])
    counts = np.bincount((u * 64).astype(int), minlength=64)
    assert stats.chisquare(counts).pvalue > P_MIN
    assert stats.kstest(u, "uniform").pvalue > P_MIN


# ---------------------------------------------------------------------------
# Logit processing
# ---------------------------------------------------------------------------
def test_bf16_conversion_bit_patterns():
    bits = [0x3F80, 0xC000, 0x7F80, 0xFF80, 0x0000, 0x8000, 0x3F81, 0x0001]
    want = np.array([1.0, -2.0, np.inf, -np.inf, 0.0, -0.0, 1.0078125, 2.0 ** -133],
                    dtype=np.float32)
    got = oracle.bf16_to_f32(bits)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_softmax_matches_library_and_closed_forms():
    rng = np.random.default_rng(1)
    for V, T in [(7, 1.0), (1000, 0.7), (32000, 1.3)]:
        z = (rng.standard_normal(V) * 3).astype(np.float32)
        p = oracle.softmax(z, T)
        ref = special.softmax(z.astype(np.float64) / T)
        assert np.max(np.abs(p - ref)) < 1e-15
        assert abs(p.sum() - 1.0) < 1e-12
    # uniform logits -> 1/V; a -inf logit gets probability 0
    assert np.allclose(oracle.softmax(np.full(10, 3.5, np.float32), 0.5), 0.1, atol=1e-15)
    z = np.array([0.0, -np.inf, 0.0], np.float32)
    assert oracle.softmax(z, 1.0).tolist() == [0.5, 0.0, 0.5]
    # two logits a, b: p = logistic((a-b)/T)
    p = oracle.softmax(np.array([1.0, 3.0], np.float32), 2.0)
    assert abs(p[0] - 1.0 / (1.0 + np.exp(1.0))) < 1e-15
    with pytest.raises(ValueError):
        oracle.softmax(np.full(4, -np.inf, np.float32), 1.0)


def test_top_k_threshold_and_ties():
    z = np.array([1.0, 3.0, 3.0, 2.0, 5.0], np.float32)
    assert oracle.kth_largest(z, 1) == 5.0
    assert oracle.kth_largest(z, 2) == 3.0
    assert oracle.kth_largest(z, 3) == 3.0
    assert oracle.kth_largest(z, 4) == 2.0
    m = oracle.top_k_mask(z, 2)  # ties with the 2nd largest are all kept
    assert m.tolist() == [-np.inf, 3.0, 3.0, -np.inf, 5.0]
    assert oracle.top_k_mask(z, 0).tolist() == z.tolist()   # k < 1: whole vocabulary
    assert oracle.top_k_mask(z, 5).tolist() == z.tolist()   # k >= V: whole vocabulary
    rng = np.random.default_rng(2)
    for k in (1, 50, 999):
        zr = rng.standard_normal(151936).astype(np.float32)
        tau = np.partition(zr, zr.size - k)[zr.size - k]
        assert oracle.kth_largest(zr, k) == tau
        assert np.count_nonzero(np.isfinite(oracle.top_k_mask(zr, k))) == np.count_nonzero(zr >= tau)


def test_argmax_lowest_index_wins_ties():
    assert oracle.argmax(np.array([0, 2, 1, 2, 2], np.float32)) == 1
    assert oracle.argmax(np.array([-np.inf, -1, -1], np.float32)) == 1
    rng = np.random.default_rng(3)
    zr = rng.integers(-3, 4, 5000).astype(np.float32)
    assert oracle.argmax(zr) == int(np.argmax(zr))


def test_repetition_penalty_reading():
    # Reading (the pages print only a subtractive frequency-penalty example):
    # logits of tokens already generated are divided by theta when positive and
    # multiplied by theta otherwise.  Values checked by hand in fp32.
    z = np.array([2.0, -2.0, 0.0, 3.0, 1.1], np.float32)
    c = np.array([1, 5, 1, 0, 2], np.int32)
    got = oracle.repetition_penalty(z, c, 1.1)
    assert got[0] == np.float32(1.8181818)
    assert got[1] == np.float32(-2.2)
    assert got[2] == 0.0 and got[3] == 3.0 and got[4] == 1.0
    assert np.array_equal(oracle.repetition_penalty(z, c, 1.0), z)


# ---------------------------------------------------------------------------
# Worked examples and the output law
# ---------------------------------------------------------------------------
def batch_of_trials(p_rows, B, K, draft_ids, q_rows=None, T=1.0, seed=0, offset=0, C=1024):
    """B identical requests with K drafts each; the K+1 target rows carry log(p)."""
    V = p_rows.shape[1]
    logits_req = np.log(p_rows).astype(np.float32)                # [K+1, V]
    logits = np.tile(logits_req, (B, 1))
    cu = np.arange(B + 1, dtype=np.int32) * K
    q = None if q_rows is None else np.tile(q_rows.astype(np.float32), (B, 1))
    T = np.full(B, T, np.float32)
    return oracle.verify_batch(logits, cu, np.asarray(draft_ids, np.int32).reshape(-1), T,
                               draft_probs=q, seed=seed, offset=offset, C=C)


def chi2_ok(counts, expected_p):
    expected_p = np.asarray(expected_p, float)
    keep = expected_p > 0
    assert counts[~keep].sum() == 0, "mass on a token with probability 0"
    n = counts[keep].sum()
    return stats.chisquare(counts[keep], n * expected_p[keep] / expected_p[keep].sum()).pvalue


def binom_ok(k, n, p):
    return stats.binomtest(int(k), int(n), p).pvalue


def test_three_token_example_accept_mass_and_residual():
    g = golden("three_token_residual.json")
    p, q = np.array(g["p"]), np.array(g["q"])
    rng = np.random.default_rng(10)
    d = rng.choice(3, size=TRIALS, p=q).astype(np.int32)
    out = batch_of_trials(np.stack([p, p]), TRIALS, 1, d, q_rows=q[None, :])
    assert out["err"] == 0
    first = out["tokens"][:, 0]
    rejected = out["num_rejected"] == 1
    # accept mass 0.8, reject 0.2
    assert binom_ok((~rejected).sum(), TRIALS, g["total_accept"]) > P_MIN
    # residual (0, 1, 0): every reject outputs B, exactly
    assert np.all(first[rejected] == 1)
    # per-token accept probabilities (1, 1, 0.5)
    for t, a in enumerate(g["accept_prob"]):
        sel = d == t
        acc = (~rejected[sel]).sum()
        if a == 1.0:
            assert acc == sel.sum()
        else:
            assert binom_ok(acc, sel.sum(), a) > P_MIN
    # accepted mass per token = min(q, p); output law = p; P_final(B) = 0.3
    acc_counts = np.bincount(first[~rejected], minlength=3)
    assert chi2_ok(acc_counts, g["accepted_mass"]) > P_MIN
    assert chi2_ok(np.bincount(first, minlength=3), p) > P_MIN
    assert abs((first == 1).mean() - g["final_B"]) < 5 * np.sqrt(0.3 * 0.7 / TRIALS)
    # num_sampled is always 1 (reject) or 2 (accept + bonus)
    assert np.array_equal(out["num_sampled"], np.where(rejected, 1, 2))


def test_four_token_no_draft_probs_example():
    g = golden("four_token_no_draft.json")
    p = np.array(g["p"])
    d = np.full(TRIALS, g["draft"], np.int32)
    out = batch_of_trials(np.stack([p, p]), TRIALS, 1, d, q_rows=None)
    assert out["err"] == 0
    first = out["tokens"][:, 0]
    rejected = out["num_rejected"] == 1
    assert binom_ok((~rejected).sum(), TRIALS, g["accept_prob"]) > P_MIN
    rec = np.bincount(first[rejected], minlength=4)
    assert rec[g["draft"]] == 0                     # the rejected draft is excluded
    assert chi2_ok(rec, g["recovered"]) > P_MIN     # (0.125, 0, 0.375, 0.5)
    assert chi2_ok(np.bincount(first, minlength=4), g["final"]) > P_MIN
    # the accept probability is p(d) itself (q = 1 for a point-mass draft)
    assert np.allclose(out["p_draft"], g["p"][g["draft"]], atol=1e-7)


def test_bonus_token_only_after_all_accepted():
    g = golden("four_token_bonus.json")
    p = np.array(g["bonus_row_p"])
    rng = np.random.default_rng(11)
    # drafts B, C against rows where each is accepted with probability p(d)
    rows = np.stack([p, p, p])
    n = 200_000
    d = np.tile(np.array(g["drafts"], np.int32), n)
    out = batch_of_trials(rows, n, 2, d, q_rows=None)
    ns, nr, tok = out["num_sampled"], out["num_rejected"], out["tokens"]
    assert np.all(nr == 2 - (ns - 1))
    all_acc = nr == 0
    assert np.all(ns[all_acc] == g["all_accepted_outputs"])
    second_rej = (nr == 1)
    assert np.all(ns[second_rej] == g["second_rejected_outputs"])
    assert np.all(tok[second_rej, 2] == -1)         # no bonus after a reject
    assert np.all(tok[all_acc, :2] == np.array(g["drafts"]))
    # bonus law: the bonus row's p; bonus-only requests (K = 0) also give p
    assert chi2_ok(np.bincount(tok[all_acc, 2], minlength=4), p) > P_MIN
    out0 = batch_of_trials(p[None, :], TRIALS, 0, np.zeros(0, np.int32))
    assert np.all(out0["num_sampled"] == 1) and np.all(out0["num_rejected"] == 0)
    assert chi2_ok(np.bincount(out0["tokens"][:, 0], minlength=4), p) > P_MIN
    del rng


def test_five_token_example():
    g = golden("five_token_residual.json")
    p, q = np.array(g["p"]), np.array(g["q"])
    rng = np.random.default_rng(12)
    d = rng.choice(5, size=TRIALS, p=q).astype(np.int32)
    out = batch_of_trials(np.stack([p, p]), TRIALS, 1, d, q_rows=q[None, :])
    first = out["tokens"][:, 0]
    rejected = out["num_rejected"] == 1
    sel = d == 0
    assert binom_ok((~rejected[sel]).sum(), sel.sum(), g["accept_the"]) > P_MIN
    res = np.array(g["residual_unnormalised"])
    assert abs(res.sum() - g["residual_total"]) < 1e-12
    assert binom_ok(rejected.sum(), TRIALS, g["residual_total"]) > P_MIN
    assert chi2_ok(np.bincount(first[rejected], minlength=5), res) > P_MIN
    assert chi2_ok(np.bincount(first, minlength=5), p) > P_MIN


def test_overlap_plus_residual_is_p_on_random_distributions():
    # min(q, p) + max(0, p - q) = p per token: the accepted outputs follow
    # min(q, p), the recovered ones max(0, p - q), and together p.
    rng = np.random.default_rng(13)
    V = 12
    p = rng.dirichlet(np.ones(V))
    q = rng.dirichlet(np.ones(V))
    d = rng.choice(V, size=TRIALS, p=q / q.sum()).astype(np.int32)
    out = batch_of_trials(np.stack([p, p]), TRIALS, 1, d, q_rows=q[None, :])
    first = out["tokens"][:, 0]
    rejected = out["num_rejected"] == 1
    overlap = np.minimum(p, q)
    resid = np.maximum(0.0, p - q)
    assert abs(overlap.sum() + resid.sum() - 1.0) < 1e-12
    assert chi2_ok(np.bincount(first[~rejected], minlength=V), overlap) > P_MIN
    assert chi2_ok(np.bincount(first[rejected], minlength=V), resid) > P_MIN
    assert binom_ok(rejected.sum(), TRIALS, resid.sum()) > P_MIN
    assert chi2_ok(np.bincount(first, minlength=V), p) > P_MIN


def race_histogram(p, C, trials, seed=21):
    """Run the oracle's race over weights p for rows g = 0..trials-1."""
    import ctypes
    w = np.ascontiguousarray(p, np.float64)
    ptr = w.ctypes.data_as(ctypes.c_void_p)
    race = oracle.lib().orc_race
    m = ctypes.c_double()
    counts = np.zeros(p.size, np.int64)
    for g in range(trials):
        counts[race(ptr, p.size, C, seed, 0, g, ctypes.byref(m))] += 1
    return counts


def merged_chi2(counts, p):
    order = np.argsort(p)
    exp_sorted = p[order] * counts.sum()
    groups = (np.cumsum(exp_sorted) // 5.0).astype(int)
    e = np.bincount(groups, weights=exp_sorted)
    o = np.bincount(groups, weights=counts[order])
    keep = e > 0
    return stats.chisquare(o[keep], e[keep] * o.sum() / e[keep].sum()).pvalue


@pytest.mark.parametrize("V,C,trials", [(4096, 256, 200_000), (1024, 128, 200_000),
                                        (1024, 1024, 100_000), (1024, 4096, 100_000)])
def test_two_level_race_law(V, C, trials):
    # Random logits; C < V races ceil(V/C) chunks then a token inside the
    # winner, C >= V is the one-level race argmax(w / E).  All must sample p
    # (bins merged to an expected count >= 5).
    rng = np.random.default_rng(14 + V + C)
    z = (rng.standard_normal(V) * 2).astype(np.float32)
    p = oracle.softmax(z, 1.0)
    assert merged_chi2(race_histogram(p, C, trials), p) > P_MIN


def test_race_levels_are_exact_for_one_chunk():
    # With a single chunk the chunk level has one candidate: the winner and the
    # margin come from the token level alone; C = V and C > V agree token for token.
    rng = np.random.default_rng(16)
    p = rng.dirichlet(np.ones(300))
    for g in range(200):
        a = oracle.race(p, 300, 9, 1, g)
        b = oracle.race(p, 4096, 9, 1, g)
        assert a == b
    # zero weights never win; all-zero weights give -1
    w = np.zeros(64)
    w[17] = 1e-300
    assert all(oracle.race(w, 16, 3, 0, g)[0] == 17 for g in range(50))
    assert oracle.race(np.zeros(64), 16, 3, 0, 0)[0] == -1


def test_race_chunk_boundaries():
    # Mass only on the first and last token of chunks (C = 8): a chunk that
    # loses an edge token, or a token raced in the wrong chunk, breaks the law.
    V, C = 64, 8
    w = np.zeros(V)
    for x, m in [(0, 1.0), (7, 2.0), (8, 3.0), (15, 1.5), (16, 0.5), (63, 2.5)]:
        w[x] = m
    counts = race_histogram(w, C, 60_000, seed=3)
    assert chi2_ok(counts, w / w.sum()) > P_MIN


def test_rows_of_a_request_are_used_in_place():
    # Distinct rows: the recovered token comes from the rejected position's row,
    # the bonus from the extra row, never from a neighbour.
    p0 = np.array([0.1, 0.2, 0.3, 0.4])
    p1 = np.array([0.45, 0.05, 0.1, 0.4])
    p2 = np.array([0.05, 0.15, 0.7, 0.1])
    n = 400_000
    d = np.tile(np.array([1, 2], np.int32), n)
    out = batch_of_trials(np.stack([p0, p1, p2]), n, 2, d, q_rows=None)
    tok, nr = out["tokens"], out["num_rejected"]
    rej0, rej1, acc = nr == 2, nr == 1, nr == 0
    assert binom_ok(rej0.sum(), n, 0.8) > P_MIN
    assert binom_ok(rej1.sum(), n, 0.2 * 0.9) > P_MIN
    assert chi2_ok(np.bincount(tok[rej0, 0], minlength=4), [0.1, 0, 0.3, 0.4]) > P_MIN
    assert chi2_ok(np.bincount(tok[rej1, 1], minlength=4), [0.45, 0.05, 0, 0.4]) > P_MIN
    assert chi2_ok(np.bincount(tok[acc, 2], minlength=4), p2) > P_MIN
    # the same with draft probabilities: the residual uses the rejected row's q
    q0 = np.array([0.25, 0.25, 0.25, 0.25])
    q1 = np.array([0.1, 0.6, 0.2, 0.1])
    rng = np.random.default_rng(17)
    dd = np.stack([rng.choice(4, n, p=q0), rng.choice(4, n, p=q1)], 1).astype(np.int32)
    out = batch_of_trials(np.stack([p0, p1, p2]), n, 2, dd.reshape(-1), q_rows=np.stack([q0, q1]))
    tok, nr = out["tokens"], out["num_rejected"]
    assert chi2_ok(np.bincount(tok[nr == 2, 0], minlength=4), np.maximum(0, p0 - q0)) > P_MIN
    assert chi2_ok(np.bincount(tok[nr == 1, 1], minlength=4), np.maximum(0, p1 - q1)) > P_MIN
    assert chi2_ok(np.bincount(tok[nr == 0, 2], minlength=4), p2) > P_MIN


def test_greedy_rule():
    V = 6
    rows = np.full((4, V), -1.0, np.float32)
    rows[0, 2] = 5.0
    rows[1, 4] = 5.0
    rows[2, 1] = 5.0
    rows[2, 3] = 5.0          # tie: argmax is the lower index, 1
    rows[3, 0] = 5.0
    cu = np.array([0, 3], np.int32)
    T = np.zeros(1, np.float32)
    # all drafts match -> 3 accepted + bonus argmax
    o = oracle.verify_batch(rows, cu, np.array([2, 4, 1], np.int32), T)
    assert o["tokens"][0].tolist() == [2, 4, 1, 0] and o["num_sampled"][0] == 4
    assert o["num_rejected"][0] == 0
    # mismatch at position 1 -> output the target argmax there and stop
    o = oracle.verify_batch(rows, cu, np.array([2, 0, 1], np.int32), T)
    assert o["tokens"][0].tolist() == [2, 4, -1, -1]
    assert o["num_sampled"][0] == 2 and o["num_rejected"][0] == 2
    # a draft equal to the higher tied index is a mismatch
    o = oracle.verify_batch(rows, cu, np.array([2, 4, 3], np.int32), T)
    assert o["tokens"][0].tolist() == [2, 4, 1, -1] and o["num_rejected"][0] == 1


def test_post_update_example_and_rollback_rule():
    g = golden("post_update_example.json")
    V, S = 16, 3
    tokens = np.array([[7, 9, 11, -1, -1]], np.int32)    # d0, d1 accepted + one more
    ns = np.array([g["num_sampled"]], np.int32)
    nr = np.array([g["num_rejected"]], np.int32)
    last = np.full(S, -5, np.int32)
    counts = np.zeros((S, V), np.int32)
    counts[1, 9] = 4
    ncomp = np.array([0, 100, 0], np.int32)
    err = oracle.post_update(np.array([1], np.int32), np.array([g["query_len"]], np.int32),
                             tokens, ns, nr, last, counts, ncomp)
    assert err == 0
    assert ncomp.tolist() == [0, 100 + g["num_computed_delta"], 0]
    assert last[1] == tokens[0, g["last_sampled_is_output_index"]]
    assert counts[1, 7] == 1 and counts[1, 9] == 5 and counts[1, 11] == 1
    assert counts.sum() == 4 + g["num_sampled"]
    # rollback rule: num_rejected = num_draft - (generated - 1)
    for c in golden("rollback_rule.json")["cases"]:
        assert c["num_draft"] - (c["generated"] - 1) == c["num_rejected"]


def test_post_update_duplicates_and_bad_slot():
    V, S = 8, 2
    tokens = np.array([[3, 3, 5], [1, -1, -1], [2, 2, 2]], np.int32)
    ns = np.array([3, 1, 0], np.int32)      # the third request sampled nothing
    nr = np.array([0, 2, 0], np.int32)
    last = np.zeros(S, np.int32)
    counts = np.zeros((S, V), np.int32)
    ncomp = np.zeros(S, np.int32)
    err = oracle.post_update(np.array([0, 5, 1], np.int32), np.array([3, 3, 3], np.int32),
                             tokens, ns, nr, last, counts, ncomp)
    assert err == oracle.ERR_SLOT
    assert counts[0].tolist() == [0, 0, 0, 2, 0, 1, 0, 0] and counts[1].sum() == 0
    assert last.tolist() == [5, 0] and ncomp.tolist() == [3, 0]


def test_batch_invariants_and_errors():
    rng = np.random.default_rng(15)
    B, V, Kmax = 40, 300, 4
    K = rng.integers(0, Kmax + 1, B)
    cu = np.concatenate([[0], np.cumsum(K)]).astype(np.int32)
    R = int(cu[-1]) + B
    logits = (rng.standard_normal((R, V)) * 2).astype(np.float32)
    d = rng.integers(-2, V + 2, int(cu[-1])).astype(np.int32)    # includes invalid ids
    T = rng.choice([0.0, 0.5, 1.0], B).astype(np.float32)
    o = oracle.verify_batch(logits, cu, d, T, seed=5, offset=3)
    assert o["err"] == 0
    ns, nr = o["num_sampled"], o["num_rejected"]
    assert np.all(ns >= 1) and np.all(ns <= K + 1) and np.all(nr == K + 1 - ns)
    for r in range(B):
        t = o["tokens"][r]
        assert np.all(t[: ns[r]] >= 0) and np.all(t[: ns[r]] < V) and np.all(t[ns[r]:] == -1)
        dd = d[cu[r]: cu[r + 1]]
        assert np.array_equal(t[: ns[r] - 1], dd[: ns[r] - 1])   # accepted prefix = drafts
        bad = (dd < 0) | (dd >= V)
        if bad.any():                                            # invalid ids never pass
            assert ns[r] - 1 <= int(np.argmax(bad))
    # determinism
    o2 = oracle.verify_batch(logits, cu, d, T, seed=5, offset=3)
    assert np.array_equal(o["tokens"], o2["tokens"])
    # errors
    bad_cu = cu.copy()
    bad_cu[3], bad_cu[4] = bad_cu[4], bad_cu[3] - 1
    assert oracle.verify_batch(logits, bad_cu, d, T)["err"] & oracle.ERR_CU
    Tn = T.copy()
    Tn[2] = -1.0
    o = oracle.verify_batch(logits, cu, d, Tn)
    assert o["err"] == oracle.ERR_TEMPERATURE and o["num_sampled"][2] == 0
    assert o["num_sampled"][3] > 0
    assert oracle.verify_batch(logits, cu, d, T, offset=1 << 32)["err"] == oracle.ERR_OFFSET
    lg = logits.copy()
    lg[cu[5] + 5] = -np.inf
    o = oracle.verify_batch(lg, cu, d, T)
    assert o["err"] == oracle.ERR_ROW and o["num_sampled"][5] == 0
