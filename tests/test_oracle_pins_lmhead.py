"""Pins for the oracle's LM-head path: the logits of the hidden states times the
LM-head weight (exact integer and dyadic cases, brute force, bf16 decoding), and
the verify step on them, tied to the separately pinned logits path and to the
output law."""
from fractions import Fraction

import numpy as np
from scipy import special, stats

import oracle

P_MIN = 1e-4


def bf16_bits(a):
    """fp32 -> bf16 bit patterns for values that bf16 holds exactly."""
    a = np.asarray(a, dtype=np.float32)
    bits = a.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "value not exact in bf16"
    return (bits >> 16).astype(np.uint16)


def bits_value(b):
    return float(np.array([int(b) << 16], dtype=np.uint32).view(np.float32)[0])


def test_logits_small_integers_brute_force():
    rng = np.random.default_rng(11)
    V, d = 23, 37
    H = rng.integers(-8, 9, size=d)
    W = rng.integers(-8, 9, size=(V, d))
    z = oracle.lm_head_logits(bf16_bits(H), bf16_bits(W))
    for x in range(V):
        want = 0
        for k in range(d):
            want += int(H[k]) * int(W[x][k])
        assert z[x] == want
    # a slice of the vocabulary gives the same values
    np.testing.assert_array_equal(oracle.lm_head_logits(bf16_bits(H), bf16_bits(W), 5, 17), z[5:17])


def test_logits_dyadic_exact():
    rng = np.random.default_rng(12)
    V, d = 9, 64
    H = rng.integers(-127, 128, size=d) * 2.0 ** -7
    W = rng.integers(-127, 128, size=(V, d)) * 2.0 ** -11
    z = oracle.lm_head_logits(bf16_bits(H), bf16_bits(W))
    for x in range(V):
        want = sum(Fraction(float(H[k])) * Fraction(float(W[x][k])) for k in range(d))
        assert Fraction(z[x]) == want  # the sum of 64 such products is exact in fp64


def test_bf16_decoding_through_one_hot_rows():
    # known bf16 bit patterns: 1.0, -2.0, 0.5, the smallest subnormal, the largest finite
    patterns = [0x3F80, 0xC000, 0x3F00, 0x0001, 0x7F7F]
    d = len(patterns)
    h = np.array(patterns, dtype=np.uint16)
    W = bf16_bits(np.eye(d, dtype=np.float32))
    z = oracle.lm_head_logits(h, W)
    assert list(z) == [1.0, -2.0, 0.5, 2.0 ** -133, (2.0 - 2.0 ** -7) * 2.0 ** 127]
    assert [bits_value(b) for b in patterns] == list(z)


def one_hot_case(seed, B=6, V=40, d=16, kmax=3, greedy_every=3):
    """Hidden states and a one-hot LM head whose logits are small integers:
    W[x] = c_x e_{pi(x)}, so z_x = c_x h_{pi(x)}, exact in fp32."""
    rng = np.random.default_rng(seed)
    K = rng.integers(0, kmax + 1, size=B)
    cu = np.concatenate([[0], np.cumsum(K)]).astype(np.int32)
    R = int(cu[-1]) + B
    H = rng.integers(-4, 5, size=(R, d)).astype(np.float32)
    pi = rng.integers(0, d, size=V)
    c = rng.integers(1, 4, size=V).astype(np.float32)
    W = np.zeros((V, d), np.float32)
    W[np.arange(V), pi] = c
    Z = (H[:, pi] * c[None, :]).astype(np.float32)
    draft = rng.integers(0, V, size=int(cu[-1])).astype(np.int32)
    T = np.where(np.arange(B) % greedy_every == 0, 0.0, 0.9).astype(np.float32)
    return bf16_bits(H), bf16_bits(W), Z, cu, draft, T


def test_one_hot_head_matches_logit_path():
    for seed in range(5):
        H, W, Z, cu, draft, T = one_hot_case(seed, V=200)
        for off in range(4):
            for C in (oracle.LM_HEAD_CHUNK, 200):
                a = oracle.lm_head_verify(H, W, cu, draft, T, seed=7, offset=off, C=C)
                b = oracle.verify_batch(Z, cu, draft, T, seed=7, offset=off, C=C)
                assert a["err"] == 0 and b["err"] == 0
                np.testing.assert_array_equal(a["tokens"], b["tokens"])
                np.testing.assert_array_equal(a["num_sampled"], b["num_sampled"])
                np.testing.assert_array_equal(a["num_rejected"], b["num_rejected"])
                np.testing.assert_array_equal(a["p_draft"], b["p_draft"])


def test_bonus_token_law():
    # one request, no drafts: the bonus token over many offsets follows softmax(z / T)
    rng = np.random.default_rng(5)
    V, d, T, N = 12, 8, 0.7, 40_000
    H = bf16_bits(rng.integers(-3, 4, size=(1, d)).astype(np.float32))
    W = bf16_bits(rng.integers(-1, 2, size=(V, d)).astype(np.float32) * 0.5)
    z = oracle.lm_head_logits(H[0], W)
    p = special.softmax(z / float(np.float32(T)))
    counts = np.zeros(V, np.int64)
    cu = np.array([0, 0], np.int32)
    for off in range(N):
        out = oracle.lm_head_verify(H, W, cu, np.zeros(0, np.int32), np.array([T], np.float32), seed=3,
                                    offset=off, C=4)
        counts[out["tokens"][0, 0]] += 1
    keep = p * N >= 5
    obs = np.append(counts[keep], counts[~keep].sum())
    exp = np.append(p[keep], p[~keep].sum()) * N
    assert stats.chisquare(obs[exp > 0], exp[exp > 0]).pvalue > P_MIN


def test_rejected_draft_never_recovered_and_accept_rate():
    rng = np.random.default_rng(6)
    V, d, T, N = 10, 8, 1.0, 20_000
    H = bf16_bits(rng.integers(-2, 3, size=(2, d)).astype(np.float32))
    W = bf16_bits(rng.integers(-1, 2, size=(V, d)).astype(np.float32))
    z0 = oracle.lm_head_logits(H[0], W)
    p0 = special.softmax(z0 / T)
    dtok = int(np.argsort(p0)[-2])
    cu = np.array([0, 1], np.int32)
    acc = 0
    rec = np.zeros(V, np.int64)
    for off in range(N):
        out = oracle.lm_head_verify(H, W, cu, np.array([dtok], np.int32), np.array([T], np.float32), seed=1,
                                    offset=off, C=4)
        if out["num_rejected"][0] == 0:
            acc += 1
            assert out["tokens"][0, 0] == dtok
        else:
            x = out["tokens"][0, 0]
            assert x != dtok
            rec[x] += 1
        assert abs(out["p_draft"][0] - p0[dtok]) < 1e-6
    # acceptance is Bernoulli(p(d)); the recovered token follows p without d
    assert stats.binomtest(acc, N, p0[dtok]).pvalue > P_MIN
    w = p0.copy()
    w[dtok] = 0.0
    w /= w.sum()
    keep = w * rec.sum() >= 5
    obs = np.append(rec[keep], rec[~keep].sum())
    exp = np.append(w[keep], w[~keep].sum()) * rec.sum()
    assert stats.chisquare(obs[exp > 0], exp[exp > 0]).pvalue > P_MIN


def test_greedy_ties_gap_and_errors():
    d = 4
    H = bf16_bits(np.array([[1, 2, 3, 4], [0, 0, 1, 0]], np.float32))
    W = bf16_bits(np.array([[0, 0, 1, 0], [1, 1, 0, 0], [0, 0, 0, 1]], np.float32))  # z0 = 3, 3, 4
    cu = np.array([0, 1], np.int32)
    out = oracle.lm_head_verify(H, W, cu, np.array([2], np.int32), np.zeros(1, np.float32))
    # row 0: argmax token 2 (z = 4) accepts d = 2; row 1: z = 1, 0, 0 -> token 0
    assert out["tokens"][0].tolist() == [2, 0] and out["num_sampled"][0] == 2
    assert out["greedy_gap"][0] == 1.0 and out["margin"][0] == np.inf
    # an exact tie goes to the lowest index, with a zero gap
    H2 = bf16_bits(np.array([[1, 2, 3, 0]], np.float32))
    W2 = bf16_bits(np.array([[0, 0, 1, 0], [1, 1, 0, 0], [0, 0, 0, 1]], np.float32))  # 3, 3, 0
    out = oracle.lm_head_verify(H2, W2, np.array([0, 0], np.int32), np.zeros(0, np.int32),
                                np.zeros(1, np.float32))
    assert out["tokens"][0, 0] == 0 and out["greedy_gap"][0] == 0.0
    # invalid temperature, non-finite logits
    out = oracle.lm_head_verify(H2, W2, np.array([0, 0], np.int32), np.zeros(0, np.int32),
                                np.array([-1.0], np.float32))
    assert out["err"] == oracle.ERR_TEMPERATURE and out["num_sampled"][0] == 0
    Hinf = H2.copy()
    Hinf[0, 0] = 0x7F80  # +inf
    out = oracle.lm_head_verify(Hinf, W2, np.array([0, 0], np.int32), np.zeros(0, np.int32),
                                np.ones(1, np.float32))
    assert out["err"] == oracle.ERR_ROW and out["tokens"][0, 0] == -1
    assert d == 4
