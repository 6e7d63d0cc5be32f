"""GPU parity of the verify step on LM-head logits (spec_verify_lm_head, through
the C ABI) against the oracle: its fp64 logits W h and its verify step on them
(no-draft-probs mode, one-level race).

Acceptance rule.  The library multiplies bf16 inputs with fp32 accumulation,
the oracle in fp64, so the logits differ by rounding:
  * the fp32 logits (dbg output) must lie within
    EPS(x) = LAMBDA sqrt(d) 2^-24 sum_k |h_k W_xk| of the fp64 ones (the
    probabilistic bound on d rounded fp32 additions, LAMBDA = 8: far below the
    change one wrong or missing product makes);
  * with every logit of a row within EPS, the race keys a (z - m) - log2 E and
    log2 p(d) move by at most 2 a EPS, i.e. a score ratio by at most
    2 EPS / T relative; a request whose oracle decision margin is below that
    (plus MARGIN for the fp32 arithmetic), or a greedy request whose top-two
    logit gap is below 2 EPS, may differ and is counted instead; every other
    request must match exactly (tokens, num_sampled, num_rejected);
  * p(d) within PROB_ATOL + p(d) 2 EPS / T.
"""
import numpy as np
import pytest
import torch

import oracle
import rejection_sampling_verify_05_amd as sv
import workloads as wl
from harness import MARGIN, PROB_ATOL

pytestmark = pytest.mark.gpu

DEV = "cuda"
LAMBDA = 8.0


def say(*a):
    print(*a, flush=True)


def bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def lm_ctx(inp, max_k=None):
    K = int(inp["K"].max().item()) if inp["B"] else 0
    return sv.spec_verify_create(inp["R"], inp["B"], max(K if max_k is None else max_k, 1), inp["V"],
                                 sv.SV_CREATE_LM_HEAD)


def lm_run(ctx, inp, seed=0, offset=0, dbg_logits=False, temperature=None, hidden=None):
    B, D, R, V = inp["B"], inp["D"], inp["R"], inp["V"]
    S = int(inp["K"].max().item()) + 1 if B else 1
    out = torch.full((B, S), -7, dtype=torch.int32, device=DEV)
    ns = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    nr = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    pd = torch.full((max(D, 1),), -7.0, dtype=torch.float32, device=DEV)
    zl = torch.full((R, V), -7.0, dtype=torch.float32, device=DEV) if dbg_logits else None
    sv.spec_verify_lm_head(ctx, inp["hidden"] if hidden is None else hidden, inp["W"], inp["draft_ids"],
                           inp["cu"], inp["temperature"] if temperature is None else temperature, out, ns, nr,
                           seed=seed, offset=offset, dbg_p_draft=pd if D else None, dbg_logits=zl)
    err = sv.spec_verify_read_error(ctx)
    return dict(tokens=out.cpu().numpy(), num_sampled=ns.cpu().numpy(), num_rejected=nr.cpu().numpy(),
                p_draft=pd.cpu().numpy()[:D], logits=None if zl is None else zl.cpu().numpy(), err=err)


def eps_rows(h, rows):
    """EPS(x) for the given rows: LAMBDA sqrt(d) 2^-24 sum_k |h_k W_xk| (fp64)."""
    Ha = np.abs(h["Hf"][rows].astype(np.float64))
    return LAMBDA * np.sqrt(Ha.shape[1]) * 2.0 ** -24 * (Ha @ h["Wabs"].T)


def host(inp):
    return dict(H=bits(inp["hidden"]), W=bits(inp["W"]), Hf=inp["hidden"].float().cpu().numpy(),
                Wabs=inp["W"].float().abs().double().cpu().numpy(), cu=inp["cu"].cpu().numpy(),
                d=inp["draft_ids"].cpu().numpy(), T=inp["temperature"].cpu().numpy())


def check(inp, h, g, seed, offset, requests, check_logits=True):
    """Compare the GPU outputs of `requests` with the oracle; returns the number
    of requests excused by the margin rule and the list of failures."""
    o = oracle.lm_head_verify(h["H"], h["W"], h["cu"], h["d"], h["T"], seed=seed, offset=offset,
                              out_stride=g["tokens"].shape[1], requests=requests)
    cu, T = h["cu"], h["T"]
    bad, excused = [], 0
    for r in requests:
        rows = np.arange(cu[r] + r, cu[r + 1] + r + 1)
        eps = eps_rows(h, rows)
        if check_logits and g["logits"] is not None:
            for k, gr in enumerate(rows):
                z64 = oracle.lm_head_logits(h["H"][gr], h["W"])
                err = np.abs(g["logits"][gr].astype(np.float64) - z64)
                if np.any(err > eps[k]):
                    x = int(np.argmax(err - eps[k]))
                    bad.append(f"row {gr}: logit {x} off by {err[x]:.3g} > {eps[k][x]:.3g}")
        e = float(eps.max()) if eps.size else 0.0
        same = (np.array_equal(g["tokens"][r], o["tokens"][r]) and g["num_sampled"][r] == o["num_sampled"][r]
                and g["num_rejected"][r] == o["num_rejected"][r])
        if T[r] > 0:
            rel = 2.0 * e / float(T[r]) + MARGIN
            near = o["margin"][r] < rel
            for i in range(cu[r], cu[r + 1]):
                pd_o = o["p_draft"][i]
                if abs(g["p_draft"][i] - pd_o) > PROB_ATOL + pd_o * rel:
                    bad.append(f"req {r} draft {i}: p(d) {g['p_draft'][i]} vs {pd_o}")
        else:
            near = o["greedy_gap"][r] < 2.0 * e
            if np.any(g["p_draft"][cu[r]:cu[r + 1]] != -1.0):
                bad.append(f"req {r}: greedy p(d) not -1")
        if not same:
            if near:
                excused += 1
            else:
                bad.append(f"req {r}: gpu {g['tokens'][r].tolist()} ns {g['num_sampled'][r]} vs oracle "
                           f"{o['tokens'][r].tolist()} ns {o['num_sampled'][r]} (margin {o['margin'][r]:.3g}, "
                           f"gap {o['greedy_gap'][r]:.3g}, eps {e:.3g})")
    return excused, bad


def structural(inp, g):
    """Properties that hold at any size: counts, the accepted prefix, token range."""
    K = inp["K"].cpu().numpy()
    cu = inp["cu"].cpu().numpy()
    d = inp["draft_ids"].cpu().numpy()
    V = inp["V"]
    assert np.all(g["num_sampled"] >= 1) and np.all(g["num_sampled"] <= K + 1)
    assert np.all(g["num_rejected"] == K + 1 - g["num_sampled"])
    for r in range(inp["B"]):
        n = g["num_sampled"][r]
        assert np.array_equal(g["tokens"][r, : n - 1], d[cu[r]: cu[r] + n - 1])
        assert 0 <= g["tokens"][r, n - 1] < V
        assert np.all(g["tokens"][r, n:] == -1)
        if n - 1 < K[r] and inp["temperature"][r].item() > 0:  # a recovered token is never the rejected draft
            assert g["tokens"][r, n - 1] != d[cu[r] + n - 1]


CASES = {
    "base": dict(B=12, K=3, V=1000, d=128),
    "tails_two_row_blocks": dict(B=50, K=4, V=777, d=192, T=0.8, greedy_every=3),
    "one_tile": dict(B=6, K=2, V=256, d=64, T=1.3),
    "tiny_vocab": dict(B=5, K=3, V=3, d=64),
    "single_token_vocab": dict(B=4, K=2, V=1, d=64),
    "peaked_high_accept": dict(B=20, K=3, V=3000, d=256, scale=8.0, draft_noise=0.01, ragged=False),
    "hot": dict(B=16, K=3, V=4100, d=128, T=0.3),
    "cold_all_greedy": dict(B=16, K=3, V=2500, d=320, greedy_every=1),
    "no_drafts": dict(B=9, K=0, V=1500, d=64, ragged=False),
    "three_row_blocks": dict(B=100, K=3, V=600, d=64, T=1.1, greedy_every=5, ragged=False),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_lm_head_parity(name):
    kw = dict(CASES[name])
    say(f"case {name}: {kw}")
    inp = wl.make_lm_head_inputs(device=DEV, **kw)
    h = host(inp)
    ctx = lm_ctx(inp)
    try:
        total = 0
        for seed, off in [(0, 0), (12345, 7), (2 ** 40 + 3, 99)]:
            g = lm_run(ctx, inp, seed=seed, offset=off, dbg_logits=True)
            assert g["err"] == 0, g["err"]
            structural(inp, g)
            ex, bad = check(inp, h, g, seed, off, range(inp["B"]), check_logits=(seed == 0))
            total += ex
            assert not bad, "\n".join(bad[:10])
            # replay: a pure function of the inputs, seed and offset
            g2 = lm_run(ctx, inp, seed=seed, offset=off)
            assert np.array_equal(g2["tokens"], g["tokens"])
        say(f"case {name}: margin-excused requests {total} of {3 * inp['B']}")
        assert total <= int(1e-4 * 3 * inp["R"])  # 0.01 % of the rows checked
    finally:
        sv.spec_verify_destroy(ctx)


def test_lm_head_strided_rows():
    # hidden states and W as row slices of wider buffers (row strides > d), d = 192
    inp = wl.make_lm_head_inputs(B=10, K=3, V=900, d=192, greedy_every=3, device=DEV)
    ctx = lm_ctx(inp)
    try:
        Hw = torch.zeros((inp["R"], 192 + 40), dtype=torch.bfloat16, device=DEV)
        Ww = torch.zeros((inp["V"], 192 + 8), dtype=torch.bfloat16, device=DEV)
        Hw[:, 8:200] = inp["hidden"]
        Ww[:, :192] = inp["W"]
        strided = dict(inp, hidden=Hw[:, 8:200], W=Ww[:, :192])
        assert strided["hidden"].stride(0) == 232 and strided["W"].stride(0) == 200
        h = host(inp)
        for seed, off in [(3, 0), (4, 5)]:
            g = lm_run(ctx, strided, seed=seed, offset=off, dbg_logits=True)
            ref = lm_run(ctx, inp, seed=seed, offset=off)
            assert g["err"] == 0
            np.testing.assert_array_equal(g["tokens"], ref["tokens"])
            ex, bad = check(inp, h, g, seed, off, range(inp["B"]))
            assert not bad and ex <= int(1e-4 * inp["R"]), "\n".join(bad[:10])
    finally:
        sv.spec_verify_destroy(ctx)


def test_lm_head_invalid_requests():
    inp = wl.make_lm_head_inputs(B=8, K=2, V=700, d=64, device=DEV)
    ctx = lm_ctx(inp)
    try:
        T = inp["temperature"].clone()
        T[3] = -1.0
        g = lm_run(ctx, inp, temperature=T)
        assert g["err"] == sv.SV_ERR_TEMPERATURE
        assert g["num_sampled"][3] == 0 and np.all(g["tokens"][3] == -1)
        assert np.all(g["num_sampled"][[0, 1, 2, 4, 5, 6, 7]] >= 1)
        Hn = inp["hidden"].clone()
        cu = inp["cu"].cpu().numpy()
        Hn[cu[5] + 5, 7] = float("nan")  # first row of request 5
        g = lm_run(ctx, inp, hidden=Hn)
        assert g["err"] == sv.SV_ERR_ROW
        assert g["num_sampled"][5] == 0 and np.all(g["tokens"][5] == -1)
        assert np.all(g["num_sampled"][[0, 1, 2, 3, 4, 6, 7]] >= 1)
        # host-side checks: hidden size not a multiple of 64, no LM-head storage
        for d_bad in (80, 96):
            bad = wl.make_lm_head_inputs(B=2, K=1, V=100, d=d_bad, device=DEV)
            with pytest.raises(sv.SpecVerifyError):
                lm_run(ctx, bad)
        plain = sv.spec_verify_create(inp["R"], inp["B"], 2, inp["V"], 0)
        try:
            with pytest.raises(sv.SpecVerifyError):
                lm_run(plain, inp)
        finally:
            sv.spec_verify_destroy(plain)
    finally:
        sv.spec_verify_destroy(ctx)


@pytest.mark.parametrize("greedy_every", [0, 4])
def test_lm_head_full_size_sampled(greedy_every):
    # The bench workload (B=256, K_r ~ U{0..3}, V=128256, d=4096), in the launch
    # configuration the bench times; the oracle checks a sample of requests,
    # the rest are checked structurally.
    inp = wl.make_lm_head_inputs(B=256, K=3, V=128256, d=4096, greedy_every=greedy_every, device=DEV)
    say(f"full size: R={inp['R']} greedy_every={greedy_every}")
    h = host(inp)
    ctx = lm_ctx(inp)
    try:
        g = lm_run(ctx, inp, seed=5, offset=3, dbg_logits=True)
        assert g["err"] == 0
        structural(inp, g)
        K = inp["K"].cpu().numpy()
        pick = [int(np.flatnonzero(K == k)[0]) for k in range(4) if np.any(K == k)] + [255]
        pick = sorted(set(pick))
        say(f"oracle requests {pick}")
        ex, bad = check(inp, h, g, 5, 3, pick)
        say(f"full size: margin-excused {ex} of {len(pick)}")
        assert not bad, "\n".join(bad[:10])
        assert ex <= int(1e-4 * inp["R"])
    finally:
        sv.spec_verify_destroy(ctx)


def test_lm_head_post_update_inside_call():
    # post_update attached to spec_verify_lm_head: the same tokens, and the same
    # state as spec_post_update applied afterwards and as the oracle's post_update.
    inp = wl.make_lm_head_inputs(B=20, K=3, V=1500, d=64, greedy_every=4, device=DEV)
    B, V = inp["B"], inp["V"]
    S = B + 5
    rng = np.random.default_rng(3)
    idx = torch.from_numpy(rng.permutation(S)[:B].astype(np.int32)).to(DEV)
    ql = (inp["K"] + 1).to(torch.int32)
    last0 = rng.integers(-1, V, S).astype(np.int32)
    ncomp0 = rng.integers(0, 100, S).astype(np.int32)
    counts0 = rng.integers(0, 3, (S, V)).astype(np.int32)
    ctx = lm_ctx(inp)
    try:
        g = lm_run(ctx, inp, seed=9, offset=4)
        assert g["err"] == 0
        want = [last0.copy(), counts0.copy(), ncomp0.copy()]
        assert oracle.post_update(idx.cpu().numpy(), ql.cpu().numpy(), g["tokens"], g["num_sampled"],
                                  g["num_rejected"], *want) == 0
        st = [torch.from_numpy(x.copy()).to(DEV) for x in (last0, counts0, ncomp0)]
        S_ = int(inp["K"].max().item()) + 1
        out = torch.full((B, S_), -7, dtype=torch.int32, device=DEV)
        ns = torch.full((B,), -7, dtype=torch.int32, device=DEV)
        nr = torch.full((B,), -7, dtype=torch.int32, device=DEV)
        pu = sv.make_post_update_args(idx, ql, out, ns, nr, st[0], st[1], st[2])
        sv.spec_verify_lm_head(ctx, inp["hidden"], inp["W"], inp["draft_ids"], inp["cu"], inp["temperature"],
                               out, ns, nr, seed=9, offset=4, post_update=pu)
        assert sv.spec_verify_read_error(ctx) == 0
        assert np.array_equal(out.cpu().numpy(), g["tokens"])
        assert np.array_equal(ns.cpu().numpy(), g["num_sampled"])
        for got, w in zip(st, want):
            assert np.array_equal(got.cpu().numpy(), w)
    finally:
        sv.spec_verify_destroy(ctx)


def test_lm_head_margin_aggregate():
    # The margin rule aggregated over enough runs that 0.01 % of the rows
    # checked is at least one: B=128 requests, K_r ~ U{0..3}, V=777, d=128,
    # every 5th request greedy; every request checked in every run.
    inp = wl.make_lm_head_inputs(B=128, K=3, V=777, d=128, T=0.9, greedy_every=5, device=DEV)
    h = host(inp)
    R = inp["R"]
    runs = max(40, -(-10_000 // R))
    bound = int(1e-4 * R * runs)
    ctx = lm_ctx(inp)
    try:
        excused = 0
        for run in range(runs):
            seed, off = 0xC0FFEE + 31 * run, 7 * run
            g = lm_run(ctx, inp, seed=seed, offset=off)
            assert g["err"] == 0
            ex, bad = check(inp, h, g, seed, off, range(inp["B"]), check_logits=False)
            assert not bad, f"run {run}: " + "\n".join(bad[:10])
            excused += ex
        say(f"LM-head aggregate: {runs} runs x {R} rows, margin-excused requests {excused}, bound {bound}")
        assert bound >= 1 and excused <= bound
    finally:
        sv.spec_verify_destroy(ctx)
