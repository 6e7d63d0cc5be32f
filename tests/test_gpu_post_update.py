"""post_update through the C ABI against the oracle's post_update (bit-exact):
last_sampled, the output-token histogram and num_computed, on verify outputs
of the workloads and on hand-made edge cases (skipped requests, tokens outside
the vocabulary, slots out of range, two updates in a row)."""
import numpy as np
import pytest
import torch

import oracle
import rejection_sampling_verify_05_amd as sv
import workloads as wl
from harness import ctx_for, run_gpu, run_draft_steps

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def gpu_post_update(ctx, idx, ql, toks, ns, nr, last, counts, ncomp):
    """Runs spec_post_update on device copies; returns host (last, counts, ncomp, err)."""
    d = {k: torch.from_numpy(np.ascontiguousarray(v)).to(DEV) for k, v in
         dict(idx=idx, ql=ql, toks=toks, ns=ns, nr=nr, last=last, counts=counts, ncomp=ncomp).items()}
    sv.spec_post_update(ctx.h, d["idx"], d["ql"], d["toks"], d["ns"], d["nr"], d["last"], d["counts"], d["ncomp"])
    err = sv.spec_verify_read_error(ctx.h)
    return d["last"].cpu().numpy(), d["counts"].cpu().numpy(), d["ncomp"].cpu().numpy(), err


def oracle_post_update(idx, ql, toks, ns, nr, last, counts, ncomp):
    last, counts, ncomp = last.copy(), counts.copy(), ncomp.copy()
    err = oracle.post_update(idx, ql, toks, ns, nr, last, counts, ncomp)
    return last, counts, ncomp, err


@pytest.mark.parametrize("cid", ["1", "2", "3"])
def test_post_update_on_verify_outputs(cid):
    w = wl.CONFIGS[cid]
    inp = wl.make_inputs(w, DEV)
    say(f"config {cid}: B={inp['B']} V={inp['V']}")
    with ctx_for(inp) as ctx:
        g = run_gpu(ctx, inp, seed=3, offset=5)
        assert g["err"] == 0
        S, V = inp["num_slots"], inp["V"]
        rng = np.random.default_rng(7)
        last = rng.integers(-1, V, S).astype(np.int32)
        ncomp = rng.integers(0, 1000, S).astype(np.int32)
        counts = inp["counts"].cpu().numpy().copy()
        counts[rng.integers(0, S, 64), rng.integers(0, V, 64)] += 3
        idx = inp["idx_mapping"].cpu().numpy()
        ql = inp["query_len"].cpu().numpy()
        args = (idx, ql, g["tokens"], g["num_sampled"], g["num_rejected"], last, counts, ncomp)
        got = gpu_post_update(ctx, *args)
        want = oracle_post_update(*args)
    assert got[3] == 0 and want[3] == 0
    assert np.array_equal(got[0], want[0])
    assert np.array_equal(got[2], want[2])
    assert np.array_equal(got[1], want[1])


def test_post_update_edge_cases_and_repeats():
    B, V, S, stride = 9, 50, 12, 4
    rng = np.random.default_rng(11)
    idx = rng.permutation(S)[:B].astype(np.int32)
    ql = rng.integers(1, 5, B).astype(np.int32)
    ns = np.array([1, 4, 0, 2, 3, 4, 1, 2, 3], np.int32)           # request 2 sampled nothing
    nr = np.maximum(ql - ns, 0).astype(np.int32)
    toks = rng.integers(0, V, (B, stride)).astype(np.int32)
    toks[1, 1] = -1                                                   # outside the vocabulary: not counted
    toks[4, 0] = V + 3
    toks[toks < -1] = -1
    for r in range(B):
        toks[r, ns[r]:] = -1
    last = np.full(S, -5, np.int32)
    counts = rng.integers(0, 3, (S, V)).astype(np.int32)
    ncomp = np.zeros(S, np.int32)
    inp = wl.make_inputs(wl.CONFIGS["1"], DEV)
    with ctx_for(inp) as ctx:
        state_g = (last, counts, ncomp)
        state_o = (last, counts, ncomp)
        for rep in range(2):  # two updates in a row accumulate
            g = gpu_post_update(ctx, idx, ql, toks, ns, nr, *state_g)
            o = oracle_post_update(idx, ql, toks, ns, nr, *state_o)
            assert g[3] == 0 and o[3] == 0
            for a, b in zip(g[:3], o[:3]):
                assert np.array_equal(a, b), f"repeat {rep}"
            state_g, state_o = g[:3], o[:3]
        # a slot outside [0, S): that request is skipped and the error bit is set
        bad = idx.copy()
        bad[3] = S + 2
        g = gpu_post_update(ctx, bad, ql, toks, ns, nr, *state_g)
        o = oracle_post_update(bad, ql, toks, ns, nr, *state_o)
        assert g[3] == sv.SV_ERR_SLOT and o[3] != 0
        for a, b in zip(g[:3], o[:3]):
            assert np.array_equal(a, b)


IN_CALL_CASES = {
    "1_draft_probs": wl.CONFIGS["1"],
    "2_greedy_mix": wl.CONFIGS["2"].with_(B=32, V=8000),
    "3_no_draft": wl.CONFIGS["3"].with_(B=48, V=20000 + 3),
    "4_topk_penalty": wl.CONFIGS["4"].with_(B=16, K=4, V=6000, history=64),
    "3p_top_p": wl.CONFIGS["3"].with_(B=24, V=9000, top_p=0.8),
    "3f_penalties": wl.CONFIGS["3"].with_(B=24, V=9000, freq=0.5, pres=0.25, history=64),
    "3d_draft_logits": wl.CONFIGS["3"].with_(B=16, V=7000, draft_logits=True),
}


@pytest.mark.parametrize("name", sorted(IN_CALL_CASES))
def test_post_update_inside_verify(name):
    # spec_verify_run with post_update attached: the same tokens as without it,
    # and the same state as spec_post_update applied afterwards (and as the
    # oracle's post_update), including the penalty paths that read the counts
    # the call updates and the residual paths that finish a request later.
    w = IN_CALL_CASES[name]
    say(f"case {name}: {w}")
    inp = wl.make_inputs(w, DEV)
    with ctx_for(inp) as ctx:
        if w.draft_logits:  # draft ids and row statistics from the draft sampler
            run_draft_steps(ctx, inp, seed=1, offset=2)
        dl = inp.get("draft_stats") is not None
        B, S, V = inp["B"], inp["num_slots"], inp["V"]
        out_stride = int(inp["K"].max().item()) + 1
        rng = np.random.default_rng(11)
        last0 = rng.integers(-1, V, S).astype(np.int32)
        ncomp0 = rng.integers(0, 1000, S).astype(np.int32)
        counts0 = inp["counts"].cpu().numpy().copy()
        penalty = any(inp.get(k) is not None for k in ("rep_penalty", "freq", "pres"))
        for seed, off in [(3, 5), (8, 0)]:
            # reference: verify, then spec_post_update (separate calls)
            g = run_gpu(ctx, inp, seed=seed, offset=off)
            assert g["err"] == 0
            ref = gpu_post_update(ctx, inp["idx_mapping"].cpu().numpy(), inp["query_len"].cpu().numpy(), g["tokens"],
                                  g["num_sampled"], g["num_rejected"], last0, counts0, ncomp0)
            want = oracle_post_update(inp["idx_mapping"].cpu().numpy(), inp["query_len"].cpu().numpy(), g["tokens"],
                                      g["num_sampled"], g["num_rejected"], last0, counts0, ncomp0)
            # in-call: the counts the call reads for penalties are the state it updates
            counts = torch.from_numpy(counts0.copy()).to(DEV)
            last = torch.from_numpy(last0.copy()).to(DEV)
            ncomp = torch.from_numpy(ncomp0.copy()).to(DEV)
            toks = torch.full((B, out_stride), -7, dtype=torch.int32, device=DEV)
            ns = torch.full((B,), -7, dtype=torch.int32, device=DEV)
            nr = torch.full((B,), -7, dtype=torch.int32, device=DEV)
            pu = sv.make_post_update_args(inp["idx_mapping"], inp["query_len"], toks, ns, nr, last, counts, ncomp)
            sv.spec_verify_run(ctx.h, inp["logits"], inp["draft_ids"], inp["cu"], inp["temperature"], toks, ns, nr,
                               draft_probs=inp["draft_probs"], top_k=inp["top_k"], rep_penalty=inp["rep_penalty"],
                               idx_mapping=inp["idx_mapping"], output_bin_counts=counts if penalty else None,
                               seed=seed, offset=off, frequency_penalty=inp.get("freq"),
                               presence_penalty=inp.get("pres"), top_p=inp.get("top_p"),
                               draft_logits=inp["draft_logits"] if dl else None,
                               draft_stats=inp["draft_stats"] if dl else None,
                               draft_temperature=inp["draft_temp"] if dl else None, post_update=pu)
            assert sv.spec_verify_read_error(ctx.h) == 0
            assert np.array_equal(toks.cpu().numpy(), g["tokens"])
            assert np.array_equal(ns.cpu().numpy(), g["num_sampled"])
            assert np.array_equal(nr.cpu().numpy(), g["num_rejected"])
            for got_t, ref_t, want_t in zip((last, counts, ncomp), ref[:3], want[:3]):
                assert np.array_equal(got_t.cpu().numpy(), ref_t)
                assert np.array_equal(got_t.cpu().numpy(), want_t)


def test_post_update_inside_verify_refuses_dbg_probs():
    inp = wl.make_inputs(wl.CONFIGS["1"], DEV)
    with ctx_for(inp) as ctx:
        B, S, V = inp["B"], inp["num_slots"], inp["V"]
        toks = torch.empty((B, 4), dtype=torch.int32, device=DEV)
        ns = torch.empty(B, dtype=torch.int32, device=DEV)
        nr = torch.empty(B, dtype=torch.int32, device=DEV)
        st = [torch.zeros(S, dtype=torch.int32, device=DEV), inp["counts"].clone(),
              torch.zeros(S, dtype=torch.int32, device=DEV)]
        pu = sv.make_post_update_args(inp["idx_mapping"], inp["query_len"], toks, ns, nr, *st)
        probs = torch.empty((inp["R"], V), dtype=torch.float32, device=DEV)
        with pytest.raises(sv.SpecVerifyError):
            sv.spec_verify_run(ctx.h, inp["logits"], inp["draft_ids"], inp["cu"], inp["temperature"], toks, ns, nr,
                               draft_probs=inp["draft_probs"], dbg_probs=probs, post_update=pu)
