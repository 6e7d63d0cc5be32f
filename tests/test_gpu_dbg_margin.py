"""The library's own decision margins (sv_verify_args.dbg_margin), through the
C ABI: per target row, the smallest relative margin of the accept test and of
the race on the sampled row, recomputed on the device.  Over each request's
rows the smallest must match the oracle's request margin within
harness.MARGIN_ATOL; rows after the sampled row and greedy requests carry
none (+inf).  Covers the modes whose races run in different kernels: the
request epilogue (bonus rows, rows without draft probabilities), its inline
residual (vocabularies of at most eight chunks), the residual kernels, top-k
candidate lists, top-p thresholds, penalties, synthetic acceptance and draft
logits."""
import numpy as np
import pytest
import torch

import rejection_sampling_verify_05_amd as sv
import workloads as wl
from harness import ctx_for, run_gpu, check_margins, run_draft_steps

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print(*a, flush=True)


C1, C2, C3, C4, C5 = (wl.CONFIGS[k] for k in ("1", "2", "3", "4", "5"))

CASES = {
    "nodraft_bf16": C3.with_(B=24, V=9000 + 8),
    "probs_inline_residual_f32": C1.with_(B=16, K=4, V=5003),
    "probs_dense_residual_bf16": C2.with_(B=16, V=20000),
    "greedy_mix": C2.with_(B=12, V=4000),
    "topk_penalty": C4.with_(B=8, K=3, V=4000, history=60),
    "topp_resident": C3.with_(B=12, V=9000 + 8, top_p=0.9),
    "topp_f32_probs": C1.with_(B=8, K=4, V=7001, top_p=0.8),
    "freq_pres": C3.with_(B=8, V=6000, history=300, freq=0.7, pres=0.4),
    "synthetic": C3.with_(B=16, V=3000, synthetic_rates=(0.9, 0.7, 0.4)),
    "student_t": C5.with_(B=8, V=8000),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_dbg_margin_matches_oracle(name):
    w = CASES[name]
    say(f"case {name}: {w}")
    inp = wl.make_inputs(w, DEV)
    with ctx_for(inp) as ctx:
        n_all = 0
        for seed, off in [(0, 0), (987654321, 13)]:
            g = run_gpu(ctx, inp, seed=seed, offset=off, dbg_margin=True)
            assert g["err"] == 0
            n, bad = check_margins(g, inp, range(inp["B"]), seed, off)
            assert not bad, "\n".join(bad[:10])
            n_all += n
        say(f"case {name}: {n_all} requests compared")
        assert n_all >= inp["B"]  # nearly every request of both runs


def test_dbg_margin_draft_logits():
    w = C3.with_(B=16, V=6000, draft_logits=True, draft_T=1.2)
    inp = wl.make_inputs(w, DEV)
    with ctx_for(inp) as ctx:
        run_draft_steps(ctx, inp, seed=4, offset=1)
        g = run_gpu(ctx, inp, seed=4, offset=1, dbg_margin=True)
    assert g["err"] == 0
    n, bad = check_margins(g, inp, range(inp["B"]), 4, 1)
    assert not bad, "\n".join(bad[:10])
    assert n >= inp["B"] // 2


def test_dbg_margin_headline_size_sampled():
    # B=256, V=128256 bf16, no draft probabilities: every row gets a margin,
    # compared on every 8th request
    inp = wl.make_inputs(C3, DEV)
    with ctx_for(inp) as ctx:
        g = run_gpu(ctx, inp, seed=7, offset=3, dbg_margin=True)
    assert g["err"] == 0
    n, bad = check_margins(g, inp, range(0, inp["B"], 8), 7, 3)
    assert not bad, "\n".join(bad[:10])
    assert n >= 28
    mr = g["margin_rows"]
    assert not np.any(mr == -7.0)  # every row written


def test_dbg_margin_refused_with_post_update():
    inp = wl.make_inputs(C1, DEV)
    with ctx_for(inp) as ctx:
        B, S = inp["B"], inp["num_slots"]
        toks = torch.empty((B, 4), dtype=torch.int32, device=DEV)
        ns = torch.empty(B, dtype=torch.int32, device=DEV)
        nr = torch.empty(B, dtype=torch.int32, device=DEV)
        st = [torch.zeros(S, dtype=torch.int32, device=DEV), inp["counts"].clone(),
              torch.zeros(S, dtype=torch.int32, device=DEV)]
        pu = sv.make_post_update_args(inp["idx_mapping"], inp["query_len"], toks, ns, nr, *st)
        mrows = torch.empty(inp["R"], dtype=torch.float32, device=DEV)
        with pytest.raises(sv.SpecVerifyError):
            sv.spec_verify_run(ctx.h, inp["logits"], inp["draft_ids"], inp["cu"], inp["temperature"], toks, ns, nr,
                               draft_probs=inp["draft_probs"], dbg_margin=mrows, post_update=pu)


def test_dbg_margin_of_flagged_requests_is_infinite():
    # requests written empty (bad temperature, bad penalty, slot out of range,
    # a row with no finite logit) took no decision: +inf on every row of
    # theirs; the valid requests keep their margins, matched to the oracle
    w = C4.with_(B=6, K=2, V=1500, history=20)
    inp = wl.make_inputs(w, DEV)
    inp["temperature"][1] = -1.0
    inp["rep_penalty"][2] = 0.0
    inp["idx_mapping"][3] = 10 ** 6
    g0 = int(inp["cu"][4].item()) + 4
    inp["logits"][g0 + 1] = float("-inf")
    with ctx_for(inp) as ctx:
        g = run_gpu(ctx, inp, dbg_margin=True)
    assert g["err"] != 0
    cu = inp["cu"].cpu().numpy()
    mr = g["margin_rows"]
    for r in (1, 2, 3, 4):
        rows = mr[cu[r] + r:cu[r + 1] + r + 1]
        assert np.all(np.isinf(rows) & (rows > 0)), (r, rows)
    n, bad = check_margins(g, inp, [0, 5])
    assert not bad, "\n".join(bad)
    assert n == 2
