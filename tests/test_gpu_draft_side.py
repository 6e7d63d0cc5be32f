"""GPU parity of draft-side sampling (spec_draft_sample, one call per draft
position) and of verification in draft-logits mode, through the C ABI, against
the oracle's draft sampler and its verification with fp64 draft
distributions.  Same acceptance rule as test_gpu_parity (harness)."""
import numpy as np
import pytest
import torch

import workloads as wl
from harness import ctx_for, run_gpu, check_requests, run_draft_steps, check_draft_tokens

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print(*a, flush=True)


C1, C2, C3, C4 = (wl.CONFIGS[k] for k in ("1", "2", "3", "4"))

CASES = {
    "bf16_nodraft_base": C3.with_(B=24, V=9000 + 8, draft_logits=True, draft_T=1.0),
    "f32_odd_vocab": C1.with_(B=8, K=4, V=5003, draft_probs=False, draft_logits=True, draft_T=0.9),
    "greedy_mix": C2.with_(B=16, V=6000, draft_probs=False, draft_logits=True),
    "topk_penalty": C4.with_(B=6, K=3, V=4000, history=40, draft_probs=False, draft_logits=True,
                             draft_top_k=0),
    "topp": C3.with_(B=12, V=6000, top_p=0.8, draft_logits=True, draft_T=1.2),
    "high_acceptance": C3.with_(B=16, V=4000, draft_logits=True, draft_noise=0.05),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_draft_side_parity(name):
    w = CASES[name]
    say(f"case {name}: {w}")
    inp = wl.make_inputs(w, DEV)
    with ctx_for(inp) as ctx:
        for seed, off in [(0, 0), (31337, 9)]:
            q = run_draft_steps(ctx, inp, seed=seed, offset=off)
            n_dm, bad = check_draft_tokens(inp, q, seed, off)
            assert not bad, "\n".join(bad[:10])
            g = run_gpu(ctx, inp, seed=seed, offset=off, dbg_probs=True)
            assert g["err"] == 0
            n_margin, bad = check_requests(g, inp, range(inp["B"]), seed, off, probs=True)
            say(f"case {name} seed {seed}: draft margin {n_dm}, verify margin {n_margin}")
            assert not bad, "\n".join(bad[:10])
            K = inp["K"].cpu().numpy()
            assert np.all(g["num_rejected"] == K + 1 - g["num_sampled"])


def test_draft_side_headline_size_sampled():
    w = C3.with_(draft_logits=True)
    inp = wl.make_inputs(w, DEV)
    with ctx_for(inp) as ctx:
        q = run_draft_steps(ctx, inp, seed=2, offset=5)
        g = run_gpu(ctx, inp, seed=2, offset=5)
    assert g["err"] == 0
    reqs = list(range(0, inp["B"], 8))
    n_dm, bad = check_draft_tokens(inp, q, 2, 5, requests=reqs)
    assert not bad, "\n".join(bad[:10])
    n_margin, bad = check_requests(g, inp, reqs, 2, 5)
    say(f"headline size: verify margin {n_margin}")
    assert not bad, "\n".join(bad[:10])


def test_draft_sample_skips_positions_beyond_k():
    w = C3.with_(B=10, V=3000, draft_logits=True, ragged=True, K=3)
    inp = wl.make_inputs(w, DEV)
    import rejection_sampling_verify_05_amd as sv
    with ctx_for(inp) as ctx:
        cu = inp["cu"]
        K = inp["K"]
        D = inp["D"]
        stats = torch.full((2 * D,), -7.0, device=DEV)
        rows = torch.clamp(cu[:-1].long() + 2, max=D - 1)
        tok = torch.full((10,), -9, dtype=torch.int32, device=DEV)
        sv.spec_draft_sample(ctx.h, inp["draft_logits"][rows].contiguous(), inp["draft_temp"], cu, tok, stats,
                             step=2)
        torch.cuda.synchronize()
    t = tok.cpu().numpy()
    k = K.cpu().numpy()
    assert np.all(t[k <= 2] == -1) and np.all(t[k > 2] >= 0)
