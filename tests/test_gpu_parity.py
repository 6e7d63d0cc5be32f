"""Parity of the HIP verify path (through the C ABI) with the CPU oracle on the
five workloads and their edge cases.  Bit-exact on tokens, num_sampled and
num_rejected outside margin requests; probabilities within 1e-6."""
import numpy as np
import pytest
import torch

import workloads as wl
from harness import ctx_for, run_gpu, check_requests, Ctx

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("cid", ["1", "2"])
def test_small_configs_full_parity(cid):
    w = wl.CONFIGS[cid]
    say(f"config {cid}: {w}")
    inp = wl.make_inputs(w, DEV)
    with ctx_for(inp) as ctx:
        g = run_gpu(ctx, inp, seed=0, offset=0, dbg_probs=True)
    assert g["err"] == 0
    n_margin, bad = check_requests(g, inp, range(inp["B"]), probs=True)
    say(f"config {cid}: margin requests {n_margin}, mismatches {len(bad)}")
    assert not bad, "\n".join(bad[:10])
    K = inp["K"].cpu().numpy()
    assert np.all(g["num_sampled"] >= 1) and np.all(g["num_sampled"] <= K + 1)
    assert np.all(g["num_rejected"] == K + 1 - g["num_sampled"])


EDGE = {
    # V below one chunk, not a multiple of 8 (no vector loads on the tail)
    "tiny_vocab": wl.CONFIGS["1"].with_(B=7, V=37, ragged=True),
    # single token vocabulary: p = 1
    "vocab_1": wl.CONFIGS["1"].with_(B=3, V=1),
    # several chunks with a ragged tail, bf16, no-draft mode, all K
    "ragged_tail_bf16": wl.CONFIGS["3"].with_(B=16, V=5000 + 3),
    # bonus-only requests (K_r = 0 everywhere)
    "bonus_only": wl.CONFIGS["3"].with_(B=9, K=0, V=3000),
    # greedy everywhere on integer-valued bf16 logits: many ties
    "greedy_ties": wl.CONFIGS["2"].with_(B=12, V=2048, greedy_every=1, scale=0.7),
    # fp32 draft-probs with V not a multiple of 4
    "f32_odd": wl.CONFIGS["1"].with_(B=6, K=5, V=4099),
    # top-k with penalty on a small vocabulary; k = 1 and k = 7
    "topk_small": wl.CONFIGS["4"].with_(B=6, K=3, V=3000, history=40),
    "topk_k1": wl.CONFIGS["4"].with_(B=5, K=2, V=2100, top_k=1, history=10),
    # top-k larger than the candidate capacity: dense threshold path
    "topk_big_k": wl.CONFIGS["4"].with_(B=4, K=2, V=9000, top_k=2000, draft_top_k=0, history=30),
    # penalty without top-k: dense penalty path
    "penalty_dense": wl.CONFIGS["4"].with_(B=5, K=3, V=4100, top_k=0, draft_top_k=0, history=300),
    # no-draft mode with top-k
    "topk_no_draft": wl.CONFIGS["3"].with_(B=8, V=3000, top_k=20, rep_penalty=1.3, history=50),
    # the top-k pass's first threshold: k = 256 (the largest k taken from the
    # threads' maxima), k = 300 (exact selection over the first 2048 tokens),
    # and a row shorter than the first 2048 tokens
    "topk_k256": wl.CONFIGS["4"].with_(B=4, K=2, V=9000, top_k=256, draft_top_k=0, history=60),
    "topk_k300": wl.CONFIGS["4"].with_(B=4, K=2, V=9000, top_k=300, draft_top_k=0, history=60),
    # k above the 256 threads of a row: the first threshold is the exact k-th
    # largest of the first tokens (fp32 and bf16 rows)
    "topk_k700": wl.CONFIGS["4"].with_(B=4, K=2, V=9000, top_k=700, draft_top_k=0, history=60),
    "topk_bf16_k300": wl.CONFIGS["3"].with_(B=4, V=9000, top_k=300, rep_penalty=1.2, history=50),
    "topk_short_row": wl.CONFIGS["4"].with_(B=5, K=2, V=1500, top_k=30, history=40),
}


@pytest.mark.parametrize("name", sorted(EDGE))
def test_edge_cases(name):
    w = EDGE[name]
    say(f"edge {name}: {w}")
    inp = wl.make_inputs(w, DEV)
    if name == "greedy_ties":
        inp["logits"] = inp["logits"].float().round().to(inp["logits"].dtype)
    with ctx_for(inp) as ctx:
        for seed, off in [(0, 0), (12345678901, 77)]:
            g = run_gpu(ctx, inp, seed=seed, offset=off, dbg_probs=True)
            assert g["err"] == 0
            n_margin, bad = check_requests(g, inp, range(inp["B"]), seed, off, probs=True)
            assert not bad, "\n".join(bad[:10])


def test_uniform_rows_and_ties_in_top_k():
    # All logits equal: top-k keeps every token (ties), so the kept set exceeds
    # the candidate capacity and the threshold path handles it; p = 1/V.
    w = wl.CONFIGS["4"].with_(B=3, K=2, V=2500, history=0, rep_penalty=1.0)
    inp = wl.make_inputs(w, DEV)
    inp["logits"][:] = 0.5
    with ctx_for(inp) as ctx:
        g = run_gpu(ctx, inp, dbg_probs=True)
    assert g["err"] == 0
    n_margin, bad = check_requests(g, inp, range(3), probs=True)
    assert not bad, "\n".join(bad)
    assert np.allclose(g["probs"], 1.0 / 2500, atol=1e-9)


def test_invalid_draft_ids_are_rejected():
    w = wl.CONFIGS["1"].with_(B=6, K=3, V=2000)
    inp = wl.make_inputs(w, DEV)
    inp["draft_ids"][0] = -1
    inp["draft_ids"][4] = 2000
    inp["draft_ids"][8] = 2 ** 31 - 1
    for mode in ("probs", "nodraft"):
        if mode == "nodraft":
            inp["draft_probs"] = None
        with ctx_for(inp) as ctx:
            g = run_gpu(ctx, inp)
        assert g["err"] == 0
        assert g["num_rejected"][0] == 3 and g["num_sampled"][0] == 1
        assert g["num_sampled"][1] <= 2 and g["num_sampled"][2] <= 3
        n_margin, bad = check_requests(g, inp, range(6))
        assert not bad, "\n".join(bad)


@pytest.mark.parametrize("V", [3000, 8192, 8200, 70000])
def test_empty_residual_races_over_p(V):
    # Every draft probability 1: max(0, p - q) is 0 everywhere, so a rejected
    # row races over p itself.  Up to 8 chunks (V <= 8192) the residual is
    # taken inside the epilogue, beyond that by the residual kernels.
    w = wl.CONFIGS["1"].with_(B=16, K=3, V=V)
    inp = wl.make_inputs(w, DEV)
    inp["draft_probs"][:] = 1.0
    with ctx_for(inp) as ctx:
        for seed, off in [(0, 0), (11, 5)]:
            g = run_gpu(ctx, inp, seed=seed, offset=off)
            assert g["err"] == 0
            n_margin, bad = check_requests(g, inp, range(inp["B"]), seed, off)
            assert not bad, "\n".join(bad)
            assert (g["num_sampled"] < inp["K"].cpu().numpy() + 1).any()  # some rows rejected


def test_request_errors_are_flagged_and_isolated():
    import rejection_sampling_verify_05_amd as sv
    w = wl.CONFIGS["4"].with_(B=6, K=2, V=1500, history=20)
    inp = wl.make_inputs(w, DEV)
    inp["temperature"][1] = -1.0
    inp["rep_penalty"][2] = 0.0
    inp["idx_mapping"][3] = 10 ** 6
    g0 = int(inp["cu"][4].item()) + 4
    inp["logits"][g0 + 1] = float("-inf")
    with ctx_for(inp) as ctx:
        g = run_gpu(ctx, inp)
    assert g["err"] == sv.SV_ERR_TEMPERATURE | sv.SV_ERR_PENALTY | sv.SV_ERR_SLOT | sv.SV_ERR_ROW
    for r in (1, 2, 3, 4):
        assert g["num_sampled"][r] == 0 and g["num_rejected"][r] == 0
        assert np.all(g["tokens"][r] == -1)
    n_margin, bad = check_requests(g, inp, [0, 5])
    assert not bad, "\n".join(bad)


def test_invalid_cu_is_flagged():
    import rejection_sampling_verify_05_amd as sv
    w = wl.CONFIGS["1"].with_(B=5, K=2, V=1100)
    inp = wl.make_inputs(w, DEV)
    inp["cu"][2] = 7   # cu = 0 2 7 6 8 10: not monotone
    with ctx_for(inp) as ctx:
        g = run_gpu(ctx, inp)
        assert g["err"] & sv.SV_ERR_CU
        # the context recovers: a valid call right after is exact
        inp2 = wl.make_inputs(w, DEV)
        g = run_gpu(ctx, inp2)
        assert g["err"] == 0
        n_margin, bad = check_requests(g, inp2, range(5))
        assert not bad, "\n".join(bad)


def test_determinism_across_launches():
    w = wl.CONFIGS["3"].with_(B=64, V=40000)
    inp = wl.make_inputs(w, DEV)
    with ctx_for(inp) as ctx:
        first = run_gpu(ctx, inp, seed=3, offset=9)
        for _ in range(100):
            g = run_gpu(ctx, inp, seed=3, offset=9)
            assert np.array_equal(g["tokens"], first["tokens"])
            assert np.array_equal(g["num_sampled"], first["num_sampled"])


def test_strided_logits_rows():
    w = wl.CONFIGS["2"].with_(B=8, V=3000)
    inp = wl.make_inputs(w, DEV)
    wide = torch.zeros((inp["R"], 3000 + 24), dtype=inp["logits"].dtype, device=DEV)
    wide[:, :3000] = inp["logits"]
    inp["logits"] = wide[:, :3000]
    with ctx_for(inp) as ctx:
        g = run_gpu(ctx, inp)
    n_margin, bad = check_requests(g, inp, range(8))
    assert not bad, "\n".join(bad)


@pytest.mark.parametrize("dtype,V", [(torch.bfloat16, 1001), (torch.bfloat16, 2053), (torch.float32, 2047),
                                     (torch.bfloat16, 9003)])
def test_topk_aligned_rows_ragged_tail(dtype, V):
    # Aligned rows (the row stride padded to whole 16-byte vectors) whose
    # length is not: the top-k pass streams whole vectors and takes the last
    # V % (16 / element size) tokens apart, also when they fall in its first
    # 2048 tokens.
    w = wl.CONFIGS["4"].with_(B=4, K=2, V=V, dtype=dtype, top_k=20, draft_top_k=0, history=30)
    inp = wl.make_inputs(w, DEV)
    wide = torch.zeros((inp["R"], (V + 7) // 8 * 8 + 8), dtype=dtype, device=DEV)
    wide[:, :V] = inp["logits"]
    inp["logits"] = wide[:, :V]
    with ctx_for(inp) as ctx:
        g = run_gpu(ctx, inp, seed=5, offset=3, dbg_probs=True)
    assert g["err"] == 0
    n_margin, bad = check_requests(g, inp, range(inp["B"]), 5, 3, probs=True)
    assert not bad, "\n".join(bad[:10])


@pytest.mark.parametrize("draft_probs", [False, True])
def test_chunk_scale_ramps(draft_probs):
    # Rows whose chunks differ in mass by far more than 2^20: logits ramp up or
    # down by 6 per 1024-token chunk, plus one row with a single spiked chunk.
    # bf16 with V a multiple of 8 takes the fast streaming pass, which then
    # meets chunks far above and far below the first chunk it saw in a row.
    w = wl.CONFIGS["3"].with_(B=8, V=40000 + 8, ragged=False, K=2)
    if draft_probs:
        w = wl.CONFIGS["1"].with_(B=8, K=2, V=40000 + 8, dtype=torch.bfloat16)
    inp = wl.make_inputs(w, DEV)
    R, V = inp["R"], inp["V"]
    chunk = torch.arange(V, device=DEV) // 1024
    lg = inp["logits"].float()
    for r in range(R):
        kind = r % 3
        if kind == 0:
            lg[r] += 6.0 * chunk
        elif kind == 1:
            lg[r] -= 6.0 * chunk
        else:
            lg[r, (chunk == 17 + r % 5)] += 60.0
    inp["logits"] = lg.to(inp["logits"].dtype)
    with ctx_for(inp) as ctx:
        for seed, off in [(0, 0), (99, 5)]:
            g = run_gpu(ctx, inp, seed=seed, offset=off, dbg_probs=True)
            assert g["err"] == 0
            n_margin, bad = check_requests(g, inp, range(inp["B"]), seed, off, probs=True)
            say(f"ramps draft_probs={draft_probs} seed {seed}: margin {n_margin}, mismatches {len(bad)}")
            assert not bad, "\n".join(bad[:10])


@pytest.mark.parametrize("scale", [0.3, 3.0])
def test_nodraft_drafts_at_heavy_tokens(scale):
    # Without draft probabilities, the rejected draft is removed from the race:
    # with drafts at each row's heaviest token, the draft's chunk holds much of
    # the row's mass, so the race must weigh that chunk without the draft (the
    # epilogue loads it only when it could win) -- at scale 0.3 nearly every
    # chunk competes, at 3.0 the heavy chunk usually wins.
    w = wl.CONFIGS["3"].with_(B=48, V=9000 + 8, scale=scale)
    inp = wl.make_inputs(w, DEV)
    cu = inp["cu"].cpu().numpy()
    lg = inp["logits"].float()
    for r in range(inp["B"]):
        for i in range(int(cu[r + 1] - cu[r])):
            g = int(cu[r]) + r + i
            inp["draft_ids"][int(cu[r]) + i] = int(torch.argmax(lg[g]).item())
    with ctx_for(inp) as ctx:
        for seed, off in [(0, 0), (3, 1), (77, 9)]:
            g = run_gpu(ctx, inp, seed=seed, offset=off)
            assert g["err"] == 0
            n_margin, bad = check_requests(g, inp, range(inp["B"]), seed, off)
            assert not bad, "\n".join(bad[:10])
