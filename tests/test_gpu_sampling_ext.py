"""GPU parity (through the C ABI) of the optional sampling settings: frequency
and presence penalties, top-p on dense rows and on top-k candidate lists, and
synthetic acceptance.  Same acceptance rule as test_gpu_parity (harness)."""
import numpy as np
import pytest
import torch

import workloads as wl
from harness import ctx_for, run_gpu, check_requests

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print(*a, flush=True)


C1, C2, C3, C4, C5 = (wl.CONFIGS[k] for k in ("1", "2", "3", "4", "5"))

CASES = {
    # penalties without top-k: general streaming pass
    "freq_pres_dense_f32": C1.with_(B=6, K=3, V=5003, history=200, freq=0.5, pres=0.3),
    "freq_pres_dense_bf16": C3.with_(B=8, V=6000, history=300, freq=0.7, pres=0.4),
    # ... the vectorised penalty pass with slices over several rows (about ten
    # 1024-token chunks per workgroup, eight chunks per row; items in column order)
    "freq_pres_fast_multirow": C3.with_(B=500, V=8192, history=100, freq=0.5, pres=0.3),
    # ... with up to nine rows per request (the pass's items go request by request)
    "freq_pres_fast_k8": C3.with_(B=200, K=8, V=8192, history=64, freq=0.4, pres=0.2),
    # penalties with top-k: lazy penalty (>= 0) and eager (negative penalty)
    "topk_freq_pres": C4.with_(B=6, K=3, V=4000, history=60, freq=0.5, pres=0.25),
    "topk_negative_freq": C4.with_(B=5, K=2, V=3000, history=60, freq=-0.5, pres=0.1, rep_penalty=1.0),
    # top-p on dense rows: bf16 (keys of 16 bits), fp32, with penalties, draft probs
    "topp_bf16_nodraft": C3.with_(B=12, V=9000 + 8, top_p=0.9),
    "topp_bf16_small_p": C3.with_(B=8, V=5000, top_p=0.3, scale=1.0),
    "topp_f32_probs": C1.with_(B=8, K=4, V=7001, top_p=0.8),
    "topp_penalty": C3.with_(B=8, V=6000, history=300, rep_penalty=1.2, freq=0.3, top_p=0.85),
    "topp_greedy_mix": C2.with_(B=12, V=4000, top_p=0.7),
    "topp_student_t": C5.with_(B=6, V=8000, top_p=0.95),
    # bf16 rows held in registers: at most 128 chunks; one chunk more takes the two-pass kernel
    "topp_resident_max_chunks": C3.with_(B=6, V=131072, top_p=0.9),
    "topp_past_resident_limit": C3.with_(B=6, V=131072 + 8, top_p=0.9),
    "topp_one_partial_chunk": C3.with_(B=10, V=1000, top_p=0.8),
    # a = log2(e) / 0.05: later chunks far above a lane's first chunk move its
    # reference up and are summed again
    "topp_low_temperature": C3.with_(B=8, V=9000 + 8, top_p=0.9, T=0.05),
    # logits near 0: the nucleus reaches past the value window (negative logits),
    # so the bucket path finds the boundary; at scale 0.01 its boundary bucket
    # holds more tokens than the LDS list
    "topp_bucket_fallback": C3.with_(B=6, V=9008, top_p=0.9, scale=0.3),
    "topp_bucket_list_overflow": C3.with_(B=4, V=9008, top_p=0.9, scale=0.01),
    # top-p on top-k candidate lists, and on top-k threshold rows (k > candidates)
    "topk_topp": C4.with_(B=6, K=3, V=4000, history=40, top_p=0.8),
    "topk_big_topp": C4.with_(B=4, K=2, V=9000, top_k=2000, draft_top_k=0, history=30, top_p=0.9),
    # synthetic acceptance
    "synthetic_nodraft": C3.with_(B=16, V=3000, synthetic_rates=(0.9, 0.7, 0.4)),
    "synthetic_probs": C1.with_(B=8, K=4, V=2000, synthetic_rates=(1.0, 0.5, 0.5, 0.0)),
    "synthetic_greedy_mix": C2.with_(B=12, V=3000, synthetic_rates=(0.8, 0.8, 0.6, 0.2)),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_sampling_settings_parity(name):
    w = CASES[name]
    say(f"case {name}: {w}")
    inp = wl.make_inputs(w, DEV)
    tot_margin = 0
    with ctx_for(inp) as ctx:
        for seed, off in [(0, 0), (987654321, 13), (5, 2 ** 31)]:
            g = run_gpu(ctx, inp, seed=seed, offset=off, dbg_probs=True)
            assert g["err"] == 0
            n_margin, bad = check_requests(g, inp, range(inp["B"]), seed, off, probs=True)
            tot_margin += n_margin
            assert not bad, "\n".join(bad[:10])
            K = inp["K"].cpu().numpy()
            assert np.all(g["num_rejected"] == K + 1 - g["num_sampled"])
    say(f"case {name}: margin requests {tot_margin}")


def test_topp_uniform_rows_take_the_row_select():
    # Every logit equal: one bucket holds the whole row (more than the LDS list),
    # so the boundary is selected straight from the row; all tokens tie and stay.
    w = C3.with_(B=3, V=6000, top_p=0.5, ragged=False, K=2)
    inp = wl.make_inputs(w, DEV)
    inp["logits"][:] = 0.25
    with ctx_for(inp) as ctx:
        g = run_gpu(ctx, inp, dbg_probs=True)
    assert g["err"] == 0
    n_margin, bad = check_requests(g, inp, range(3), probs=True)
    assert not bad, "\n".join(bad)
    assert np.allclose(g["probs"], 1.0 / 6000, atol=1e-9)


def test_topp_masked_vocabulary_tail():
    # Logits past a cut are -inf (a masked vocabulary); one row is all -inf and
    # its request is flagged, the others keep their nucleus among the rest.
    import rejection_sampling_verify_05_amd as sv
    w = C3.with_(B=8, V=9008, top_p=0.85)
    inp = wl.make_inputs(w, DEV)
    inp["logits"][:, 5000:] = float("-inf")
    g0 = int(inp["cu"][3].item()) + 3  # first target row of request 3
    inp["logits"][g0] = float("-inf")
    with ctx_for(inp) as ctx:
        g = run_gpu(ctx, inp, seed=3, offset=7, dbg_probs=True)
    assert g["err"] == sv.SV_ERR_ROW
    assert g["num_sampled"][3] == 0 and np.all(g["tokens"][3] == -1)
    ok = [r for r in range(8) if r != 3]
    n_margin, bad = check_requests(g, inp, ok, 3, 7, probs=True)
    assert not bad, "\n".join(bad)
    assert np.all(g["tokens"][ok][g["tokens"][ok] >= 0] < 5000)


def test_topp_at_large_vocab_sampled_rows():
    w = C3.with_(B=64, top_p=0.9)
    inp = wl.make_inputs(w, DEV)
    with ctx_for(inp) as ctx:
        g = run_gpu(ctx, inp, seed=1, offset=4)
    assert g["err"] == 0
    n_margin, bad = check_requests(g, inp, list(range(0, 64, 4)), 1, 4)
    say(f"large vocab top-p: margin requests {n_margin}")
    assert not bad, "\n".join(bad[:10])


def test_setting_errors_are_flagged():
    import rejection_sampling_verify_05_amd as sv
    w = C1.with_(B=5, K=2, V=1500, history=20, freq=0.5, top_p=0.9)
    inp = wl.make_inputs(w, DEV)
    inp["freq"][1] = float("nan")
    inp["top_p"][2] = float("nan")
    with ctx_for(inp) as ctx:
        g = run_gpu(ctx, inp)
        assert g["err"] == sv.SV_ERR_PENALTY | sv.SV_ERR_TOP_P
        for r in (1, 2):
            assert g["num_sampled"][r] == 0 and np.all(g["tokens"][r] == -1)
        n_margin, bad = check_requests(g, inp, [0, 3, 4])
        assert not bad, "\n".join(bad)
        # increasing or out-of-range synthetic rates are refused on the host
        for rates in ([0.5, 0.6], [1.2, 0.5], [0.5, float("nan")]):
            inp["synthetic_rates"] = rates
            with pytest.raises(sv.SpecVerifyError):
                run_gpu(ctx, inp)
