"""The allocation-free entry point (spec_verify_run_noalloc, through the C
ABI) against spec_verify_run on the same inputs.  The two share kernels and
grids, so their outputs must be identical.  Each workload runs two calls in a
row, the second with a smaller input, so the fixed scratch array holds the
first call's contents when the second starts.  The workloads cover the plain
no-draft path, draft probabilities (residual tables), top-p (row states), and
post_update inside the call.  Capacity limits and the device error word are
checked too."""
import numpy as np
import pytest
import torch

import rejection_sampling_verify_05_amd as sv
import workloads as wl
from harness import Ctx, run_gpu, check_all

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def run_noalloc(inp, seed, offset, out_stride, errs, stream=None):
    B, D = inp["B"], inp["D"]
    out = torch.full((B, out_stride), -7, dtype=torch.int32, device=DEV)
    ns = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    nr = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    pd = torch.full((max(D, 1),), -7.0, dtype=torch.float32, device=DEV)
    sv.spec_verify_run_noalloc(inp["logits"], inp["draft_ids"], inp["cu"], inp["temperature"], out, ns, nr,
                               draft_probs=inp["draft_probs"], seed=seed, offset=offset,
                               dbg_p_draft=pd if D else None, top_p=inp.get("top_p"),
                               synthetic_rates=inp.get("synthetic_rates"), device_errors=errs, stream=stream)
    torch.cuda.synchronize()
    return dict(tokens=out.cpu().numpy(), num_sampled=ns.cpu().numpy(), num_rejected=nr.cpu().numpy(),
                p_draft=pd[:D].cpu().numpy())


PAIRS = {
    "no_draft": (wl.CONFIGS["3"].with_(B=200, V=50000), wl.CONFIGS["3"].with_(B=37, V=50000)),
    "draft_probs": (wl.CONFIGS["1"].with_(B=48, K=4, V=20000, dtype=torch.bfloat16),
                    wl.CONFIGS["1"].with_(B=9, K=4, V=7000)),
    "top_p": (wl.CONFIGS["3p"].with_(B=40, V=30000), wl.CONFIGS["3p"].with_(B=11, V=12000)),
    "headline_then_small": (wl.CONFIGS["3"], wl.CONFIGS["3"].with_(B=20, V=128256)),
}


@pytest.mark.parametrize("name", sorted(PAIRS))
def test_noalloc_matches_spec_verify_run(name):
    errs = torch.zeros(1, dtype=torch.int32, device=DEV)
    for k, w in enumerate(PAIRS[name]):
        inp = wl.make_inputs(w, DEV, salt=k)
        stride = int(inp["K"].max().item()) + 1
        say(f"{name} call {k}: B={inp['B']} R={inp['R']} V={inp['V']}")
        for seed, off in [(5, 0), (2 ** 33 + 7, 41)]:
            g = run_noalloc(inp, seed, off, stride, errs)
            assert int(errs.item()) == 0
            with Ctx(inp["R"], inp["B"], stride - 1, inp["V"]) as ctx:
                ref = run_gpu(ctx, inp, seed=seed, offset=off, out_stride=stride)
            assert ref["err"] == 0
            for key in ("tokens", "num_sampled", "num_rejected", "p_draft"):
                assert np.array_equal(g[key], ref[key]), (name, k, key)
        if name != "headline_then_small":
            n_margin, bad = check_all(dict(g, err=0), inp, range(inp["B"]), seed, off)
            assert not bad, "\n".join(bad[:10])


def test_noalloc_post_update_and_errors():
    w = wl.CONFIGS["3"].with_(B=64, V=16384, greedy_every=4)
    inp = wl.make_inputs(w, DEV)
    B, V, S = inp["B"], inp["V"], inp["num_slots"]
    states = []
    for mode in ("ctx", "noalloc"):
        st = [torch.zeros(S, dtype=torch.int32, device=DEV), inp["counts"].clone(),
              torch.zeros(S, dtype=torch.int32, device=DEV)]
        out = torch.full((B, 4), -7, dtype=torch.int32, device=DEV)
        ns = torch.full((B,), -7, dtype=torch.int32, device=DEV)
        nr = torch.full((B,), -7, dtype=torch.int32, device=DEV)
        pu = sv.make_post_update_args(inp["idx_mapping"], inp["query_len"], out, ns, nr, *st)
        errs = torch.zeros(1, dtype=torch.int32, device=DEV)
        with Ctx(inp["R"], B, 3, V) as ctx:
            for off in range(3):
                if mode == "ctx":
                    sv.spec_verify_run(ctx.h, inp["logits"], inp["draft_ids"], inp["cu"], inp["temperature"], out,
                                       ns, nr, seed=8, offset=off, post_update=pu)
                else:
                    sv.spec_verify_run_noalloc(inp["logits"], inp["draft_ids"], inp["cu"], inp["temperature"], out,
                                               ns, nr, seed=8, offset=off, post_update=pu, device_errors=errs)
            torch.cuda.synchronize()
        assert int(errs.item()) == 0
        states.append([x.cpu().numpy() for x in st] + [out.cpu().numpy()])
    for a, b in zip(*states):
        assert np.array_equal(a, b)
    # device-side errors land in the caller's word; the call's other requests are unaffected
    bad = dict(inp)
    bad["temperature"] = inp["temperature"].clone()
    bad["temperature"][5] = -2.0
    errs = torch.zeros(1, dtype=torch.int32, device=DEV)
    g = run_noalloc(bad, 1, 1, 4, errs)
    assert int(errs.item()) == sv.SV_ERR_TEMPERATURE
    assert g["num_sampled"][5] == 0 and np.all(g["tokens"][5] == -1)
    # limits: top-k, and more rows than the fixed array holds
    with pytest.raises(sv.SpecVerifyError) as e:
        big = wl.make_inputs(wl.CONFIGS["4"].with_(B=2, K=2, V=3000, history=5), DEV)
        sv.spec_verify_run_noalloc(big["logits"], big["draft_ids"], big["cu"], big["temperature"],
                                   torch.empty((2, 3), dtype=torch.int32, device=DEV),
                                   torch.empty(2, dtype=torch.int32, device=DEV),
                                   torch.empty(2, dtype=torch.int32, device=DEV), top_k=big["top_k"],
                                   draft_probs=big["draft_probs"], device_errors=errs)
    assert e.value.status == sv.SV_ECAPACITY
    B, K, V = 4000, 4, 1024  # 20000 rows: more than SV_NOALLOC_MAX_ROWS
    R = B * (K + 1)
    lg = torch.empty((R, V), dtype=torch.bfloat16, device=DEV)
    cu = torch.arange(0, B * K + 1, K, dtype=torch.int32, device=DEV)
    with pytest.raises(sv.SpecVerifyError) as e:
        sv.spec_verify_run_noalloc(lg, torch.zeros(B * K, dtype=torch.int32, device=DEV), cu,
                                   torch.ones(B, dtype=torch.float32, device=DEV),
                                   torch.empty((B, K + 1), dtype=torch.int32, device=DEV),
                                   torch.empty(B, dtype=torch.int32, device=DEV),
                                   torch.empty(B, dtype=torch.int32, device=DEV), device_errors=errs)
    assert e.value.status == sv.SV_ECAPACITY
