"""The seeded input generators: deterministic, the stated shapes and layout."""
import torch

import workloads as wl


def test_deterministic_and_shaped():
    for cid in ("1", "2"):
        w = wl.CONFIGS[cid]
        a = wl.make_inputs(w, "cpu")
        b = wl.make_inputs(w, "cpu")
        assert torch.equal(a["logits"].float(), b["logits"].float())
        assert torch.equal(a["draft_ids"], b["draft_ids"])
        assert a["logits"].shape == (a["R"], w.V) and a["logits"].dtype == w.dtype
        assert a["R"] == a["D"] + a["B"] == w.B * (w.K + 1)
        assert torch.allclose(a["draft_probs"].sum(1), torch.ones(a["D"]), atol=1e-5)
    c = wl.make_inputs(wl.CONFIGS["2"], "cpu", salt=1)
    assert not torch.equal(c["logits"].float(), a["logits"].float())


def test_ragged_layout_and_greedy_mix():
    w = wl.CONFIGS["3"].with_(B=64, V=512)
    a = wl.make_inputs(w, "cpu")
    K = a["K"]
    assert int(K.min()) >= 0 and int(K.max()) <= 3 and len(set(K.tolist())) > 1
    assert torch.equal(a["cu"][1:] - a["cu"][:-1], K)
    assert a["draft_probs"] is None and a["R"] == int(K.sum()) + 64
    g = wl.make_inputs(wl.CONFIGS["2"].with_(B=8, V=300), "cpu")
    assert (g["temperature"] == 0).sum() == 2


def test_history_counts():
    w = wl.CONFIGS["4"].with_(B=6, K=2, V=700)
    a = wl.make_inputs(w, "cpu")
    cnt = a["counts"]
    assert int(cnt[a["idx_mapping"].long()].sum(1).min()) == w.history
    assert int(cnt.sum()) == w.B * w.history
    assert len(set(a["idx_mapping"].tolist())) == w.B
