"""Seeded synthetic inputs for the verify step.

This module only produces inputs: target logits, draft tokens (and the draft
distribution they were sampled from), per-request settings and post_update
state.  It holds none of the verify method's arithmetic; the draft softmax
below is the draft model's output distribution, an input of the method.  Both
the HIP path and the CPU oracle are fed the tensors made here.

Workloads (sizes and distributions of the five benchmark configurations):
  1  tiny         B=4,    K=3,        V=1024,   fp32 N(0,2^2),  draft probs, T=1.0
  2  mixed        B=64,   K=4,        V=32000,  bf16 N(0,2^2),  draft probs, T=0.8,
                  every 4th request greedy (T=0)
  3  no-draft     B=256,  K_r~U{0..3}, V=128256, bf16 N(0,3^2), draft ids only, T=1.0
  3' no-draft-k3  as 3 with K_r = 3
  4  topk-pen     B=512,  K=8,        V=151936, fp32 N(0,2^2),  draft probs, top-k 50,
                  T=0.7, repetition penalty 1.1 from a 512-token history per request
  5  stress       B=1024, K=5,        V=256000, bf16 3*t_3,     draft probs, T=1.0

LM-head workloads (make_lm_head_inputs): hidden states N(0,1) and an LM-head
weight N(0, (scale / sqrt(d))^2), both bf16, so the target logits W h are about
N(0, scale^2) (scale 3 as config 3); config 3's request mix (B=256, K_r ~
U{0..3}, V=128256) with d=4096, the hidden size of the models with that
vocabulary.  Drafts: d = argmax(W h + N(0,1)) (the fp32 product here is only
an input generator).

Draft side: draft logits = target + N(0,1) (config 5: 0.9*target + N(0,0.5^2));
in draft-probs mode q = softmax(draft logits / T_draft) (config 4: over the
draft's own top 50) and d ~ q; in the no-draft mode (and for greedy requests)
d = argmax(draft logits).  All randomness comes from one torch.Generator
seeded with 1000 + config id (plus the caller's salt), on the device the
tensors are made on.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    cid: str
    name: str
    B: int
    K: int               # drafts per request (max when ragged)
    V: int
    dtype: torch.dtype   # target logits dtype
    logits: str          # "normal" or "student_t3"
    scale: float
    T: float
    draft_probs: bool
    ragged: bool = False
    greedy_every: int = 0        # every n-th request greedy (0: none)
    draft_T: float = 1.0
    draft_top_k: int = 0
    top_k: int = 0
    rep_penalty: float = 1.0
    history: int = 0             # tokens in each request's output history (counts)
    draft_mix: float = 1.0       # draft logits = mix * target + noise_scale * N(0,1)
    draft_noise: float = 1.0
    freq: float = 0.0            # frequency penalty of most requests (every 5th: none)
    pres: float = 0.0            # presence penalty of most requests (every 5th: none)
    top_p: float = 1.0           # top-p of most requests (every 7th: none)
    synthetic_rates: tuple = ()  # synthetic acceptance rates of positions 1.. (empty: off)
    draft_logits: bool = False   # keep the draft logits (target dtype) for draft-side sampling

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def rows_hint(self) -> int:
        return self.B * ((self.K / 2 if self.ragged else self.K) + 1)


CONFIGS = {
    "1": Workload("1", "tiny", 4, 3, 1024, torch.float32, "normal", 2.0, 1.0, True),
    "2": Workload("2", "mixed", 64, 4, 32000, torch.bfloat16, "normal", 2.0, 0.8, True,
                  greedy_every=4, draft_T=0.8),
    "3": Workload("3", "no-draft", 256, 3, 128256, torch.bfloat16, "normal", 3.0, 1.0, False,
                  ragged=True),
    "3k3": Workload("3k3", "no-draft-k3", 256, 3, 128256, torch.bfloat16, "normal", 3.0, 1.0,
                    False),
    "4": Workload("4", "topk-pen", 512, 8, 151936, torch.float32, "normal", 2.0, 0.7, True,
                  draft_T=0.7, draft_top_k=50, top_k=50, rep_penalty=1.1, history=512),
    "5": Workload("5", "stress", 1024, 5, 256000, torch.bfloat16, "student_t3", 3.0, 1.0, True,
                  draft_mix=0.9, draft_noise=0.5),
}
# The headline and top-k workloads with the optional sampling settings switched
# on (measurement of those paths; same sizes as their base workloads).
CONFIGS.update({
    "3p": CONFIGS["3"].with_(cid="3p", name="no-draft top-p 0.9", top_p=0.9),
    "3f": CONFIGS["3"].with_(cid="3f", name="no-draft freq 0.5 pres 0.3", freq=0.5, pres=0.3, history=512),
    "3s": CONFIGS["3"].with_(cid="3s", name="no-draft synthetic (0.8, 0.6, 0.4)", synthetic_rates=(0.8, 0.6, 0.4)),
    "3d": CONFIGS["3"].with_(cid="3d", name="draft-side sampling, draft logits bf16 at T 1", draft_logits=True),
    "4f": CONFIGS["4"].with_(cid="4f", name="topk-pen freq 0.5 pres 0.25", freq=0.5, pres=0.25),
    "4p": CONFIGS["4"].with_(cid="4p", name="topk-pen top-p 0.8", top_p=0.8),
})


def _seed_of(cid: str) -> int:
    return 1000 + {"1": 1, "2": 2, "3": 3, "3k3": 3, "4": 4, "5": 5}.get(cid.rstrip("pfsd"), 9)


def make_inputs(w: Workload, device="cpu", salt: int = 0, slots_extra: int = 64) -> dict:
    """Build every tensor of one verify step (plus post_update state) for
    workload `w` on `device`.  Deterministic in (w, device type, salt)."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(_seed_of(w.cid) * 1000003 + salt)
    B, V = w.B, w.V

    if w.ragged:
        K = torch.randint(0, w.K + 1, (B,), generator=gen, device=dev)
    else:
        K = torch.full((B,), w.K, device=dev)
    cu = torch.zeros(B + 1, dtype=torch.int32, device=dev)
    cu[1:] = torch.cumsum(K, 0).to(torch.int32)
    D = int(cu[-1].item())
    R = D + B

    # target logits, generated in fp32 and rounded (RNE) to the target dtype
    if w.logits == "normal":
        t32 = torch.randn((R, V), generator=gen, device=dev) * w.scale
    else:  # Student-t with 3 degrees of freedom: N / sqrt(chi2_3 / 3)
        t32 = torch.randn((R, V), generator=gen, device=dev)
        chi = torch.zeros((R, V), device=dev)
        for _ in range(3):
            chi.add_(torch.randn((R, V), generator=gen, device=dev).square_())
        t32.div_(chi.div_(3.0).sqrt_()).mul_(w.scale)
        del chi
    logits = t32.to(w.dtype)
    del t32

    # per-request settings
    T = torch.full((B,), w.T, dtype=torch.float32, device=dev)
    if w.greedy_every:
        T[:: w.greedy_every] = 0.0
    top_k = torch.full((B,), w.top_k, dtype=torch.int32, device=dev) if w.top_k else None
    S = B + slots_extra
    idx_mapping = torch.randperm(S, generator=gen, device=dev)[:B].to(torch.int32)
    counts = torch.zeros((S, V), dtype=torch.int32, device=dev)
    if w.history:
        hist = torch.randint(0, V, (B, w.history), generator=gen, device=dev)
        rows = idx_mapping.long().unsqueeze(1).expand(B, w.history)
        counts.index_put_((rows.reshape(-1), hist.reshape(-1)),
                          torch.ones(B * w.history, dtype=torch.int32, device=dev), accumulate=True)
    rep = torch.full((B,), w.rep_penalty, dtype=torch.float32, device=dev) if w.rep_penalty != 1.0 else None
    every = lambda n, v, off: torch.where(torch.arange(B, device=dev) % n == 0, torch.full((B,), off, device=dev),
                                          torch.full((B,), v, device=dev)).to(torch.float32)
    freq = every(5, w.freq, 0.0) if w.freq else None
    pres = every(5, w.pres, 0.0) if w.pres else None
    top_p = every(7, w.top_p, 1.0) if w.top_p < 1.0 else None

    # draft side: draft position i of request r sits on target row cu[r] + r + i
    req = torch.repeat_interleave(torch.arange(B, device=dev), K)
    pos = torch.arange(D, device=dev) - cu[:-1].long()[req]
    drow = cu[:-1].long()[req] + req + pos
    draft_ids = torch.zeros(D, dtype=torch.int32, device=dev)
    draft_probs = None
    draft_logits = None
    draft_temp = None
    if D:
        dl = logits[drow].float() * w.draft_mix
        dl.add_(torch.randn(dl.shape, generator=gen, device=dev), alpha=w.draft_noise)
        greedy_req = (T == 0)[req]
        if w.draft_logits:  # drafts are drawn later by the draft-side sampler
            draft_logits = dl.to(w.dtype)
            draft_temp = torch.where(T == 0, torch.zeros_like(T), torch.full_like(T, w.draft_T))
        if w.draft_probs:
            if w.draft_top_k:
                kth = torch.topk(dl, w.draft_top_k, dim=1).values[:, -1:]
                dl.masked_fill_(dl < kth, float("-inf"))
            draft_probs = torch.softmax(dl / w.draft_T, dim=1)
            sampled = torch.multinomial(draft_probs, 1, generator=gen).squeeze(1)
            draft_ids = torch.where(greedy_req, dl.argmax(1), sampled).to(torch.int32)
        else:
            draft_ids = dl.argmax(1).to(torch.int32)
        del dl

    return dict(
        workload=w, logits=logits, cu=cu, draft_ids=draft_ids, draft_probs=draft_probs,
        temperature=T, top_k=top_k, rep_penalty=rep, idx_mapping=idx_mapping, counts=counts,
        freq=freq, pres=pres, top_p=top_p, draft_logits=draft_logits, draft_temp=draft_temp,
        synthetic_rates=list(w.synthetic_rates) if w.synthetic_rates else None,
        query_len=(K + 1).to(torch.int32), K=K.to(torch.int32), R=R, D=D, B=B, V=V,
        num_slots=S,
    )


def make_lm_head_inputs(B: int, K: int, V: int, d: int, ragged: bool = True, T: float = 1.0,
                        greedy_every: int = 0, scale: float = 3.0, draft_noise: float = 1.0,
                        device="cpu", seed: int = 1003) -> dict:
    """Hidden states [R, d] and an LM-head weight [V, d] (bf16), request layout,
    temperatures and draft ids for spec_verify_lm_head."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    if ragged:
        Kr = torch.randint(0, K + 1, (B,), generator=gen, device=dev)
    else:
        Kr = torch.full((B,), K, device=dev)
    cu = torch.zeros(B + 1, dtype=torch.int32, device=dev)
    cu[1:] = torch.cumsum(Kr, 0).to(torch.int32)
    D = int(cu[-1].item())
    R = D + B
    hidden = torch.randn((R, d), generator=gen, device=dev).to(torch.bfloat16)
    W = (torch.randn((V, d), generator=gen, device=dev) * (scale / d ** 0.5)).to(torch.bfloat16)
    Tt = torch.full((B,), T, dtype=torch.float32, device=dev)
    if greedy_every:
        Tt[::greedy_every] = 0.0
    req = torch.repeat_interleave(torch.arange(B, device=dev), Kr)
    pos = torch.arange(D, device=dev) - cu[:-1].long()[req]
    drow = cu[:-1].long()[req] + req + pos
    draft_ids = torch.zeros(D, dtype=torch.int32, device=dev)
    for s0 in range(0, D, 256):  # drafts: argmax of a noisy copy of the target logits
        rows = drow[s0:s0 + 256]
        z = hidden[rows].float() @ W.float().t()
        z.add_(torch.randn(z.shape, generator=gen, device=dev), alpha=draft_noise)
        draft_ids[s0:s0 + 256] = z.argmax(1).to(torch.int32)
        del z
    return dict(hidden=hidden, W=W, cu=cu, draft_ids=draft_ids, temperature=Tt, K=Kr.to(torch.int32),
                R=R, D=D, B=B, V=V, d=d)


def to_numpy(inp: dict, rows=None) -> dict:
    """Host copies for the oracle.  bf16 logits become their uint16 bit patterns
    (the oracle widens them itself).  rows: optional index tensor of target rows."""
    import numpy as np
    lg = inp["logits"] if rows is None else inp["logits"][rows]
    if lg.dtype == torch.bfloat16:
        lg_np = lg.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    else:
        lg_np = lg.contiguous().cpu().numpy()
    out = {"logits": lg_np}
    for k in ("cu", "draft_ids", "temperature", "top_k", "rep_penalty", "idx_mapping", "query_len", "K",
              "freq", "pres", "top_p"):
        v = inp.get(k)
        out[k] = None if v is None else v.cpu().numpy()
    out["synthetic_rates"] = inp.get("synthetic_rates")
    return out
