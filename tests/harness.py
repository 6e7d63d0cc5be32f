"""Helpers shared by the GPU parity tests, the smoke check and the bench's CPU
leg: run one verify step through the C ABI, run the oracle on the same inputs,
and compare under the acceptance rule.

Acceptance rule (per request):
  * greedy requests, num_sampled, num_rejected and tokens: bit-exact, except
    requests whose oracle decision margin is below MARGIN (relative), which
    are counted and reported instead;
  * with top-p, the kept set depends on whether the mass above a token is
    below top_p; the library sums fp32 probabilities, the oracle fp64 ones, so
    where some row's mass above lies within TOPP_TOL of top_p the request is
    also accepted when it matches the oracle run with top_p moved by +-TOPP_TOL
    (counted with the margin requests);
  * p(d) of every draft and the processed probabilities: within PROB_ATOL.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import rejection_sampling_verify_05_amd as sv

MARGIN = 1e-5
PROB_ATOL = 1e-6
TOPP_TOL = 4e-6
MARGIN_ATOL = 2e-5  # library margins are fp32 quantities, the oracle's fp64


class Ctx:
    """A library context sized for one workload (destroyed on close)."""

    def __init__(self, max_rows, max_reqs, max_k, max_vocab, topk=False):
        self.h = sv.spec_verify_create(max_rows, max_reqs, max_k, max_vocab,
                                       sv.SV_CREATE_TOPK if topk else 0)

    def close(self):
        if self.h is not None:
            sv.spec_verify_destroy(self.h)
            self.h = None

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.close()


def has_penalty(inp):
    return any(inp.get(k) is not None for k in ("rep_penalty", "freq", "pres"))


def ctx_for(inp, extra_rows=0):
    w = inp["workload"]
    return Ctx(inp["R"] + extra_rows, inp["B"], max(int(inp["K"].max().item()) if inp["B"] else 0, 1),
               inp["V"], topk=inp["top_k"] is not None)


def run_gpu(ctx: Ctx, inp: dict, seed=0, offset=0, dbg_probs=False, out_stride=None,
            stream=None, dbg_margin=False):
    """One spec_verify_run; returns host numpy outputs.  dbg_probs: True (every
    row's probabilities come back as "probs"), or a list of target rows (only
    those come back, as "probs_rows").  dbg_margin: the library's per-row
    decision margins come back as "margin_rows"."""
    B, D, V = inp["B"], inp["D"], inp["V"]
    dev = inp["logits"].device
    if out_stride is None:
        out_stride = int(inp["K"].max().item()) + 1 if B else 1
    out = torch.full((B, out_stride), -7, dtype=torch.int32, device=dev)
    ns = torch.full((B,), -7, dtype=torch.int32, device=dev)
    nr = torch.full((B,), -7, dtype=torch.int32, device=dev)
    pd = torch.full((max(D, 1),), -7.0, dtype=torch.float32, device=dev)
    probs = torch.full((inp["R"], V), -7.0, dtype=torch.float32, device=dev) if dbg_probs is not None and \
        dbg_probs is not False else None
    mrows = torch.full((inp["R"],), -7.0, dtype=torch.float32, device=dev) if dbg_margin else None
    sv.spec_verify_run(ctx.h, inp["logits"], inp["draft_ids"], inp["cu"], inp["temperature"],
                       out, ns, nr, draft_probs=inp["draft_probs"], top_k=inp["top_k"],
                       rep_penalty=inp["rep_penalty"], idx_mapping=inp["idx_mapping"],
                       output_bin_counts=inp["counts"] if has_penalty(inp) else None,
                       seed=seed, offset=offset, dbg_p_draft=pd if D else None, dbg_probs=probs,
                       frequency_penalty=inp.get("freq"), presence_penalty=inp.get("pres"),
                       top_p=inp.get("top_p"), synthetic_rates=inp.get("synthetic_rates"),
                       draft_logits=inp.get("draft_logits") if inp.get("draft_stats") is not None else None,
                       draft_stats=inp.get("draft_stats"),
                       draft_temperature=inp.get("draft_temp") if inp.get("draft_stats") is not None else None,
                       dbg_margin=mrows, stream=stream)
    err = sv.spec_verify_read_error(ctx.h, stream)
    res = dict(tokens=out.cpu().numpy(), num_sampled=ns.cpu().numpy(),
               num_rejected=nr.cpu().numpy(), p_draft=pd[:D].cpu().numpy(), err=err)
    if mrows is not None:
        res["margin_rows"] = mrows.cpu().numpy()
    if probs is not None:
        if dbg_probs is True:
            res["probs"] = probs.cpu().numpy()
        else:  # only these target rows come back to the host
            res["probs_rows"] = {int(r): probs[int(r)].cpu().numpy() for r in dbg_probs}
    return res


def run_draft_steps(ctx: Ctx, inp: dict, seed=0, offset=0):
    """Draw every draft token with spec_draft_sample, one call per draft
    position, from the rows of inp["draft_logits"]; fills inp["draft_ids"] and
    inp["draft_stats"] and returns the per-draft-row q(d) (host)."""
    B, D, V = inp["B"], inp["D"], inp["V"]
    dev = inp["logits"].device
    cu = inp["cu"]
    K = inp["K"]
    kmax = int(K.max().item()) if B else 0
    stats = torch.full((2 * max(D, 1),), -7.0, dtype=torch.float32, device=dev)
    qd = torch.zeros(max(D, 1), dtype=torch.float32, device=dev)
    ids = torch.full((max(D, 1),), -7, dtype=torch.int32, device=dev)
    r_idx = torch.arange(B, device=dev)
    for step in range(kmax):
        rows = torch.clamp(cu[:-1].long() + step, max=max(D - 1, 0))  # requests without this step read any row
        dl = inp["draft_logits"][rows].contiguous()
        tok = torch.full((B,), -7, dtype=torch.int32, device=dev)
        q = torch.full((B,), -7.0, dtype=torch.float32, device=dev)
        sv.spec_draft_sample(ctx.h, dl, inp["draft_temp"], cu, tok, stats, step=step, out_q=q, seed=seed,
                             offset=offset, draft_ids=ids)
        has = K > step
        dst = cu[:-1].long()[has] + step
        assert bool((ids[dst] == tok[has]).all())  # written at the draft rows by the library
        qd[dst] = q[has]
        assert bool((tok[~has] == -1).all())
    inp["draft_ids"] = ids[:D]
    inp["draft_stats"] = stats[: 2 * D]
    return qd[:D].cpu().numpy()


def check_draft_tokens(inp: dict, q_gpu, seed=0, offset=0, C=oracle.RACE_CHUNK, requests=None):
    """Compare the GPU draft tokens and q(d) with the oracle's draft sampler;
    returns (n_margin, mismatches)."""
    cu = inp["cu"].cpu().numpy()
    lg = inp["draft_logits"]
    rows = lg.contiguous().view(torch.int16).cpu().numpy().view(np.uint16) if lg.dtype == torch.bfloat16 \
        else lg.contiguous().cpu().numpy()
    ids = inp["draft_ids"].cpu().numpy()
    Tq = inp["draft_temp"].cpu().numpy()
    bad, n_margin = [], 0
    for r in (range(inp["B"]) if requests is None else requests):
        for dr in range(int(cu[r]), int(cu[r + 1])):
            d, q, mg = oracle.draft_sample(rows[dr], float(Tq[r]), seed, offset, dr, C)
            if d != ids[dr]:
                if mg < MARGIN:
                    n_margin += 1
                else:
                    bad.append(f"draft row {dr}: gpu {ids[dr]} oracle {d} margin {mg:.3g}")
            elif abs(float(q_gpu[dr]) - q) > PROB_ATOL:
                bad.append(f"draft row {dr}: q(d) gpu {q_gpu[dr]} oracle {q}")
    return n_margin, bad


class HostInputs:
    """Host copies of one verify call's inputs, taken once (bf16 logits as their
    bit patterns), so that the oracle can run over many requests in threads."""

    def __init__(self, inp: dict):
        lg = inp["logits"]
        self.logits = (lg.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
                       if lg.dtype == torch.bfloat16 else lg.contiguous().cpu().numpy())
        self.cu = inp["cu"].cpu().numpy()
        self.draft_ids = inp["draft_ids"].cpu().numpy()
        self.temperature = inp["temperature"].cpu().numpy()
        self.draft_probs = None if inp["draft_probs"] is None else inp["draft_probs"].float().cpu().numpy()
        tens = lambda k: None if inp.get(k) is None else inp[k].cpu().numpy()
        self.top_k, self.rep_penalty = tens("top_k"), tens("rep_penalty")
        self.freq, self.pres, self.top_p = tens("freq"), tens("pres"), tens("top_p")
        self.idx_mapping = inp["idx_mapping"].cpu().numpy()
        self.counts = inp["counts"].cpu().numpy() if has_penalty(inp) else None


class OracleRequest:
    """Oracle state of one request: processed probabilities are computed once,
    decisions can then be replayed for many (seed, offset).  host: optional
    HostInputs of the same call (no device reads then)."""

    def __init__(self, inp: dict, r: int, host=None):
        if isinstance(host, HostInputs):
            self._from_host(inp, r, host)
            return
        cu = inp["cu"].cpu().numpy() if host is None else host["cu"]
        self.r = r
        self.c0, self.c1 = int(cu[r]), int(cu[r + 1])
        self.K = self.c1 - self.c0
        self.g0 = self.c0 + r
        rows = slice(self.g0, self.g0 + self.K + 1)
        lg = inp["logits"][rows]
        if lg.dtype == torch.bfloat16:
            self.rows = lg.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        else:
            self.rows = lg.contiguous().cpu().numpy()
        self.T = float(inp["temperature"][r].item())
        self.top_k = int(inp["top_k"][r].item()) if inp["top_k"] is not None else 0
        self.theta = None
        counts = None
        if inp["rep_penalty"] is not None:
            self.theta = float(inp["rep_penalty"][r].item())
        self.freq = float(inp["freq"][r].item()) if inp.get("freq") is not None else 0.0
        self.pres = float(inp["pres"][r].item()) if inp.get("pres") is not None else 0.0
        self.top_p = float(inp["top_p"][r].item()) if inp.get("top_p") is not None else 1.0
        if has_penalty(inp):
            slot = int(inp["idx_mapping"][r].item())
            counts = inp["counts"][slot].cpu().numpy()
        self.counts = counts
        self.syn = inp.get("synthetic_rates")
        self.d = inp["draft_ids"][self.c0:self.c1].cpu().numpy()
        self.q = None
        if inp["draft_probs"] is not None and self.K:
            self.q = inp["draft_probs"][self.c0:self.c1].float().cpu().numpy()
        self.q64 = None
        if inp.get("draft_stats") is not None and self.K:
            tq = float(inp["draft_temp"][r].item())
            if tq > 0:  # greedy drafts carry no distribution: the draft-ids-only rules
                dl = inp["draft_logits"][self.c0:self.c1]
                dl = dl.contiguous().view(torch.int16).cpu().numpy().view(np.uint16) if dl.dtype == torch.bfloat16 \
                    else dl.contiguous().cpu().numpy()
                self.q64 = oracle.draft_q_rows(dl, tq)
        self.P, self.amax, self.err, self.topp_margin = self.prepare(0.0)

    def _from_host(self, inp: dict, r: int, h: HostInputs):
        self.r = r
        self.c0, self.c1 = int(h.cu[r]), int(h.cu[r + 1])
        self.K = self.c1 - self.c0
        self.g0 = self.c0 + r
        self.rows = h.logits[self.g0:self.g0 + self.K + 1]
        self.T = float(h.temperature[r])
        self.top_k = int(h.top_k[r]) if h.top_k is not None else 0
        self.theta = float(h.rep_penalty[r]) if h.rep_penalty is not None else None
        self.freq = float(h.freq[r]) if h.freq is not None else 0.0
        self.pres = float(h.pres[r]) if h.pres is not None else 0.0
        self.top_p = float(h.top_p[r]) if h.top_p is not None else 1.0
        self.counts = h.counts[int(h.idx_mapping[r])] if h.counts is not None else None
        self.syn = inp.get("synthetic_rates")
        self.d = h.draft_ids[self.c0:self.c1]
        self.q = h.draft_probs[self.c0:self.c1] if (h.draft_probs is not None and self.K) else None
        self.q64 = None
        assert inp.get("draft_stats") is None, "draft-logits mode: use the device constructor"
        self.P, self.amax, self.err, self.topp_margin = self.prepare(0.0)

    def prepare(self, shift):
        return oracle.prepare_request_ex(self.rows, self.T, self.top_k, self.theta, self.counts,
                                         freq=self.freq, pres=self.pres, top_p=self.top_p,
                                         top_p_shift=shift)

    def near_topp_boundary(self):
        return bool(np.any(self.topp_margin < TOPP_TOL))

    def decide_shifted(self, shift, seed=0, offset=0, C=oracle.RACE_CHUNK):
        P, amax, err, _ = self.prepare(shift)
        return oracle.decide_request(P, amax, self.T, self.d, self.q, self.g0, seed, offset, C,
                                     synthetic_rates=self.syn, draft_q64=self.q64)

    def decide(self, seed=0, offset=0, C=oracle.RACE_CHUNK):
        return oracle.decide_request(self.P, self.amax, self.T, self.d, self.q, self.g0, seed,
                                     offset, C, synthetic_rates=self.syn, draft_q64=self.q64)


def compare_request(g: dict, r: int, o_tokens, o_ns, o_nr, o_margin, out_stride):
    """Returns 'ok', 'margin' or a mismatch description."""
    want = list(o_tokens) + [-1] * (out_stride - len(o_tokens))
    got = g["tokens"][r].tolist()
    same = got == want and g["num_sampled"][r] == o_ns and g["num_rejected"][r] == o_nr
    if same:
        return "ok"
    if o_margin < MARGIN:
        return "margin"
    return (f"request {r}: gpu tokens {got} ns {g['num_sampled'][r]} nr {g['num_rejected'][r]}; "
            f"oracle {want} ns {o_ns} nr {o_nr} margin {o_margin:.3g}")


def _p_draft_err(gp, o, shift):
    P = o.prepare(shift)[0]
    exact = np.array([P[i, d] if 0 <= d < P.shape[1] else 0.0 for i, d in enumerate(o.d)])
    return float(np.max(np.abs(gp.astype(np.float64) - exact)))


def check_requests(g: dict, inp: dict, requests, seed=0, offset=0, probs=False):
    """Compare the GPU outputs of `requests` with the oracle; returns (n_margin,
    mismatches list).  Also checks p(d) and (optionally) processed probs."""
    out_stride = g["tokens"].shape[1]
    bad, n_margin = [], 0
    for r in requests:
        o = OracleRequest(inp, r)
        assert o.err == 0, f"oracle rejected request {r}: {o.err}"
        toks, ns, nr, mg, pd = o.decide(seed, offset)
        res = compare_request(g, r, toks, ns, nr, mg, out_stride)
        if res not in ("ok", "margin") and o.near_topp_boundary():
            for shift in (-TOPP_TOL, TOPP_TOL):
                t2, ns2, nr2, mg2, _ = o.decide_shifted(shift, seed, offset)
                if compare_request(g, r, t2, ns2, nr2, mg2, out_stride) in ("ok", "margin"):
                    res = "margin"
                    break
        if res == "margin":
            n_margin += 1
        elif res != "ok":
            bad.append(res)
        if o.K and o.T > 0:
            gp = g["p_draft"][o.c0:o.c1]
            err = np.max(np.abs(gp.astype(np.float64) - pd.astype(np.float64)))
            # the oracle's p_draft is fp32-rounded; compare against its fp64 value
            P = o.P
            exact = np.array([P[i, d] if 0 <= d < P.shape[1] else 0.0 for i, d in enumerate(o.d)])
            err = np.max(np.abs(gp.astype(np.float64) - exact))
            if err > PROB_ATOL and o.near_topp_boundary():
                err = min(err, *(_p_draft_err(gp, o, s) for s in (-TOPP_TOL, TOPP_TOL)))
            if err > PROB_ATOL:
                bad.append(f"request {r}: p(d) error {err:.3g}")
        if probs and "probs" in g:
            gp = g["probs"][o.g0:o.g0 + o.K + 1].astype(np.float64)
            err = np.max(np.abs(gp - o.P))
            if err > PROB_ATOL and o.near_topp_boundary():
                err = min(err, *(np.max(np.abs(gp - o.prepare(s)[0])) for s in (-TOPP_TOL, TOPP_TOL)))
            if err > PROB_ATOL:
                bad.append(f"request {r}: probability error {err:.3g}")
    return n_margin, bad


def check_margins(g: dict, inp: dict, requests, seed=0, offset=0, atol=MARGIN_ATOL):
    """Compare the library's per-row decision margins (run_gpu with
    dbg_margin) with the oracle's request margins: the smallest over a
    request's rows must match the oracle's within atol; rows after the sampled
    one carry no decision (+inf), and neither do greedy requests.  Requests
    whose tokens differ from the oracle's by a margin (or top-p boundary)
    excuse are skipped.  Returns (number compared, mismatch list)."""
    mr = g["margin_rows"]
    out_stride = g["tokens"].shape[1]
    bad, n = [], 0
    for r in requests:
        o = OracleRequest(inp, r)
        toks, ns, nr, mg, _ = o.decide(seed, offset)
        if compare_request(g, r, toks, ns, nr, mg, out_stride) != "ok" or o.near_topp_boundary():
            continue
        rows = mr[o.g0:o.g0 + o.K + 1].astype(np.float64)
        j = int(g["num_sampled"][r]) - 1
        if not np.all(np.isinf(rows[j + 1:])):
            bad.append(f"request {r}: rows after the sampled row {j} carry margins {rows[j + 1:]}")
        dev = float(rows.min())
        if np.isinf(mg) or np.isinf(dev):
            if not (np.isinf(mg) and np.isinf(dev)):
                bad.append(f"request {r}: margin gpu {dev} oracle {mg}")
        elif abs(dev - mg) > atol:
            bad.append(f"request {r}: margin gpu {dev:.9g} oracle {mg:.9g} (rows {rows})")
        n += 1
    return n, bad


def check_one(g: dict, inp: dict, r: int, host: HostInputs, seed=0, offset=0, probs_rows=None):
    """check_requests for one request, from host copies; returns (is_margin, mismatch list)."""
    out_stride = g["tokens"].shape[1]
    bad = []
    o = OracleRequest(inp, r, host)
    if o.err != 0:
        return False, [f"oracle rejected request {r}: {o.err}"]
    toks, ns, nr, mg, pd = o.decide(seed, offset)
    res = compare_request(g, r, toks, ns, nr, mg, out_stride)
    if res not in ("ok", "margin") and o.near_topp_boundary():
        for shift in (-TOPP_TOL, TOPP_TOL):
            t2, ns2, nr2, mg2, _ = o.decide_shifted(shift, seed, offset)
            if compare_request(g, r, t2, ns2, nr2, mg2, out_stride) in ("ok", "margin"):
                res = "margin"
                break
    if res not in ("ok", "margin"):
        bad.append(res)
    if o.K and o.T > 0:
        gp = g["p_draft"][o.c0:o.c1].astype(np.float64)
        exact = np.array([o.P[i, d] if 0 <= d < o.P.shape[1] else 0.0 for i, d in enumerate(o.d)])
        err = float(np.max(np.abs(gp - exact)))
        if err > PROB_ATOL and o.near_topp_boundary():
            err = min(err, *(_p_draft_err(gp.astype(np.float32), o, s) for s in (-TOPP_TOL, TOPP_TOL)))
        if err > PROB_ATOL:
            bad.append(f"request {r}: p(d) error {err:.3g}")
    if probs_rows is not None:
        for i in range(o.K + 1):
            row = probs_rows.get(o.g0 + i)
            if row is not None:
                err = float(np.max(np.abs(row.astype(np.float64) - o.P[i])))
                if err > PROB_ATOL:
                    bad.append(f"request {r} row {o.g0 + i}: probability error {err:.3g}")
    return res == "margin", bad


def check_all(g: dict, inp: dict, requests, seed=0, offset=0, probs_rows=None, workers=16, host=None):
    """check_requests over many requests with the oracle in a thread pool (its C
    calls release the GIL).  probs_rows: {target row: device probabilities} to
    compare with the oracle's fp64 ones.  Returns (n_margin, mismatches)."""
    from concurrent.futures import ThreadPoolExecutor
    host = host or HostInputs(inp)
    with ThreadPoolExecutor(max_workers=workers) as ex:
        res = list(ex.map(lambda r: check_one(g, inp, r, host, seed, offset, probs_rows), requests))
    return sum(m for m, _ in res), [b for _, bl in res for b in bl]
