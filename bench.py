#!/usr/bin/env python3
"""Benchmark of the speculative-decoding verify step on one MI355X.

One step = spec_verify_run with post_update applied inside the call (or,
with --separate-post-update, spec_verify_run then spec_post_update) over one
batch of the headline
workload (B=256 requests, K_r uniform in {0..3}, V=128256, bf16 target logits
N(0, 3^2), no draft probabilities).  Inputs are resident in HBM before the
timed region; the step rotates over several distinct input copies (more than
1 GB in total) so that the 256 MB Infinity Cache cannot serve the logits.

Prints one JSON line: verified logit rows/s over the timed steps; the
first pass over the rows (the streaming statistics kernel, or the top-k pass
when top-k is on) with its achieved algorithmic HBM bandwidth against the
8 TB/s peak (its duration from dispatch-stamped HIP events on the launch
stream, over a second, instrumented pass of the same steps), next to the
same kernel's figure from the committed rocprofv3 trace of this workload;
the whole verify call's and the epilogue kernel's durations; the acceptance
measured on the outputs; and the CPU oracle's rate on a bounded sample of the
same workload, single-threaded and over a process pool on the host's cores
(timed before the GPU is touched).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
PROFILES = os.path.join(ROOT, "profiles")
# FETCH_SIZE / WRITE_SIZE counter record of the streaming kernel on the headline workload
COUNTERS = os.path.join(PROFILES, "stats_fast_kernel_bf16_B256_V128256_counters.md")
CSRC = "rejection_sampling_verify_05_amd/csrc/"
_COMMON = [CSRC + "sv_common.h", CSRC + "sv_device.h", CSRC + "sv_internal.h", "rejection_sampling_verify_05_amd/build.py"]
# The sources a profile record was taken on, per kernel: a record stays valid
# while these files are unchanged.
KERNEL_SOURCES = [CSRC + "sv_stats.hip"] + _COMMON
KERNEL_SOURCES_TOPK = [CSRC + "sv_topk.hip", CSRC + "sv_tiles.h"] + _COMMON
KERNEL_SOURCES_TOPP = [CSRC + "sv_topp.hip", CSRC + "sv_tiles.h"] + _COMMON


# ... and of the LM-head GEMM on its workload
COUNTERS_LM = os.path.join(ROOT, "profiles", "lm_gemm_kernel_B256_V128256_d4096_counters.md")
KERNEL_SOURCES_LM = ["rejection_sampling_verify_05_amd/csrc/sv_lmhead.hip", "rejection_sampling_verify_05_amd/csrc/sv_device.h",
                     "rejection_sampling_verify_05_amd/csrc/sv_internal.h", "rejection_sampling_verify_05_amd/build.py"]


def kernel_source_hash(sources=None) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def read_record(path, sources=None):
    """The `- key: value` record of a profiles/ summary, or None when the file is
    missing or was taken on different kernel sources."""
    if not path or not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].split(": ", 1)
            rec[k.strip("` ")] = v.strip().strip("`")
    if rec.get("kernel_source_sha256") != kernel_source_hash(sources):
        return None
    return rec


def recorded_traffic_per_row(path=None, sources=None):
    """HBM bytes per target row measured by the counter runs, or None when the
    record is missing or was taken on different kernel sources."""
    rec = read_record(path or COUNTERS, sources)
    return None if rec is None else float(rec["hbm_bytes_per_target_row"])


# Per-workload profiles/ summaries: the first pass over the rows, named for the
# kernel and the workload.
WORKLOAD_PROFILE = {
    "2": ("stats_fast_kernel_bf16_B64_K4_V32000", KERNEL_SOURCES),
    "3": ("stats_fast_kernel_bf16_B256_V128256", KERNEL_SOURCES),
    "3k3": ("stats_fast_kernel_bf16_B256_K3_V128256", KERNEL_SOURCES),
    "4": ("topk_kernel_f32_B512_K8_V151936", KERNEL_SOURCES_TOPK),
    "5": ("stats_fast_kernel_bf16_B1024_K5_V256000", KERNEL_SOURCES),
    "3f": ("stats_fast_kernel_pen_bf16_B256_V128256", KERNEL_SOURCES),
    "3p": ("topp_resident_kernel_bf16_B256_V128256", KERNEL_SOURCES_TOPP),
}


def profile_paths(cid):
    """(counter record, trace record, the sources both were taken on) of a workload."""
    if cid not in WORKLOAD_PROFILE:
        return None, None, None
    base, sources = WORKLOAD_PROFILE[cid]
    return os.path.join(PROFILES, base + "_counters.md"), os.path.join(PROFILES, base + "_trace.md"), sources


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))  # the GPU machine gives one GPU's process 16 cores


_POOL_INPUT = None


def _oracle_slice(task):
    """Oracle verify call on requests [a, b) of the pool's input batch (run in a
    forked worker; the batch is inherited, not sent)."""
    import oracle
    a, b, offset = task
    h = _POOL_INPUT
    cu = h["cu"]
    g0, g1 = int(cu[a]) + a, int(cu[b]) + b
    d0, d1 = int(cu[a]), int(cu[b])
    sl = lambda v, lo, hi: None if v is None else v[lo:hi]
    oracle.verify_batch(h["logits"][g0:g1], cu[a:b + 1] - cu[a], h["draft_ids"][d0:d1],
                        h["temperature"][a:b], draft_probs=sl(h["draft_probs"], d0, d1),
                        top_k=sl(h["top_k"], a, b), rep_penalty=sl(h["rep_penalty"], a, b),
                        idx_mapping=sl(h["idx_mapping"], a, b), counts=h["counts"], seed=1234, offset=offset,
                        freq=sl(h["freq"], a, b), pres=sl(h["pres"], a, b), top_p=sl(h["top_p"], a, b),
                        synthetic_rates=h["synthetic_rates"], max_k=h["max_k"])
    return g1 - g0


def cpu_baseline_leg(w, seconds):
    """The oracle on a bounded sample of workload w, made on the host with the
    same generator recipe (the GPU is not touched): request slices in one
    process for half the budget, then the same slices over a fork pool of the
    host's cores for the other half (at least one slice, resp. one slice per
    worker, so that the largest workloads stay bounded)."""
    import multiprocessing as mp
    import time as _t
    global _POOL_INPUT
    inp = wl_make_host_inputs(w)
    h = inp["host"]
    B = inp["B"]
    _POOL_INPUT = h
    workers = host_workers()
    per = max(1, -(-B // (4 * workers)))  # requests per slice
    slices = [(a, min(B, a + per)) for a in range(0, B, per)]
    t0 = _t.perf_counter()
    n1 = rows1 = 0
    while True:
        a, b = slices[n1 % len(slices)]
        rows1 += _oracle_slice((a, b, n1 // len(slices)))
        n1 += 1
        if _t.perf_counter() - t0 >= seconds / 2:
            break
    s1 = _t.perf_counter() - t0
    ctx = mp.get_context("fork")
    rows_n = n_tasks = 0
    with ctx.Pool(workers) as pool:
        pool.map(_oracle_slice, [(a, b, 63) for a, b in slices[:workers]])  # workers started and warm
        t1 = _t.perf_counter()
        k = 0
        while True:
            tasks = [(*slices[(k + i) % len(slices)], (k + i) // len(slices)) for i in range(workers)]
            rows_n += sum(pool.map(_oracle_slice, tasks))
            n_tasks += workers
            k += workers
            if _t.perf_counter() - t1 >= seconds / 2:
                break
        sn = _t.perf_counter() - t1
    _POOL_INPUT = None
    return {"value": rows_n / sn, "unit": "rows/s", "cores": workers, "kind": "oracle",
            "cpu_model": cpu_model(),
            "single_process": {"value": rows1 / s1, "unit": "rows/s", "cores": 1,
                               "sample": f"{n1} slice(s) of {per} requests ({rows1} rows), {s1:.1f} s"},
            "sample": f"{n_tasks} slices of {per} requests of workload {w.cid} ({rows_n} rows; B={B}) over a fork "
                      f"pool of {workers} processes, {sn:.1f} s; inputs made on the host with the same generator "
                      "recipe as the GPU copies (same distribution, other draws); C oracle, fp64"}


def wl_make_host_inputs(w):
    """Host copy of workload w for the oracle leg (numpy views, as the oracle takes them)."""
    import workloads as wl
    inp = wl.make_inputs(w, "cpu", salt=0)
    h = wl.to_numpy(inp)
    penalty = any(inp[k] is not None for k in ("rep_penalty", "freq", "pres"))
    h["counts"] = inp["counts"].numpy() if penalty else None
    h["draft_probs"] = None if inp["draft_probs"] is None else inp["draft_probs"].numpy()
    h["max_k"] = w.K
    return {"host": h, "B": inp["B"], "R": inp["R"]}


def copy_calibration():
    """torch's copy kernel on 256 MiB, three times: a known-size reference for
    the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="3", help="workload id (1, 2, 3, 3k3, 4, 5; with optional "
                    "settings: 3p top-p, 3f frequency/presence penalties, 3s synthetic acceptance, "
                    "3d draft-side sampling plus draft-logits verification, 4f and 4p; 3h: the "
                    "LM-head path, logits computed from hidden states d=4096 in the step)")
    ap.add_argument("--copies", type=int, default=0, help="input copies to rotate (0: >= 1 GB)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle sample budget")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--separate-post-update", action="store_true",
                    help="run post_update as its own call after spec_verify_run instead of inside it")
    ap.add_argument("--cpu-leg", action="store_true",
                    help="only the oracle baseline (run by the benchmark itself in a child process that "
                         "never touches the GPU, so its process pool can fork); prints its JSON and exits")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="before warmup, run torch's copy kernel on 256 MiB three times (a known-size "
                         "reference for the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); "
              "the verify step shards by request with no exchange, so run one process per GPU.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads as wl

    if args.cpu_leg:
        print(json.dumps(cpu_baseline_leg(wl.CONFIGS[args.workload], args.cpu_seconds)), flush=True)
        return

    from rejection_sampling_verify_05_amd import build as libbuild
    if not os.path.exists(libbuild.OUTPUT):
        libbuild.build_library()
    import rejection_sampling_verify_05_amd as sv

    torch.cuda.set_device(0)
    if args.workload == "3h":
        return bench_lm_head(args)
    w = wl.CONFIGS[args.workload]
    first = wl.make_inputs(w, "cuda", salt=0)
    per_copy = first["logits"].numel() * first["logits"].element_size()
    ncopies = args.copies or max(4, -(-(1 << 30) // per_copy))
    copies = [first] + [wl.make_inputs(w, "cuda", salt=i) for i in range(1, ncopies)]
    out_stride = w.K + 1
    max_rows = max(c["R"] for c in copies)
    ctx = sv.spec_verify_create(max_rows, w.B, w.K, w.V, sv.SV_CREATE_TOPK if w.top_k else 0)

    stream = torch.cuda.current_stream()
    S = first["num_slots"]
    last = torch.zeros(S, dtype=torch.int32, device="cuda")
    ncomp = torch.zeros(S, dtype=torch.int32, device="cuda")
    counts = first["counts"].clone()
    outs = []
    penalty = any(first[k] is not None for k in ("rep_penalty", "freq", "pres"))
    for c in copies:
        o = dict(tokens=torch.empty((w.B, out_stride), dtype=torch.int32, device="cuda"),
                 ns=torch.empty(w.B, dtype=torch.int32, device="cuda"),
                 nr=torch.empty(w.B, dtype=torch.int32, device="cuda"))
        o["vargs"] = sv.make_verify_args(
            c["logits"], c["draft_ids"], c["cu"], c["temperature"], o["tokens"], o["ns"], o["nr"],
            draft_probs=c["draft_probs"], top_k=c["top_k"], rep_penalty=c["rep_penalty"],
            idx_mapping=c["idx_mapping"], output_bin_counts=c["counts"] if penalty else None,
            seed=1234, offset=0, frequency_penalty=c["freq"], presence_penalty=c["pres"], top_p=c["top_p"],
            synthetic_rates=c["synthetic_rates"])
        if w.draft_logits:
            # Draft-side sampling: one call per draft position over that position's
            # draft-logit rows (gathered once, before timing), writing the draft ids
            # and row statistics the verify call then reads in draft-logits mode.
            D = c["D"]
            stats = torch.zeros(2 * max(D, 1), dtype=torch.float32, device="cuda")
            o["dargs"] = []
            for step in range(w.K):
                rows = torch.clamp(c["cu"][:-1].long() + step, max=max(D - 1, 0))
                dl = c["draft_logits"][rows].contiguous()
                o.setdefault("keep", []).append(dl)
                o["dargs"].append(sv.make_draft_args(
                    dl, c["draft_temp"], c["cu"], torch.empty(w.B, dtype=torch.int32, device="cuda"), stats,
                    step=step, seed=1234, offset=0, draft_ids=c["draft_ids"]))
                o["keep"].append(o["dargs"][-1])
            o["keep"].append(stats)
            o["vargs"] = sv.make_verify_args(
                c["logits"], c["draft_ids"], c["cu"], c["temperature"], o["tokens"], o["ns"], o["nr"],
                seed=1234, offset=0, draft_logits=c["draft_logits"], draft_stats=stats,
                draft_temperature=c["draft_temp"])
        o["pargs"] = sv.make_post_update_args(c["idx_mapping"], c["query_len"], o["tokens"], o["ns"],
                                              o["nr"], last, counts, ncomp)
        if not args.separate_post_update:  # the bookkeeping inside the verify call
            o["vargs"].post_update = ctypes.addressof(o["pargs"])
            o["vargs"]._post_update = o["pargs"]
        outs.append(o)

    def step(i):
        o = outs[i % ncopies]
        for da in o.get("dargs", ()):
            da.offset = i
            sv.spec_draft_sample(ctx, da, stream=stream)
        o["vargs"].offset = i
        sv.spec_verify_run(ctx, o["vargs"], stream=stream)
        if args.separate_post_update:
            sv.spec_post_update(ctx, o["pargs"], stream=stream)

    if args.copy_calibration:
        copy_calibration()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    assert sv.spec_verify_read_error(ctx) == 0

    # Timed region: K steps between two synchronisations, nothing else on the
    # stream.  `value` and ms_per_step come from it.
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    rows = 0
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for k in range(args.steps):
        i = args.warmup + k
        step(i)
        rows += copies[i % ncopies]["R"]
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    assert sv.spec_verify_read_error(ctx) == 0

    # The same K steps again, instrumented: the library launches its streaming
    # and epilogue kernels with start/stop HIP events stamped by the dispatch
    # on the launch stream (spec_verify_profile_*), and torch events on the
    # same stream bracket each whole verify call.  The events add gaps between
    # launches, which is why `value` comes from the clean pass above.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    sv.spec_verify_profile_start(ctx, args.steps)
    torch.cuda.synchronize()
    for k in range(args.steps):
        i = args.warmup + k
        o = outs[i % ncopies]
        o["vargs"].offset = i
        ev[k][0].record(stream)
        sv.spec_verify_run(ctx, o["vargs"], stream=stream)
        ev[k][1].record(stream)
        if args.separate_post_update:
            sv.spec_post_update(ctx, o["pargs"], stream=stream)
    torch.cuda.synchronize()
    verify_ms = np.array([a.elapsed_time(b) for a, b in ev])
    stream_ms, epi_ms = sv.spec_verify_profile_read(ctx, args.steps)
    stream_ms, epi_ms = np.array(stream_ms), np.array(epi_ms)
    assert len(stream_ms) == args.steps
    assert sv.spec_verify_read_error(ctx) == 0

    # Dominant kernel: the first pass over the rows (the streaming statistics
    # pass, the top-k pass, or the register-resident top-p pass).  Its algorithmic bytes are one read of every
    # target row, R V s (s = 2 for bf16, 4 for fp32), plus, for the statistics
    # pass with penalties, the counts row of each penalised request (V 4).
    esize = first["logits"].element_size()
    # With top-p on aligned bf16 rows of at most 128 chunks and no top-k or
    # penalty, the library's first (and only) pass over the rows is the
    # register-resident top-p pass.
    resident = (w.top_p < 1.0 and not w.top_k and not penalty and esize == 2 and w.V % 8 == 0
                and -(-w.V // 1024) <= 128)
    kernel = "topk_kernel (top-k pass: every row read once)" if w.top_k else \
        "topp_resident_kernel (top-p call: every row held in registers, read once)" if resident else \
        "stats_fast_kernel (streaming softmax statistics)"

    def launch_bytes(c):
        b = c["R"] * w.V * esize
        if penalty and not w.top_k:
            pen = torch.zeros(w.B, dtype=torch.bool)
            for k in ("rep_penalty", "freq", "pres"):
                if c[k] is not None:
                    pen |= (c[k].cpu() != (1.0 if k == "rep_penalty" else 0.0))
            b += int(pen.sum()) * w.V * 4
        return b

    per_copy_bytes = [launch_bytes(c) for c in copies]
    bytes_per = float(np.mean([per_copy_bytes[(args.warmup + k) % ncopies] for k in range(args.steps)]))
    rows_per = rows / args.steps
    R_mean = float(np.mean([copies[(args.warmup + k) % ncopies]["R"] for k in range(args.steps)]))
    # Every verify call of this process (warmup, timed pass, instrumented pass):
    # what a profiler run of the whole process averages over.
    every = list(range(args.warmup)) + [args.warmup + k for k in range(args.steps)] * 2
    launches = {"count": len(every),
                "rows_mean": round(float(np.mean([copies[i % ncopies]["R"] for i in every])), 2),
                "bytes_mean": round(float(np.mean([per_copy_bytes[i % ncopies] for i in every])), 1)}
    achieved = bytes_per / (float(np.mean(stream_ms)) * 1e-3) / 1e9
    cpath, tpath, srcs = profile_paths(w.cid)
    per_row = recorded_traffic_per_row(cpath, srcs) if cpath else None
    traffic = None if per_row is None else int(per_row * R_mean)
    trace = read_record(tpath, srcs)
    prof = None
    if trace is not None:
        avg_ns = float(trace["kernel_avg_ns"])
        rb = float(trace["bytes_per_launch"])
        prof = {"avg_us": round(avg_ns / 1e3, 3), "achieved": round(rb / avg_ns, 1),
                "frac": round(rb / avg_ns / HBM_PEAK_GBS, 4), "dispatches": int(trace["dispatches"]),
                "source": os.path.relpath(tpath, ROOT)}
    value = rows / (total_ms * 1e-3)

    # Acceptance measured on the outputs of the instrumented pass's last step
    # of each input copy: accepted drafts per draft position.
    acc_n = np.zeros(w.K + 1)
    acc_d = np.zeros(w.K + 1)
    for c, o in zip(copies, outs):
        Kr = c["K"].cpu().numpy()
        ns = o["ns"].cpu().numpy()
        T = c["temperature"].cpu().numpy()
        for i in range(w.K):
            has = Kr > i
            acc_d[i] += has.sum()
            acc_n[i] += (has & (ns - 1 > i)).sum()
    per_pos = [round(float(a / d), 4) if d else None for a, d in zip(acc_n[:w.K], acc_d[:w.K])]

    def pct(a):
        return {"mean": round(float(np.mean(a)) * 1e3, 2), "p10": round(float(np.percentile(a, 10)) * 1e3, 2),
                "p50": round(float(np.median(a)) * 1e3, 2), "p90": round(float(np.percentile(a, 90)) * 1e3, 2)}

    sv.spec_verify_destroy(ctx)

    # CPU baseline after the GPU part (which then runs on a GPU that is not
    # coming out of idle), in a child process that never touches the GPU: its
    # process pool forks from there.
    cpu = None
    if not args.no_cpu:
        import subprocess
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-leg", "--workload", args.workload,
                            "--cpu-seconds", str(args.cpu_seconds)], capture_output=True, text=True,
                           timeout=args.cpu_seconds * 10 + 300)
        if r.returncode != 0:
            raise RuntimeError(f"oracle baseline leg failed:\n{r.stderr[-2000:]}")
        cpu = json.loads(r.stdout.strip().splitlines()[-1])

    line = {
        "metric": "verified logit rows/sec + achieved HBM GB/s (B=256, K=3, V=128256)",
        "value": round(value, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B={w.B}, K_r {'~U{0..%d}' % w.K if w.ragged else '=%d' % w.K}, "
                               f"V={w.V}, {'bf16' if w.dtype == torch.bfloat16 else 'fp32'} logits, "
                               f"{'draft probs' if w.draft_probs else ('draft logits, drafts sampled in the step' if w.draft_logits else 'draft ids only')}",
                   "global_batch": w.B, "rows_per_step": round(rows_per, 1), "input_copies": ncopies,
                   "post_update": "separate call" if args.separate_post_update else "inside the verify call",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": kernel,
                     "kernel_us": pct(stream_ms), "bytes_per_launch": int(bytes_per),
                     "bytes_rule": f"R*V*{esize} (each target row read once)" +
                                   (" + V*4 per penalised request (its counts row)" if penalty and not w.top_k else ""),
                     "rocprof": prof},
        "step_achieved_GBs": round(bytes_per / (total_ms / args.steps * 1e-3) / 1e9, 1),
        "verify_call_us": pct(verify_ms),
        "epilogue_kernel_us": pct(epi_ms),
        "acceptance_per_position": per_pos,
        "cpu_baseline": cpu,
        "launches_all_passes": launches,
        "wall_s": round(wall, 3),
    }
    print(json.dumps(line), flush=True)


def pct(a):
    import numpy as np
    return {"mean": round(float(np.mean(a)) * 1e3, 2), "p10": round(float(np.percentile(a, 10)) * 1e3, 2),
            "p50": round(float(np.median(a)) * 1e3, 2), "p90": round(float(np.percentile(a, 90)) * 1e3, 2)}


def bench_lm_head(args):
    """One step = spec_verify_lm_head (the LM-head GEMM with the verify
    statistics in its epilogue, then the per-request decisions) with post_update
    inside the call (or as its own call with --separate-post-update),
    on config 3's request mix with hidden size 4096.  The LM-head weight (1.05 GB)
    is one resident tensor, as in serving; the hidden states rotate over copies.
    Also times, as context, the same step with the logits materialised: torch's
    bf16 matmul (hipBLASLt) then spec_verify_run on the logits."""
    import numpy as np
    import torch

    import workloads as wl
    import rejection_sampling_verify_05_amd as sv

    B, K, V, d = 256, 3, 128256, 4096
    ncopies = args.copies or 4
    copies = [wl.make_lm_head_inputs(B=B, K=K, V=V, d=d, device="cuda", seed=1003 + i) for i in range(ncopies)]
    W = copies[0]["W"]
    for c in copies[1:]:
        c["W"] = W  # one weight, several batches of hidden states
    max_rows = max(c["R"] for c in copies)
    ctx = sv.spec_verify_create(max_rows, B, K, V, sv.SV_CREATE_LM_HEAD)
    stream = torch.cuda.current_stream()
    S = B + 64
    last = torch.zeros(S, dtype=torch.int32, device="cuda")
    ncomp = torch.zeros(S, dtype=torch.int32, device="cuda")
    counts = torch.zeros((S, V), dtype=torch.int32, device="cuda")
    idx_mapping = torch.arange(B, dtype=torch.int32, device="cuda")
    outs = []
    for c in copies:
        o = dict(tokens=torch.empty((B, K + 1), dtype=torch.int32, device="cuda"),
                 ns=torch.empty(B, dtype=torch.int32, device="cuda"),
                 nr=torch.empty(B, dtype=torch.int32, device="cuda"))
        o["largs"] = sv.make_lm_head_args(c["hidden"], W, c["draft_ids"], c["cu"], c["temperature"], o["tokens"],
                                          o["ns"], o["nr"], seed=1234, offset=0)
        o["pargs"] = sv.make_post_update_args(idx_mapping, (c["K"] + 1).to(torch.int32), o["tokens"], o["ns"],
                                              o["nr"], last, counts, ncomp)
        if not args.separate_post_update:  # the bookkeeping inside the call
            o["largs"].post_update = ctypes.addressof(o["pargs"])
            o["largs"]._post_update = o["pargs"]
        outs.append(o)

    def step(i):
        o = outs[i % ncopies]
        o["largs"].offset = i
        sv.spec_verify_lm_head(ctx, o["largs"], stream=stream)
        if args.separate_post_update:
            sv.spec_post_update(ctx, o["pargs"], stream=stream)

    if args.copy_calibration:
        copy_calibration()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    assert sv.spec_verify_read_error(ctx) == 0
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    rows = 0
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for k in range(args.steps):
        i = args.warmup + k
        step(i)
        rows += copies[i % ncopies]["R"]
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    assert sv.spec_verify_read_error(ctx) == 0

    # Instrumented pass: dispatch-stamped events around the GEMM and the request kernel.
    sv.spec_verify_profile_start(ctx, args.steps)
    torch.cuda.synchronize()
    for k in range(args.steps):
        step(args.warmup + k)
    torch.cuda.synchronize()
    gemm_ms, req_ms = sv.spec_verify_profile_read(ctx, args.steps)
    gemm_ms, req_ms = np.array(gemm_ms), np.array(req_ms)
    assert len(gemm_ms) == args.steps

    # Context: logits materialised by torch's bf16 matmul, then the verify call.
    vctx = sv.spec_verify_create(max_rows, B, K, V, 0)
    logits = [torch.empty((c["R"], V), dtype=torch.bfloat16, device="cuda") for c in copies]
    vargs = [sv.make_verify_args(logits[j], c["draft_ids"], c["cu"], c["temperature"], outs[j]["tokens"],
                                 outs[j]["ns"], outs[j]["nr"], seed=1234, offset=0)
             for j, c in enumerate(copies)]
    nref = min(args.steps, 50)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(nref)]
    for k in range(nref + 5):
        j = k % ncopies
        e = ev[k - 5] if k >= 5 else None
        if e:
            e[0].record(stream)
        torch.mm(copies[j]["hidden"], W.t(), out=logits[j])
        if e:
            e[1].record(stream)
        vargs[j].offset = k
        sv.spec_verify_run(vctx, vargs[j], stream=stream)
        if e:
            e[2].record(stream)
    torch.cuda.synchronize()
    mm_ms = np.array([a.elapsed_time(b) for a, b, _ in ev])
    vr_ms = np.array([b.elapsed_time(c) for _, b, c in ev])
    sv.spec_verify_destroy(vctx)
    del logits

    R_mean = float(np.mean([copies[(args.warmup + k) % ncopies]["R"] for k in range(args.steps)]))
    flops = 2.0 * R_mean * V * d
    per_row = recorded_traffic_per_row(COUNTERS_LM, KERNEL_SOURCES_LM)
    traffic = None if per_row is None else int(per_row * R_mean)
    achieved = flops / (float(np.mean(gemm_ms)) * 1e-3) / 1e12

    cpu = None
    if not args.no_cpu:
        import oracle
        c = copies[0]
        H = c["hidden"].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        Wb = W.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        cu, dids, T = c["cu"].cpu().numpy(), c["draft_ids"].cpu().numpy(), c["temperature"].cpu().numpy()
        t_start = time.perf_counter()
        n_req, cpu_rows = 0, 0
        while True:
            oracle.lm_head_verify(H, Wb, cu, dids, T, seed=1234, offset=0, out_stride=K + 1, requests=[n_req])
            cpu_rows += int(cu[n_req + 1] - cu[n_req]) + 1
            n_req += 1
            if time.perf_counter() - t_start >= args.cpu_seconds or n_req == B:
                break
        cpu_s = time.perf_counter() - t_start
        cpu = {"value": cpu_rows / cpu_s, "unit": "rows/s", "cores": 1, "kind": "oracle",
               "sample": f"requests 0..{n_req - 1} of one batch ({cpu_rows} rows: fp64 LM-head logits and the "
                         f"verify step), single-threaded C oracle, {cpu_s:.1f} s"}

    sv.spec_verify_destroy(ctx)
    line = {
        "metric": "verified logit rows/sec + achieved HBM GB/s (B=256, K=3, V=128256)",
        "value": round(rows / (total_ms * 1e-3), 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"LM-head path: B={B}, K_r ~U{{0..{K}}}, V={V}, hidden size {d}, bf16 hidden "
                               "states and LM-head weight, logits computed in the step (never stored), "
                               "draft ids only",
                   "global_batch": B, "rows_per_step": round(rows / args.steps, 1), "input_copies": ncopies,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                     "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "kernel": "lm_gemm_kernel (LM-head GEMM with the verify statistics in its epilogue)",
                     "kernel_us": pct(gemm_ms), "flops_per_launch": int(flops),
                     "flops_rule": "2 R V d (the product W h of every target row)"},
        "request_kernel_us": pct(req_ms),
        "materialised_logits_context_us": {"torch_matmul_bf16": pct(mm_ms), "spec_verify_run": pct(vr_ms)},
        "cpu_baseline": cpu,
        "wall_s": round(wall, 3),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
