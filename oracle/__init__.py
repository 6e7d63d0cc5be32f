"""CPU oracle for the speculative-decoding verify step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product library
(``rejection_sampling_verify_05_amd``) never imports, links or calls it, and the
two share no code: the arithmetic lives in ``oracle.c`` (plain C, fp64 for
probabilities and race scores), and this module only marshals NumPy arrays into
it through ctypes.

What each function follows on the pages is documented in ``oracle.h`` /
``oracle.c``.  Pins (worked examples, identities, known-answer vectors,
chi-square tests of the output law) live in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# SV_ORACLE_LIB names another build of oracle.c to load (the mutation check
# loads deliberately broken copies this way); default: the in-tree build.
_DEFAULT_SO = os.path.join(_HERE, "liborc.so")
_SO = os.environ.get("SV_ORACLE_LIB") or _DEFAULT_SO

RACE_CHUNK = 1024
LM_HEAD_CHUNK = 64  # race chunk width of the LM-head path
TAG_ACCEPT, TAG_CHUNK, TAG_TOKEN, TAG_DRAFT_CHUNK, TAG_DRAFT_TOKEN = 0, 1, 2, 3, 4
F32, BF16 = 0, 1
ERR_CU, ERR_TEMPERATURE, ERR_PENALTY, ERR_ROW, ERR_SLOT, ERR_OFFSET = 1, 2, 4, 8, 16, 32
ERR_TOP_P = 64

_lib = None


class _ReqOpts(ctypes.Structure):
    _fields_ = [("top_k", ctypes.c_int32), ("theta", ctypes.c_void_p), ("freq", ctypes.c_float),
                ("pres", ctypes.c_float), ("top_p", ctypes.c_float), ("top_p_shift", ctypes.c_double)]


class _BatchOpts(ctypes.Structure):
    _fields_ = [("freq", ctypes.c_void_p), ("pres", ctypes.c_void_p), ("top_p", ctypes.c_void_p),
                ("synthetic_rates", ctypes.c_void_p)]


GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra"]


def compile_to(src: str, out: str, extra=()) -> str:
    """Compile a copy of oracle.c (src) into the shared library `out`."""
    tmp = out + ".tmp"
    r = subprocess.run(["gcc", *GCC_FLAGS, *extra, "-o", tmp, src, "-lm"], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed on {src}:\n{r.stderr}")
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile oracle.c into liborc.so with gcc (no FMA contraction)."""
    if force or not os.path.exists(_DEFAULT_SO):
        compile_to(_SRC, _DEFAULT_SO)
    return _DEFAULT_SO


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        P = ctypes.c_void_p
        i32, i64, u32, u64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64
        f32, f64 = ctypes.c_float, ctypes.c_double
        L.orc_philox4x32_10.argtypes = [P, P, P]
        L.orc_philox4x32_10.restype = None
        L.orc_philox4x32_10_n.argtypes = [P, i64, P, P]
        L.orc_philox4x32_10_n.restype = None
        L.orc_word.argtypes = [u64, u32, u32, u32, u32]
        L.orc_word.restype = u32
        L.orc_uniform_accept.argtypes = [u32]
        L.orc_uniform_accept.restype = f64
        L.orc_uniform_race.argtypes = [u32]
        L.orc_uniform_race.restype = f64
        L.orc_exp_noise.argtypes = [u64, u32, u32, u32, u32]
        L.orc_exp_noise.restype = f64
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f32.restype = f32
        L.orc_repetition_penalty.argtypes = [P, P, i32, f32]
        L.orc_repetition_penalty.restype = None
        L.orc_kth_largest.argtypes = [P, i32, i32]
        L.orc_kth_largest.restype = f32
        L.orc_top_k_mask.argtypes = [P, i32, i32]
        L.orc_top_k_mask.restype = None
        L.orc_argmax.argtypes = [P, i32]
        L.orc_argmax.restype = i32
        L.orc_softmax.argtypes = [P, i32, f64, P]
        L.orc_softmax.restype = ctypes.c_int
        L.orc_race.argtypes = [P, i32, i32, u64, u32, u32, P]
        L.orc_race.restype = i32
        L.orc_prepare_request.argtypes = [P, ctypes.c_int, i64, i32, i32, f32, i32, P, P, P, P]
        L.orc_prepare_request.restype = ctypes.c_int
        L.orc_decide_request.argtypes = [P, P, i32, i32, f32, P, P, i64, u32, u64, u32, i32,
                                         P, P, P, P]
        L.orc_decide_request.restype = f64
        L.orc_verify_batch.argtypes = [P, ctypes.c_int, i64, i32, i32, P, i64, P, P, i32, i32,
                                       P, P, P, P, P, i32, u64, u64, i32, P, i32, P, P, P, P]
        L.orc_verify_batch.restype = u32
        L.orc_frequency_presence_penalty.argtypes = [P, P, i32, f32, f32]
        L.orc_frequency_presence_penalty.restype = None
        L.orc_top_p_keep.argtypes = [P, i32, f64, f64, P, P]
        L.orc_top_p_keep.restype = i32
        L.orc_synthetic_rates.argtypes = [f64, i32, P]
        L.orc_synthetic_rates.restype = ctypes.c_int
        L.orc_prepare_request_ex.argtypes = [P, ctypes.c_int, i64, i32, i32, f32, P, P, P, P, P]
        L.orc_prepare_request_ex.restype = ctypes.c_int
        L.orc_decide_request_ex.argtypes = [P, P, i32, i32, f32, P, P, i64, u32, u64, u32, i32, P,
                                            P, P, P, P]
        L.orc_decide_request_ex.restype = f64
        L.orc_verify_batch_ex.argtypes = [P, ctypes.c_int, i64, i32, i32, P, i64, P, P, i32, i32,
                                          P, P, P, P, P, i32, u64, u64, i32, P, P, i32, P, P, P, P]
        L.orc_verify_batch_ex.restype = u32
        L.orc_race_tags.argtypes = [P, i32, i32, u64, u32, u32, u32, u32, P]
        L.orc_race_tags.restype = i32
        L.orc_draft_sample.argtypes = [P, ctypes.c_int, i32, f32, u64, u32, u32, i32, P, P]
        L.orc_draft_sample.restype = i32
        L.orc_decide_request_q64.argtypes = [P, P, i32, i32, f32, P, P, u32, u64, u32, i32, P, P, P,
                                             P, P]
        L.orc_decide_request_q64.restype = f64
        L.orc_lm_head_logits.argtypes = [P, P, i64, i32, i32, i32, P]
        L.orc_lm_head_logits.restype = None
        L.orc_lm_head_verify.argtypes = [P, i64, P, i64, i32, i32, P, P, i32, P, u64, u64, i32, P, i32, P,
                                         P, P, P, P, P]
        L.orc_lm_head_verify.restype = ctypes.c_uint32
        L.orc_draft_q_rows.argtypes = [P, ctypes.c_int, i64, i32, i32, f32, P]
        L.orc_draft_q_rows.restype = ctypes.c_int
        L.orc_post_update.argtypes = [P, P, P, i32, P, P, i32, i32, i32, P, P, P]
        L.orc_post_update.restype = u32
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


# ---- random stream ---------------------------------------------------------
def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.asarray(ctr, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def philox4x32_10_n(ctr, key) -> np.ndarray:
    """Philox blocks of counters [n, 4] (uint32) under one key [2]; returns [n, 4] uint32."""
    c = np.ascontiguousarray(ctr, dtype=np.uint32).reshape(-1, 4)
    k = np.asarray(key, dtype=np.uint32)
    out = np.zeros_like(c)
    lib().orc_philox4x32_10_n(_ptr(c), c.shape[0], _ptr(k), _ptr(out))
    return out


def word(seed: int, offset: int, g: int, tag: int, idx: int) -> int:
    return int(lib().orc_word(seed, offset, g, tag, idx))


def uniform_accept(w: int) -> float:
    return float(lib().orc_uniform_accept(w))


def uniform_race(w: int) -> float:
    return float(lib().orc_uniform_race(w))


def exp_noise(seed: int, offset: int, g: int, tag: int, idx: int) -> float:
    return float(lib().orc_exp_noise(seed, offset, g, tag, idx))


# ---- logit processing ------------------------------------------------------
def bf16_to_f32(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([lib().orc_bf16_to_f32(int(v)) for v in b], dtype=np.float32)


def repetition_penalty(z, counts, theta: float) -> np.ndarray:
    zz = _c(z, np.float32).copy()
    cc = _c(counts, np.int32)
    lib().orc_repetition_penalty(_ptr(zz), _ptr(cc), zz.size, theta)
    return zz


def kth_largest(z, k: int) -> float:
    zz = _c(z, np.float32)
    return float(lib().orc_kth_largest(_ptr(zz), zz.size, k))


def top_k_mask(z, k: int) -> np.ndarray:
    zz = _c(z, np.float32).copy()
    lib().orc_top_k_mask(_ptr(zz), zz.size, k)
    return zz


def frequency_presence_penalty(z, counts, freq: float, pres: float) -> np.ndarray:
    zz = _c(z, np.float32).copy()
    cc = _c(counts, np.int32)
    lib().orc_frequency_presence_penalty(_ptr(zz), _ptr(cc), zz.size, freq, pres)
    return zz


def top_p_keep(p, top_p: float, shift: float = 0.0):
    """Returns (keep bool array, margin, number kept) of the nucleus set of p."""
    pp = _c(p, np.float64)
    keep = np.zeros(pp.size, dtype=np.uint8)
    m = ctypes.c_double(0.0)
    n = lib().orc_top_p_keep(_ptr(pp), pp.size, float(top_p), float(shift), _ptr(keep), ctypes.byref(m))
    return keep.astype(bool), float(m.value), int(n)


def synthetic_rates(L: float, K: int) -> np.ndarray:
    r = np.zeros(max(K, 1), dtype=np.float32)
    if lib().orc_synthetic_rates(float(L), int(K), _ptr(r)) != 0:
        raise ValueError("mean acceptance length outside [1, K + 1]")
    return r[:K]


def argmax(z) -> int:
    zz = _c(z, np.float32)
    return int(lib().orc_argmax(_ptr(zz), zz.size))


def softmax(z, T: float) -> np.ndarray:
    zz = _c(z, np.float32)
    p = np.zeros(zz.size, dtype=np.float64)
    err = lib().orc_softmax(_ptr(zz), zz.size, float(T), _ptr(p))
    if err:
        raise ValueError("row has no finite maximum")
    return p


def race(w, C: int, seed: int, offset: int, g: int):
    ww = _c(w, np.float64)
    m = ctypes.c_double(0.0)
    x = lib().orc_race(_ptr(ww), ww.size, C, seed, offset, g, ctypes.byref(m))
    return int(x), float(m.value)


def race_tags(w, C: int, seed: int, offset: int, g: int, tag_chunk: int, tag_token: int):
    ww = _c(w, np.float64)
    m = ctypes.c_double(0.0)
    x = lib().orc_race_tags(_ptr(ww), ww.size, C, seed, offset, g, tag_chunk, tag_token, ctypes.byref(m))
    return int(x), float(m.value)


# ---- draft side ------------------------------------------------------------
def draft_sample(row, T: float, seed: int, offset: int, key: int, C: int = RACE_CHUNK):
    """row: [V] float32 or uint16 (bf16 bits).  Returns (token, q(token), margin)."""
    rr = np.ascontiguousarray(row).reshape(-1)
    dtype = BF16 if rr.dtype == np.uint16 else F32
    q = ctypes.c_double(0.0)
    m = ctypes.c_double(0.0)
    d = lib().orc_draft_sample(_ptr(rr), dtype, rr.size, float(T), seed, offset, key, C, ctypes.byref(q),
                               ctypes.byref(m))
    return int(d), float(q.value), float(m.value)


def draft_q_rows(rows, T: float):
    """fp64 draft distributions softmax(z / T) of [K, V] draft logits (float32 or bf16 bits)."""
    rr = np.ascontiguousarray(rows)
    K, V = rr.shape
    Q = np.zeros((K, V), dtype=np.float64)
    if K:
        err = lib().orc_draft_q_rows(_ptr(rr), BF16 if rr.dtype == np.uint16 else F32, V, K, V, float(T), _ptr(Q))
        if err:
            raise ValueError("draft row has no finite maximum")
    return Q


# ---- LM head ----------------------------------------------------------------
def lm_head_logits(h_bits, W_bits, x0: int = 0, x1=None) -> np.ndarray:
    """fp64 logits of one row: h [d] and W [V, d] as bf16 bit patterns (uint16)."""
    h = np.ascontiguousarray(h_bits, dtype=np.uint16).reshape(-1)
    W = np.ascontiguousarray(W_bits, dtype=np.uint16)
    V, d = W.shape
    assert h.size == d
    x1 = V if x1 is None else x1
    z = np.zeros(x1 - x0, dtype=np.float64)
    lib().orc_lm_head_logits(_ptr(h), _ptr(W), d, d, x0, x1, _ptr(z))
    return z


def lm_head_verify(hidden_bits, W_bits, cu, draft_ids, temperature, seed: int = 0, offset: int = 0,
                   out_stride=None, requests=None, C: int = LM_HEAD_CHUNK):
    """Verify step on LM-head logits (no-draft-probs mode, two-level race of chunk width C).
    hidden_bits [R, d] and W_bits [V, d]: bf16 bit patterns (uint16).  requests:
    optional iterable of the request ids to compute (others stay -1 / 0).
    Returns a dict with tokens [B, out_stride], num_sampled, num_rejected,
    margin [B], greedy_gap [B], p_draft [D] and the error mask."""
    H = np.ascontiguousarray(hidden_bits, dtype=np.uint16)
    W = np.ascontiguousarray(W_bits, dtype=np.uint16)
    R, d = H.shape
    V, d2 = W.shape
    assert d == d2
    cu = _c(cu, np.int32)
    B = cu.size - 1
    D = R - B
    if out_stride is None:
        out_stride = (int(np.max(np.diff(cu))) if B > 0 else 0) + 1
    dd = _c(draft_ids, np.int32) if D > 0 else np.zeros(1, np.int32)
    T = _c(temperature, np.float32)
    tokens = np.full((B, out_stride), -1, dtype=np.int32)
    ns = np.zeros(B, dtype=np.int32)
    nr = np.zeros(B, dtype=np.int32)
    mg = np.zeros(B, dtype=np.float64)
    gg = np.zeros(B, dtype=np.float64)
    pd = np.zeros(max(D, 1), dtype=np.float32)
    only = None
    if requests is not None:
        only = np.zeros(max(B, 1), dtype=np.uint8)
        only[list(requests)] = 1
    err = lib().orc_lm_head_verify(_ptr(H), d, _ptr(W), d, d, V, _ptr(dd), _ptr(cu), B, _ptr(T), seed,
                                   offset, int(C), _ptr(tokens), out_stride, _ptr(ns), _ptr(nr), _ptr(mg),
                                   _ptr(gg), _ptr(pd), _ptr(only))
    return dict(tokens=tokens, num_sampled=ns, num_rejected=nr, margin=mg, greedy_gap=gg,
                p_draft=pd[:D], err=int(err))


# ---- one request -----------------------------------------------------------
def prepare_request_ex(rows, T: float, top_k: int = 0, theta=None, counts=None, freq: float = 0.0,
                       pres: float = 0.0, top_p: float = 1.0, top_p_shift: float = 0.0):
    """rows: [K+1, V] float32, or uint16 bf16 bits.  Returns (P [K+1,V] f64, amax,
    err, top-p margin per row)."""
    dtype = BF16 if rows.dtype == np.uint16 else F32
    rr = np.ascontiguousarray(rows)
    n, V = rr.shape
    P = np.zeros((n, V), dtype=np.float64)
    amax = np.zeros(n, dtype=np.int32)
    tm = np.zeros(n, dtype=np.float64)
    th = None if theta is None else np.array([theta], dtype=np.float32)
    cc = _c(counts, np.int32)
    o = _ReqOpts(int(top_k), None if th is None else th.ctypes.data, float(freq), float(pres),
                 float(top_p), float(top_p_shift))
    err = lib().orc_prepare_request_ex(_ptr(rr), dtype, V, n - 1, V, float(T), ctypes.byref(o),
                                       _ptr(cc), _ptr(P), _ptr(amax), _ptr(tm))
    return P, amax, int(err), tm


def prepare_request(rows, T: float, top_k: int = 0, theta=None, counts=None, **kw):
    """rows: [K+1, V] float32, or uint16 bf16 bits.  Returns (P [K+1,V] f64, amax, err).
    Keyword settings as prepare_request_ex (freq, pres, top_p, top_p_shift)."""
    P, amax, err, _ = prepare_request_ex(rows, T, top_k, theta, counts, **kw)
    return P, amax, err


def decide_request(P, amax, T: float, draft_ids, draft_probs=None, g0: int = 0, seed: int = 0,
                   offset: int = 0, C: int = RACE_CHUNK, synthetic_rates=None, draft_q64=None):
    """Returns (tokens list, num_sampled, num_rejected, margin, p_draft).  draft_q64:
    fp64 draft distributions [K, V] (from draft logits) in place of draft_probs."""
    n, V = P.shape
    K = n - 1
    PP = np.ascontiguousarray(P, dtype=np.float64)
    am = _c(amax, np.int32)
    d = _c(np.asarray(draft_ids).reshape(-1), np.int32) if K > 0 else np.zeros(1, np.int32)
    q = _c(draft_probs, np.float32)
    sr = None if synthetic_rates is None else np.ascontiguousarray(synthetic_rates, np.float32)
    if sr is not None:
        assert sr.size >= K
    tokens = np.full(K + 1, -1, dtype=np.int32)
    ns = ctypes.c_int32(0)
    nr = ctypes.c_int32(0)
    pd = np.zeros(max(K, 1), dtype=np.float32)
    if draft_q64 is not None:
        Q = np.ascontiguousarray(draft_q64, dtype=np.float64)
        mg = lib().orc_decide_request_q64(_ptr(PP), _ptr(am), K, V, float(T), _ptr(d), _ptr(Q), g0, seed,
                                          offset, C, _ptr(sr), _ptr(tokens), ctypes.byref(ns),
                                          ctypes.byref(nr), _ptr(pd))
    else:
        mg = lib().orc_decide_request_ex(_ptr(PP), _ptr(am), K, V, float(T), _ptr(d), _ptr(q),
                                         V if q is None else q.shape[-1], g0, seed, offset, C, _ptr(sr),
                                         _ptr(tokens), ctypes.byref(ns), ctypes.byref(nr), _ptr(pd))
    return tokens[: ns.value].tolist(), ns.value, nr.value, float(mg), pd[:K]


# ---- whole call ------------------------------------------------------------
def verify_batch(logits, cu, draft_ids, temperature, draft_probs=None, top_k=None,
                 rep_penalty=None, idx_mapping=None, counts=None, seed: int = 0,
                 offset: int = 0, max_k=None, out_stride=None, C: int = RACE_CHUNK,
                 freq=None, pres=None, top_p=None, synthetic_rates=None):
    """Whole verify call on host arrays.  logits: [R, V] float32 or uint16 (bf16
    bits).  Returns a dict with tokens [B, out_stride], num_sampled, num_rejected,
    margin [B], p_draft [D] and the error mask."""
    lg = np.ascontiguousarray(logits)
    dtype = BF16 if lg.dtype == np.uint16 else F32
    R, V = lg.shape
    cu = _c(cu, np.int32)
    B = cu.size - 1
    D = R - B
    if max_k is None:
        max_k = int(np.max(np.diff(cu))) if B > 0 else 0
    if out_stride is None:
        out_stride = max_k + 1
    d = _c(draft_ids, np.int32) if D > 0 else np.zeros(1, np.int32)
    q = _c(draft_probs, np.float32)
    T = _c(temperature, np.float32)
    tk = _c(top_k, np.int32)
    rp = _c(rep_penalty, np.float32)
    im = _c(idx_mapping, np.int32)
    cc = _c(counts, np.int32)
    S = 0 if cc is None else cc.shape[0]
    tokens = np.full((B, out_stride), -1, dtype=np.int32)
    ns = np.zeros(B, dtype=np.int32)
    nr = np.zeros(B, dtype=np.int32)
    mg = np.zeros(B, dtype=np.float64)
    pd = np.zeros(max(D, 1), dtype=np.float32)
    fq, pr, tp = _c(freq, np.float32), _c(pres, np.float32), _c(top_p, np.float32)
    sr = None
    if synthetic_rates is not None:
        sr = np.zeros(max(int(max_k), 1), np.float32)
        sr[: len(synthetic_rates)] = synthetic_rates
    x = _BatchOpts(*(None if a is None else a.ctypes.data for a in (fq, pr, tp, sr)))
    err = lib().orc_verify_batch_ex(_ptr(lg), dtype, V, R, V, _ptr(q), V, _ptr(d), _ptr(cu), B,
                                    int(max_k), _ptr(T), _ptr(tk), _ptr(rp), _ptr(im), _ptr(cc), S,
                                    seed, offset, C, ctypes.byref(x), _ptr(tokens), out_stride,
                                    _ptr(ns), _ptr(nr), _ptr(mg), _ptr(pd))
    return dict(tokens=tokens, num_sampled=ns, num_rejected=nr, margin=mg, p_draft=pd[:D],
                err=int(err))


def post_update(idx_mapping, query_len, tokens, num_sampled, num_rejected, last_sampled,
                counts, num_computed):
    """In-place post_update on host arrays (int32).  Returns the error mask."""
    im = _c(idx_mapping, np.int32)
    ql = _c(query_len, np.int32)
    tk = _c(tokens, np.int32)
    ns = _c(num_sampled, np.int32)
    nr = _c(num_rejected, np.int32)
    for a in (last_sampled, counts, num_computed):
        assert a.dtype == np.int32 and a.flags.c_contiguous
    B = im.size
    S, V = counts.shape
    return int(lib().orc_post_update(_ptr(im), _ptr(ql), _ptr(tk), tk.shape[1], _ptr(ns),
                                     _ptr(nr), B, V, S, _ptr(last_sampled), _ptr(counts),
                                     _ptr(num_computed)))
