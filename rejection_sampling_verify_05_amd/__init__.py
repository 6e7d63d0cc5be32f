"""Python binding of the MI355X speculative-decoding verify library.

The library is the C ABI declared in ``include/specverify.h`` and built into
``libspecverify.so`` (HIP, gfx950) next to this file.  This module only
marshals arguments: torch tensors supply device pointers and the stream, and
every step of the verify path runs in the library's kernels.  There is no
fallback: if the shared library is missing or fails to load, every entry
point raises.

Entry points (same names as the C ABI):
    spec_verify_create, spec_verify_destroy, spec_verify_run,
    spec_post_update, spec_verify_strerror, spec_verify_read_error,
    spec_verify_synthetic_rates, spec_verify_profile_start, spec_verify_profile_read,
    spec_draft_sample, spec_verify_lm_head, spec_verify_debug_philox,
    spec_verify_debug_exp_noise, spec_verify_run_noalloc
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "SV_OK", "SV_EINVAL", "SV_ECAPACITY", "SV_EDTYPE", "SV_EHIP", "SV_EINPUT",
    "SV_F32", "SV_BF16", "SV_CREATE_TOPK", "SV_RACE_CHUNK", "SV_MAX_DRAFTS",
    "SV_ERR_CU", "SV_ERR_TEMPERATURE", "SV_ERR_PENALTY", "SV_ERR_ROW", "SV_ERR_SLOT", "SV_ERR_TOP_P",
    "SpecVerifyError", "VerifyArgs", "PostUpdateArgs", "lib", "library_path",
    "spec_verify_create", "spec_verify_destroy", "spec_verify_run", "spec_post_update",
    "spec_verify_strerror", "spec_verify_read_error", "spec_verify_synthetic_rates",
    "DraftArgs", "spec_draft_sample", "SV_CREATE_LM_HEAD", "LmHeadArgs", "spec_verify_lm_head",
    "spec_verify_debug_philox", "spec_verify_debug_exp_noise", "spec_verify_run_noalloc",
]

SV_OK, SV_EINVAL, SV_ECAPACITY, SV_EDTYPE, SV_EHIP, SV_EINPUT = 0, -1, -2, -3, -4, -5
SV_F32, SV_BF16 = 0, 1
SV_CREATE_TOPK = 1
SV_CREATE_LM_HEAD = 2
SV_LM_HEAD_CHUNK = 64
SV_RACE_CHUNK = 1024
SV_MAX_DRAFTS = 64
SV_TOPK_CANDIDATES = 1024
SV_NOALLOC_MAX_ROWS, SV_NOALLOC_MAX_REQS = 16384, 4096
SV_NOALLOC_MAX_CHUNKS, SV_NOALLOC_MAX_RESID = 1 << 21, 1 << 20
SV_ERR_CU, SV_ERR_TEMPERATURE, SV_ERR_PENALTY, SV_ERR_ROW, SV_ERR_SLOT = 1, 2, 4, 8, 16
SV_ERR_TOP_P = 64

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libspecverify.so")


def library_path() -> str:
    return _SO


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {spec_verify_strerror(status)} ({status})")


class VerifyArgs(ctypes.Structure):
    """Mirror of ``sv_verify_args``."""
    _fields_ = [
        ("target_logits", ctypes.c_void_p),
        ("draft_probs", ctypes.c_void_p),
        ("draft_ids", ctypes.c_void_p),
        ("cu_num_draft", ctypes.c_void_p),
        ("temperature", ctypes.c_void_p),
        ("top_k", ctypes.c_void_p),
        ("rep_penalty", ctypes.c_void_p),
        ("idx_mapping", ctypes.c_void_p),
        ("output_bin_counts", ctypes.c_void_p),
        ("out_tokens", ctypes.c_void_p),
        ("out_num_sampled", ctypes.c_void_p),
        ("out_num_rejected", ctypes.c_void_p),
        ("dbg_p_draft", ctypes.c_void_p),
        ("dbg_probs", ctypes.c_void_p),
        ("logits_row_stride", ctypes.c_int64),
        ("draft_row_stride", ctypes.c_int64),
        ("seed", ctypes.c_uint64),
        ("offset", ctypes.c_uint64),
        ("logits_dtype", ctypes.c_int32),
        ("num_rows", ctypes.c_int32),
        ("num_reqs", ctypes.c_int32),
        ("vocab_size", ctypes.c_int32),
        ("out_stride", ctypes.c_int32),
        ("num_slots", ctypes.c_int32),
        ("frequency_penalty", ctypes.c_void_p),
        ("presence_penalty", ctypes.c_void_p),
        ("top_p", ctypes.c_void_p),
        ("synthetic_rates", ctypes.c_void_p),  # host pointer
        ("draft_logits", ctypes.c_void_p),
        ("draft_stats", ctypes.c_void_p),
        ("draft_temperature", ctypes.c_void_p),
        ("draft_logits_stride", ctypes.c_int64),
        ("draft_logits_dtype", ctypes.c_int32),
        ("post_update", ctypes.c_void_p),
        ("dbg_margin", ctypes.c_void_p),
    ]


class DraftArgs(ctypes.Structure):
    """Mirror of ``sv_draft_args``."""
    _fields_ = [
        ("draft_logits", ctypes.c_void_p),
        ("temperature", ctypes.c_void_p),
        ("cu_num_draft", ctypes.c_void_p),
        ("out_tokens", ctypes.c_void_p),
        ("out_q", ctypes.c_void_p),
        ("draft_stats", ctypes.c_void_p),
        ("draft_ids", ctypes.c_void_p),
        ("logits_row_stride", ctypes.c_int64),
        ("seed", ctypes.c_uint64),
        ("offset", ctypes.c_uint64),
        ("logits_dtype", ctypes.c_int32),
        ("num_reqs", ctypes.c_int32),
        ("vocab_size", ctypes.c_int32),
        ("step", ctypes.c_int32),
    ]


class LmHeadArgs(ctypes.Structure):
    """Mirror of ``sv_lm_head_args``."""
    _fields_ = [
        ("hidden", ctypes.c_void_p),
        ("lm_head", ctypes.c_void_p),
        ("draft_ids", ctypes.c_void_p),
        ("cu_num_draft", ctypes.c_void_p),
        ("temperature", ctypes.c_void_p),
        ("out_tokens", ctypes.c_void_p),
        ("out_num_sampled", ctypes.c_void_p),
        ("out_num_rejected", ctypes.c_void_p),
        ("dbg_p_draft", ctypes.c_void_p),
        ("dbg_logits", ctypes.c_void_p),
        ("hidden_row_stride", ctypes.c_int64),
        ("lm_head_row_stride", ctypes.c_int64),
        ("seed", ctypes.c_uint64),
        ("offset", ctypes.c_uint64),
        ("hidden_size", ctypes.c_int32),
        ("num_rows", ctypes.c_int32),
        ("num_reqs", ctypes.c_int32),
        ("vocab_size", ctypes.c_int32),
        ("out_stride", ctypes.c_int32),
        ("post_update", ctypes.c_void_p),
    ]


class PostUpdateArgs(ctypes.Structure):
    """Mirror of ``sv_post_update_args``."""
    _fields_ = [
        ("idx_mapping", ctypes.c_void_p),
        ("query_len", ctypes.c_void_p),
        ("tokens", ctypes.c_void_p),
        ("num_sampled", ctypes.c_void_p),
        ("num_rejected", ctypes.c_void_p),
        ("last_sampled", ctypes.c_void_p),
        ("output_bin_counts", ctypes.c_void_p),
        ("num_computed_tokens", ctypes.c_void_p),
        ("num_reqs", ctypes.c_int32),
        ("tokens_stride", ctypes.c_int32),
        ("vocab_size", ctypes.c_int32),
        ("num_slots", ctypes.c_int32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libspecverify.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            raise ImportError(f"{_SO} is missing: build it with __graft_entry__.build() "
                              "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(_SO)
        P = ctypes.c_void_p
        L.spec_verify_create.argtypes = [ctypes.POINTER(P), ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_uint32]
        L.spec_verify_create.restype = ctypes.c_int
        L.spec_verify_destroy.argtypes = [P]
        L.spec_verify_destroy.restype = None
        L.spec_verify_run.argtypes = [P, ctypes.POINTER(VerifyArgs), P]
        L.spec_verify_run.restype = ctypes.c_int
        L.spec_post_update.argtypes = [P, ctypes.POINTER(PostUpdateArgs), P]
        L.spec_post_update.restype = ctypes.c_int
        L.spec_verify_strerror.argtypes = [ctypes.c_int]
        L.spec_verify_strerror.restype = ctypes.c_char_p
        L.spec_verify_read_error.argtypes = [P, ctypes.POINTER(ctypes.c_uint32), P]
        L.spec_verify_read_error.restype = ctypes.c_int
        L.spec_draft_sample.argtypes = [P, ctypes.POINTER(DraftArgs), P]
        L.spec_draft_sample.restype = ctypes.c_int
        L.spec_verify_lm_head.argtypes = [P, ctypes.POINTER(LmHeadArgs), P]
        L.spec_verify_lm_head.restype = ctypes.c_int
        L.spec_verify_synthetic_rates.argtypes = [ctypes.c_float, ctypes.c_int32, P]
        L.spec_verify_synthetic_rates.restype = ctypes.c_int
        L.spec_verify_profile_start.argtypes = [P, ctypes.c_int32]
        L.spec_verify_profile_start.restype = ctypes.c_int
        L.spec_verify_profile_read.argtypes = [P, P, P, ctypes.POINTER(ctypes.c_int32)]
        L.spec_verify_profile_read.restype = ctypes.c_int
        L.spec_verify_run_noalloc.argtypes = [ctypes.POINTER(VerifyArgs), P, P]
        L.spec_verify_run_noalloc.restype = ctypes.c_int
        L.spec_verify_debug_philox.argtypes = [P, ctypes.c_int64, ctypes.c_uint64, P, P]
        L.spec_verify_debug_philox.restype = ctypes.c_int
        L.spec_verify_debug_exp_noise.argtypes = [P, ctypes.c_int64, P, P]
        L.spec_verify_debug_exp_noise.restype = ctypes.c_int
        _lib = L
    return _lib


# ---------------------------------------------------------------------------
# Marshalling helpers
# ---------------------------------------------------------------------------
def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev(t, dtype, name, ndim=None, contiguous=True):
    import torch
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# ---------------------------------------------------------------------------
# Entry points
# ---------------------------------------------------------------------------
def spec_verify_strerror(status: int) -> str:
    return lib().spec_verify_strerror(int(status)).decode()


def spec_verify_create(max_rows: int, max_reqs: int, max_k: int, max_vocab: int,
                       flags: int = 0) -> ctypes.c_void_p:
    ctx = ctypes.c_void_p()
    st = lib().spec_verify_create(ctypes.byref(ctx), max_rows, max_reqs, max_k, max_vocab, flags)
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_create")
    return ctx


def spec_verify_destroy(ctx) -> None:
    """Frees the context and clears the handle, so a second call is a no-op."""
    if ctx is None or not getattr(ctx, "value", ctx):
        return
    lib().spec_verify_destroy(ctx)
    if isinstance(ctx, ctypes.c_void_p):
        ctx.value = None


def make_verify_args(target_logits, draft_ids, cu_num_draft, temperature, out_tokens,
                     out_num_sampled, out_num_rejected, *, draft_probs=None, top_k=None,
                     rep_penalty=None, idx_mapping=None, output_bin_counts=None, seed=0,
                     offset=0, dbg_p_draft=None, dbg_probs=None, frequency_penalty=None,
                     presence_penalty=None, top_p=None, synthetic_rates=None, draft_logits=None,
                     draft_stats=None, draft_temperature=None, post_update=None,
                     dbg_margin=None) -> VerifyArgs:
    """Fill an sv_verify_args from torch tensors (no copies, no compute).
    post_update: a PostUpdateArgs (make_post_update_args) applied inside the call."""
    import torch
    if target_logits.dim() != 2 or not target_logits.is_cuda or target_logits.stride(1) != 1:
        raise ValueError("target_logits must be a 2-D CUDA tensor with unit column stride")
    if target_logits.dtype == torch.float32:
        dt = SV_F32
    elif target_logits.dtype == torch.bfloat16:
        dt = SV_BF16
    else:
        raise TypeError("target_logits must be float32 or bfloat16")
    R, V = target_logits.shape
    _dev(draft_ids, torch.int32, "draft_ids", 1)
    _dev(cu_num_draft, torch.int32, "cu_num_draft", 1)
    _dev(temperature, torch.float32, "temperature", 1)
    _dev(out_tokens, torch.int32, "out_tokens", 2)
    _dev(out_num_sampled, torch.int32, "out_num_sampled", 1)
    _dev(out_num_rejected, torch.int32, "out_num_rejected", 1)
    if draft_probs is not None:
        _dev(draft_probs, torch.float32, "draft_probs", 2, contiguous=False)
        if draft_probs.stride(1) != 1:
            raise ValueError("draft_probs must have unit column stride")
    _dev(top_k, torch.int32, "top_k", 1)
    _dev(rep_penalty, torch.float32, "rep_penalty", 1)
    _dev(frequency_penalty, torch.float32, "frequency_penalty", 1)
    _dev(presence_penalty, torch.float32, "presence_penalty", 1)
    _dev(top_p, torch.float32, "top_p", 1)
    _dev(draft_stats, torch.float32, "draft_stats", 1)
    _dev(draft_temperature, torch.float32, "draft_temperature", 1)
    if draft_logits is not None:
        if draft_logits.dim() != 2 or not draft_logits.is_cuda or draft_logits.stride(1) != 1:
            raise ValueError("draft_logits must be a 2-D CUDA tensor with unit column stride")
        if draft_logits.dtype not in (torch.float32, torch.bfloat16):
            raise TypeError("draft_logits must be float32 or bfloat16")
    _dev(idx_mapping, torch.int32, "idx_mapping", 1)
    _dev(output_bin_counts, torch.int32, "output_bin_counts", 2)
    _dev(dbg_p_draft, torch.float32, "dbg_p_draft", 1)
    _dev(dbg_probs, torch.float32, "dbg_probs", 2)
    _dev(dbg_margin, torch.float32, "dbg_margin", 1)
    B = cu_num_draft.numel() - 1
    a = VerifyArgs()
    a.target_logits = target_logits.data_ptr()
    a.draft_probs = None if draft_probs is None else draft_probs.data_ptr()
    a.draft_ids = draft_ids.data_ptr() if draft_ids.numel() else None
    a.cu_num_draft = cu_num_draft.data_ptr()
    a.temperature = temperature.data_ptr()
    a.top_k = None if top_k is None else top_k.data_ptr()
    a.rep_penalty = None if rep_penalty is None else rep_penalty.data_ptr()
    a.idx_mapping = None if idx_mapping is None else idx_mapping.data_ptr()
    a.output_bin_counts = None if output_bin_counts is None else output_bin_counts.data_ptr()
    a.out_tokens = out_tokens.data_ptr()
    a.out_num_sampled = out_num_sampled.data_ptr()
    a.out_num_rejected = out_num_rejected.data_ptr()
    a.dbg_p_draft = None if dbg_p_draft is None else dbg_p_draft.data_ptr()
    a.dbg_probs = None if dbg_probs is None else dbg_probs.data_ptr()
    a.dbg_margin = None if dbg_margin is None else dbg_margin.data_ptr()
    a.logits_row_stride = target_logits.stride(0)
    a.draft_row_stride = 0 if draft_probs is None else draft_probs.stride(0)
    a.seed = int(seed)
    a.offset = int(offset)
    a.logits_dtype = dt
    a.num_rows = R
    a.num_reqs = B
    a.vocab_size = V
    a.out_stride = out_tokens.shape[1]
    a.num_slots = 0 if output_bin_counts is None else output_bin_counts.shape[0]
    a.frequency_penalty = None if frequency_penalty is None else frequency_penalty.data_ptr()
    a.presence_penalty = None if presence_penalty is None else presence_penalty.data_ptr()
    a.top_p = None if top_p is None else top_p.data_ptr()
    if draft_logits is not None:
        a.draft_logits = draft_logits.data_ptr()
        a.draft_logits_stride = draft_logits.stride(0)
        a.draft_logits_dtype = SV_BF16 if draft_logits.dtype == torch.bfloat16 else SV_F32
    a.draft_stats = None if draft_stats is None else draft_stats.data_ptr()
    a.draft_temperature = None if draft_temperature is None else draft_temperature.data_ptr()
    if synthetic_rates is not None:
        # host array: copied by the library during the call
        vals = [float(v) for v in synthetic_rates]
        buf = (ctypes.c_float * max(len(vals), 1))(*vals)
        a._synthetic_buf = buf
        a.synthetic_rates = ctypes.cast(buf, ctypes.c_void_p).value
    if post_update is not None:
        if not isinstance(post_update, PostUpdateArgs):
            raise TypeError("post_update must be a PostUpdateArgs")
        a._post_update = post_update  # keeps the host struct alive with the args
        a.post_update = ctypes.addressof(post_update)
    return a


def spec_verify_run(ctx, *args, stream=None, **kwargs) -> None:
    """spec_verify_run(ctx, target_logits, draft_ids, cu_num_draft, temperature,
    out_tokens, out_num_sampled, out_num_rejected, *, draft_probs=None, top_k=None,
    rep_penalty=None, idx_mapping=None, output_bin_counts=None, seed=0, offset=0,
    dbg_p_draft=None, dbg_probs=None, frequency_penalty=None, presence_penalty=None,
    top_p=None, synthetic_rates=None (a host sequence), draft_logits=None,
    draft_stats=None, draft_temperature=None, post_update=None, dbg_margin=None,
    stream=None), or spec_verify_run(ctx, VerifyArgs)."""
    a = args[0] if len(args) == 1 and isinstance(args[0], VerifyArgs) else make_verify_args(*args, **kwargs)
    st = lib().spec_verify_run(ctx, ctypes.byref(a), _stream_handle(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_run")


def spec_verify_run_noalloc(*args, device_errors, stream=None, **kwargs) -> None:
    """spec_verify_run without a context (the library's fixed scratch array);
    device_errors: an int32 device tensor of one element that the kernels OR
    their SV_ERR_* bits into (the caller zeroes and reads it).  Arguments as
    spec_verify_run, passed as make_verify_args' (or one VerifyArgs)."""
    import torch
    _dev(device_errors, torch.int32, "device_errors")
    if device_errors.numel() < 1:
        raise ValueError("device_errors needs one element")
    a = args[0] if len(args) == 1 and isinstance(args[0], VerifyArgs) else make_verify_args(*args, **kwargs)
    st = lib().spec_verify_run_noalloc(ctypes.byref(a), _ptr(device_errors), _stream_handle(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_run_noalloc")


def make_post_update_args(idx_mapping, query_len, tokens, num_sampled, num_rejected,
                          last_sampled, output_bin_counts, num_computed_tokens) -> PostUpdateArgs:
    import torch
    for t, n, d in [(idx_mapping, "idx_mapping", 1), (query_len, "query_len", 1),
                    (tokens, "tokens", 2), (num_sampled, "num_sampled", 1),
                    (num_rejected, "num_rejected", 1), (last_sampled, "last_sampled", 1),
                    (output_bin_counts, "output_bin_counts", 2),
                    (num_computed_tokens, "num_computed_tokens", 1)]:
        _dev(t, torch.int32, n, d)
    a = PostUpdateArgs()
    a.idx_mapping = idx_mapping.data_ptr()
    a.query_len = query_len.data_ptr()
    a.tokens = tokens.data_ptr()
    a.num_sampled = num_sampled.data_ptr()
    a.num_rejected = num_rejected.data_ptr()
    a.last_sampled = last_sampled.data_ptr()
    a.output_bin_counts = output_bin_counts.data_ptr()
    a.num_computed_tokens = num_computed_tokens.data_ptr()
    a.num_reqs = idx_mapping.numel()
    a.tokens_stride = tokens.shape[1]
    a.vocab_size = output_bin_counts.shape[1]
    a.num_slots = output_bin_counts.shape[0]
    return a


def spec_post_update(ctx, *args, stream=None) -> None:
    """spec_post_update(ctx, idx_mapping, query_len, tokens, num_sampled, num_rejected,
    last_sampled, output_bin_counts, num_computed_tokens, stream=None), or with a
    PostUpdateArgs."""
    a = args[0] if len(args) == 1 and isinstance(args[0], PostUpdateArgs) else make_post_update_args(*args)
    st = lib().spec_post_update(ctx, ctypes.byref(a), _stream_handle(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_post_update")


def make_draft_args(draft_logits, temperature, cu_num_draft, out_tokens, draft_stats, *, step: int,
                    out_q=None, seed=0, offset=0, draft_ids=None) -> DraftArgs:
    """Fill an sv_draft_args from torch tensors (no copies, no compute)."""
    import torch
    if draft_logits.dim() != 2 or not draft_logits.is_cuda or draft_logits.stride(1) != 1:
        raise ValueError("draft_logits must be a 2-D CUDA tensor with unit column stride")
    if draft_logits.dtype == torch.float32:
        dt = SV_F32
    elif draft_logits.dtype == torch.bfloat16:
        dt = SV_BF16
    else:
        raise TypeError("draft_logits must be float32 or bfloat16")
    _dev(temperature, torch.float32, "temperature", 1)
    _dev(cu_num_draft, torch.int32, "cu_num_draft", 1)
    _dev(out_tokens, torch.int32, "out_tokens", 1)
    _dev(out_q, torch.float32, "out_q", 1)
    _dev(draft_stats, torch.float32, "draft_stats", 1)
    _dev(draft_ids, torch.int32, "draft_ids", 1)
    a = DraftArgs()
    a.draft_logits = draft_logits.data_ptr()
    a.temperature = temperature.data_ptr()
    a.cu_num_draft = cu_num_draft.data_ptr()
    a.out_tokens = out_tokens.data_ptr()
    a.out_q = None if out_q is None else out_q.data_ptr()
    a.draft_stats = draft_stats.data_ptr()
    a.draft_ids = None if draft_ids is None else draft_ids.data_ptr()
    a.logits_row_stride = draft_logits.stride(0)
    a.seed = int(seed)
    a.offset = int(offset)
    a.logits_dtype = dt
    a.num_reqs = draft_logits.shape[0]
    a.vocab_size = draft_logits.shape[1]
    a.step = int(step)
    return a


def spec_draft_sample(ctx, *args, stream=None, **kwargs) -> None:
    """spec_draft_sample(ctx, draft_logits [B, V], temperature [B], cu_num_draft [B+1],
    out_tokens [B], draft_stats [2 D], step=i, out_q=None, seed=0, offset=0,
    draft_ids=None, stream=None), or spec_draft_sample(ctx, DraftArgs)."""
    a = args[0] if len(args) == 1 and isinstance(args[0], DraftArgs) else make_draft_args(*args, **kwargs)
    st = lib().spec_draft_sample(ctx, ctypes.byref(a), _stream_handle(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_draft_sample")


def make_lm_head_args(hidden, lm_head, draft_ids, cu_num_draft, temperature, out_tokens,
                      out_num_sampled, out_num_rejected, *, seed=0, offset=0, dbg_p_draft=None,
                      dbg_logits=None, post_update=None) -> LmHeadArgs:
    """Fill an sv_lm_head_args from torch tensors (no copies, no compute).
    hidden [R, d] and lm_head [V, d] are bfloat16 with unit column stride."""
    import torch
    for t, n in ((hidden, "hidden"), (lm_head, "lm_head")):
        if t.dim() != 2 or not t.is_cuda or t.stride(1) != 1 or t.dtype != torch.bfloat16:
            raise ValueError(f"{n} must be a 2-D bfloat16 CUDA tensor with unit column stride")
    if hidden.shape[1] != lm_head.shape[1]:
        raise ValueError("hidden and lm_head disagree on the hidden size")
    _dev(draft_ids, torch.int32, "draft_ids", 1)
    _dev(cu_num_draft, torch.int32, "cu_num_draft", 1)
    _dev(temperature, torch.float32, "temperature", 1)
    _dev(out_tokens, torch.int32, "out_tokens", 2)
    _dev(out_num_sampled, torch.int32, "out_num_sampled", 1)
    _dev(out_num_rejected, torch.int32, "out_num_rejected", 1)
    _dev(dbg_p_draft, torch.float32, "dbg_p_draft", 1)
    _dev(dbg_logits, torch.float32, "dbg_logits", 2)
    a = LmHeadArgs()
    a.hidden = hidden.data_ptr()
    a.lm_head = lm_head.data_ptr()
    a.draft_ids = None if draft_ids is None or draft_ids.numel() == 0 else draft_ids.data_ptr()
    a.cu_num_draft = cu_num_draft.data_ptr()
    a.temperature = temperature.data_ptr()
    a.out_tokens = out_tokens.data_ptr()
    a.out_num_sampled = out_num_sampled.data_ptr()
    a.out_num_rejected = out_num_rejected.data_ptr()
    a.dbg_p_draft = None if dbg_p_draft is None else dbg_p_draft.data_ptr()
    a.dbg_logits = None if dbg_logits is None else dbg_logits.data_ptr()
    a.hidden_row_stride = hidden.stride(0)
    a.lm_head_row_stride = lm_head.stride(0)
    a.seed = int(seed)
    a.offset = int(offset)
    a.hidden_size = hidden.shape[1]
    a.num_rows = hidden.shape[0]
    a.num_reqs = cu_num_draft.shape[0] - 1
    a.vocab_size = lm_head.shape[0]
    a.out_stride = out_tokens.shape[1]
    if post_update is not None:
        if not isinstance(post_update, PostUpdateArgs):
            raise TypeError("post_update must be a PostUpdateArgs")
        a._post_update = post_update
        a.post_update = ctypes.addressof(post_update)
    return a


def spec_verify_lm_head(ctx, *args, stream=None, **kwargs) -> None:
    """spec_verify_lm_head(ctx, hidden [R, d], lm_head [V, d], draft_ids [D],
    cu_num_draft [B+1], temperature [B], out_tokens [B, S], out_num_sampled [B],
    out_num_rejected [B], seed=0, offset=0, dbg_p_draft=None, dbg_logits=None,
    stream=None), or spec_verify_lm_head(ctx, LmHeadArgs)."""
    a = args[0] if len(args) == 1 and isinstance(args[0], LmHeadArgs) else make_lm_head_args(*args, **kwargs)
    st = lib().spec_verify_lm_head(ctx, ctypes.byref(a), _stream_handle(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_lm_head")


def spec_verify_synthetic_rates(mean_length: float, k: int) -> list:
    """Minimum-variance unconditional acceptance rates for a mean acceptance length."""
    buf = (ctypes.c_float * max(int(k), 1))()
    st = lib().spec_verify_synthetic_rates(float(mean_length), int(k), ctypes.cast(buf, ctypes.c_void_p))
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_synthetic_rates")
    return [buf[i] for i in range(int(k))]


def spec_verify_read_error(ctx, stream=None) -> int:
    """Synchronise the stream and return (and clear) the device error bits."""
    flags = ctypes.c_uint32(0)
    st = lib().spec_verify_read_error(ctx, ctypes.byref(flags), _stream_handle(stream))
    if st not in (SV_OK, SV_EINPUT):
        raise SpecVerifyError(st, "spec_verify_read_error")
    return int(flags.value)


def spec_verify_profile_start(ctx, max_calls: int) -> None:
    """Record HIP events around the streaming and epilogue kernels of the next
    max_calls spec_verify_run calls (on their own stream)."""
    st = lib().spec_verify_profile_start(ctx, int(max_calls))
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_profile_start")


def spec_verify_profile_read(ctx, max_calls: int):
    """Wait for the recorded events; return (stream_ms, epilogue_ms) lists of
    per-call kernel durations in milliseconds, and stop recording."""
    a = (ctypes.c_float * max_calls)()
    b = (ctypes.c_float * max_calls)()
    n = ctypes.c_int32(0)
    st = lib().spec_verify_profile_read(ctx, ctypes.cast(a, ctypes.c_void_p), ctypes.cast(b, ctypes.c_void_p),
                                        ctypes.byref(n))
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_profile_read")
    return list(a[:n.value]), list(b[:n.value])


def spec_verify_debug_philox(counters, key: int, out=None, stream=None):
    """Philox4x32-10 blocks of the library for int32/uint32 device counters [n, 4]
    under a 64-bit key; returns (or fills) an int32 [n, 4] tensor of the words."""
    import torch
    if counters.dim() != 2 or counters.shape[1] != 4:
        raise ValueError("counters must be [n, 4]")
    _dev(counters, counters.dtype, "counters")
    if counters.element_size() != 4:
        raise TypeError("counters must hold 32-bit words")
    if out is None:
        out = torch.empty((counters.shape[0], 4), dtype=torch.int32, device=counters.device)
    _dev(out, torch.int32, "out", 2)
    st = lib().spec_verify_debug_philox(_ptr(counters), counters.shape[0], key & 0xFFFFFFFFFFFFFFFF, _ptr(out),
                                        _stream_handle(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_debug_philox")
    return out


def spec_verify_debug_exp_noise(words, out=None, stream=None):
    """The library's fp32 Exp(1) noise for 32-bit device words [n]; returns a float32 [n] tensor."""
    import torch
    _dev(words, words.dtype, "words", 1)
    if words.element_size() != 4:
        raise TypeError("words must be 32-bit")
    if out is None:
        out = torch.empty(words.shape[0], dtype=torch.float32, device=words.device)
    _dev(out, torch.float32, "out", 1)
    st = lib().spec_verify_debug_exp_noise(_ptr(words), words.shape[0], _ptr(out), _stream_handle(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_debug_exp_noise")
    return out
