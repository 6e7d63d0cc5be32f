/*
 * specverify.h -- C ABI of the MI355X (gfx950) speculative-decoding verify step.
 *
 * One call of spec_verify_run verifies a batch of B requests.  Request r
 * proposed K_r draft tokens; the target model produced K_r + 1 logit rows for
 * it (one per draft position plus the extra "bonus" row), packed request after
 * request into target_logits [R, V] with R = sum_r (K_r + 1).  Request r owns
 * rows cu[r] + r ... cu[r+1] + r, where cu = cu_num_draft is the prefix sum of
 * the K_r (the layout of the target logits and the cu_num_logits prefix sums
 * in "【vllm】DeepSeekMTP、eagle", sample() walk-through; bonus rows are the last
 * row of each request as in "vLLM 投机解码（Eagle / MTP）实现与运行流程", 8.2).
 *
 * For each request the library computes, on the device:
 *   1. processed logits z: repetition penalty, frequency penalty, presence
 *      penalty (each optional), then top-k (optional) (8.2 of the second page:
 *      processors, constraints, then softmax; the frequency penalty is the
 *      first page's penalties walk-through, z -= penalty * count);
 *   2. p = softmax(z / T) per row (T = temperature[r]); T == 0 selects the
 *      greedy rule of 8.3 (argmax of z, lowest index on ties); then top-p
 *      (optional; clamped to [1e-6, 1] as in the Mini-SGLang sampler
 *      conventions): a token stays iff the tokens strictly more probable than
 *      it hold less than top_p of the mass, and p is renormalised over them;
 *   3. for i = 0..K_r-1: accept draft d_i iff it is a valid id, q_i(d_i) > 0
 *      and p_i(d_i) >= u_i * q_i(d_i) (q = 1 without draft probabilities),
 *      u_i a Philox uniform on ((0,1]; 8.3, stochastic branch, and the
 *      residual-distribution Q&A of the same page); stop at the first reject j.
 *      Synthetic acceptance ("speculative decoding in vLLM", 7.2) replaces this
 *      test by u_i * a_i <= a_{i+1} (fp64) for unconditional per-position
 *      rates a (a_0 = 1), so position i + 1 is accepted with probability
 *      a_{i+1}; everything else is unchanged;
 *   4. after a reject: the recovered token from max(0, p_j - q_j), or, with no
 *      draft probabilities, from p_j with d_j removed (NO_DRAFT_PROBS Q&A);
 *      if every draft passed: the bonus token from row K_r (bonus Q&A);
 *      sampling is a two-level exponential race argmax(w / E), E ~ Exp(1),
 *      over chunks of SV_RACE_CHUNK tokens and then over the winning chunk's
 *      tokens (its law is exactly w / sum w);
 *   5. outputs: out_tokens[r][0..num_sampled) = accepted drafts then the
 *      recovered or bonus token, -1 after; num_sampled = accepted + 1;
 *      num_rejected = K_r - accepted.
 * spec_post_update then applies the per-request bookkeeping of the first page's
 * postprocess walk-through: last_sampled, output_bin_counts and
 * num_computed_tokens += query_len - num_rejected.
 *
 * Random stream: Philox4x32-10 (Salmon et al., SC'11), key = (seed lo, seed
 * hi), counter = (idx >> 2, target row g, tag, offset), word idx & 3; tag 0 is
 * the accept uniform of row g (idx 0), tag 1 the chunk race (idx = chunk), tag
 * 2 the token race (idx = token).  Accept uniform ((w >> 8) + 1) * 2^-24, race
 * uniform (w >> 8) * 2^-24 with E = -ln U.  Results are a pure function of
 * (inputs, seed, offset): the same call replays bit for bit.
 *
 * Conventions for every entry point:
 *   - pointers in argument structs are DEVICE pointers unless stated; the
 *     caller owns them and they must stay valid until the stream reaches the
 *     work enqueued by the call;
 *   - calls are stream-ordered and asynchronous; nothing synchronises the host
 *     except spec_verify_read_error;
 *   - a context is used by one stream at a time (not re-entrant);
 *   - host-side checks (pointers, sizes, capacities, dtype) run before any
 *     launch and return SV_EINVAL / SV_ECAPACITY / SV_EDTYPE with nothing
 *     enqueued; a failed launch returns SV_EHIP;
 *   - device-side checks set bits in the context's error word (read with
 *     spec_verify_read_error).  A request whose temperature, penalty, slot or
 *     rows are invalid gets num_sampled = num_rejected = 0 and a row of -1; an
 *     invalid cu_num_draft leaves that call's outputs unspecified.  Every
 *     memory access stays inside the buffers described here in all cases.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library exports only the entry points below (it is built with hidden
 * default visibility). */
#if defined(__GNUC__)
#define SV_API __attribute__((visibility("default")))
#else
#define SV_API
#endif

#define SV_RACE_CHUNK 1024        /* tokens per chunk of the two-level race        */
#define SV_MAX_DRAFTS 64          /* largest max_k a context accepts               */
#define SV_TOPK_CANDIDATES 1024   /* top-k rows with more kept tokens use the dense path */
#define SV_LM_HEAD_CHUNK 64       /* tokens per race chunk of spec_verify_lm_head          */

typedef struct sv_ctx sv_ctx; /* opaque; owns the device scratch */
struct sv_post_update_args;   /* defined with spec_post_update below */

/* Return codes. */
enum {
  SV_OK = 0,
  SV_EINVAL = -1,    /* bad pointer, size or scalar                       */
  SV_ECAPACITY = -2, /* exceeds the capacities given to spec_verify_create */
  SV_EDTYPE = -3,    /* unknown logits dtype                               */
  SV_EHIP = -4,      /* a HIP runtime call or kernel launch failed         */
  SV_EINPUT = -5     /* device-side input check failed (see error bits)    */
};

/* Logits element types. */
enum { SV_F32 = 0, SV_BF16 = 1 };

/* Bits of the device error word. */
enum {
  SV_ERR_CU = 1u << 0,          /* cu_num_draft is not a valid prefix sum for this call */
  SV_ERR_TEMPERATURE = 1u << 1, /* temperature < 0, NaN or infinite                      */
  SV_ERR_PENALTY = 1u << 2,     /* repetition penalty <= 0, NaN or infinite              */
  SV_ERR_ROW = 1u << 3,         /* a processed logit row has no finite maximum           */
  SV_ERR_SLOT = 1u << 4,        /* idx_mapping outside [0, num_slots)                    */
  SV_ERR_TOP_P = 1u << 6        /* top_p is NaN                                          */
};

/* spec_verify_create flags. */
enum {
  SV_CREATE_TOPK = 1u << 0,    /* reserve top-k candidate storage (needed for top_k != NULL)  */
  SV_CREATE_LM_HEAD = 1u << 1 /* reserve the LM-head path's tile records (spec_verify_lm_head) */
};
/*
 * Create a context sized for calls with at most max_rows target rows,
 * max_reqs requests, max_k drafts per request (<= SV_MAX_DRAFTS) and a
 * vocabulary of at most max_vocab tokens.  Allocates device scratch on the
 * current device (chunk tables of ceil(max_vocab / SV_RACE_CHUNK) entries per
 * row, per-request counters; with SV_CREATE_TOPK also SV_TOPK_CANDIDATES
 * candidates per row).  *out receives the context.  Errors: SV_EINVAL (NULL
 * out, non-positive size), SV_ECAPACITY (max_k > SV_MAX_DRAFTS), SV_EHIP.
 */
SV_API int spec_verify_create(sv_ctx **out, int32_t max_rows, int32_t max_reqs, int32_t max_k,
                       int32_t max_vocab, uint32_t flags);

/* Free a context (synchronises the device first).  NULL is ignored. */
SV_API void spec_verify_destroy(sv_ctx *ctx);

typedef struct sv_verify_args {
  const void *target_logits;        /* [num_rows, logits_row_stride], dtype logits_dtype    */
  const float *draft_probs;         /* [D, draft_row_stride] fp32, or NULL: no-draft-probs  */
                                    /* mode (q is the point mass at the draft), D = R - B   */
  const int32_t *draft_ids;         /* [D]; ids outside [0, V) are simply rejected         */
  const int32_t *cu_num_draft;      /* [num_reqs + 1]; cu[0] = 0, nondecreasing,            */
                                    /* cu[B] = D, K_r <= out_stride - 1                     */
  const float *temperature;         /* [num_reqs]; 0 = greedy, > 0 sampled                  */
  const int32_t *top_k;             /* [num_reqs] or NULL; k < 1 or k >= V disables         */
  const float *rep_penalty;         /* [num_reqs] or NULL; 1 = none                         */
  const int32_t *idx_mapping;       /* [num_reqs] batch row -> state slot (with a penalty)  */
  const int32_t *output_bin_counts; /* [num_slots, vocab_size] (read here, with a penalty)  */
  int32_t *out_tokens;              /* [num_reqs, out_stride], -1 padded                    */
  int32_t *out_num_sampled;         /* [num_reqs]                                           */
  int32_t *out_num_rejected;        /* [num_reqs]                                           */
  float *dbg_p_draft;               /* [D] p_i(d_i) (-1 for greedy requests) or NULL        */
  float *dbg_probs;                 /* [num_rows, vocab_size] processed probabilities or   */
                                    /* NULL; slow, for parity checks only                   */
  int64_t logits_row_stride;        /* elements between rows, >= vocab_size                */
  int64_t draft_row_stride;         /* elements between draft rows, >= vocab_size           */
  uint64_t seed;                    /* Philox key                                           */
  uint64_t offset;                  /* per-call step, must be < 2^32                        */
  int32_t logits_dtype;             /* SV_F32 or SV_BF16                                    */
  int32_t num_rows;                 /* R = cu[B] + B                                        */
  int32_t num_reqs;                 /* B                                                    */
  int32_t vocab_size;               /* V <= max_vocab                                       */
  int32_t out_stride;               /* row length of out_tokens, <= max_k + 1               */
  int32_t num_slots;                /* rows of output_bin_counts (0 without a penalty)      */
  const float *frequency_penalty;   /* [num_reqs] or NULL; z -= f * count, 0 = none          */
  const float *presence_penalty;    /* [num_reqs] or NULL; z -= f where count > 0, 0 = none  */
  const float *top_p;               /* [num_reqs] or NULL; clamped to [1e-6, 1], 1 = none    */
  const float *synthetic_rates;     /* HOST pointer [out_stride - 1] or NULL: synthetic      */
                                    /* acceptance with these unconditional rates of draft   */
                                    /* positions 1.., each in [0, 1], non-increasing        */
  /* Draft-logits mode (instead of draft_probs; all three given or none):               */
  const void *draft_logits;         /* [D, draft_logits_stride], dtype draft_logits_dtype   */
  const float *draft_stats;         /* [2 D] (m, s) per draft row, from spec_draft_sample   */
  const float *draft_temperature;   /* [num_reqs] temperature the drafts were drawn at; 0:  */
                                    /* greedy drafts (then as draft ids only)               */
  int64_t draft_logits_stride;      /* elements between draft-logit rows, >= vocab_size     */
  int32_t draft_logits_dtype;       /* SV_F32 or SV_BF16                                    */
  /* HOST pointer or NULL: apply post_update (see spec_post_update) for this    */
  /* step inside the call, from its own outputs, as soon as each request's      */
  /* tokens are final; its idx_mapping, query_len, last_sampled,                */
  /* output_bin_counts, num_computed_tokens and num_slots are used (num_reqs    */
  /* and vocab_size must match; tokens, num_sampled, num_rejected and           */
  /* tokens_stride are ignored).  Not with dbg_probs.                           */
  const struct sv_post_update_args *post_update;
  /* [num_rows] or NULL: per target row, the smallest relative margin of the  */
  /* random decisions taken on it, in the library's own fp32 quantities (slow; */
  /* parity checks only; not with post_update).  Accept test of draft i:      */
  /* |p - u q| / max(p, u q) ("vLLM 投机解码（Eagle / MTP）实现与运行流程",      */
  /* section 8.3); the race of the sampled row: 1 - s2 / s1 of the best and     */
  /* second-best race scores at the chunk level and at the token level (1     */
  /* with a single candidate), each race recomputed over the whole row; 0     */
  /* when that recomputation picks another token than the one written.        */
  /* INFINITY: no random decision (greedy requests, rows after the sampled    */
  /* one, requests written empty); synthetic acceptance has no accept margin. */
  float *dbg_margin;
} sv_verify_args;

/*
 * Enqueue one verify step on `stream` (see the top of this file).  Reads the
 * target logits once per row in a streaming pass; in draft-probs mode it also
 * reads the full draft row of each rejected request.  With top_p and neither
 * top_k nor a penalty, 16-byte aligned bf16 rows of at most 131072 tokens are
 * held on chip and read once in all; otherwise rows that have no top-k
 * candidate list are read again: two (bf16 without penalties) or four more
 * passes find the nucleus threshold, and one more recomputes their
 * statistics under it.  A penalty array other than NULL needs idx_mapping,
 * output_bin_counts and num_slots >= 1.  Errors: SV_EINVAL (also synthetic
 * rates outside [0, 1], not finite or increasing; post_update with dbg_probs,
 * dbg_margin or mismatched sizes), SV_ECAPACITY, SV_EDTYPE, SV_EHIP (nothing
 * enqueued on the first three).  With post_update the bookkeeping of the step
 * is done by the call's last kernels (one launch fewer than calling
 * spec_post_update afterwards; the same results).
 */
SV_API int spec_verify_run(sv_ctx *ctx, const sv_verify_args *args, hipStream_t stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, serving loops that must not allocate, harnesses that forbid it.
 * The same verify step as spec_verify_run, with the same kernels and the
 * same results, without a context.  Its scratch (chunk tables, row
 * statistics, residual tables, row states) is one fixed device array of the
 * library, of about 21 MB, which each GPU the library runs on holds until the
 * process ends.  The first call on a device looks up that device's copy of
 * the array.  The call allocates nothing, on the device or the host.
 *
 * Limits (SV_ECAPACITY beyond them, nothing enqueued):
 * - at most SV_NOALLOC_MAX_ROWS target rows and SV_NOALLOC_MAX_REQS requests;
 * - rows x ceil(V / SV_RACE_CHUNK) <= SV_NOALLOC_MAX_CHUNKS;
 * - requests x ceil(V / SV_RACE_CHUNK) <= SV_NOALLOC_MAX_RESID;
 * - no top_k (its candidate lists need SV_TOPK_CANDIDATES entries per row).
 * Other settings are as for spec_verify_run, except that profiling is not
 * available.
 *
 * device_errors: a DEVICE uint32 word that the call's kernels OR their
 * SV_ERR_* bits into.  The caller zeroes it and reads it.
 *
 * Every call on one GPU shares that GPU's array, and the array keeps the
 * last call's contents.  Calls whose work overlaps on one GPU (on different
 * streams, or from different host threads without ordering) race and give
 * unspecified results.  Calls ordered on one stream are safe.
 * Errors: as spec_verify_run, plus SV_EINVAL for a NULL device_errors.
 */
#define SV_NOALLOC_MAX_ROWS 16384
#define SV_NOALLOC_MAX_REQS 4096
#define SV_NOALLOC_MAX_CHUNKS (1 << 21)
#define SV_NOALLOC_MAX_RESID (1 << 20)
SV_API int spec_verify_run_noalloc(const sv_verify_args *args, uint32_t *device_errors, hipStream_t stream);

struct sv_post_update_args {
  const int32_t *idx_mapping;   /* [num_reqs] batch row -> state slot                     */
  const int32_t *query_len;     /* [num_reqs] tokens scheduled for the request this step  */
  const int32_t *tokens;        /* [num_reqs, tokens_stride] out_tokens of the verify step */
  const int32_t *num_sampled;   /* [num_reqs]                                             */
  const int32_t *num_rejected;  /* [num_reqs]                                             */
  int32_t *last_sampled;        /* [num_slots] in/out                                     */
  int32_t *output_bin_counts;   /* [num_slots, vocab_size] in/out                         */
  int32_t *num_computed_tokens; /* [num_slots] in/out                                     */
  int32_t num_reqs;
  int32_t tokens_stride;
  int32_t vocab_size;
  int32_t num_slots;
};
typedef struct sv_post_update_args sv_post_update_args;

/*
 * post_update ("【vllm】DeepSeekMTP、eagle", postprocess / _post_update_kernel):
 * for every request with num_sampled > 0 and slot s = idx_mapping[r]:
 * output_bin_counts[s][t] += 1 for each sampled token t in [0, V) (a token
 * sampled twice counts twice), last_sampled[s] = the last sampled token,
 * num_computed_tokens[s] += query_len[r] - num_rejected[r].  Slots outside
 * [0, num_slots) are skipped and raise SV_ERR_SLOT.  Two requests of one call
 * must not share a slot (counts stay exact, last_sampled is then either one).
 * Errors: SV_EINVAL, SV_EHIP.
 */
SV_API int spec_post_update(sv_ctx *ctx, const sv_post_update_args *args, hipStream_t stream);

/*
 * Draft-side sampling (NEXT row of the verify step; "speculative decoding in
 * vLLM", 7.1: probabilistic drafting needs the draft distribution at
 * verification).  For one draft step, request r's draft token is drawn from
 * q = softmax(z_r / T_r) over its row of draft_logits by the same two-level
 * race as the verifier, on Philox counter row cu[r] + step (its row in the
 * verify call's draft arrays) with tags 3 (chunks) and 4 (tokens); T_r = 0
 * takes the argmax (lowest index).  Outputs: out_tokens[r] (-1 when step >=
 * K_r or the request is invalid), out_q[r] = q(d) (1 for greedy; may be NULL),
 * draft_ids[cu[r] + step] = d when draft_ids is given (the verify call's draft
 * ids), and draft_stats[2 (cu[r] + step) + {0, 1}] = (m, s), the row's scale and
 * mass: q(x) = 2^(log2(e) / T (z_x - m)) / s.  Keep the draft logits rows and
 * pass them with draft_stats and the same temperatures to spec_verify_run
 * (draft-logits mode): no probability rows are stored.  Reads each draft row
 * once.  Errors: SV_EINVAL, SV_ECAPACITY (num_reqs beyond max_reqs or
 * max_rows, vocab beyond max_vocab), SV_EDTYPE, SV_EHIP.
 */
typedef struct sv_draft_args {
  const void *draft_logits;     /* [num_reqs, logits_row_stride] this step's draft logits */
  const float *temperature;     /* [num_reqs] draft temperature, >= 0                      */
  const int32_t *cu_num_draft;  /* [num_reqs + 1] prefix sums of the verify call          */
  int32_t *out_tokens;          /* [num_reqs]                                             */
  float *out_q;                 /* [num_reqs] or NULL                                     */
  float *draft_stats;           /* [2 D] written at the drafted rows                      */
  int32_t *draft_ids;           /* [D] or NULL: d also written at draft row cu[r] + step  */
  int64_t logits_row_stride;    /* elements between rows, >= vocab_size                   */
  uint64_t seed;                /* Philox key                                             */
  uint64_t offset;              /* per-call step, must be < 2^32                          */
  int32_t logits_dtype;         /* SV_F32 or SV_BF16                                      */
  int32_t num_reqs;
  int32_t vocab_size;
  int32_t step;                 /* draft position sampled by this call, >= 0              */
} sv_draft_args;

SV_API int spec_draft_sample(sv_ctx *ctx, const sv_draft_args *args, hipStream_t stream);

/*
 * Host helper for synthetic acceptance ("speculative decoding in vLLM", 7.2):
 * the minimum-variance unconditional rates for a mean acceptance length L in
 * [1, k + 1] (accepted drafts + 1).  The accepted count then takes only the two
 * integers around L - 1: rates[i] (position i + 1) is 1 up to floor(L - 1),
 * then the fractional part, then 0.  rates is a HOST array of k floats.
 * Returns SV_OK, or SV_EINVAL (L out of range or not finite, k < 0, NULL).
 */
SV_API int spec_verify_synthetic_rates(float mean_length, int32_t k, float *rates);

/*
 * Verify step on LM-head logits (NEXT row of the verify step).  The target
 * logits are z = W h: the hidden states of the target rows times the LM-head
 * weight ("【vllm】DeepSeekMTP、eagle", compute_logits: the LM head maps the
 * hidden states of the logit positions to [num_logit_pos, vocab_size]).  The
 * library computes them with bf16 inputs and fp32 accumulation on the matrix
 * cores and reduces them in the same kernel to the verify step's statistics
 * ("speculative decoding in vLLM", 7.4: max, argmax and sum of exp per target
 * row), so the [num_rows, vocab_size] logits are never written to memory.
 * Then, as spec_verify_run in no-draft-probs mode without penalties, top-k or
 * top-p: greedy requests (T = 0) compare each draft with the row's argmax
 * (lowest index on ties); sampled requests accept d_i iff it is a valid id and
 * p_i(d_i) >= u_i, and the recovered token (p_j with d_j removed) or the bonus
 * token is drawn by the two-level exponential race of spec_verify_run with
 * chunks of SV_LM_HEAD_CHUNK tokens (the race of the NO_DRAFT_PROBS Q&A of
 * "vLLM 投机解码（Eagle / MTP）实现与运行流程"; tags 1 and 2 of the row's
 * Philox stream; the law is exactly p): the GEMM leaves per (row, chunk) the
 * maximum logit, the chunk's mass and its argmax, and the winning chunk's
 * logits are recomputed from W and h for the token race.  Outputs as
 * spec_verify_run.  The context must be created with SV_CREATE_LM_HEAD
 * (records of ceil(max_vocab / SV_LM_HEAD_CHUNK) x 16 bytes per row).  Cost:
 * one pass over W (V d bf16) per 256 target rows, shared through L2 by the
 * workgroups of one token tile, 2 R V d flops, and SV_LM_HEAD_CHUNK rows of W
 * per sampled request.
 * Errors: SV_EINVAL (NULL pointer, hidden_size not a positive multiple of 64,
 * strides below hidden_size or not multiples of 8, bases not 16-byte aligned,
 * offset >= 2^32), SV_ECAPACITY (sizes beyond the context, or no
 * SV_CREATE_LM_HEAD), SV_EHIP.  Device-side: SV_ERR_CU, SV_ERR_TEMPERATURE, and
 * SV_ERR_ROW for a request with a non-finite logit.
 */
typedef struct sv_lm_head_args {
  const void *hidden;           /* [num_rows, hidden_row_stride] bf16 hidden states of the  */
                                /* target rows (rows ordered as target_logits)              */
  const void *lm_head;          /* [vocab_size, lm_head_row_stride] bf16 LM-head weight     */
  const int32_t *draft_ids;     /* [D], D = num_rows - num_reqs                             */
  const int32_t *cu_num_draft;  /* [num_reqs + 1] as in spec_verify_run                     */
  const float *temperature;     /* [num_reqs]; 0 = greedy                                   */
  int32_t *out_tokens;          /* [num_reqs, out_stride], -1 padded                        */
  int32_t *out_num_sampled;     /* [num_reqs]                                               */
  int32_t *out_num_rejected;    /* [num_reqs]                                               */
  float *dbg_p_draft;           /* [D] p_i(d_i) (-1 for greedy requests) or NULL            */
  float *dbg_logits;            /* [num_rows, vocab_size] fp32 logits or NULL (parity only) */
  int64_t hidden_row_stride;    /* elements, >= hidden_size, multiple of 8                  */
  int64_t lm_head_row_stride;   /* elements, >= hidden_size, multiple of 8                  */
  uint64_t seed;                /* Philox key                                               */
  uint64_t offset;              /* per-call step, < 2^32                                    */
  int32_t hidden_size;          /* d, a multiple of 64                                      */
  int32_t num_rows;             /* R = cu[B] + B                                            */
  int32_t num_reqs;             /* B                                                        */
  int32_t vocab_size;           /* V <= max_vocab                                           */
  int32_t out_stride;           /* row length of out_tokens, <= max_k + 1                   */
  const struct sv_post_update_args *post_update; /* HOST pointer or NULL: post_update of   */
                                /* this step inside the call, as in sv_verify_args          */
} sv_lm_head_args;

SV_API int spec_verify_lm_head(sv_ctx *ctx, const sv_lm_head_args *args, hipStream_t stream);

/* Static string for a return code. */
SV_API const char *spec_verify_strerror(int status);

/*
 * Synchronise `stream`, copy the device error word into *host_flags (a host
 * pointer) and clear it.  Returns SV_OK when no bit was set, SV_EINPUT when
 * some were, SV_EINVAL / SV_EHIP on failure.  For tests and debugging: it
 * blocks the host.
 */
SV_API int spec_verify_read_error(sv_ctx *ctx, uint32_t *host_flags, hipStream_t stream);

/*
 * Measurement.  spec_verify_profile_start makes the next `max_calls` calls of
 * spec_verify_run launch their first pass over the target rows (the top-k
 * pass when top-k is on, else the streaming statistics kernel) and the request
 * epilogue kernel (of spec_verify_lm_head: the fused LM-head GEMM and its
 * request kernel) with start/stop HIP events that the launch stamps at the
 * kernel's own start and end on the call's stream (hipExtLaunchKernel), so an
 * interval is that kernel's execution time.  The events are created here
 * (timing only: no system-scope fence, so they add no cache writeback to the
 * kernels they bracket), owned by the context, destroyed with it or by the
 * next start.
 * spec_verify_profile_read waits for those events, writes the per-call
 * durations in milliseconds to the host arrays stream_ms[] and epilogue_ms[]
 * (each with room for max_calls entries; either may be NULL), stores the
 * number of recorded calls in *n_calls and stops recording.  Returns SV_OK,
 * SV_EINVAL (null context, max_calls < 1 or > 65536, nothing started) or
 * SV_EHIP.
 */
SV_API int spec_verify_profile_start(sv_ctx *ctx, int32_t max_calls);
SV_API int spec_verify_profile_read(sv_ctx *ctx, float *stream_ms, float *epilogue_ms, int32_t *n_calls);

/*
 * Debug and test entry points: the library's own random stream and race noise,
 * value for value, so that tests can compare them directly with the published
 * Philox4x32-10 known-answer vectors (Salmon et al., SC'11) and with an
 * independent implementation.  Neither needs a context.
 *
 * spec_verify_debug_philox: out[i] = Philox4x32-10(counters[i], key) for i < n,
 * where counters and out are DEVICE arrays of n blocks of four uint32 words
 * (word 0 first), both 16-byte aligned, and key is split as (key lo, key hi)
 * like the seed of sv_verify_args.
 * spec_verify_debug_exp_noise: out[i] = the fp32 Exp(1) noise E = -ln U that
 * the races use for the Philox word words[i], U = (words[i] >> 8) * 2^-24
 * (+inf for U = 0); words and out are DEVICE arrays of n elements.
 * Both are stream-ordered.  Returns SV_OK, SV_EINVAL (n < 0, a null or
 * misaligned pointer with n > 0) or SV_EHIP.
 */
SV_API int spec_verify_debug_philox(const uint32_t *counters, int64_t n, uint64_t key, uint32_t *out,
                             hipStream_t stream);
SV_API int spec_verify_debug_exp_noise(const uint32_t *words, int64_t n, float *out, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* SPECVERIFY_H */
