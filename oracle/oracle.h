/*
 * oracle.h -- CPU reference ("oracle") for the speculative-decoding verify step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this code: only the tests, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no source with the HIP library (its own Philox,
 * its own softmax, its own race), and it is deliberately plain: one request at a
 * time, full rows, fp64 for probabilities and race scores, fp32 (IEEE,
 * round-to-nearest-even, no contraction) only where the method fixes fp32
 * arithmetic on logits.
 *
 * What it computes, and where the pages define it:
 *  - softmax of the processed target logits at temperature T
 *      ("vLLM 投机解码（Eagle / MTP）实现与运行流程", section 八 8.2: processors,
 *      then sampling constraints, then softmax);
 *  - accept draft d with probability min(1, p(d)/q(d)), stop at the first reject
 *      (same page, 8.3, stochastic branch; the Q&A "原理解释：残差分布与拒绝采样");
 *  - recovered token from max(0, p - q) / sum, or, with no draft probabilities,
 *      from p with the rejected draft removed (same page, Q&A on NO_DRAFT_PROBS,
 *      4-token example two);
 *  - bonus token from the extra target row when every draft passes (same page,
 *      Q&A on the bonus token, 4-token example one);
 *  - greedy rule for temperature 0 (same page, 8.3, greedy branch);
 *  - post_update: last sampled token, output-token histogram, and
 *      num_computed += query_len - num_rejected ("【vllm】DeepSeekMTP、eagle",
 *      postprocess / _post_update_kernel walk-through);
 *  - optional settings: the frequency penalty of the first page's penalties
 *      walk-through (logit -= penalty * count), a presence penalty (a constant
 *      for every token seen; a reading), top-p on the probabilities (clamped to
 *      [1e-6, 1] as in the Mini-SGLang walk-through's sampler conventions; the
 *      kept set is every token whose strictly more probable tokens hold less
 *      than top_p of the mass), and synthetic acceptance with per-position
 *      unconditional rates or a mean acceptance length ("speculative decoding
 *      in vLLM", 7.2);
 *  - draft-side sampling ("speculative decoding in vLLM", 7.1: probabilistic
 *      drafting needs the draft distribution at verification): each draft token
 *      is drawn from q = softmax(z / T) by the same two-level race on noise of
 *      its own tags, and verification may take q rows computed from the draft
 *      logits instead of stored probabilities;
 *  - sampling by an exponential race argmax(w / E), E ~ Exp(1)
 *      (Q&A on NO_DRAFT_PROBS: the recovered-token kernel draws Exp(1) noise and
 *      takes argmax(prob / q)); here run as a two-level race (chunk, then token)
 *      whose law is exactly w / sum(w).
 *
 * The random stream is Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
 * Random Numbers: As Easy as 1, 2, 3", SC'11), written here from that paper.
 */
#ifndef SPEC_VERIFY_ORACLE_H
#define SPEC_VERIFY_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ORC_OK = 0,
  ORC_ERR_CU = 1u << 0,          /* cu_num_draft not a valid prefix sum           */
  ORC_ERR_TEMPERATURE = 1u << 1, /* temperature negative or not finite            */
  ORC_ERR_PENALTY = 1u << 2,     /* repetition penalty <= 0 or not finite          */
  ORC_ERR_ROW = 1u << 3,         /* a processed row has no finite maximum          */
  ORC_ERR_SLOT = 1u << 4,        /* idx_mapping outside [0, num_slots)             */
  ORC_ERR_OFFSET = 1u << 5,      /* offset does not fit in 32 bits                 */
  ORC_ERR_TOP_P = 1u << 6,       /* top_p is NaN                                  */
};

enum { ORC_TAG_ACCEPT = 0, ORC_TAG_CHUNK = 1, ORC_TAG_TOKEN = 2, ORC_TAG_DRAFT_CHUNK = 3, ORC_TAG_DRAFT_TOKEN = 4 };
enum { ORC_F32 = 0, ORC_BF16 = 1 };

/* Optional per-request settings beyond temperature.  Processing order of the
 * logits: repetition penalty, frequency penalty, presence penalty, top-k, then
 * temperature and softmax, then top-p on the probabilities. */
typedef struct orc_req_opts {
  int32_t top_k;      /* < 1 or >= V: off                                        */
  const float *theta; /* repetition penalty, or NULL (1: off)                    */
  float freq;         /* frequency penalty: z -= freq * count (0: off)           */
  float pres;         /* presence penalty: z -= pres where count > 0 (0: off)    */
  float top_p;        /* nucleus mass, clamped to [1e-6, 1]; 1: off; NaN: error  */
  double top_p_shift; /* keep iff mass above < top_p + shift; 0 for the method,  */
                      /* other values only to bracket rounding in tests          */
} orc_req_opts;

/* Batch-level optional settings for orc_verify_batch_ex (NULL arrays: off). */
typedef struct orc_batch_opts {
  const float *freq;            /* [B] frequency penalties or NULL             */
  const float *pres;            /* [B] presence penalties or NULL              */
  const float *top_p;           /* [B] nucleus masses or NULL                  */
  const float *synthetic_rates; /* [max_k] unconditional acceptance rates of   */
                                /* draft positions 1..max_k, or NULL           */
} orc_batch_opts;

/* ---- random stream ----------------------------------------------------- */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
/* n blocks, counters and outputs [n][4], one key. */
void orc_philox4x32_10_n(const uint32_t *ctr, int64_t n, const uint32_t key[2], uint32_t *out);
/* Word idx&3 of Philox(counter = (idx>>2, g, tag, offset), key = (seed lo, seed hi)). */
uint32_t orc_word(uint64_t seed, uint32_t offset, uint32_t g, uint32_t tag, uint32_t idx);
double orc_uniform_accept(uint32_t w); /* ((w>>8)+1) * 2^-24, in (0, 1] */
double orc_uniform_race(uint32_t w);   /* (w>>8) * 2^-24, in [0, 1)     */
double orc_exp_noise(uint64_t seed, uint32_t offset, uint32_t g, uint32_t tag, uint32_t idx);

/* ---- logit processing (fp32, IEEE RNE) ---------------------------------- */
float orc_bf16_to_f32(uint16_t bits);
void orc_repetition_penalty(float *z, const int32_t *counts, int32_t V, float theta);
float orc_kth_largest(const float *z, int32_t V, int32_t k);
void orc_top_k_mask(float *z, int32_t V, int32_t k);
int32_t orc_argmax(const float *z, int32_t V);
void orc_frequency_presence_penalty(float *z, const int32_t *counts, int32_t V, float freq,
                                    float pres);
/* Nucleus (top-p) set of the probabilities p[0..V): keep[x] = 1 iff the mass of
 * the tokens strictly more probable than x is below top_p + shift (ties at the
 * boundary are all kept).  *margin receives the smallest |mass above - top_p|
 * over the distinct probability values.  Returns the number of kept tokens. */
int32_t orc_top_p_keep(const double *p, int32_t V, double top_p, double shift, uint8_t *keep,
                       double *margin);
/* Minimum-variance unconditional acceptance rates for a target mean acceptance
 * length L in [1, K + 1] (accepted drafts + 1): rates[i] for position i + 1.
 * Returns 0, or -1 when L is out of range or not finite. */
int orc_synthetic_rates(double L, int32_t K, float *rates);
/* p = softmax(z / T) in fp64; returns 0, or ORC_ERR_ROW if max(z) is not finite. */
int orc_softmax(const float *z, int32_t V, double T, double *p);

/* ---- sampling ---------------------------------------------------------- */
/* Two-level exponential race over weights w[0..V) with chunk width C.
 * Returns the winning token (or -1 if every weight is 0); *margin receives the
 * smallest relative gap 1 - r2/r1 between the best and second-best score at the
 * two levels (1 when a level has a single candidate). */
int32_t orc_race(const double *w, int32_t V, int32_t C, uint64_t seed, uint32_t offset,
                 uint32_t g, double *margin);
/* The same race with the noise of the given chunk and token tags. */
int32_t orc_race_tags(const double *w, int32_t V, int32_t C, uint64_t seed, uint32_t offset,
                      uint32_t g, uint32_t tag_chunk, uint32_t tag_token, double *margin);

/* ---- draft side -------------------------------------------------------- */
/* Draft-side sampling of one draft row: q = softmax(z / T) in fp64 (T = 0:
 * the argmax, q(d) = 1), d from the two-level race over q with the draft tags
 * (3 and 4) at counter row `key` (the draft's row in the verify call).  *q_token
 * receives q(d); *margin the race margin (+inf for T = 0).  Returns d, or -1
 * (no finite logit). */
int32_t orc_draft_sample(const void *row, int dtype, int32_t V, float T, uint64_t seed,
                         uint32_t offset, uint32_t key, int32_t C, double *q_token, double *margin);

/* ---- LM head (row f2) ---------------------------------------------------- */
/* Logits of one row from its hidden state and the LM-head weight: z_x =
 * sum_k h_k W[x][k] over bf16 inputs (bit patterns), products and sums in fp64
 * (the plain definition of the matrix product), for tokens x in [x0, x1). */
void orc_lm_head_logits(const uint16_t *h, const uint16_t *W, int64_t wstride, int32_t d, int32_t x0,
                        int32_t x1, double *z);
/* The verify step on LM-head logits, no-draft-probs mode: hidden [R, d] with row
 * stride hstride, W [V, d] with row stride wstride (bf16 bits); per request the
 * logits of its rows by orc_lm_head_logits, then greedy (first fp64 argmax) or
 * p = softmax(z / T) in fp64, and the decisions of orc_decide_request with the
 * two-level race of chunk width C.  Outputs as orc_verify_batch; greedy_gap [B]
 * (or NULL) receives each greedy request's smallest top-1 / top-2 logit gap over
 * the rows it used (+inf otherwise).  only [B] (or NULL): requests with only[r]
 * == 0 are skipped (outputs left at -1 / 0).  Returns the ORC_ERR_* mask. */
uint32_t orc_lm_head_verify(const uint16_t *hidden, int64_t hstride, const uint16_t *W,
                            int64_t wstride, int32_t d, int32_t V, const int32_t *draft_ids,
                            const int32_t *cu, int32_t B, const float *temperature, uint64_t seed,
                            uint64_t offset, int32_t C, int32_t *out_tokens, int32_t out_stride,
                            int32_t *num_sampled, int32_t *num_rejected, double *margin,
                            double *greedy_gap, float *p_draft, const uint8_t *only);

/* fp64 draft distributions softmax(z / T) of K draft rows (stride in elements). */
int orc_draft_q_rows(const void *rows, int dtype, int64_t stride, int32_t K, int32_t V, float T,
                     double *Q);

/* ---- one request ------------------------------------------------------- */
/* Process the K+1 target rows of one request (penalty, top-k, then softmax at T,
 * or argmax when T == 0).  rows: [K+1, V] logits (dtype ORC_F32/ORC_BF16) with
 * row stride `stride` elements; counts: histogram row or NULL.
 * Outputs P [K+1, V] (fp64 probabilities; one-hot at the argmax when T == 0)
 * and amax [K+1].  Returns an ORC_ERR_* mask (0 on success). */
int orc_prepare_request(const void *rows, int dtype, int64_t stride, int32_t K, int32_t V,
                        float T, int32_t top_k, const float *theta, const int32_t *counts,
                        double *P, int32_t *amax);

/* orc_prepare_request with the settings of orc_req_opts (o may be NULL).
 * topp_margin [K+1] (or NULL) receives each row's top-p margin (+inf when
 * top-p is off or the row is greedy). */
int orc_prepare_request_ex(const void *rows, int dtype, int64_t stride, int32_t K, int32_t V,
                           float T, const orc_req_opts *o, const int32_t *counts, double *P,
                           int32_t *amax, double *topp_margin);

/* Accept/reject decisions and the recovered / bonus token for one request whose
 * rows were prepared by orc_prepare_request.  draft_probs: [K, V] fp32 rows with
 * stride dstride, or NULL for the no-draft-probs mode.  g0: global index of the
 * request's first target row.  Writes tokens[0..num_sampled), p_draft[K] (the
 * target probability of each draft; -1 for temperature 0).  Returns the
 * request's decision margin (+inf when no random decision was taken). */
double orc_decide_request(const double *P, const int32_t *amax, int32_t K, int32_t V, float T,
                          const int32_t *draft_ids, const float *draft_probs, int64_t dstride,
                          uint32_t g0, uint64_t seed, uint32_t offset, int32_t C,
                          int32_t *tokens, int32_t *num_sampled, int32_t *num_rejected,
                          float *p_draft);

/* orc_decide_request with synthetic acceptance: when syn_rates (K unconditional
 * rates of positions 1..K, non-increasing, in [0, 1]) is not NULL, draft i is
 * accepted iff it is a valid id and u_i * a_i <= a_{i+1} (a_0 = 1, exact in
 * fp64), in place of the probability test or the greedy comparison; the
 * recovered and bonus tokens are unchanged. */
double orc_decide_request_ex(const double *P, const int32_t *amax, int32_t K, int32_t V, float T,
                             const int32_t *draft_ids, const float *draft_probs, int64_t dstride,
                             uint32_t g0, uint64_t seed, uint32_t offset, int32_t C,
                             const float *syn_rates, int32_t *tokens, int32_t *num_sampled,
                             int32_t *num_rejected, float *p_draft);
/* orc_decide_request_ex with fp64 draft distributions Q [K, V] (rows computed
 * from draft logits), used in place of draft_probs when Q is not NULL. */
double orc_decide_request_q64(const double *P, const int32_t *amax, int32_t K, int32_t V, float T,
                              const int32_t *draft_ids, const double *Q, uint32_t g0, uint64_t seed,
                              uint32_t offset, int32_t C, const float *syn_rates, int32_t *tokens,
                              int32_t *num_sampled, int32_t *num_rejected, float *p_draft);

/* ---- whole call -------------------------------------------------------- */
/* Mirrors the library's verify entry point with host arrays.  out_tokens is
 * [B, out_stride] padded with -1.  margin [B] and p_draft [D] may be NULL.
 * Returns the OR of the ORC_ERR_* bits raised (requests that raise an error
 * produce num_sampled = num_rejected = 0). */
uint32_t orc_verify_batch(const void *logits, int dtype, int64_t stride, int32_t num_rows,
                          int32_t V, const float *draft_probs, int64_t dstride,
                          const int32_t *draft_ids, const int32_t *cu, int32_t B,
                          int32_t max_k, const float *temperature, const int32_t *top_k,
                          const float *rep_penalty, const int32_t *idx_mapping,
                          const int32_t *counts, int32_t num_slots, uint64_t seed,
                          uint64_t offset, int32_t C, int32_t *out_tokens, int32_t out_stride,
                          int32_t *num_sampled, int32_t *num_rejected, double *margin,
                          float *p_draft);

/* orc_verify_batch with the optional settings of orc_batch_opts (x may be NULL;
 * a request with a frequency or presence penalty needs its histogram slot). */
uint32_t orc_verify_batch_ex(const void *logits, int dtype, int64_t stride, int32_t num_rows,
                             int32_t V, const float *draft_probs, int64_t dstride,
                             const int32_t *draft_ids, const int32_t *cu, int32_t B,
                             int32_t max_k, const float *temperature, const int32_t *top_k,
                             const float *rep_penalty, const int32_t *idx_mapping,
                             const int32_t *counts, int32_t num_slots, uint64_t seed,
                             uint64_t offset, int32_t C, const orc_batch_opts *x,
                             int32_t *out_tokens, int32_t out_stride, int32_t *num_sampled,
                             int32_t *num_rejected, double *margin, float *p_draft);

/* post_update on host arrays (batch order).  Requests with num_sampled <= 0 or a
 * slot outside [0, num_slots) are skipped; returns ORC_ERR_SLOT if any slot was
 * out of range. */
uint32_t orc_post_update(const int32_t *idx_mapping, const int32_t *query_len,
                         const int32_t *tokens, int32_t tokens_stride,
                         const int32_t *num_sampled, const int32_t *num_rejected, int32_t B,
                         int32_t V, int32_t num_slots, int32_t *last_sampled, int32_t *counts,
                         int32_t *num_computed);

#ifdef __cplusplus
}
#endif
#endif
