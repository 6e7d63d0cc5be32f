/*
 * oracle.c -- CPU reference for the speculative-decoding verify step.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h): used by the tests, the smoke check
 * and the benchmark's CPU-baseline leg, never by the product path.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off -fno-fast-math
 * (no FMA contraction, so every fp32 operation on logits rounds once, as IEEE
 * round-to-nearest-even; probabilities and race scores are fp64).
 *
 * Citations name the page and its section; "page 2" is "vLLM 投机解码（Eagle / MTP）
 * 实现与运行流程", "page 1" is "【vllm】DeepSeekMTP、eagle", "page 3" is
 * "speculative decoding in vLLM" (section 七, verification), "page 4" is the
 * Mini-SGLang walk-through (sampler conventions).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Philox4x32-10, from Salmon et al., SC'11.  Each round multiplies counter    */
/* words 0 and 2 by the two round multipliers, swaps the halves of the 64-bit  */
/* products across lanes and xors in the other two counter words and the key; */
/* the key is advanced by the two Weyl constants between rounds.               */
/* ------------------------------------------------------------------------ */
#define PHILOX_MUL_A 0xD2511F53u
#define PHILOX_MUL_B 0xCD9E8D57u
#define PHILOX_WEYL_A 0x9E3779B9u
#define PHILOX_WEYL_B 0xBB67AE85u

void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    uint64_t prod_a = (uint64_t)PHILOX_MUL_A * (uint64_t)x0;
    uint64_t prod_b = (uint64_t)PHILOX_MUL_B * (uint64_t)x2;
    uint32_t hi_a = (uint32_t)(prod_a >> 32), lo_a = (uint32_t)prod_a;
    uint32_t hi_b = (uint32_t)(prod_b >> 32), lo_b = (uint32_t)prod_b;
    uint32_t y0 = hi_b ^ x1 ^ k0;
    uint32_t y1 = lo_b;
    uint32_t y2 = hi_a ^ x3 ^ k1;
    uint32_t y3 = lo_a;
    x0 = y0;
    x1 = y1;
    x2 = y2;
    x3 = y3;
    k0 += PHILOX_WEYL_A;
    k1 += PHILOX_WEYL_B;
  }
  out[0] = x0;
  out[1] = x1;
  out[2] = x2;
  out[3] = x3;
}

/* n blocks at once (counters and outputs [n][4]), same key: a loop over the above. */
void orc_philox4x32_10_n(const uint32_t *ctr, int64_t n, const uint32_t key[2], uint32_t *out) {
  for (int64_t i = 0; i < n; ++i) orc_philox4x32_10(ctr + 4 * i, key, out + 4 * i);
}

/* Counter layout: (idx >> 2, target row g, tag, call offset); word idx & 3.
 * Key: the two 32-bit halves of the 64-bit seed. */
uint32_t orc_word(uint64_t seed, uint32_t offset, uint32_t g, uint32_t tag, uint32_t idx) {
  uint32_t ctr[4] = {idx >> 2, g, tag, offset};
  uint32_t key[2] = {(uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32)};
  uint32_t out[4];
  orc_philox4x32_10(ctr, key, out);
  return out[idx & 3u];
}

/* Accept uniform on the 2^-24 grid, excluding 0: a draft with p = 0 is never
 * accepted, and u = 1 accepts only when p >= q. */
double orc_uniform_accept(uint32_t w) { return ldexp((double)((w >> 8) + 1u), -24); }

/* Race uniform on the 2^-24 grid, excluding 1 (E = -ln U is then never 0). */
double orc_uniform_race(uint32_t w) { return ldexp((double)(w >> 8), -24); }

/* Exp(1) noise E = -ln U; U = 0 gives E = +inf (a score of 0 that never wins
 * against a positive score). */
double orc_exp_noise(uint64_t seed, uint32_t offset, uint32_t g, uint32_t tag, uint32_t idx) {
  double u = orc_uniform_race(orc_word(seed, offset, g, tag, idx));
  if (u == 0.0) return INFINITY;
  return -log(u);
}

/* ------------------------------------------------------------------------ */
/* Logit processing                                                          */
/* ------------------------------------------------------------------------ */

/* bf16 is the upper half of an IEEE binary32. */
float orc_bf16_to_f32(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Multiplicative repetition penalty on every token seen in the output so far
 * (page 1, penalties section: applied to logits before sampling, from the
 * per-request output_bin_counts histogram).  A positive logit is divided by
 * theta, a non-positive one multiplied by theta, both in fp32. */
void orc_repetition_penalty(float *z, const int32_t *counts, int32_t V, float theta) {
  for (int32_t x = 0; x < V; ++x) {
    if (counts[x] > 0) {
      if (z[x] > 0.0f)
        z[x] = z[x] / theta;
      else
        z[x] = z[x] * theta;
    }
  }
}

static int cmp_float_desc(const void *a, const void *b) {
  float fa = *(const float *)a, fb = *(const float *)b;
  return (fa < fb) - (fa > fb);
}

/* k-th largest value of z counting duplicates (1 <= k <= V), via a sort. */
float orc_kth_largest(const float *z, int32_t V, int32_t k) {
  float *tmp = (float *)malloc(sizeof(float) * (size_t)V);
  memcpy(tmp, z, sizeof(float) * (size_t)V);
  qsort(tmp, (size_t)V, sizeof(float), cmp_float_desc);
  float tau = tmp[k - 1];
  free(tmp);
  return tau;
}

/* Top-k (page 4: top_k < 1 means the whole vocabulary): every logit below the
 * k-th largest is removed; ties with the k-th largest are all kept. */
void orc_top_k_mask(float *z, int32_t V, int32_t k) {
  if (k < 1 || k >= V) return;
  float tau = orc_kth_largest(z, V, k);
  for (int32_t x = 0; x < V; ++x)
    if (z[x] < tau) z[x] = -INFINITY;
}

/* First index of the maximum (lowest index wins ties). */
int32_t orc_argmax(const float *z, int32_t V) {
  int32_t best = 0;
  for (int32_t x = 1; x < V; ++x)
    if (z[x] > z[best]) best = x;
  return best;
}

/* Frequency and presence penalties from the output histogram.  The frequency
 * form is the walk-through of page 1 (penalties section: with penalty 0.5 a
 * token seen once loses 0.5, seen twice loses 1.0): z -= freq * count, the
 * product rounded to fp32 first.  The presence penalty subtracts a constant
 * from every token seen at least once (a reading: the pages name no formula). */
void orc_frequency_presence_penalty(float *z, const int32_t *counts, int32_t V, float freq,
                                    float pres) {
  for (int32_t x = 0; x < V; ++x) {
    if (counts[x] > 0) {
      float t = freq * (float)counts[x];
      z[x] = z[x] - t;
      z[x] = z[x] - pres;
    }
  }
}

static _Thread_local const double *g_sort_p; /* qsort context: probabilities, descending (per thread) */
static int cmp_idx_p_desc(const void *a, const void *b) {
  int32_t ia = *(const int32_t *)a, ib = *(const int32_t *)b;
  double pa = g_sort_p[ia], pb = g_sort_p[ib];
  if (pa != pb) return pa < pb ? 1 : -1;
  return (ia > ib) - (ia < ib);
}

/* Nucleus set: walk the distinct probability values from the largest down,
 * carrying the mass of everything strictly above; a value is kept while that
 * mass is below top_p (+ shift).  Ties share one decision. */
int32_t orc_top_p_keep(const double *p, int32_t V, double top_p, double shift, uint8_t *keep,
                       double *margin) {
  int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)V);
  for (int32_t x = 0; x < V; ++x) idx[x] = x;
  g_sort_p = p;
  qsort(idx, (size_t)V, sizeof(int32_t), cmp_idx_p_desc);
  double above = 0.0, mg = INFINITY;
  int32_t n = 0;
  for (int32_t i = 0; i < V;) {
    int32_t j = i;
    while (j < V && p[idx[j]] == p[idx[i]]) ++j;
    int kept = p[idx[i]] > 0.0 && (i == 0 || above < top_p + shift); /* the top value always stays */
    if (p[idx[i]] > 0.0 && fabs(above - top_p) < mg) mg = fabs(above - top_p);
    for (int32_t t = i; t < j; ++t) {
      keep[idx[t]] = (uint8_t)kept;
      n += kept;
    }
    for (int32_t t = i; t < j; ++t) above += p[idx[t]];
    i = j;
  }
  free(idx);
  if (margin) *margin = mg;
  return n;
}

/* Synthetic acceptance (page 3, 7.2): a target mean acceptance length L in
 * [1, K + 1] becomes the minimum-variance per-position rates.  The number of
 * accepted drafts N has mean L - 1; its variance is smallest when N takes only
 * the two integers around L - 1, which gives unconditional rates P(N >= i) of
 * 1 up to floor(L - 1), then the fractional part, then 0. */
int orc_synthetic_rates(double L, int32_t K, float *rates) {
  if (!(L >= 1.0) || !(L <= (double)K + 1.0)) return -1;
  double n0 = floor(L - 1.0);
  double f = (L - 1.0) - n0;
  for (int32_t i = 1; i <= K; ++i) {
    double a = (double)i <= n0 ? 1.0 : ((double)i == n0 + 1.0 ? f : 0.0);
    rates[i - 1] = (float)a;
  }
  return 0;
}

/* Temperature-scaled softmax in fp64 (page 2, 8.2). */
int orc_softmax(const float *z, int32_t V, double T, double *p) {
  double m = -INFINITY;
  for (int32_t x = 0; x < V; ++x) {
    double t = (double)z[x] / T;
    if (t > m) m = t;
  }
  if (!isfinite(m)) return ORC_ERR_ROW;
  double s = 0.0;
  for (int32_t x = 0; x < V; ++x) {
    p[x] = exp((double)z[x] / T - m);
    s += p[x];
  }
  for (int32_t x = 0; x < V; ++x) p[x] /= s;
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Exponential race.  argmax_x w_x / E_x with E_x ~ Exp(1) i.i.d. picks x with  */
/* probability w_x / sum(w) (page 2, NO_DRAFT_PROBS Q&A: no normalisation is   */
/* needed before the argmax).  Two levels: first a chunk c with weight M_c =   */
/* sum of w over the chunk, raced with one Exp(1) per chunk, then a token      */
/* inside the winning chunk raced with one Exp(1) per token; the product of    */
/* the two laws is (M_c / sum M)(w_x / M_c) = w_x / sum(w).  Ties go to the    */
/* lowest index.  C >= V reduces to the one-level race over all tokens.        */
/* ------------------------------------------------------------------------ */
static void keep_top2(double score, int32_t idx, double *b1, int32_t *i1, double *b2) {
  if (*i1 < 0 || score > *b1) {
    if (*i1 >= 0) *b2 = *b1;
    *b1 = score;
    *i1 = idx;
  } else if (score > *b2) {
    *b2 = score;
  }
}

static double level_margin(double b1, double b2, int have_second) {
  if (!have_second) return 1.0;
  if (!(b1 > 0.0)) return 0.0;
  return 1.0 - b2 / b1;
}

int32_t orc_race_tags(const double *w, int32_t V, int32_t C, uint64_t seed, uint32_t offset,
                      uint32_t g, uint32_t tag_chunk, uint32_t tag_token, double *margin) {
  int32_t nchunks = (V + C - 1) / C;
  double b1 = 0.0, b2 = -1.0;
  int32_t c_best = -1, ncand = 0;
  for (int32_t c = 0; c < nchunks; ++c) {
    int32_t lo = c * C, hi = lo + C < V ? lo + C : V;
    double M = 0.0;
    for (int32_t x = lo; x < hi; ++x) M += w[x];
    if (!(M > 0.0)) continue;
    double score = M / orc_exp_noise(seed, offset, g, tag_chunk, (uint32_t)c);
    keep_top2(score, c, &b1, &c_best, &b2);
    ++ncand;
  }
  if (c_best < 0) {
    if (margin) *margin = 1.0;
    return -1;
  }
  double m1 = level_margin(b1, b2, ncand > 1);

  double t1 = 0.0, t2 = -1.0;
  int32_t x_best = -1, tcand = 0;
  int32_t lo = c_best * C, hi = lo + C < V ? lo + C : V;
  for (int32_t x = lo; x < hi; ++x) {
    if (!(w[x] > 0.0)) continue;
    double score = w[x] / orc_exp_noise(seed, offset, g, tag_token, (uint32_t)x);
    keep_top2(score, x, &t1, &x_best, &t2);
    ++tcand;
  }
  double m2 = level_margin(t1, t2, tcand > 1);
  if (margin) *margin = m1 < m2 ? m1 : m2;
  return x_best;
}

int32_t orc_race(const double *w, int32_t V, int32_t C, uint64_t seed, uint32_t offset,
                 uint32_t g, double *margin) {
  return orc_race_tags(w, V, C, seed, offset, g, ORC_TAG_CHUNK, ORC_TAG_TOKEN, margin);
}

/* ------------------------------------------------------------------------ */
/* One request                                                               */
/* ------------------------------------------------------------------------ */
static void load_row(const void *rows, int dtype, int64_t stride, int32_t i, int32_t V, float *z) {
  if (dtype == ORC_BF16) {
    const uint16_t *r = (const uint16_t *)rows + (int64_t)i * stride;
    for (int32_t x = 0; x < V; ++x) z[x] = orc_bf16_to_f32(r[x]);
  } else {
    const float *r = (const float *)rows + (int64_t)i * stride;
    memcpy(z, r, sizeof(float) * (size_t)V);
  }
}

/* Order of processing (page 2, 8.2): logits processors (the repetition,
 * frequency and presence penalties) -> sampling constraints (top-k) ->
 * temperature and softmax -> top-p on the probabilities (page 4: top-p is
 * clamped to [1e-6, 1], 1 meaning no restriction), renormalised over the kept
 * tokens.  Temperature 0 selects the greedy rule, which needs only the argmax
 * of the processed logits (top-p never removes the argmax). */
int orc_prepare_request_ex(const void *rows, int dtype, int64_t stride, int32_t K, int32_t V,
                           float T, const orc_req_opts *o, const int32_t *counts, double *P,
                           int32_t *amax, double *topp_margin) {
  orc_req_opts none = {0, NULL, 0.0f, 0.0f, 1.0f, 0.0};
  if (!o) o = &none;
  for (int32_t i = 0; i <= K && topp_margin; ++i) topp_margin[i] = INFINITY;
  if (!(T >= 0.0f) || !isfinite(T)) return ORC_ERR_TEMPERATURE;
  if (o->theta && !(isfinite(*o->theta) && *o->theta > 0.0f)) return ORC_ERR_PENALTY;
  if (!isfinite(o->freq) || !isfinite(o->pres)) return ORC_ERR_PENALTY;
  if (isnan(o->top_p)) return ORC_ERR_TOP_P;
  const float top_p = o->top_p < 1e-6f ? 1e-6f : o->top_p;
  const int use_top_p = top_p < 1.0f && T > 0.0f;
  int err = 0;
  float *z = (float *)malloc(sizeof(float) * (size_t)V);
  uint8_t *keep = use_top_p ? (uint8_t *)malloc((size_t)V) : NULL;
  for (int32_t i = 0; i <= K; ++i) {
    load_row(rows, dtype, stride, i, V, z);
    if (o->theta && counts && *o->theta != 1.0f) orc_repetition_penalty(z, counts, V, *o->theta);
    if (counts && (o->freq != 0.0f || o->pres != 0.0f))
      orc_frequency_presence_penalty(z, counts, V, o->freq, o->pres);
    orc_top_k_mask(z, V, o->top_k);
    amax[i] = orc_argmax(z, V);
    double *p = P + (int64_t)i * V;
    if (!isfinite(z[amax[i]])) {
      err |= ORC_ERR_ROW;
      continue;
    }
    if (T == 0.0f) {
      for (int32_t x = 0; x < V; ++x) p[x] = 0.0;
      p[amax[i]] = 1.0;
      continue;
    }
    err |= orc_softmax(z, V, (double)T, p);
    if (use_top_p) {
      double mg = INFINITY;
      orc_top_p_keep(p, V, (double)top_p, o->top_p_shift, keep, &mg);
      if (topp_margin) topp_margin[i] = mg;
      double s = 0.0;
      for (int32_t x = 0; x < V; ++x)
        if (keep[x]) s += p[x];
      for (int32_t x = 0; x < V; ++x) p[x] = keep[x] ? p[x] / s : 0.0;
    }
  }
  free(keep);
  free(z);
  return err;
}

int orc_prepare_request(const void *rows, int dtype, int64_t stride, int32_t K, int32_t V,
                        float T, int32_t top_k, const float *theta, const int32_t *counts,
                        double *P, int32_t *amax) {
  orc_req_opts o = {top_k, theta, 0.0f, 0.0f, 1.0f, 0.0};
  return orc_prepare_request_ex(rows, dtype, stride, K, V, T, &o, counts, P, amax, NULL);
}

/* Synthetic accept test of draft position i (0-based): unconditional rates a
 * of positions 1..K, a_0 = 1; accept iff u * a_i <= a_{i+1}, i.e. with the
 * conditional probability a_{i+1} / a_i, so that position i + 1 is reached and
 * accepted with probability a_{i+1} (page 3, 7.2).  The product of two fp32
 * values is exact in fp64. */
static int synthetic_accept(const float *a, int32_t i, double u) {
  double prev = i == 0 ? 1.0 : (double)a[i - 1];
  return u * prev <= (double)a[i];
}

/* q_i(x) of draft row i: fp32 draft probabilities, fp64 rows, or none (NULL). */
static double draft_q(const float *draft_probs, int64_t dstride, const double *Q, int32_t V, int32_t i,
                      int32_t x) {
  if (Q) return Q[(int64_t)i * V + x];
  return (double)draft_probs[(int64_t)i * dstride + x];
}

static double decide(const double *P, const int32_t *amax, int32_t K, int32_t V, float T,
                     const int32_t *draft_ids, const float *draft_probs, int64_t dstride,
                     const double *Q, uint32_t g0, uint64_t seed, uint32_t offset, int32_t C,
                     const float *syn_rates, int32_t *tokens, int32_t *num_sampled,
                     int32_t *num_rejected, float *p_draft) {
  const int has_q = draft_probs != NULL || Q != NULL;
  double margin = INFINITY;

  if (T == 0.0f) {
    /* Greedy (page 2, 8.3): output the target argmax at each position, stop
     * after the first position whose draft differs; bonus argmax if none did.
     * In synthetic mode the rate test replaces the comparison and accepted
     * positions output the draft itself. */
    for (int32_t i = 0; i < K; ++i)
      if (p_draft) p_draft[i] = -1.0f;
    for (int32_t i = 0; i < K; ++i) {
      int acc;
      if (syn_rates) {
        int32_t d = draft_ids[i];
        double u = orc_uniform_accept(orc_word(seed, offset, g0 + (uint32_t)i, ORC_TAG_ACCEPT, 0));
        acc = d >= 0 && d < V && synthetic_accept(syn_rates, i, u);
        tokens[i] = acc ? d : amax[i];
      } else {
        acc = draft_ids[i] == amax[i];
        tokens[i] = amax[i];
      }
      if (!acc) {
        *num_sampled = i + 1;
        *num_rejected = K - i;
        return margin;
      }
    }
    tokens[K] = amax[K];
    *num_sampled = K + 1;
    *num_rejected = 0;
    return margin;
  }

  /* Target probability of every draft (page 2, 8.3: target_prob at the draft). */
  if (p_draft)
    for (int32_t i = 0; i < K; ++i) {
      int32_t d = draft_ids[i];
      p_draft[i] = (d >= 0 && d < V) ? (float)P[(int64_t)i * V + d] : 0.0f;
    }

  /* Accept loop (page 2, 8.3 and the Q&A on min(1, p/q)): draft i is accepted
   * when it is a valid id, q(d) > 0 and p(d) >= u * q(d); q = 1 without draft
   * probabilities (NO_DRAFT_PROBS Q&A).  Synthetic mode: the rate test.  The
   * first reject ends the loop. */
  int32_t j = K;
  for (int32_t i = 0; i < K; ++i) {
    int32_t d = draft_ids[i];
    int valid = d >= 0 && d < V;
    double u = orc_uniform_accept(orc_word(seed, offset, g0 + (uint32_t)i, ORC_TAG_ACCEPT, 0));
    if (syn_rates) {
      if (!valid || !synthetic_accept(syn_rates, i, u)) {
        j = i;
        break;
      }
      continue;
    }
    double q = 1.0;
    if (has_q) q = valid ? draft_q(draft_probs, dstride, Q, V, i, d) : 0.0;
    if (!valid || !(q > 0.0)) {
      j = i;
      break;
    }
    double p = P[(int64_t)i * V + d];
    double uq = u * q;
    double mg = fabs(p - uq) / (p > uq ? p : uq);
    if (mg < margin) margin = mg;
    if (!(p >= uq)) {
      j = i;
      break;
    }
  }
  for (int32_t i = 0; i < j; ++i) tokens[i] = draft_ids[i];

  /* The sampled row: recovered token at the reject, else the bonus row
   * (page 2, Q&A on the bonus token: only when every draft was accepted). */
  double *w = (double *)malloc(sizeof(double) * (size_t)V);
  const double *pj = P + (int64_t)j * V;
  if (j < K) {
    int32_t d = draft_ids[j];
    double total = 0.0;
    if (has_q) {
      /* Residual max(0, p - q), unnormalised (page 2, residual Q&A; page 3, 7.0). */
      for (int32_t x = 0; x < V; ++x) {
        double r = pj[x] - draft_q(draft_probs, dstride, Q, V, j, x);
        w[x] = r > 0.0 ? r : 0.0;
        total += w[x];
      }
    } else {
      /* q is the point mass at d: the residual is p with d removed. */
      for (int32_t x = 0; x < V; ++x) w[x] = pj[x];
      if (d >= 0 && d < V) w[d] = 0.0;
      for (int32_t x = 0; x < V; ++x) total += w[x];
    }
    /* A reject with no residual mass can only come from rounding; race over p. */
    if (!(total > 0.0))
      for (int32_t x = 0; x < V; ++x) w[x] = pj[x];
  } else {
    for (int32_t x = 0; x < V; ++x) w[x] = pj[x];
  }
  double mg = 1.0;
  tokens[j] = orc_race(w, V, C, seed, offset, g0 + (uint32_t)j, &mg);
  if (mg < margin) margin = mg;
  free(w);
  *num_sampled = j + 1;
  *num_rejected = K - j;
  return margin;
}


double orc_decide_request_ex(const double *P, const int32_t *amax, int32_t K, int32_t V, float T,
                             const int32_t *draft_ids, const float *draft_probs, int64_t dstride,
                             uint32_t g0, uint64_t seed, uint32_t offset, int32_t C,
                             const float *syn_rates, int32_t *tokens, int32_t *num_sampled,
                             int32_t *num_rejected, float *p_draft) {
  return decide(P, amax, K, V, T, draft_ids, draft_probs, dstride, NULL, g0, seed, offset, C, syn_rates,
                tokens, num_sampled, num_rejected, p_draft);
}

double orc_decide_request_q64(const double *P, const int32_t *amax, int32_t K, int32_t V, float T,
                              const int32_t *draft_ids, const double *Q, uint32_t g0, uint64_t seed,
                              uint32_t offset, int32_t C, const float *syn_rates, int32_t *tokens,
                              int32_t *num_sampled, int32_t *num_rejected, float *p_draft) {
  return decide(P, amax, K, V, T, draft_ids, NULL, 0, Q, g0, seed, offset, C, syn_rates, tokens,
                num_sampled, num_rejected, p_draft);
}

double orc_decide_request(const double *P, const int32_t *amax, int32_t K, int32_t V, float T,
                          const int32_t *draft_ids, const float *draft_probs, int64_t dstride,
                          uint32_t g0, uint64_t seed, uint32_t offset, int32_t C,
                          int32_t *tokens, int32_t *num_sampled, int32_t *num_rejected,
                          float *p_draft) {
  return orc_decide_request_ex(P, amax, K, V, T, draft_ids, draft_probs, dstride, g0, seed, offset,
                               C, NULL, tokens, num_sampled, num_rejected, p_draft);
}

/* ------------------------------------------------------------------------ */
/* Draft side (row f4): the draft token of one draft row is sampled from     */
/* q = softmax(z / T) with the same two-level race as the verifier, on noise  */
/* of its own tags, so the verifier can take q from the draft logits and the  */
/* row's softmax statistics instead of stored probabilities (page 3, 7.1:     */
/* probabilistic drafting needs the full draft distribution at verification). */
/* ------------------------------------------------------------------------ */
int32_t orc_draft_sample(const void *row, int dtype, int32_t V, float T, uint64_t seed,
                         uint32_t offset, uint32_t key, int32_t C, double *q_token, double *margin) {
  float *z = (float *)malloc(sizeof(float) * (size_t)V);
  load_row(row, dtype, (int64_t)V, 0, V, z);
  int32_t d = orc_argmax(z, V);
  if (!isfinite(z[d])) {
    free(z);
    return -1;
  }
  if (T == 0.0f) {
    free(z);
    if (q_token) *q_token = 1.0;
    if (margin) *margin = INFINITY;
    return d;
  }
  double *q = (double *)malloc(sizeof(double) * (size_t)V);
  orc_softmax(z, V, (double)T, q);
  double mg = 1.0;
  d = orc_race_tags(q, V, C, seed, offset, key, ORC_TAG_DRAFT_CHUNK, ORC_TAG_DRAFT_TOKEN, &mg);
  if (q_token) *q_token = d >= 0 ? q[d] : 0.0;
  if (margin) *margin = mg;
  free(q);
  free(z);
  return d;
}

/* fp64 draft distributions of K draft rows: softmax(z / T) (page 3, 7.1). */
int orc_draft_q_rows(const void *rows, int dtype, int64_t stride, int32_t K, int32_t V, float T,
                     double *Q) {
  float *z = (float *)malloc(sizeof(float) * (size_t)V);
  int err = 0;
  for (int32_t i = 0; i < K; ++i) {
    load_row(rows, dtype, stride, i, V, z);
    err |= orc_softmax(z, V, (double)T, Q + (int64_t)i * V);
  }
  free(z);
  return err;
}

/* ------------------------------------------------------------------------ */
/* LM head (row f2): the logits the verifier streams are the product of the  */
/* target rows' hidden states with the LM-head weight (page 3, 7.4: the       */
/* stats kernel works on the target logits; page 1: the logits come from the  */
/* LM head).  The plain definition, in fp64.                                 */
/* ------------------------------------------------------------------------ */
void orc_lm_head_logits(const uint16_t *h, const uint16_t *W, int64_t wstride, int32_t d, int32_t x0,
                        int32_t x1, double *z) {
  double *hd = (double *)malloc(sizeof(double) * (size_t)d);
  for (int32_t k = 0; k < d; ++k) hd[k] = (double)orc_bf16_to_f32(h[k]);
  for (int32_t x = x0; x < x1; ++x) {
    const uint16_t *w = W + (int64_t)x * wstride;
    double acc = 0.0;
    for (int32_t k = 0; k < d; ++k) acc += hd[k] * (double)orc_bf16_to_f32(w[k]);
    z[x - x0] = acc;
  }
  free(hd);
}

/* The verify step on LM-head logits (row f2): for each request the logits of
 * its K+1 rows come from orc_lm_head_logits (fp64, never rounded to fp32),
 * then the no-draft-probs rules of 8.3 of "vLLM 投机解码（Eagle / MTP）实现与运行
 * 流程" with the two-level race of chunk width C (the NO_DRAFT_PROBS Q&A's
 * argmax(w / E), run over chunks and then tokens): greedy rows take the first
 * fp64 argmax, sampled rows p = softmax(z / T) in fp64.  *gap receives, per
 * request, the smallest fp64 logit gap between the best and second-best token
 * of a greedy row it used (+inf for sampled requests or V = 1). */
static int32_t argmax64(const double *z, int32_t V, double *gap) {
  int32_t best = 0;
  for (int32_t x = 1; x < V; ++x)
    if (z[x] > z[best]) best = x;
  double second = -INFINITY;
  for (int32_t x = 0; x < V; ++x)
    if (x != best && z[x] > second) second = z[x];
  *gap = z[best] - second;
  return best;
}

uint32_t orc_lm_head_verify(const uint16_t *hidden, int64_t hstride, const uint16_t *W,
                            int64_t wstride, int32_t d, int32_t V, const int32_t *draft_ids,
                            const int32_t *cu, int32_t B, const float *temperature, uint64_t seed,
                            uint64_t offset, int32_t C, int32_t *out_tokens, int32_t out_stride,
                            int32_t *num_sampled, int32_t *num_rejected, double *margin,
                            double *greedy_gap, float *p_draft, const uint8_t *only) {
  uint32_t err = 0;
  if ((offset >> 32) != 0) return ORC_ERR_OFFSET;
  for (int32_t r = 0; r < B; ++r) {
    for (int32_t t = 0; t < out_stride; ++t) out_tokens[(int64_t)r * out_stride + t] = -1;
    num_sampled[r] = num_rejected[r] = 0;
    if (margin) margin[r] = INFINITY;
    if (greedy_gap) greedy_gap[r] = INFINITY;
  }
  for (int32_t r = 0; r <= B; ++r)
    if (cu[r] < 0 || (r > 0 && cu[r] < cu[r - 1]) || (r > 0 && cu[r] - cu[r - 1] > out_stride - 1))
      return ORC_ERR_CU;
  if (cu[0] != 0) return ORC_ERR_CU;
  for (int32_t r = 0; r < B; ++r) {
    if (only && !only[r]) continue;
    const int32_t K = cu[r + 1] - cu[r];
    const int64_t g0 = (int64_t)cu[r] + r;
    const float T = temperature[r];
    if (!(T >= 0.0f) || !isfinite(T)) {
      err |= ORC_ERR_TEMPERATURE;
      continue;
    }
    double *Z = (double *)malloc(sizeof(double) * (size_t)(K + 1) * (size_t)V);
    double *P = (double *)malloc(sizeof(double) * (size_t)(K + 1) * (size_t)V);
    int32_t *amax = (int32_t *)malloc(sizeof(int32_t) * (size_t)(K + 1));
    int bad = 0;
    for (int32_t i = 0; i <= K; ++i) {
      double *z = Z + (int64_t)i * V, *p = P + (int64_t)i * V;
      orc_lm_head_logits(hidden + (g0 + i) * hstride, W, wstride, d, 0, V, z);
      for (int32_t x = 0; x < V; ++x)
        if (!isfinite(z[x])) bad = 1;
      double gap;
      amax[i] = argmax64(z, V, &gap);
      if (T == 0.0f) {
        for (int32_t x = 0; x < V; ++x) p[x] = x == amax[i] ? 1.0 : 0.0;
      } else {
        double m = z[amax[i]] / (double)T, s = 0.0;
        for (int32_t x = 0; x < V; ++x) {
          p[x] = exp(z[x] / (double)T - m);
          s += p[x];
        }
        for (int32_t x = 0; x < V; ++x) p[x] /= s;
      }
    }
    if (bad) {
      err |= ORC_ERR_ROW;
      free(Z), free(P), free(amax);
      continue;
    }
    int32_t ns = 0, nr = 0;
    float *pd = p_draft ? p_draft + cu[r] : NULL;
    float pd_tmp[64];
    const double mg = orc_decide_request(P, amax, K, V, T, draft_ids + cu[r], NULL, V, (uint32_t)g0,
                                         seed, (uint32_t)offset, C, out_tokens + (int64_t)r * out_stride,
                                         &ns, &nr, pd ? pd : pd_tmp);
    num_sampled[r] = ns;
    num_rejected[r] = nr;
    if (margin) margin[r] = mg;
    if (greedy_gap && T == 0.0f) {
      /* the rows whose argmax decided something: 0 .. num_sampled - 1 */
      double gmin = INFINITY, gap;
      for (int32_t i = 0; i < ns; ++i) {
        argmax64(Z + (int64_t)i * V, V, &gap);
        if (gap < gmin) gmin = gap;
      }
      greedy_gap[r] = gmin;
    }
    free(Z), free(P), free(amax);
  }
  return err;
}

/* ------------------------------------------------------------------------ */
/* Whole call                                                                */
/* ------------------------------------------------------------------------ */
uint32_t orc_verify_batch_ex(const void *logits, int dtype, int64_t stride, int32_t num_rows,
                             int32_t V, const float *draft_probs, int64_t dstride,
                             const int32_t *draft_ids, const int32_t *cu, int32_t B,
                             int32_t max_k, const float *temperature, const int32_t *top_k,
                             const float *rep_penalty, const int32_t *idx_mapping,
                             const int32_t *counts, int32_t num_slots, uint64_t seed,
                             uint64_t offset, int32_t C, const orc_batch_opts *x,
                             int32_t *out_tokens, int32_t out_stride, int32_t *num_sampled,
                             int32_t *num_rejected, double *margin, float *p_draft) {
  uint32_t err = 0;
  int32_t D = num_rows - B;
  orc_batch_opts none = {NULL, NULL, NULL, NULL};
  if (!x) x = &none;
  for (int32_t r = 0; r < B; ++r) {
    for (int32_t t = 0; t < out_stride; ++t) out_tokens[(int64_t)r * out_stride + t] = -1;
    num_sampled[r] = 0;
    num_rejected[r] = 0;
    if (margin) margin[r] = INFINITY;
  }
  if (offset >> 32) return ORC_ERR_OFFSET;

  /* cu_num_draft: prefix sums of the per-request draft counts (page 1, the
   * rejection_sample inputs), so request r owns target rows cu[r]+r .. cu[r+1]+r,
   * the last of which is its bonus row. */
  int cu_ok = cu[0] == 0 && cu[B] == D;
  for (int32_t r = 0; r < B && cu_ok; ++r)
    if (cu[r + 1] < cu[r] || cu[r + 1] - cu[r] > max_k || cu[r + 1] - cu[r] + 1 > out_stride)
      cu_ok = 0;
  if (!cu_ok) return ORC_ERR_CU;

  for (int32_t r = 0; r < B; ++r) {
    int32_t K = cu[r + 1] - cu[r];
    int32_t g0 = cu[r] + r;
    float T = temperature[r];
    orc_req_opts o = {top_k ? top_k[r] : 0, rep_penalty ? &rep_penalty[r] : NULL,
                      x->freq ? x->freq[r] : 0.0f, x->pres ? x->pres[r] : 0.0f,
                      x->top_p ? x->top_p[r] : 1.0f, 0.0};
    /* A valid penalty other than the identity reads the request's histogram row. */
    int needs_counts = (o.theta && isfinite(*o.theta) && *o.theta > 0.0f && *o.theta != 1.0f) ||
                       (isfinite(o.freq) && o.freq != 0.0f) || (isfinite(o.pres) && o.pres != 0.0f);
    const int32_t *counts_row = NULL;
    if (needs_counts) {
      int32_t slot = idx_mapping[r];
      if (slot < 0 || slot >= num_slots) {
        err |= ORC_ERR_SLOT;
        continue;
      }
      counts_row = counts + (int64_t)slot * V;
    }
    double *P = (double *)malloc(sizeof(double) * (size_t)(K + 1) * (size_t)V);
    int32_t *amax = (int32_t *)malloc(sizeof(int32_t) * (size_t)(K + 1));
    const void *rows = dtype == ORC_BF16 ? (const void *)((const uint16_t *)logits + (int64_t)g0 * stride)
                                         : (const void *)((const float *)logits + (int64_t)g0 * stride);
    int e = orc_prepare_request_ex(rows, dtype, stride, K, V, T, &o, counts_row, P, amax, NULL);
    if (e) {
      err |= (uint32_t)e;
    } else {
      const float *q = draft_probs ? draft_probs + (int64_t)cu[r] * dstride : NULL;
      double mg = orc_decide_request_ex(P, amax, K, V, T, draft_ids + cu[r], q, dstride,
                                        (uint32_t)g0, seed, (uint32_t)offset, C, x->synthetic_rates,
                                        out_tokens + (int64_t)r * out_stride, &num_sampled[r],
                                        &num_rejected[r], p_draft ? p_draft + cu[r] : NULL);
      if (margin) margin[r] = mg;
    }
    free(P);
    free(amax);
  }
  return err;
}

uint32_t orc_verify_batch(const void *logits, int dtype, int64_t stride, int32_t num_rows,
                          int32_t V, const float *draft_probs, int64_t dstride,
                          const int32_t *draft_ids, const int32_t *cu, int32_t B,
                          int32_t max_k, const float *temperature, const int32_t *top_k,
                          const float *rep_penalty, const int32_t *idx_mapping,
                          const int32_t *counts, int32_t num_slots, uint64_t seed,
                          uint64_t offset, int32_t C, int32_t *out_tokens, int32_t out_stride,
                          int32_t *num_sampled, int32_t *num_rejected, double *margin,
                          float *p_draft) {
  return orc_verify_batch_ex(logits, dtype, stride, num_rows, V, draft_probs, dstride, draft_ids,
                             cu, B, max_k, temperature, top_k, rep_penalty, idx_mapping, counts,
                             num_slots, seed, offset, C, NULL, out_tokens, out_stride, num_sampled,
                             num_rejected, margin, p_draft);
}

/* post_update (page 1, _post_update_kernel): for each request, add its sampled
 * tokens to the slot's histogram, record the last sampled token, and advance
 * num_computed_tokens by query_len - num_rejected. */
uint32_t orc_post_update(const int32_t *idx_mapping, const int32_t *query_len,
                         const int32_t *tokens, int32_t tokens_stride,
                         const int32_t *num_sampled, const int32_t *num_rejected, int32_t B,
                         int32_t V, int32_t num_slots, int32_t *last_sampled, int32_t *counts,
                         int32_t *num_computed) {
  uint32_t err = 0;
  for (int32_t r = 0; r < B; ++r) {
    int32_t n = num_sampled[r];
    if (n <= 0) continue;
    int32_t s = idx_mapping[r];
    if (s < 0 || s >= num_slots) {
      err |= ORC_ERR_SLOT;
      continue;
    }
    const int32_t *tok = tokens + (int64_t)r * tokens_stride;
    for (int32_t i = 0; i < n; ++i)
      if (tok[i] >= 0 && tok[i] < V) counts[(int64_t)s * V + tok[i]] += 1;
    last_sampled[s] = tok[n - 1];
    num_computed[s] += query_len[r] - num_rejected[r];
  }
  return err;
}
