/*
 * Drives every entry point of the CPU oracle (oracle/oracle.c) on small
 * seeded inputs, in every mode, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer.  The sanitizers abort on the first out-of-bounds
 * access, use after free, leak or undefined operation.  The driver itself
 * checks only a few invariants (token ranges, counts), and prints "ok" at the end.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double unif(void) {
  rng ^= rng << 13;
  rng ^= rng >> 7;
  rng ^= rng << 17;
  return (double)(rng >> 11) * 0x1p-53;
}
static double gauss(void) {
  double u = unif() + 1e-300, v = unif();
  return sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v);
}

#define CHECK(c)                                                  \
  do {                                                            \
    if (!(c)) {                                                   \
      fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      exit(2);                                                    \
    }                                                             \
  } while (0)

static void batch(int dtype, int B, int K, int V, int with_q, int topk, int pen, int topp, int syn, int greedy) {
  int32_t *cu = malloc(sizeof(int32_t) * (B + 1));
  cu[0] = 0;
  for (int r = 0; r < B; ++r) cu[r + 1] = cu[r] + (K ? (int)(unif() * (K + 1)) % (K + 1) : 0);
  const int D = cu[B], R = D + B, S = B + 3;
  float *lf = malloc(sizeof(float) * (size_t)R * V);
  uint16_t *lb = malloc(sizeof(uint16_t) * (size_t)R * V);
  for (int64_t i = 0; i < (int64_t)R * V; ++i) {
    lf[i] = (float)(2.0 * gauss());
    uint32_t u;
    memcpy(&u, &lf[i], 4);
    lb[i] = (uint16_t)(u >> 16);
  }
  int32_t *ids = malloc(sizeof(int32_t) * (D + 1));
  for (int i = 0; i < D; ++i) ids[i] = (int)(unif() * (V + 2)) - 1; /* some out of range */
  float *q = NULL;
  if (with_q) {
    q = malloc(sizeof(float) * (size_t)(D + 1) * V);
    for (int i = 0; i < D; ++i) {
      double s = 0;
      for (int x = 0; x < V; ++x) s += (q[(int64_t)i * V + x] = (float)unif());
      for (int x = 0; x < V; ++x) q[(int64_t)i * V + x] /= (float)s;
    }
  }
  float *T = malloc(sizeof(float) * B), *rp = malloc(sizeof(float) * B), *fq = malloc(sizeof(float) * B);
  float *pr = malloc(sizeof(float) * B), *tp = malloc(sizeof(float) * B);
  int32_t *tk = malloc(sizeof(int32_t) * B), *im = malloc(sizeof(int32_t) * B);
  for (int r = 0; r < B; ++r) {
    T[r] = greedy && r % 3 == 0 ? 0.0f : 0.8f;
    rp[r] = 1.1f;
    fq[r] = 0.5f;
    pr[r] = 0.25f;
    tp[r] = 0.7f;
    tk[r] = topk;
    im[r] = (r * 7) % S;
  }
  T[B - 1] = greedy ? -1.0f : T[B - 1]; /* one invalid temperature in greedy batches */
  int32_t *counts = calloc((size_t)S * V, sizeof(int32_t));
  for (int i = 0; i < S * 5; ++i) counts[(int64_t)(i % S) * V + (int)(unif() * V) % V] += 1;
  float rates[8] = {0.9f, 0.7f, 0.5f, 0.4f, 0.2f, 0.1f, 0.0f, 0.0f};
  orc_batch_opts x = {pen ? fq : NULL, pen ? pr : NULL, topp ? tp : NULL, syn ? rates : NULL};
  const int os = K + 1;
  int32_t *tok = malloc(sizeof(int32_t) * B * os), *ns = malloc(sizeof(int32_t) * B), *nr = malloc(sizeof(int32_t) * B);
  double *mg = malloc(sizeof(double) * B);
  float *pd = malloc(sizeof(float) * (D + 1));
  uint32_t err = orc_verify_batch_ex(dtype ? (const void *)lb : (const void *)lf, dtype, V, R, V, q, V, ids, cu, B, K,
                                     T, topk ? tk : NULL, pen ? rp : NULL, im, counts, S, 12345, 7, 64, &x, tok, os,
                                     ns, nr, mg, pd);
  for (int r = 0; r < B; ++r) {
    CHECK(ns[r] >= 0 && ns[r] <= cu[r + 1] - cu[r] + 1);
    for (int t = 0; t < ns[r]; ++t) CHECK(tok[r * os + t] >= -1 && tok[r * os + t] < V);
  }
  if (greedy) CHECK(err & ORC_ERR_TEMPERATURE);
  int32_t *last = calloc(S, sizeof(int32_t)), *nc = calloc(S, sizeof(int32_t));
  int32_t *ql = malloc(sizeof(int32_t) * B);
  for (int r = 0; r < B; ++r) ql[r] = cu[r + 1] - cu[r] + 1;
  orc_post_update(im, ql, tok, os, ns, nr, B, V, S, last, counts, nc);
  free(last), free(nc), free(ql);
  free(cu), free(lf), free(lb), free(ids), free(q), free(T), free(rp), free(fq), free(pr), free(tp), free(tk),
      free(im), free(counts), free(tok), free(ns), free(nr), free(mg), free(pd);
}

int main(void) {
  /* random stream */
  uint32_t c[8] = {1, 2, 3, 4, 5, 6, 7, 8}, k[2] = {9, 10}, o[8];
  orc_philox4x32_10(c, k, o);
  orc_philox4x32_10_n(c, 2, k, o);
  CHECK(orc_uniform_accept(0) > 0.0 && orc_uniform_race(0xFFFFFFFFu) < 1.0);
  CHECK(orc_exp_noise(1, 2, 3, 1, 4) > 0.0);
  CHECK(orc_bf16_to_f32(0x3F80) == 1.0f);
  /* logit processing */
  enum { V = 300 };
  float z[V];
  int32_t cnt[V];
  double p[V];
  uint8_t keep[V];
  for (int x = 0; x < V; ++x) {
    z[x] = (float)gauss();
    cnt[x] = x % 4;
  }
  orc_repetition_penalty(z, cnt, V, 1.2f);
  orc_frequency_presence_penalty(z, cnt, V, 0.3f, 0.1f);
  CHECK(orc_kth_largest(z, V, 7) <= orc_kth_largest(z, V, 1));
  orc_top_k_mask(z, V, 40);
  CHECK(orc_argmax(z, V) >= 0);
  CHECK(orc_softmax(z, V, 0.9, p) == 0);
  double tm;
  CHECK(orc_top_p_keep(p, V, 0.6, 0.0, keep, &tm) >= 1);
  float rates[6];
  CHECK(orc_synthetic_rates(2.5, 6, rates) == 0 && orc_synthetic_rates(9.0, 6, rates) != 0);
  /* races: C below, at and above V; a single token; no weight */
  double w[V], m;
  for (int x = 0; x < V; ++x) w[x] = unif() * (x % 3 != 0);
  for (int C = 1; C <= 2 * V; C = C * 3 + 1) CHECK(orc_race(w, V, C, 5, 6, 7, &m) >= 0);
  CHECK(orc_race_tags(w, 1, 64, 5, 6, 7, 3, 4, &m) == -1 || 1);
  memset(w, 0, sizeof w);
  CHECK(orc_race(w, V, 64, 5, 6, 7, &m) == -1);
  /* draft side */
  double qt;
  CHECK(orc_draft_sample(z, ORC_F32, V, 1.0f, 3, 4, 5, 64, &qt, &m) >= 0);
  CHECK(orc_draft_sample(z, ORC_F32, V, 0.0f, 3, 4, 5, 64, &qt, &m) >= 0);
  double Q[2 * V];
  float z2[2 * V];
  for (int x = 0; x < 2 * V; ++x) z2[x] = (float)gauss();
  CHECK(orc_draft_q_rows(z2, ORC_F32, V, 2, V, 0.7f, Q) == 0);
  /* one request, every mode */
  enum { K = 3 };
  float rows[(K + 1) * V];
  for (int i = 0; i < (K + 1) * V; ++i) rows[i] = (float)(2.0 * gauss());
  double P[(K + 1) * V], tmg[K + 1];
  int32_t amax[K + 1], ids[K] = {3, V + 5, 17}, toks[K + 1], ns, nr;
  float pd[K], qrows[K * V], theta = 1.1f;
  for (int i = 0; i < K * V; ++i) qrows[i] = 1.0f / V;
  orc_req_opts op = {20, &theta, 0.5f, 0.2f, 0.8f, 0.0};
  CHECK(orc_prepare_request_ex(rows, ORC_F32, V, K, V, 0.7f, &op, cnt, P, amax, tmg) == 0);
  orc_decide_request(P, amax, K, V, 0.7f, ids, qrows, V, 11, 1, 2, 64, toks, &ns, &nr, pd);
  orc_decide_request(P, amax, K, V, 0.7f, ids, NULL, V, 11, 1, 2, 64, toks, &ns, &nr, pd);
  orc_decide_request_ex(P, amax, K, V, 0.7f, ids, NULL, V, 11, 1, 2, 64, rates, toks, &ns, &nr, pd);
  orc_decide_request_q64(P, amax, K, V, 0.7f, ids, Q, 11, 1, 2, 64, NULL, toks, &ns, &nr, pd);
  CHECK(orc_prepare_request(rows, ORC_F32, V, K, V, 0.0f, 0, NULL, NULL, P, amax) == 0);
  orc_decide_request(P, amax, K, V, 0.0f, ids, NULL, V, 11, 1, 2, 64, toks, &ns, &nr, pd);
  CHECK(ns >= 1 && ns <= K + 1);
  /* LM head */
  enum { LD = 64, LV = 130, LB = 5 };
  uint16_t H[(LB * 4) * LD], W[LV * LD];
  for (int i = 0; i < LB * 4 * LD; ++i) H[i] = (uint16_t)(0x3C00 + (int)(unif() * 0x800));
  for (int i = 0; i < LV * LD; ++i) W[i] = (uint16_t)((unif() < 0.5 ? 0xBC00 : 0x3C00) + (int)(unif() * 0x400));
  double lz[LV];
  orc_lm_head_logits(H, W, LD, LD, 3, LV, lz);
  int32_t lcu[LB + 1] = {0, 1, 3, 3, 6, 8}, lids[8] = {1, 2, 3, 4, 5, 6, 7, 8}, ltok[LB * 4], lns[LB], lnr[LB];
  float lT[LB] = {1.0f, 0.0f, 0.7f, 1.3f, 0.0f}, lpd[8];
  double lmg[LB], lgap[LB];
  uint8_t only[LB] = {1, 1, 0, 1, 1};
  CHECK(orc_lm_head_verify(H, LD, W, LD, LD, LV, lids, lcu, LB, lT, 9, 9, 64, ltok, 4, lns, lnr, lmg, lgap, lpd,
                           only) == 0);
  /* whole calls: fp32 / bf16, draft probs / none, top-k, penalties, top-p, synthetic, greedy */
  batch(ORC_F32, 9, 3, 1000, 1, 0, 0, 0, 0, 0);
  batch(ORC_BF16, 11, 4, 2100, 0, 0, 0, 0, 0, 1);
  batch(ORC_F32, 7, 2, 1500, 1, 30, 1, 0, 0, 0);
  batch(ORC_BF16, 8, 3, 1300, 0, 0, 1, 1, 0, 0);
  batch(ORC_F32, 6, 5, 900, 1, 0, 0, 0, 1, 1);
  batch(ORC_BF16, 5, 0, 700, 0, 10, 0, 1, 0, 0);
  batch(ORC_F32, 4, 2, 1, 1, 0, 0, 0, 0, 0);
  /* an invalid layout and an out-of-range offset are errors, not accesses */
  float one[4] = {0, 0, 0, 0};
  int32_t bcu[3] = {0, 2, 1}, bid[2] = {0, 0}, bt[6], bn[2], br[2];
  float bT[2] = {1.0f, 1.0f};
  CHECK(orc_verify_batch(one, ORC_F32, 2, 2, 2, NULL, 2, bid, bcu, 2, 2, bT, NULL, NULL, NULL, NULL, 0, 1, 0, 64, bt, 3,
                         bn, br, NULL, NULL) == ORC_ERR_CU);
  CHECK(orc_verify_batch(one, ORC_F32, 2, 2, 2, NULL, 2, bid, bcu, 2, 2, bT, NULL, NULL, NULL, NULL, 0, 1,
                         (uint64_t)1 << 33, 64, bt, 3, bn, br, NULL, NULL) == ORC_ERR_OFFSET);
  printf("ok\n");
  return 0;
}
