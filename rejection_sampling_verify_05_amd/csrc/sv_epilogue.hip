// sv_epilogue.hip -- request epilogue, residual pass, post_update and the debug kernels.
//
// Data flow of one spec_verify_run (all on one stream):
//   topk_kernel   (only with top_k)      one workgroup per target row: exact
//                 k-th largest processed logit tau and, when at most
//                 kCandCap tokens reach tau, the kept tokens sorted by id.
//   stats_kernel  the streaming pass.  A persistent grid reads every chunk of
//   (or the       kChunk logits once, each workgroup a balanced contiguous
//   fast variant) slice, and stores per chunk (max, sum exp2(a (z - max))) --
//                 or (max, argmax) for greedy rows -- in the chunk table.
//   epilogue_kernel  one workgroup per request: row softmax statistics from
//                 the chunk table, the accept tests, the first reject, and
//                 the bonus / recovered race.
//   resid_kernel, resid_race_kernel  (draft-probs mode) residual
//                 max(0, p - q) chunk masses of each rejected request's row,
//                 then the race.
//   dbg_kernel    (optional) writes the processed probabilities.
//
// The method follows "vLLM 投机解码（Eagle / MTP）实现与运行流程" section 八
// (8.2 order of processing, 8.3 greedy and stochastic rules), its Q&A on the
// residual distribution, the bonus token and NO_DRAFT_PROBS, and
// "【vllm】DeepSeekMTP、eagle" for post_update.  The sampling race is the
// exponential-race argmax(w / E) of the NO_DRAFT_PROBS Q&A, run over chunks
// and then tokens.
#include <stdint.h>

#include "sv_common.h"

namespace sv {

namespace {

constexpr int kTabCache = 2048;  // chunk-table entries the epilogue kernel keeps in LDS

// Candidate lists of compact (top-k) rows, staged in LDS by the epilogue.
template <bool CAND>
struct CandBuf {
  float cw[kCandCap];  // candidate weights
  int ci[kCandCap];    // candidate token ids
};
template <>
struct CandBuf<false> {};

// LDS of the request epilogue: TC chunk-table entries cached; CAND: room for
// the candidate lists of compact rows (not needed by the plain variant).
template <int TC, bool CAND>
struct EpiSharedT {
  static constexpr int kCache = TC;
  BlockScratch red;
  float m[kMaxDrafts + 1];
  float s[kMaxDrafts + 1];
  float tau[kMaxDrafts + 1];
  float sx[kMaxDrafts + 1];
  int amax[kMaxDrafts + 1];
  int state[kMaxDrafts + 1];
  int d[kMaxDrafts + 1];
  int rj[kMaxDrafts + 1];  // accept test of draft i failed (1) or passed (0)
  float rt[kInlineResidNC];  // residual chunk masses (vocabularies of at most kInlineResidNC chunks)
  float zc[kWaves][kChunk];  // speculative chunks of rows 0..3 (raw logits, token order)
  float zx[kWaves][kChunk];  // the draft tokens' chunks of rows 0..3
  float w1s[kWaves];         // best chunk other than the draft token's: score
  int w1c[kWaves];           //   and index (-1: none)
  int cd[kWaves];            // the draft token's chunk when excluded, else -1
  float rcd[kWaves];         // 1/E of that chunk in the chunk race
  union {
    float2 tab[TC];  // dense rows: chunk tables of the request's rows
    CandBuf<CAND> cand;
  } u;
};
using EpiShared = EpiSharedT<kTabCache, true>;

// Race over a compact candidate list (token ids ascending in sh.u.cand.ci,
// weights in sh.u.cand.cw, n entries); all threads call it.  Same law and
// random words as the dense race: chunk masses are the sums over the
// candidates of each chunk.
__device__ __forceinline__ int compact_race(const Params &p, uint32_t g, int n, EpiShared &sh) {
  __syncthreads();
  const float *cw = sh.u.cand.cw;
  const int *ci = sh.u.cand.ci;
  ArgMax best{-1.0f, 0x7FFFFFFF};
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const int c = ci[i] / kChunk;
    if (i > 0 && ci[i - 1] / kChunk == c) continue;  // not the first candidate of its chunk
    float M = 0.0f;
    for (int t = i; t < n && ci[t] / kChunk == c; ++t) M += cw[t];
    if (M > 0.0f) {
      const uint4 w4 = rng_block(p, (uint32_t)c >> 2, g, kTagChunk);
      ArgMax o{race_score(M, pick(w4, c & 3)), c};
      if (better(o, best)) best = o;
    }
  }
  const ArgMax cb = block_argmax(best, sh.red);
  if (cb.s < 0.0f) return -1;
  const int cstar = cb.i;
  ArgMax tb{-1.0f, 0x7FFFFFFF};
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const int x = ci[i];
    if (x / kChunk != cstar || !(cw[i] > 0.0f)) continue;
    const uint4 w4 = rng_block(p, (uint32_t)x >> 2, g, kTagToken);
    ArgMax o{race_score(cw[i], pick(w4, x & 3)), x};
    if (better(o, tb)) tb = o;
  }
  const ArgMax b = block_argmax(tb, sh.red);
  return b.s < 0.0f ? -1 : b.i;
}

// ---------------------------------------------------------------------------
// Request epilogue: one workgroup per request, after the streaming pass.
//
// Round trips: (1) the request's cu entries and temperature; (2) the chunk
// tables and the draft ids; (3) for each of the first four rows, speculatively,
// the logits of the chunks its race could need: the chunk that wins the race
// among the chunks without the draft token, and the draft token's own chunk
// (z_d, and the chunk mass without d), plus single loads of z_d and q(d) for the
// other rows.  The speculative chunks go to LDS; the accept tests then pick
// the row j to sample and the whole workgroup finishes its race from LDS.  A
// rejected row past the fourth, or a bonus row past the fourth, takes one more
// round trip; compact (top-k) rows race over their candidate lists.
// ---------------------------------------------------------------------------

// Speculative state of one row while its wave waits for the loads.
struct RowSpec {
  float zc[16];   // logits of chunk c1 (stochastic) or of the lowest max chunk (greedy)
  float zx[16];   // logits of the draft token's chunk cd
  ArgMax w1;      // best chunk other than cd: (score, c1); c1 = -1 if none
  int cd;         // draft token's chunk when it is excluded, else -1
  float rcd;      // 1/E of chunk cd in the chunk race
};

// Row statistics of row i from its chunk table (dense) or candidates (compact):
// scale m (the largest chunk reference r_c; the row maximum for greedy rows and
// compact rows) and Σ exp2(a (z - m)); greedy dense rows also get the lowest
// chunk holding the maximum.  One wave; results uniform.
template <class EF>
__device__ __forceinline__ void row_stats(const Params &p, const Req &q, int g, int st, bool greedy, EF ent,
                                          float &m, float &s, int &lc) {
  const int lane = threadIdx.x & 63;
  s = 0.0f;
  lc = 0x7FFFFFFF;
  if (st >= 0) {
    const float *cv = p.cand_val + (int64_t)g * kCandCap;
    float lm = kNegInf;
    for (int t = lane; t < st; t += 64) lm = fmaxf(lm, cv[t]);
    m = wave_max(lm);
    float ls = 0.0f;
    for (int t = lane; t < st; t += 64) ls += exp2_acc(q.a * (cv[t] - m));
    s = wave_sum(ls);
    return;
  }
  float lm = kNegInf;
  for (int c = lane; c < p.NC; c += 64) lm = fmaxf(lm, ent(c).x);
  m = wave_max(lm);
  if (greedy) {
    int l = 0x7FFFFFFF;
    for (int c = lane; c < p.NC; c += 64)
      if (ent(c).x == m) l = min(l, c);
    lc = wave_min_i(l);
  } else if (m > kNegInf) {
    float ls = 0.0f;
    for (int c = lane; c < p.NC; c += 64) {
      const float2 e = ent(c);
      if (e.x > kNegInf) ls += e.y * exp2_acc(q.a * (e.x - m));
    }
    s = wave_sum(ls);
  }
}

// Speculative part for dense stochastic row i (no-draft-probs rows and bonus
// rows): the chunk race without the draft token's chunk, then the loads of
// the winning chunk and of the draft token's chunk (penalties applied).
template <class EF>
__device__ __forceinline__ void spec_issue(const Params &p, const Req &q, int i, int d, float m, EF ent, RowSpec &rs,
                                           const ChunkNoise &cn, const Proc &pr) {
  const int g = q.g0 + i;
  const bool excl = i < q.K && !q.has_q && d >= 0 && d < p.V;
  rs.cd = excl ? d / kChunk : -1;
  rs.rcd = 0.0f;
  rs.w1 = wave_chunk_race(p, g, ent, q.a, m, rs.cd, cn, &rs.rcd);
  const int c1 = rs.w1.s < 0.0f ? -1 : rs.w1.i;
  if (c1 >= 0 || excl) load_chunk16_pen_pair(p, g, c1, rs.cd, pr, rs.zc, rs.zx);
}

// After the loads of spec_issue: z_d and the mass of d's chunk without d, in
// the scale of that chunk's table entry r = ent(c_d).x:
// exp2(fma(z, a, -hi)) exp2(-lo) with a r = hi + lo (pr: the processing left
// after the penalties).
__device__ __forceinline__ void spec_draft_record(const Params &p, const Req &q, int d, const Proc &pr,
                                                  const RowSpec &rs, float ref, float &zd, float &sx) {
  const int lane = threadIdx.x & 63;
  const float a = q.a, hi = a * ref, lo = __builtin_fmaf(a, ref, -hi);
  float acc = 0.0f, zl = kNegInf;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int x = c16_tok(rs.cd, e, lane);
    const float z = x < p.V ? apply_proc(rs.zx[e], x, pr) : kNegInf;
    if (x == d)
      zl = z;
    else
      acc += exp2_acc(__builtin_fmaf(z, a, -hi));
  }
  sx = ref > kNegInf ? wave_sum(acc) * exp2_acc(-lo) : 0.0f;
  zd = wave_max(zl);
}

// Moves a wave's speculative chunks and race state for row i to LDS slot `slot`.
template <class SH>
__device__ __forceinline__ void spec_publish(const RowSpec &rs, int slot, SH &sh) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    *reinterpret_cast<float4 *>(&sh.zc[slot][t * 256 + 4 * lane]) =
        make_float4(rs.zc[4 * t], rs.zc[4 * t + 1], rs.zc[4 * t + 2], rs.zc[4 * t + 3]);
    *reinterpret_cast<float4 *>(&sh.zx[slot][t * 256 + 4 * lane]) =
        make_float4(rs.zx[4 * t], rs.zx[4 * t + 1], rs.zx[4 * t + 2], rs.zx[4 * t + 3]);
  }
  if (lane == 0) {
    sh.w1s[slot] = rs.w1.s;
    sh.w1c[slot] = rs.w1.i;
    sh.cd[slot] = rs.cd;
    sh.rcd[slot] = rs.rcd;
  }
}

// Final race of row j from LDS slot `slot` (all threads): the chunk of d
// competes with its mass without d (sx); if nothing is left without d, the race
// is over p_j.
template <class EF, class SH>
__device__ __forceinline__ int spec_finish(const Params &p, const Req &q, int j, int dj, float m, float sx,
                                           const Proc &pr, EF ent, int slot, SH &sh) {
  const int gs = q.g0 + j;
  const float a = q.a;
  ArgMax win{sh.w1s[slot], sh.w1c[slot]};
  const int cd = sh.cd[slot];
  bool excl = cd >= 0;
  if (excl) {
    const float2 e = ent(cd);
    const float rd = sh.rcd[slot];  // 1/E of chunk cd, drawn by the chunk race
    const float Wd = e.x > kNegInf ? sx * exp2_acc(a * (e.x - m)) : 0.0f;
    if (Wd > 0.0f) {
      ArgMax o{Wd * rd, cd};
      if (better(o, win)) win = o;
    }
    if (win.s < 0.0f) {  // nothing left once d_j is removed (rounding): race over p_j
      excl = false;
      const float Wf = e.x > kNegInf ? e.y * exp2_acc(a * (e.x - m)) : 0.0f;
      if (Wf > 0.0f) win = ArgMax{Wf * rd, cd};
    }
  }
  if (win.s < 0.0f) return -1;
  const int cstar = win.i;
  const float hi = a * ent(cstar).x;
  const float *zs = cstar == cd ? sh.zx[slot] : sh.zc[slot];  // penalties applied
  return block_token_race(p, gs, cstar, zs, proc_after_pen(pr), a, hi, (excl && cstar == cd) ? dj : -1, sh.red);
}

// Speculative rows: with at most four rows, row w for wave w; with more, rows
// 0, 1, 2 and the bonus row (the likeliest to be sampled after row 0 when the
// acceptance rate is high).  spec_slot: the wave (LDS slot) of row i, or -1.
__device__ __forceinline__ int spec_row(int w, int nrow) { return nrow <= kWaves || w < kWaves - 1 ? w : nrow - 1; }
__device__ __forceinline__ int spec_slot(int i, int nrow) {
  if (nrow <= kWaves) return i;
  return i < kWaves - 1 ? i : (i == nrow - 1 ? kWaves - 1 : -1);
}

// The residual of rejected row j of request q in this workgroup (rows of at
// most kInlineResidNC chunks, draft distributions given): chunk masses of
// w = max(0, p_j - q_j), wave w taking chunks w, w + 4, ... two at a time
// with all their loads issued first, then the chunk race and the token race
// over w; an empty residual (rounding) races over p_j.  The arithmetic and
// random words are those of resid_kernel and resid_race_kernel.
template <class EF, class SH>
__device__ __forceinline__ void inline_residual(const Params &p, const Req &q, int j, int gs, float m, float s,
                                                const Proc &pr, int64_t out_j, EF entry, SH &sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float inv_s = 1.0f / s, a = q.a;
  const int64_t dr = q.c0 + j;  // the draft row of position j
  const bool probs = p.draft_probs != nullptr;
  const bool qvec = probs ? ((uintptr_t)p.draft_probs % 16 == 0 && p.dstride % 4 == 0) : p.dvec_ok;
  const float mq = probs ? 0.0f : p.draft_stats[2 * dr], inv_sq = probs ? 1.0f : 1.0f / p.draft_stats[2 * dr + 1];
  auto draft_chunk = [&](int c, float (&qx)[16]) {
    if (probs)
      load_chunk16_at(p.draft_probs, SV_F32, p.dstride, qvec, p.V, dr, c, qx);
    else
      load_chunk16_at(p.draft_logits, p.ddtype, p.dlstride, qvec, p.V, dr, c, qx);
  };
  for (int c0 = wave; c0 < p.NC; c0 += 2 * kWaves) {
    const int c1 = c0 + kWaves;  // may be past the row: its values are not used
    float za[16], zb[16], qa[16], qb[16];
    load_chunk16_pair(p, gs, c0, c1 < p.NC ? c1 : c0, za, zb);
    draft_chunk(c0, qa);
    draft_chunk(c1 < p.NC ? c1 : c0, qb);
    float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int x0 = c16_tok(c0, e, lane), x1 = c16_tok(c1, e, lane);
      const float q0 = probs ? qa[e] : exp2_acc(q.aq * (qa[e] - mq)) * inv_sq;
      const float q1 = probs ? qb[e] : exp2_acc(q.aq * (qb[e] - mq)) * inv_sq;
      if (x0 < p.V) acc0 += fmaxf(exp2_acc(a * (apply_proc(za[e], x0, pr) - m)) * inv_s - q0, 0.0f);
      if (x1 < p.V) acc1 += fmaxf(exp2_acc(a * (apply_proc(zb[e], x1, pr) - m)) * inv_s - q1, 0.0f);
    }
    const float w0 = wave_sum(acc0), w1 = wave_sum(acc1);
    if (lane == 0) {
      sh.rt[c0] = w0;
      if (c1 < p.NC) sh.rt[c1] = w1;
    }
  }
  __syncthreads();
  const bool fallback = !(block_sum(tid < p.NC ? sh.rt[tid] : 0.0f, sh.red) > 0.0f);
  const int cstar = block_chunk_race(p, (uint32_t)gs, p.NC, [&](int c) -> float {
    if (!fallback) return sh.rt[c];
    const float2 e = entry(j, c);
    return e.x > kNegInf ? e.y * exp2_acc(a * (e.x - m)) : 0.0f;
  }, sh.red);
  int x = -1;
  if (cstar >= 0) {
    const int x0 = cstar * kChunk + 4 * tid;
    float z[4], qx[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {  // all loads first
      const int xc = min(x0 + k, p.V - 1);
      z[k] = load_logit(p, gs, xc);
      qx[k] = draft_q_of(p, q, j, xc);
    }
    const uint4 w4 = rng_block(p, (uint32_t)x0 >> 2, (uint32_t)gs, kTagToken);
    ArgMax best{-1.0f, 0x7FFFFFFF};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int xx = x0 + k;
      if (xx < p.V) {
        const float px = exp2_acc(a * (apply_proc(z[k], xx, pr) - m)) * inv_s;
        const float wx = fallback ? px : fmaxf(px - qx[k], 0.0f);
        if (wx > 0.0f) {
          const ArgMax o{race_score(wx, pick(w4, k)), xx};
          if (better(o, best)) best = o;
        }
      }
    }
    const ArgMax bb = block_argmax(best, sh.red);
    x = bb.s < 0.0f ? -1 : bb.i;
  }
  if (tid == 0) p.out_tokens[out_j] = x;
  fused_post_update(p, q.r, q.K, j, x, [&](int i) { return sh.d[i]; });
}

// PLAIN: the call has no top-k and at most four rows per request; the
// settings it does not use are then constants, and their paths compile away.
// With PLAIN, TP: the call has top-p, so each row carries the top-p pass's
// threshold tau (tokens below it are out of the race; the row's chunk table
// already holds the kept masses); PEN: the call has penalties, which the
// request's settings keep (else they are the identity); QD: the call has
// draft distributions (else q = 1).  FEW: at most four rows per request (with
// QD alone, more rows are allowed).
template <bool PLAIN, bool TP, bool PEN, bool QD, bool FEW, class SH>
__device__ __forceinline__ void request_epilogue(const Params &p, const Req &q_in, SH &sh) {
  constexpr int TC = SH::kCache;
  Req q = q_in;
  if (PLAIN) {
    if (!PEN) {
      q.proc.counts = nullptr;
      q.proc.theta = 1.0f;
      q.proc.freq = 0.0f;
      q.proc.pres = 0.0f;
    }
    q.proc.tau = kNegInf;
    if (!QD) q.has_q = false;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = q.K, r = q.r, nrow = K + 1;

  if (!q.cu_ok || p.cu[0] != 0 || p.cu[p.B] != p.D) {
    if (tid == 0) raise_err(p, SV_ERR_CU);
    write_empty(p, r);
    return;
  }
  // FEW: at most four rows per request (cu_ok bounds K by out_stride - 1):
  // every row has a wave of its own.
  if (PLAIN && FEW) __builtin_assume(nrow <= kWaves);
  if (q.mode == kModeInvalid) {
    if (tid == 0) raise_err(p, q.errbits);
    write_empty(p, r);
    return;
  }
  const bool greedy = q.mode == kModeGreedy;

  // Row states (top-k pass results), draft ids and the chunk tables.
  for (int i = tid; i < nrow; i += kThreads) {
    const int g = q.g0 + i;
    const int st = (PLAIN && !TP) ? kRowDense : row_state(p, g);
    sh.state[i] = st;
    sh.tau[i] = (st == kRowDense) ? kNegInf : p.cand_tau[g];
    sh.d[i] = i < K ? p.draft_ids[q.c0 + i] : -1;
  }
  const bool cached = nrow * p.NC <= TC;
  float2 tv[TC / kThreads];
  if (cached) {  // all table loads issued first
#pragma unroll
    for (int m = 0; m < TC / kThreads; ++m) {
      const int t = tid + m * kThreads;
      const int i = t / p.NC, c = t - i * p.NC;
      tv[m] = t < nrow * p.NC ? p.chunk_tab[(int64_t)(q.g0 + i) * p.nc_stride + c] : make_float2(0.0f, 0.0f);
    }
  }
  // While the tables are in flight: the chunk-race noise of this wave's
  // speculative row (it depends only on the row).
  const int srow = spec_row(wave, nrow);
  const ChunkNoise cn = chunk_noise(p, q.g0 + min(srow, nrow - 1));
  // ... and its accept uniform (rows taken later draw theirs when they come)
  const double u_srow = srow < K ? u_accept(rng_block(p, 0, (uint32_t)(q.g0 + srow), kTagAccept).x) : 1.0;
  if (cached) {
#pragma unroll
    for (int m = 0; m < TC / kThreads; ++m) {
      const int t = tid + m * kThreads;
      if (t < nrow * p.NC) sh.u.tab[t] = tv[m];
    }
  }
  __syncthreads();
  auto entry = [&](int i, int c) -> float2 {
    return cached ? sh.u.tab[i * p.NC + c] : p.chunk_tab[(int64_t)(q.g0 + i) * p.nc_stride + c];
  };

  // Wave w first takes its speculative row spec_row(w) -- rows 0..3, or with
  // more than four rows 0, 1, 2 and the bonus row K -- with the speculative
  // loads; then, round robin, the rows nobody speculates on, with only what
  // the accept tests need.
  RowSpec rs;
#pragma unroll
  for (int e = 0; e < 16; ++e) rs.zc[e] = rs.zx[e] = 0.0f;
  rs.cd = -1;
  rs.w1 = ArgMax{-1.0f, 0x7FFFFFFF};
  for (int i = srow, phase = 0;;) {
    bool spec = phase == 0;
    if (spec && i >= nrow) {  // no speculative row for this wave
      phase = 1;
      i = wave;
      continue;
    }
    if (!spec) {
      while (i < nrow && spec_slot(i, nrow) >= 0) i += kWaves;
      if (i >= nrow) break;
    }
    const int g = q.g0 + i;
    const int st = (PLAIN && !TP) ? kRowDense : sh.state[i];
    const int d = sh.d[i];
    auto ent = [&](int c) { return entry(i, c); };
    float m, s;
    int lc = 0x7FFFFFFF;
    Proc pr = q.proc;
    pr.tau = (PLAIN && !TP) ? kNegInf : sh.tau[i];
    int am = 0x7FFFFFFF;
    float zd = kNegInf, qd = 1.0f, sx = 0.0f;
    const bool valid_d = i < K && d >= 0 && d < p.V;
    // Speculative dense stochastic rows of at most 256 chunks: statistics and
    // chunk race from one read of the table (spec_issue's race is then done).
    const bool fused = st < 0 && !greedy && spec && (!q.has_q || i == K) && p.NC <= 256;
    if (fused) {
      const bool excl = i < q.K && !q.has_q && valid_d;
      rs.cd = excl ? d / kChunk : -1;
      rs.rcd = 0.0f;
      row_stats_race(p, ent, q.a, rs.cd, cn, m, s, rs.w1, &rs.rcd);
    } else {
      row_stats(p, q, g, st, greedy, ent, m, s, lc);
    }
    if (fused) {
      const int c1 = rs.w1.s < 0.0f ? -1 : rs.w1.i;
      // The draft token's chunk (left out of the race above) can win only if
      // its whole mass beats c1's score; else its mass without d is not
      // needed, d stays out of the race, and only z_d is loaded.
      bool need_cd = rs.cd >= 0;
      if (need_cd && c1 >= 0) {
        const float2 ec = ent(rs.cd);
        const float Wcd = ec.x > kNegInf ? ec.y * exp2_acc(q.a * (ec.x - m)) : 0.0f;
        need_cd = Wcd * rs.rcd >= rs.w1.s * (1.0f - 1e-5f);  // (a margin for the rounding of the two masses)
      }
      if (need_cd) {
        load_chunk16_pen_pair(p, g, c1, rs.cd, pr, rs.zc, rs.zx);
        spec_draft_record(p, q, d, proc_after_pen(pr), rs, ent(rs.cd).x, zd, sx);
      } else {
        // z_d (and its count) issued before the chunk, so that both arrive in one round trip
        const float zr = valid_d ? load_logit(p, g, d) : 0.0f;
        const int nd = (valid_d && pr.counts != nullptr) ? pr.counts[d] : 0;
        if (c1 >= 0) load_chunk16_pen(p, g, c1, pr, rs.zc);
        if (valid_d) {
          const float z = nd > 0 ? penalize(zr, nd, pr) : zr;
          zd = z < pr.tau ? kNegInf : z;
        }
        rs.cd = -1;
      }
      spec_publish(rs, wave, sh);
    } else if (st < 0 && greedy) {
      if (lc < p.NC) {
        load_chunk16_pen(p, g, lc, pr, rs.zc);
        am = wave_first_equal(p, lc, rs.zc, proc_after_pen(pr), m);
      }
    } else if (st < 0 && spec && (!q.has_q || i == K)) {
      spec_issue(p, q, i, d, m, ent, rs, cn, pr);
      if (rs.cd >= 0) spec_draft_record(p, q, d, proc_after_pen(pr), rs, ent(rs.cd).x, zd, sx);
      spec_publish(rs, wave, sh);
    } else if (valid_d) {
      // single loads: z_d (and q(d)) for the accept test
      zd = apply_proc(load_logit(p, g, d), d, pr);
      if (q.has_q) qd = draft_q_of(p, q, i, d);
    }
    // The accept test of draft i by the wave that has its row ("vLLM 投机解码
    // （Eagle / MTP）实现与运行流程", 8.3): greedy, the draft equals the argmax;
    // stochastic, a valid draft with q > 0 and p(d) >= u q (q = 1 without
    // draft distributions); synthetic, u a_i <= a_{i+1} (a_0 = 1), exact in fp64.
    bool rej = false;
    float pdv = -1.0f;  // p(d) for dbg_p_draft (-1: greedy)
    if (i < K) {
      const double u = (greedy && !p.synthetic) ? 1.0 : (i == srow ? u_srow : u_accept(rng_block(p, 0, (uint32_t)g, kTagAccept).x));
      if (p.synthetic) {
        const double prev = i == 0 ? 1.0 : (double)p.syn[i - 1];
        rej = !(valid_d && u * prev <= (double)p.syn[i]);
        if (!greedy) pdv = valid_d ? exp2_acc(q.a * (zd - m)) / s : 0.0f;
      } else if (greedy) {
        rej = d != am;
      } else {
        float pd = 0.0f;
        double qv = q.has_q ? 0.0 : 1.0;
        if (valid_d) {
          pd = exp2_acc(q.a * (zd - m)) / s;
          if (q.has_q) qv = (double)qd;
        }
        rej = !(valid_d && qv > 0.0 && (double)pd >= u * qv);
        pdv = pd;
      }
    }
    if (lane == 0) {
      sh.m[i] = m;
      sh.s[i] = s;
      sh.amax[i] = am;
      sh.sx[i] = sx;
      sh.rj[i] = rej ? 1 : 0;
      if (i < K && p.dbg_p_draft) p.dbg_p_draft[q.c0 + i] = pdv;
      p.row_info[g] = make_float4(m, s, __int_as_float(am), __int_as_float(st));
    }
    if (spec) {
      phase = 1;
      i = wave;
    } else {
      i += kWaves;
    }
  }
  __syncthreads();
  // The row checks and the sampled row j (the first rejected draft, else the
  // bonus row), in every wave from the rows' records: no further barrier.
  bool bad = __ballot(lane < nrow && !__builtin_isfinite(sh.m[lane])) != 0;
  if (nrow > 64) bad = bad || !__builtin_isfinite(sh.m[64]);
  if (bad) {
    if (tid == 0) raise_err(p, SV_ERR_ROW);
    write_empty(p, r);
    return;
  }
  const unsigned long long rmask = __ballot(lane < K && sh.rj[lane] != 0);
  const int j = rmask ? (__ffsll((long long)rmask) - 1) : K;

  // Accepted prefix, padding and counts.
  for (int t = tid; t < p.out_stride; t += kThreads) {
    const int v = t < j ? sh.d[t] : -1;
    if (t != j) p.out_tokens[(int64_t)r * p.out_stride + t] = v;
  }
  if (tid == 0) {
    p.out_ns[r] = j + 1;
    p.out_nr[r] = K - j;
  }
  const int64_t out_j = (int64_t)r * p.out_stride + j;

  auto accepted = [&](int i) { return sh.d[i]; };
  if (greedy) {
    if (tid == 0) p.out_tokens[out_j] = sh.amax[j];
    fused_post_update(p, r, K, j, sh.amax[j], accepted);
    return;
  }

  const int gs = q.g0 + j;
  const bool rejected = j < K;
  const int dj = rejected ? sh.d[j] : -1;
  const float m = sh.m[j], s = sh.s[j];
  Proc pr = q.proc;
  pr.tau = (PLAIN && !TP) ? kNegInf : sh.tau[j];
  const int st = (PLAIN && !TP) ? kRowDense : sh.state[j];
  const float a = q.a;

  if constexpr (!PLAIN) {
  if (st >= 0) {
    // Compact top-k row: the race runs over the kept tokens only.
    __syncthreads();  // the LDS chunk-table cache is reused for the candidates
    const float *cv = p.cand_val + (int64_t)gs * kCandCap;
    const int32_t *cix = p.cand_idx + (int64_t)gs * kCandCap;
    const bool qres = rejected && q.has_q;
    float part = 0.0f;
    for (int t = tid; t < st; t += kThreads) {
      const int x = cix[t];
      const float pxv = exp2_acc(a * (cv[t] - m)) / s;
      float w = pxv;
      if (rejected) {
        if (qres)
          w = fmaxf(pxv - draft_q_of(p, q, j, x), 0.0f);
        else if (x == dj)
          w = 0.0f;
      }
      sh.u.cand.ci[t] = x;
      sh.u.cand.cw[t] = w;
      part += w;
    }
    const float total = block_sum(part, sh.red);
    if (!(total > 0.0f)) {  // residual empty by rounding: race over p
      for (int t = tid; t < st; t += kThreads) sh.u.cand.cw[t] = exp2_acc(a * (cv[t] - m)) / s;
    }
    const int x = compact_race(p, (uint32_t)gs, st, sh);
    if (tid == 0) p.out_tokens[out_j] = x;
    fused_post_update(p, r, K, j, x, accepted);
    return;
  }
  }

  if (rejected && q.has_q && p.NC <= kInlineResidNC) {
    inline_residual(p, q, j, gs, m, s, pr, out_j, entry, sh);
    return;
  }
  if (rejected && q.has_q) {
    // Dense residual: handed to resid_kernel (needs the full draft row).
    if (tid == 0) {
      p.res_req[r] = make_int4(gs, j, dj, (int)p.epoch);
      p.res_list[1 + atomicAdd(p.res_list, 1)] = r;  // at most one entry per request: fits in max_reqs
    }
    return;
  }

  // Dense race over p_j (bonus row, or the rejected row with d_j removed).
  auto entj = [&](int c) { return entry(j, c); };
  int slot = spec_slot(j, nrow);
  float sxj = sh.sx[j];
  if (slot < 0) {  // no speculative state for this row: same steps, loads now
    if (wave == 0) {
      spec_issue(p, q, j, dj, m, entj, rs, chunk_noise(p, q.g0 + j), pr);
      float zd = kNegInf;
      sxj = 0.0f;
      if (rs.cd >= 0) spec_draft_record(p, q, dj, proc_after_pen(pr), rs, entj(rs.cd).x, zd, sxj);
      spec_publish(rs, 0, sh);
      if (lane == 0) sh.sx[j] = sxj;
    }
    __syncthreads();
    slot = 0;
    sxj = sh.sx[j];
  }
  const int x = spec_finish(p, q, j, dj, m, sxj, pr, entj, slot, sh);
  if (tid == 0) p.out_tokens[out_j] = x;
  fused_post_update(p, r, K, j, x, accepted);
}

// ---------------------------------------------------------------------------
// Residual pass (draft-probs mode, dense rows).  The epilogue lists each
// rejected request (res_list: a count, then request ids) and records its row in
// res_req with this call's epoch.  resid_kernel: chunk masses of
// w = max(0, p_j - q_j), persistent over (listed request, segment of cps chunks)
// items; resid_race_kernel: the race over them (one workgroup per request,
// active when its res_req entry carries this call's epoch).
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(kThreads) void resid_kernel(Params p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nact = p.res_list[0];
  // persistent: work item w = (active request w / nseg, segment w % nseg)
  for (int w = blockIdx.x; w < nact * p.nseg; w += gridDim.x) {
    const int r = p.res_list[1 + w / p.nseg];
    const int seg = w % p.nseg;
    const int4 rq = p.res_req[r];
    const Req q = load_req(p, r);
    const int gs = rq.x, j = rq.y;
    const float4 ri = p.row_info[gs];
    const float m = ri.x, inv_s = 1.0f / ri.y, a = q.a;
    Proc pr = q.proc;
    if (row_has_tau(__float_as_int(ri.w))) pr.tau = p.cand_tau[gs];
    float *rt = p.res_tab + (int64_t)r * p.nc_stride;
    for (int c = seg * p.cps + wave; c < min(p.NC, (seg + 1) * p.cps); c += kWaves) {
      // 16 tokens per lane, all loads issued before any use
      float z[16], qx[16];
      load_chunk16(p, gs, c, z);
      if (p.draft_probs != nullptr) {
#pragma unroll
        for (int e = 0; e < 16; ++e) qx[e] = draft_q_of(p, q, j, min(c16_tok(c, e, lane), p.V - 1));
      } else {  // draft-logits mode: the draft row's chunk with vector loads
        const int64_t dr = q.c0 + j;
        load_chunk16_at(p.draft_logits, p.ddtype, p.dlstride, p.dvec_ok, p.V, dr, c, qx);
        const float mq = p.draft_stats[2 * dr], inv_sq = 1.0f / p.draft_stats[2 * dr + 1];
#pragma unroll
        for (int e = 0; e < 16; ++e) qx[e] = exp2_acc(q.aq * (qx[e] - mq)) * inv_sq;
      }
      float acc = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int x = c16_tok(c, e, lane);
        if (x < p.V) {
          const float px = exp2_acc(a * (apply_proc(z[e], x, pr) - m)) * inv_s;
          acc += fmaxf(px - qx[e], 0.0f);
        }
      }
      const float Wc = wave_sum(acc);
      if (lane == 0) rt[c] = Wc;
    }
  }
}

__global__ __launch_bounds__(kThreads) void resid_race_kernel(Params p) {
  __shared__ BlockScratch red;
  const int r = blockIdx.x;
  if (r == 0 && threadIdx.x == 0) p.res_list[0] = 0;  // the residual pass has read it: zero for the next call
  const int4 rq = p.res_req[r];
  if (rq.w != (int)p.epoch) return;
  const Req q = load_req(p, r);
  const int gs = rq.x, j = rq.y;
  const float4 ri = p.row_info[gs];
  const float m = ri.x, inv_s = 1.0f / ri.y, a = q.a;
  Proc pr = q.proc;
  if (row_has_tau(__float_as_int(ri.w))) pr.tau = p.cand_tau[gs];
  const float *rt = p.res_tab + (int64_t)r * p.nc_stride;
  // An empty residual (rounding) falls back to racing over p_j.
  float part = 0.0f;
  for (int c = threadIdx.x; c < p.NC; c += kThreads) part += rt[c];
  const bool fallback = !(block_sum(part, red) > 0.0f);
  const float2 *tab = p.chunk_tab + (int64_t)gs * p.nc_stride;
  const int cstar = block_chunk_race(p, (uint32_t)gs, p.NC, [&](int c) -> float {
    if (!fallback) return rt[c];
    const float2 e = tab[c];
    return e.x > kNegInf ? e.y * exp2_acc(a * (e.x - m)) : 0.0f;
  }, red);
  int x = -1;
  if (cstar >= 0) {
    const int x0 = cstar * kChunk + 4 * (int)threadIdx.x;
    float z[4], qx[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {  // all loads first
      const int xc = min(x0 + k, p.V - 1);
      z[k] = load_logit(p, gs, xc);
      qx[k] = draft_q_of(p, q, j, xc);
    }
    const uint4 w4 = rng_block(p, (uint32_t)x0 >> 2, (uint32_t)gs, kTagToken);
    ArgMax best{-1.0f, 0x7FFFFFFF};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int xx = x0 + k;
      if (xx < p.V) {
        const float px = exp2_acc(a * (apply_proc(z[k], xx, pr) - m)) * inv_s;
        const float wx = fallback ? px : fmaxf(px - qx[k], 0.0f);
        if (wx > 0.0f) {
          ArgMax o{race_score(wx, pick(w4, k)), xx};
          if (better(o, best)) best = o;
        }
      }
    }
    const ArgMax bb = block_argmax(best, red);
    x = bb.s < 0.0f ? -1 : bb.i;
  }
  if (threadIdx.x == 0) p.out_tokens[(int64_t)r * p.out_stride + j] = x;
  fused_post_update(p, r, q.K, j, x, [&](int i) { return p.draft_ids[q.c0 + i]; });
}

// Request epilogue kernel: one workgroup per request, after the stats pass.
template <bool PLAIN, bool TP, bool PEN, bool QD, bool FEW = true>
__global__ __launch_bounds__(kThreads) void epilogue_kernel(Params p) {
  __shared__ EpiShared sh;
  request_epilogue<PLAIN, TP, PEN, QD, FEW>(p, load_req(p, blockIdx.x), sh);
}

// ---------------------------------------------------------------------------
// Debug probabilities (parity checks): p of every processed token.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void dbg_kernel(Params p) {
  const int g = blockIdx.y;
  const int x = blockIdx.x * kThreads + threadIdx.x;
  if (x >= p.V) return;
  const int r = find_request(p.cu, p.B, g);
  const Req q = load_req(p, r);
  float v = 0.0f;
  if (q.cu_ok && q.mode != kModeInvalid) {
    const float4 ri = p.row_info[g];
    const int st = __float_as_int(ri.w);
    if (q.mode == kModeGreedy) {
      v = (x == __float_as_int(ri.z)) ? 1.0f : 0.0f;
    } else {
      Proc pr = q.proc;
      if (st != kRowDense) pr.tau = p.cand_tau[g];
      v = exp2_acc(q.a * (apply_proc(load_logit(p, g, x), x, pr) - ri.x)) / ri.y;
    }
  }
  p.dbg_probs[(int64_t)g * p.V + x] = v;
}

// ---------------------------------------------------------------------------
// Debug decision margins (parity checks): one workgroup per target row, after
// every other kernel of the call.  Row i of a sampled request gets the
// smallest relative margin of the random decisions taken on it: its accept
// test when i < K_r and i <= j (|p - u q| / max(p, u q), from the row
// statistics the epilogue stored and the same p(d), q(d) and u), and, on the
// sampled row j, the race: its weights (p_j, the residual max(0, p_j - q_j),
// or p_j without d_j) recomputed token by token over the whole row, the chunk
// and token races run again with their best and second-best scores, margin
// 1 - s2 / s1 per level (1 with a single candidate).  If that recomputation
// picks another token than the one written, the margin is 0.
// ---------------------------------------------------------------------------
struct Top2 {
  float s1, s2;  // best and second-best score (-1: none)
  int i1;        // index of the best (lowest index among equal scores)
  int n;         // candidates
};

__device__ __forceinline__ void top2_add(Top2 &t, float s, int i) {
  ++t.n;
  if (t.i1 < 0 || s > t.s1 || (s == t.s1 && i < t.i1)) {
    if (t.i1 >= 0) t.s2 = t.s1;
    t.s1 = s;
    t.i1 = i;
  } else if (s > t.s2) {
    t.s2 = s;
  }
}

__device__ __forceinline__ double top2_margin(const Top2 &t) {
  if (t.n < 2) return 1.0;
  if (!(t.s1 > 0.0f)) return 0.0;
  return 1.0 - (double)t.s2 / (double)t.s1;
}

__global__ __launch_bounds__(kThreads) void margin_kernel(Params p) {
  __shared__ BlockScratch red;
  __shared__ float ts[kChunk];
  __shared__ Top2 wt[kWaves];
  const int g = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = find_request(p.cu, p.B, g);
  const Req q = load_req(p, r);
  const int i = g - q.g0;
  const int j = p.out_ns[r] - 1;  // the sampled row (-1: request written empty)
  double mg = __builtin_inf();
  if (q.cu_ok && q.mode == kModeSample && i >= 0 && i <= q.K && i <= j && j <= q.K) {
    const float4 ri = p.row_info[g];
    const float m = ri.x, s = ri.y;
    Proc pr = q.proc;
    if (__float_as_int(ri.w) != kRowDense) pr.tau = p.cand_tau[g];
    const float a = q.a;
    const int d = i < q.K ? p.draft_ids[q.c0 + i] : -1;
    const bool valid_d = d >= 0 && d < p.V;
    // Accept test of draft i, in the epilogue's arithmetic.
    if (i < q.K && !p.synthetic && valid_d) {
      const double qd = q.has_q ? (double)draft_q_of(p, q, i, d) : 1.0;
      if (qd > 0.0) {
        const float pd = exp2_acc(a * (apply_proc(load_logit(p, g, d), d, pr) - m)) / s;
        const double uq = u_accept(rng_block(p, 0, (uint32_t)g, kTagAccept).x) * qd;
        mg = __builtin_fabs((double)pd - uq) / __builtin_fmax((double)pd, uq);
      }
    }
    if (i == j) {
      const bool rej = j < q.K;
      const float inv_s = 1.0f / s;
      auto weight = [&](int x, bool resid) -> float {
        const float px = exp2_acc(a * (apply_proc(load_logit(p, g, x), x, pr) - m)) * inv_s;
        if (!resid) return px;
        if (q.has_q) return fmaxf(px - draft_q_of(p, q, j, x), 0.0f);
        return x == d ? 0.0f : px;
      };
      // An empty residual (rounding) races over p_j, as in the epilogue.
      float part = 0.0f;
      if (rej)
        for (int x = tid; x < p.V; x += kThreads) part += weight(x, true);
      const bool resid = rej && block_sum(part, red) > 0.0f;
      // Chunk level: wave w takes chunks w, w + kWaves, ...
      Top2 ct{-1.0f, -1.0f, -1, 0};
      for (int c = wave; c < p.NC; c += kWaves) {
        float acc = 0.0f;
        for (int e = 0; e < kChunk / 64; ++e) {
          const int x = c * kChunk + e * 64 + lane;
          if (x < p.V) acc += weight(x, resid);
        }
        const float W = wave_sum(acc);
        if (W > 0.0f) top2_add(ct, race_score(W, pick(rng_block(p, (uint32_t)c >> 2, (uint32_t)g, kTagChunk), c & 3)), c);
      }
      if (lane == 0) wt[wave] = ct;
      __syncthreads();
      Top2 cb{-1.0f, -1.0f, -1, 0};
      for (int w = 0; w < kWaves; ++w) {  // merge (every thread, same order)
        const Top2 o = wt[w];
        if (o.n == 0) continue;
        const int n = cb.n + o.n;
        top2_add(cb, o.s1, o.i1);
        if (o.s2 > cb.s2) cb.s2 = o.s2;
        cb.n = n;
      }
      double mr = top2_margin(cb);
      int xs = -1;
      if (cb.i1 >= 0) {
        // Token level in the winning chunk.
        for (int t = tid; t < kChunk; t += kThreads) {
          const int x = cb.i1 * kChunk + t;
          const float w = x < p.V ? weight(x, resid) : 0.0f;
          ts[t] = w > 0.0f ? race_score(w, pick(rng_block(p, (uint32_t)x >> 2, (uint32_t)g, kTagToken), x & 3)) : -1.0f;
        }
        __syncthreads();
        Top2 tb{-1.0f, -1.0f, -1, 0};
        for (int t = 0; t < kChunk; ++t)
          if (ts[t] >= 0.0f) top2_add(tb, ts[t], t);
        mr = __builtin_fmin(mr, top2_margin(tb));
        xs = tb.i1 < 0 ? -1 : cb.i1 * kChunk + tb.i1;
      }
      if (xs != p.out_tokens[(int64_t)r * p.out_stride + j]) mr = 0.0;
      mg = __builtin_fmin(mg, mr);
    }
  }
  if (tid == 0) p.dbg_margin[g] = (float)mg;
}

// ---------------------------------------------------------------------------
// post_update ("【vllm】DeepSeekMTP、eagle", _post_update_kernel walk-through).
// ---------------------------------------------------------------------------
// One thread per (request, output slot): every load is issued at once (indices
// clamped into range), the histogram updates are fire-and-forget atomics, and
// the thread holding the last sampled token also writes last_sampled and
// advances num_computed.
__global__ __launch_bounds__(kThreads) void post_update_kernel(PostParams p) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t total = (int64_t)p.B * p.tokens_stride;
  if (i >= total) return;
  const int r = (int)(i / p.tokens_stride), t = (int)(i - (int64_t)r * p.tokens_stride);
  const int n = p.num_sampled[r];
  const int s = p.idx_mapping[r];
  const int tok = p.tokens[i];
  const int ql = p.query_len[r];
  const int nr = p.num_rejected[r];
  const int nn = min(n, p.tokens_stride);
  if (nn <= 0 || t >= nn) return;
  if (s < 0 || s >= p.num_slots) {
    if (t == 0) atomicOr(p.err, SV_ERR_SLOT);
    return;
  }
  if (tok >= 0 && tok < p.V) atomicAdd(&p.counts[(int64_t)s * p.V + tok], 1);
  if (t == nn - 1) {
    p.last_sampled[s] = tok;
    atomicAdd(&p.num_computed[s], ql - nr);
  }
}

// ---------------------------------------------------------------------------
// Debug: the library's own random stream and Exp(1) noise, value for value
// (tests compare them with the published known-answer vectors and the oracle).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void dbg_philox_kernel(const uint4 *ctr, int64_t n, uint32_t k0, uint32_t k1,
                                                             uint4 *out) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads)
    out[i] = philox10(ctr[i], k0, k1);
}

__global__ __launch_bounds__(kThreads) void dbg_noise_kernel(const uint32_t *words, int64_t n, float *out) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads)
    out[i] = exp_noise(words[i]);
}

}  // namespace

hipError_t launch_epilogue(const Params &p, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  const bool qd = p.draft_probs != nullptr || p.draft_logits != nullptr;
  const void *fn;
  if (!plain_call(p))
    fn = reinterpret_cast<const void *>(&epilogue_kernel<false, false, false, false>);
  else if (qd)  // (draft distributions with top-p or penalties: not a plain call)
    fn = p.out_stride <= kWaves ? reinterpret_cast<const void *>(&epilogue_kernel<true, false, false, true>)
                                : reinterpret_cast<const void *>(&epilogue_kernel<true, false, false, true, false>);
  else if (p.has_topp)
    fn = pen_call(p) ? reinterpret_cast<const void *>(&epilogue_kernel<true, true, true, false>)
                     : reinterpret_cast<const void *>(&epilogue_kernel<true, true, false, false>);
  else
    fn = pen_call(p) ? reinterpret_cast<const void *>(&epilogue_kernel<true, false, true, false>)
                     : reinterpret_cast<const void *>(&epilogue_kernel<true, false, false, false>);
  return launch_timed(fn, dim3((unsigned)p.B), p, s, t0, t1);
}

__global__ void zero_count_kernel(int *count) { *count = 0; }

hipError_t launch_zero_count(int *count, hipStream_t s) {
  zero_count_kernel<<<dim3(1), dim3(1), 0, s>>>(count);
  return hipGetLastError();
}

hipError_t launch_resid(const Params &p, hipStream_t s) {
  const dim3 grid((unsigned)p.resid_grid);
  if (p.dtype == 1)
    resid_kernel<1><<<grid, dim3(kThreads), 0, s>>>(p);
  else
    resid_kernel<0><<<grid, dim3(kThreads), 0, s>>>(p);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  resid_race_kernel<<<dim3((unsigned)p.B), dim3(kThreads), 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_dbg_probs(const Params &p, hipStream_t s) {
  const dim3 grid((unsigned)((p.V + kThreads - 1) / kThreads), (unsigned)p.R);
  dbg_kernel<<<grid, dim3(kThreads), 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_dbg_margin(const Params &p, hipStream_t s) {
  margin_kernel<<<dim3((unsigned)p.R), dim3(kThreads), 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_post_update(const PostParams &p, hipStream_t s) {
  const int64_t total = (int64_t)p.B * p.tokens_stride;
  post_update_kernel<<<dim3((unsigned)((total + kThreads - 1) / kThreads)), dim3(kThreads), 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_dbg_philox(const uint32_t *ctr, int64_t n, uint64_t key, uint32_t *out, hipStream_t s) {
  const int64_t blocks = (n + kThreads - 1) / kThreads;
  dbg_philox_kernel<<<dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(kThreads), 0, s>>>(
      reinterpret_cast<const uint4 *>(ctr), n, (uint32_t)(key & 0xFFFFFFFFu), (uint32_t)(key >> 32),
      reinterpret_cast<uint4 *>(out));
  return hipGetLastError();
}

hipError_t launch_dbg_noise(const uint32_t *words, int64_t n, float *out, hipStream_t s) {
  const int64_t blocks = (n + kThreads - 1) / kThreads;
  dbg_noise_kernel<<<dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(kThreads), 0, s>>>(words, n, out);
  return hipGetLastError();
}

}  // namespace sv
