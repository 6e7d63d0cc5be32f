// sv_kernels.hip -- gfx950 kernels of the speculative-decoding verify step.
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

#include "sv_device.h"

namespace sv {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------------------
// Per-request state
// ---------------------------------------------------------------------------
struct Req {
  int r, K, g0, c0;  // request, drafts, first target row, first draft index
  int mode;          // kModeSample / kModeGreedy / kModeInvalid
  float a;           // log2(e) / T
  unsigned errbits;  // device errors this request raises
  bool cu_ok;        // its own cu entries are consistent
  Proc proc;         // penalty part (tau set per row)
};

// Fills a Req from the request's cu entries and temperature, plus the optional
// penalty settings (one more round trip, only when a penalty is given).
__device__ __forceinline__ Req make_req(const Params &p, int r, int c0, int c1, float T) {
  Req q;
  q.r = r;
  q.c0 = c0;
  q.K = c1 - c0;
  q.g0 = c0 + r;
  q.cu_ok = c0 >= 0 && c0 <= c1 && c1 <= p.D && q.K <= p.out_stride - 1;
  q.errbits = 0;
  q.proc.counts = nullptr;
  q.proc.theta = 1.0f;
  q.proc.tau = kNegInf;
  q.a = 0.0f;
  if (!(T >= 0.0f) || !__builtin_isfinite(T)) {
    q.mode = kModeInvalid;
    q.errbits |= SV_ERR_TEMPERATURE;
  } else if (T == 0.0f) {
    q.mode = kModeGreedy;
  } else {
    q.mode = kModeSample;
    q.a = kLog2e / T;
  }
  if (p.rep_penalty != nullptr) {
    const float th = p.rep_penalty[r];
    if (!(th > 0.0f) || !__builtin_isfinite(th)) {
      q.mode = kModeInvalid;
      q.errbits |= SV_ERR_PENALTY;
    } else if (th != 1.0f) {
      const int slot = p.idx_mapping[r];
      if (slot < 0 || slot >= p.num_slots) {
        q.mode = kModeInvalid;
        q.errbits |= SV_ERR_SLOT;
      } else {
        q.proc.counts = p.counts + (int64_t)slot * p.V;
        q.proc.theta = th;
      }
    }
  }
  return q;
}

__device__ __forceinline__ Req load_req(const Params &p, int r) { return make_req(p, r, p.cu[r], p.cu[r + 1], p.temperature[r]); }

// Request owning target row g: the r with f(r) = cu[r] + r <= g < f(r + 1),
// f strictly increasing.  One wide load of a 64-request window around the
// linear guess g B / R (one round trip when the K_r are not far from uniform);
// otherwise a wave-parallel 64-ary search, one wide load per level.  The load
// that finds r also fetches cu[r+1] and the temperature.  Every lane of the
// wave must call it; the result is uniform.
__device__ __forceinline__ Req lookup_req(const Params &p, int g) {
  const int lane = threadIdx.x & 63;
  {
    int base = (int)((int64_t)g * p.B / p.R) - 32;
    base = max(0, min(base, p.B - 64));
    const int idx = base + lane;
    const bool in = idx < p.B;
    const int c = in ? p.cu[idx] : 0x7FFFFFFF;
    const int cn = in ? p.cu[idx + 1] : 0;
    const float T = in ? p.temperature[idx] : 0.0f;
    const int last_lane = min(63, p.B - 1 - base);
    const bool lo_ok = __builtin_amdgcn_readlane(c, 0) + base <= g;
    const bool hi_ok = __builtin_amdgcn_readlane(cn, last_lane) + base + last_lane + 1 > g;
    if (lo_ok && hi_ok) {
      const unsigned long long m = __ballot(in && c + idx <= g);
      const int last = m ? 63 - __clzll((long long)m) : 0;
      return make_req(p, base + last, __builtin_amdgcn_readlane(c, last), __builtin_amdgcn_readlane(cn, last),
                      __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, T), last)));
    }
  }
  int stride = 1;
  while (stride * 64 < p.B) stride *= 64;
  int base = 0;
  for (;;) {
    const int idx = base + lane * stride;
    const bool in = idx < p.B;
    int c = 0, cn = 0;
    float T = 0.0f;
    if (in) {
      c = p.cu[idx];
      if (stride == 1) {
        cn = p.cu[idx + 1];
        T = p.temperature[idx];
      }
    }
    const unsigned long long m = __ballot(in && c + idx <= g);
    const int last = m ? 63 - __clzll((long long)m) : 0;
    if (stride == 1) {
      const int r = base + last;
      return make_req(p, r, __builtin_amdgcn_readlane(c, last), __builtin_amdgcn_readlane(cn, last),
                      __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, T), last)));
    }
    base += last * stride;
    stride /= 64;
  }
}

__device__ __forceinline__ int row_state(const Params &p, int g) { return p.has_topk ? p.cand_n[g] : kRowDense; }

__device__ __forceinline__ float exp2_acc(float t) { return __builtin_amdgcn_exp2f(t); }

// ---------------------------------------------------------------------------
// Chunk decoding.  A wave reads one chunk of kChunk tokens with 16-byte loads:
// bf16: lane l holds tokens [8l, 8l+8) and [512+8l, 512+8l+8);
// fp32: lane l holds tokens [4l + 256 v, 4l + 256 v + 4), v = 0..3.
// Element e of a lane has the chunk-local index below (increasing in e).
// ---------------------------------------------------------------------------
template <int DT>
struct Layout;
template <>
struct Layout<1> {
  static constexpr int kVec = 2;
  static constexpr int kBytes = 2;
  __device__ static __forceinline__ int local(int e, int lane) { return (e >> 3) * 512 + lane * 8 + (e & 7); }
  __device__ static __forceinline__ float elem(const u32x4 *raw, int e) {
    const u32x4 v = raw[e >> 3];
    const int k = e & 7;
    const uint32_t w = (k >> 1) == 0 ? v.x : (k >> 1) == 1 ? v.y : (k >> 1) == 2 ? v.z : v.w;
    return (k & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
  }
};
template <>
struct Layout<0> {
  static constexpr int kVec = 4;
  static constexpr int kBytes = 4;
  __device__ static __forceinline__ int local(int e, int lane) { return (e >> 2) * 256 + lane * 4 + (e & 3); }
  __device__ static __forceinline__ float elem(const u32x4 *raw, int e) {
    const u32x4 v = raw[e >> 2];
    const int k = e & 3;
    return __uint_as_float(k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w);
  }
};

// ---------------------------------------------------------------------------
// Races.  RACE(w, g): chunk c* = argmax_c M_c / E(g, 1, c) over chunks with
// M_c > 0, then token x* = argmax_{x in c*} w_x / E(g, 2, x) over w_x > 0.
// Scores are fp32 (race_score); ties go to the lowest index.
// ---------------------------------------------------------------------------
constexpr int kTabCache = 2048;  // chunk-table entries the epilogue keeps in LDS

struct EpiShared {
  BlockScratch red;
  float m[kMaxDrafts + 1];
  float s[kMaxDrafts + 1];
  float tau[kMaxDrafts + 1];
  float zd[kMaxDrafts + 1];
  float qd[kMaxDrafts + 1];
  float sx[kMaxDrafts + 1];
  int amax[kMaxDrafts + 1];
  int state[kMaxDrafts + 1];
  int d[kMaxDrafts + 1];
  int j;
  int bad;
  int flag;
  float zc[kWaves][kChunk];  // speculative chunks of rows 0..3 (raw logits, token order)
  float zx[kWaves][kChunk];  // the draft tokens' chunks of rows 0..3
  float w1s[kWaves];         // best chunk other than the draft token's: score
  int w1c[kWaves];           //   and index (-1: none)
  int cd[kWaves];            // the draft token's chunk when excluded, else -1
  union {
    float2 tab[kTabCache];  // dense rows: chunk tables of the request's rows
    struct {
      float cw[kCandCap];   // compact rows: candidate weights
      int ci[kCandCap];     // compact rows: candidate token ids
    } cand;
  } u;
};

// Block-level chunk race (all threads call it); thread t takes chunks t,
// t + 256, ...; W(c) >= 0.  Returns -1 if no chunk has positive weight.
template <class WF>
__device__ __forceinline__ int block_chunk_race(const Params &p, uint32_t g, int NC, WF W, BlockScratch &red) {
  ArgMax best{-1.0f, 0x7FFFFFFF};
  for (int c = threadIdx.x; c < NC; c += kThreads) {
    const float Wc = W(c);
    if (Wc > 0.0f) {
      const uint4 w4 = rng_block(p, (uint32_t)c >> 2, g, kTagChunk);
      ArgMax o{race_score(Wc, pick(w4, c & 3)), c};
      if (better(o, best)) best = o;
    }
  }
  const ArgMax b = block_argmax(best, red);
  return b.s < 0.0f ? -1 : b.i;
}

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

__device__ __forceinline__ void write_empty(const Params &p, int r) {
  for (int t = threadIdx.x; t < p.out_stride; t += kThreads) p.out_tokens[(int64_t)r * p.out_stride + t] = -1;
  if (threadIdx.x == 0) {
    p.out_ns[r] = 0;
    p.out_nr[r] = 0;
  }
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

// Chunk c of row g, 16 tokens per lane: lane l holds c C + 256 t + 4 l + k for
// t, k < 4 (one Philox block per 4 tokens); positions past V read token V - 1.
__device__ __forceinline__ int c16_tok(int c, int e, int lane) { return c * kChunk + (e >> 2) * 256 + 4 * lane + (e & 3); }
// The dtype test stays outside the loads so that all 16 issue back to back.
__device__ __forceinline__ void load_chunk16(const Params &p, int g, int c, float (&z)[16]) {
  const int lane = threadIdx.x & 63;
  if (p.dtype == 1) {
    const uint16_t *row = static_cast<const uint16_t *>(p.logits) + (int64_t)g * p.lstride;
#pragma unroll
    for (int e = 0; e < 16; ++e) z[e] = bf16_bits_to_f32(row[min(c16_tok(c, e, lane), p.V - 1)]);
  } else {
    const float *row = static_cast<const float *>(p.logits) + (int64_t)g * p.lstride;
#pragma unroll
    for (int e = 0; e < 16; ++e) z[e] = row[min(c16_tok(c, e, lane), p.V - 1)];
  }
}

// Wave-level chunk race of row g over its chunk table (W_c = s_c exp2(a (m_c - m))),
// chunk `skip` left out.  Lane l draws the words of chunks 4l..4l+3.
template <class EF>
__device__ __forceinline__ ArgMax wave_chunk_race(const Params &p, int g, EF ent, float a, float m, int skip) {
  const int lane = threadIdx.x & 63;
  ArgMax best{-1.0f, 0x7FFFFFFF};
  for (int c0 = 4 * lane; c0 < p.NC; c0 += 256) {
    const uint4 w4 = rng_block(p, (uint32_t)c0 >> 2, (uint32_t)g, kTagChunk);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = c0 + k;
      if (c < p.NC && c != skip) {
        const float2 e = ent(c);
        if (e.x > kNegInf) {
          const float Wc = e.y * exp2_acc(a * (e.x - m));
          if (Wc > 0.0f) {
            ArgMax o{Wc / exp_noise(pick(w4, k)), c};
            if (better(o, best)) best = o;
          }
        }
      }
    }
  }
  return wave_argmax(best);
}

// Token race over chunk c of row g whose raw logits are in LDS (zs, token
// order): weights exp2(fma(z', a, -hi)) on the processed z' (hi = a m_c; a
// factor common to the chunk cancels), token `skip` left out.  Thread t takes
// tokens 4t..4t+3 (one Philox block).  All threads call it; -1 if no token has
// weight.
__device__ __forceinline__ int block_token_race(const Params &p, int g, int c, const float *zs, const Proc &pr,
                                                float a, float hi, int skip, BlockScratch &red) {
  const int t4 = 4 * threadIdx.x;
  const int x0 = c * kChunk + t4;
  const uint4 w4 = rng_block(p, (uint32_t)x0 >> 2, (uint32_t)g, kTagToken);
  const float4 z4 = *reinterpret_cast<const float4 *>(zs + t4);
  const float zz[4] = {z4.x, z4.y, z4.z, z4.w};
  ArgMax best{-1.0f, 0x7FFFFFFF};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int x = x0 + k;
    const bool ok = x < p.V && x != skip;
    const float wx = ok ? exp2_acc(__builtin_fmaf(apply_proc(zz[k], min(x, p.V - 1), pr), a, -hi)) : 0.0f;
    const ArgMax o{race_score(wx, pick(w4, k)), x};
    if (wx > 0.0f && better(o, best)) best = o;
  }
  const ArgMax b = block_argmax(best, red);
  return b.s < 0.0f ? -1 : b.i;
}

// Lowest token of chunk c (held in z) whose processed logit equals m; INT_MAX if none.
__device__ __forceinline__ int wave_first_equal(const Params &p, int c, const float (&z)[16], const Proc &pr, float m) {
  const int lane = threadIdx.x & 63;
  int li = 0x7FFFFFFF;
#pragma unroll
  for (int e = 15; e >= 0; --e) {
    const int x = c16_tok(c, e, lane);
    if (x < p.V && apply_proc(z[e], x, pr) == m) li = x;
  }
  return wave_min_i(li);
}

// Speculative state of one row while its wave waits for the loads.
struct RowSpec {
  float zc[16];   // logits of chunk c1 (stochastic) or of the lowest max chunk (greedy)
  float zx[16];   // logits of the draft token's chunk cd
  ArgMax w1;      // best chunk other than cd: (score, c1); c1 = -1 if none
  int cd;         // draft token's chunk when it is excluded, else -1
};

// Row statistics of row i from its chunk table (dense) or candidates (compact):
// maximum m and Σ exp2(a (z - m)); greedy dense rows also get the lowest
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
// the winning chunk and of the draft token's chunk.
template <class EF>
__device__ __forceinline__ void spec_issue(const Params &p, const Req &q, int i, int d, float m, EF ent, RowSpec &rs) {
  const int g = q.g0 + i;
  const bool excl = i < q.K && !p.draft_probs && d >= 0 && d < p.V;
  rs.cd = excl ? d / kChunk : -1;
  rs.w1 = wave_chunk_race(p, g, ent, q.a, m, rs.cd);
  const int c1 = rs.w1.s < 0.0f ? -1 : rs.w1.i;
  if (c1 >= 0) load_chunk16(p, g, c1, rs.zc);
  if (excl) load_chunk16(p, g, rs.cd, rs.zx);
}

// After the loads of spec_issue: z_d and the mass of d's chunk without d, in
// the chunk entry's scale (exp2(fma(z, a, -hi)) exp2(-lo), a m_c = hi + lo).
__device__ __forceinline__ void spec_draft_record(const Params &p, const Req &q, int d, const Proc &pr,
                                                  const RowSpec &rs, float &zd, float &sx) {
  const int lane = threadIdx.x & 63;
  float z[16];
  float mx = kNegInf, zl = kNegInf;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int x = c16_tok(rs.cd, e, lane);
    z[e] = x < p.V ? apply_proc(rs.zx[e], x, pr) : kNegInf;
    mx = fmaxf(mx, z[e]);
    if (x == d) zl = z[e];
  }
  const float mc = wave_max(mx);
  const float a = q.a, hi = a * mc, lo = __builtin_fmaf(a, mc, -hi);
  float acc = 0.0f;
  if (mc > kNegInf) {
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (c16_tok(rs.cd, e, lane) != d) acc += exp2_acc(__builtin_fmaf(z[e], a, -hi));
  }
  sx = mc > kNegInf ? wave_sum(acc) * exp2_acc(-lo) : 0.0f;
  zd = wave_max(zl);
}

// Moves a wave's speculative chunks and race state for row i to LDS slot `slot`.
__device__ __forceinline__ void spec_publish(const RowSpec &rs, int slot, EpiShared &sh) {
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
  }
}

// Final race of row j from LDS slot `slot` (all threads): the chunk of d
// competes with its mass without d (sx); if nothing is left without d, the race
// is over p_j.
template <class EF>
__device__ __forceinline__ int spec_finish(const Params &p, const Req &q, int j, int dj, float m, float sx,
                                           const Proc &pr, EF ent, int slot, EpiShared &sh) {
  const int gs = q.g0 + j;
  const float a = q.a;
  ArgMax win{sh.w1s[slot], sh.w1c[slot]};
  const int cd = sh.cd[slot];
  bool excl = cd >= 0;
  if (excl) {
    const float2 e = ent(cd);
    const uint32_t wd = pick(rng_block(p, (uint32_t)cd >> 2, (uint32_t)gs, kTagChunk), cd & 3);
    const float Wd = e.x > kNegInf ? sx * exp2_acc(a * (e.x - m)) : 0.0f;
    if (Wd > 0.0f) {
      ArgMax o{race_score(Wd, wd), cd};
      if (better(o, win)) win = o;
    }
    if (win.s < 0.0f) {  // nothing left once d_j is removed (rounding): race over p_j
      excl = false;
      const float Wf = e.x > kNegInf ? e.y * exp2_acc(a * (e.x - m)) : 0.0f;
      if (Wf > 0.0f) win = ArgMax{race_score(Wf, wd), cd};
    }
  }
  if (win.s < 0.0f) return -1;
  const int cstar = win.i;
  const float hi = a * ent(cstar).x;
  const float *zs = cstar == cd ? sh.zx[slot] : sh.zc[slot];
  return block_token_race(p, gs, cstar, zs, pr, a, hi, (excl && cstar == cd) ? dj : -1, sh.red);
}

__device__ __forceinline__ void request_epilogue(const Params &p, const Req &q, EpiShared &sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = q.K, r = q.r, nrow = K + 1;

  if (!q.cu_ok || p.cu[0] != 0 || p.cu[p.B] != p.D) {
    if (tid == 0) raise_err(p, SV_ERR_CU);
    write_empty(p, r);
    return;
  }
  if (q.mode == kModeInvalid) {
    if (tid == 0) raise_err(p, q.errbits);
    write_empty(p, r);
    return;
  }
  const bool greedy = q.mode == kModeGreedy;

  // Row states (top-k pass results), draft ids and the chunk tables.
  for (int i = tid; i < nrow; i += kThreads) {
    const int g = q.g0 + i;
    const int st = row_state(p, g);
    sh.state[i] = st;
    sh.tau[i] = (st == kRowDense) ? kNegInf : p.cand_tau[g];
    sh.d[i] = i < K ? p.draft_ids[q.c0 + i] : -1;
  }
  const bool cached = nrow * p.NC <= kTabCache;
  if (cached) {
    for (int t = tid; t < nrow * p.NC; t += kThreads) {
      const int i = t / p.NC, c = t - i * p.NC;
      sh.u.tab[t] = p.chunk_tab[(int64_t)(q.g0 + i) * p.nc_stride + c];
    }
  }
  __syncthreads();
  auto entry = [&](int i, int c) -> float2 {
    return cached ? sh.u.tab[i * p.NC + c] : p.chunk_tab[(int64_t)(q.g0 + i) * p.nc_stride + c];
  };

  // Each wave takes rows wave, wave + 4, ...  Its first row gets the
  // speculative loads; the others only what the accept tests need.
  RowSpec rs;
#pragma unroll
  for (int e = 0; e < 16; ++e) rs.zc[e] = rs.zx[e] = 0.0f;
  rs.cd = -1;
  rs.w1 = ArgMax{-1.0f, 0x7FFFFFFF};
  for (int i = wave; i < nrow; i += kWaves) {
    const int g = q.g0 + i;
    const int st = sh.state[i];
    const int d = sh.d[i];
    auto ent = [&](int c) { return entry(i, c); };
    float m, s;
    int lc;
    row_stats(p, q, g, st, greedy, ent, m, s, lc);
    Proc pr = q.proc;
    pr.tau = sh.tau[i];
    int am = 0x7FFFFFFF;
    float zd = kNegInf, qd = 1.0f, sx = 0.0f;
    const bool valid_d = i < K && d >= 0 && d < p.V;
    if (st < 0 && greedy) {
      if (lc < p.NC) {
        load_chunk16(p, g, lc, rs.zc);
        am = wave_first_equal(p, lc, rs.zc, pr, m);
      }
    } else if (st < 0 && i == wave && (!p.draft_probs || i == K)) {
      spec_issue(p, q, i, d, m, ent, rs);
      if (rs.cd >= 0) spec_draft_record(p, q, d, pr, rs, zd, sx);
      spec_publish(rs, i, sh);
    } else if (valid_d) {
      // single loads: z_d (and q(d)) for the accept test
      zd = apply_proc(load_logit(p, g, d), d, pr);
      if (p.draft_probs) qd = p.draft_probs[(int64_t)(q.c0 + i) * p.dstride + d];
    }
    if (lane == 0) {
      sh.m[i] = m;
      sh.s[i] = s;
      sh.amax[i] = am;
      sh.zd[i] = zd;
      sh.qd[i] = qd;
      sh.sx[i] = sx;
      p.row_info[g] = make_float4(m, s, __int_as_float(am), __int_as_float(st));
    }
  }
  __syncthreads();
  if (tid == 0) {
    int bad = 0;
    for (int i = 0; i < nrow; ++i) bad |= !__builtin_isfinite(sh.m[i]);
    sh.bad = bad;
  }

  // Accept tests: lane i of wave 0 takes draft position i.
  if (wave == 0) {
    bool rej = false;
    if (lane < K) {
      const int d = sh.d[lane];
      const int g = q.g0 + lane;
      if (greedy) {
        rej = d != sh.amax[lane];
        if (p.dbg_p_draft) p.dbg_p_draft[q.c0 + lane] = -1.0f;
      } else {
        const bool valid = d >= 0 && d < p.V;
        float pd = 0.0f;
        double qd = p.draft_probs ? 0.0 : 1.0;
        if (valid) {
          pd = exp2_acc(q.a * (sh.zd[lane] - sh.m[lane])) / sh.s[lane];
          if (p.draft_probs) qd = (double)sh.qd[lane];
        }
        const double u = u_accept(rng_block(p, 0, (uint32_t)g, kTagAccept).x);
        rej = !(valid && qd > 0.0 && (double)pd >= u * qd);
        if (p.dbg_p_draft) p.dbg_p_draft[q.c0 + lane] = pd;
      }
    }
    const unsigned long long mask = __ballot(rej);
    if (lane == 0) sh.j = mask ? (__ffsll((long long)mask) - 1) : K;
  }
  __syncthreads();
  if (sh.bad) {
    if (tid == 0) raise_err(p, SV_ERR_ROW);
    write_empty(p, r);
    return;
  }
  const int j = sh.j;

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

  if (greedy) {
    if (tid == 0) p.out_tokens[out_j] = sh.amax[j];
    return;
  }

  const int gs = q.g0 + j;
  const bool rejected = j < K;
  const int dj = rejected ? sh.d[j] : -1;
  const float m = sh.m[j], s = sh.s[j];
  Proc pr = q.proc;
  pr.tau = sh.tau[j];
  const int st = sh.state[j];
  const float a = q.a;

  if (st >= 0) {
    // Compact top-k row: the race runs over the kept tokens only.
    __syncthreads();  // the LDS chunk-table cache is reused for the candidates
    const float *cv = p.cand_val + (int64_t)gs * kCandCap;
    const int32_t *cix = p.cand_idx + (int64_t)gs * kCandCap;
    const float *qrow = (rejected && p.draft_probs) ? p.draft_probs + (int64_t)(q.c0 + j) * p.dstride : nullptr;
    float part = 0.0f;
    for (int t = tid; t < st; t += kThreads) {
      const int x = cix[t];
      const float pxv = exp2_acc(a * (cv[t] - m)) / s;
      float w = pxv;
      if (rejected) {
        if (qrow)
          w = fmaxf(pxv - qrow[x], 0.0f);
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
    return;
  }

  if (rejected && p.draft_probs) {
    // Dense residual: handed to resid_kernel (needs the full draft row).
    if (tid == 0) p.res_req[r] = make_int4(gs, j, dj, (int)p.epoch);
    return;
  }

  // Dense race over p_j (bonus row, or the rejected row with d_j removed).
  auto entj = [&](int c) { return entry(j, c); };
  int slot = j;
  float sxj = sh.sx[j];
  if (j >= kWaves) {  // no speculative state for this row: same steps, loads now
    if (wave == 0) {
      spec_issue(p, q, j, dj, m, entj, rs);
      float zd = kNegInf;
      sxj = 0.0f;
      if (rs.cd >= 0) spec_draft_record(p, q, dj, pr, rs, zd, sxj);
      spec_publish(rs, 0, sh);
      if (lane == 0) sh.sx[j] = sxj;
    }
    __syncthreads();
    slot = 0;
    sxj = sh.sx[j];
  }
  const int x = spec_finish(p, q, j, dj, m, sxj, pr, entj, slot, sh);
  if (tid == 0) p.out_tokens[out_j] = x;
}

// ---------------------------------------------------------------------------
// Streaming statistics pass.
//
// Persistent and balanced: the grid is the resident workgroup count, and
// workgroup w owns the contiguous slice [w N / G, (w+1) N / G) of the N = R NC
// chunks, row-major.  Its waves take every 4th chunk of the slice through a
// three-deep load pipeline and write each chunk's (max, scaled mass) entry to
// the chunk table.  Nothing here depends on the draft tokens: the request
// epilogue kernel, launched next on the same stream, reads the tables.
// ---------------------------------------------------------------------------
struct RowInfo {
  int g, r, i, c0, K, g0, mode, st;  // mode kModeInvalid: row skipped
  float a, theta, tau;
  const int32_t *counts;
};
constexpr int kRowCache = kSliceRows;  // rows of a slice looked up before streaming

__device__ __forceinline__ RowInfo row_info_of(const Params &p, const Req &q, int g) {
  RowInfo ri;
  ri.g = g;
  ri.r = q.r;
  ri.i = g - q.g0;
  ri.c0 = q.c0;
  ri.K = q.K;
  ri.g0 = q.g0;
  const bool ok = q.cu_ok && ri.i >= 0 && ri.i <= q.K && q.mode != kModeInvalid;
  ri.mode = ok ? q.mode : kModeInvalid;
  ri.st = ok ? row_state(p, g) : kRowDense;
  ri.a = q.a;
  ri.theta = q.proc.theta;
  ri.counts = q.proc.counts;
  ri.tau = (ok && ri.st == kRowThreshold) ? p.cand_tau[g] : kNegInf;
  return ri;
}

template <int DT>
__device__ __forceinline__ void issue_chunk(const Params &p, int64_t f, int64_t end, u32x4 (&v)[Layout<DT>::kVec]) {
  using L = Layout<DT>;
  if (f >= end || !p.vec_ok) return;
  const int64_t g = f / p.NC;
  const int c = (int)(f - g * p.NC);
  if ((c + 1) * kChunk > p.V) return;
  const int lane = threadIdx.x & 63;
  const u32x4 *src = reinterpret_cast<const u32x4 *>(static_cast<const char *>(p.logits) +
                                                    (g * p.lstride + (int64_t)c * kChunk) * L::kBytes);
#pragma unroll
  for (int h = 0; h < L::kVec; ++h) v[h] = __builtin_nontemporal_load(&src[h * 64 + lane]);
}

// Statistics of chunk c of row ri.g into the chunk table: (max, sum of
// exp2(a (z - max))).  Greedy rows carry a = 0 and only their maxima are used.
template <int DT>
__device__ __forceinline__ void chunk_stats(const Params &p, const RowInfo &ri, int c, const u32x4 (&v)[Layout<DT>::kVec]) {
  using L = Layout<DT>;
  const int lane = threadIdx.x & 63;
  const int g = ri.g;
  Proc pr;
  pr.counts = ri.counts;
  pr.theta = ri.theta;
  pr.tau = ri.tau;
  float z[16];
  if (p.vec_ok && (c + 1) * kChunk <= p.V) {
#pragma unroll
    for (int e = 0; e < 16; ++e) z[e] = L::elem(v, e);
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int x = c * kChunk + L::local(e, lane);
      z[e] = x < p.V ? load_logit(p, g, x) : kNegInf;
    }
  }
  if (pr.counts != nullptr || pr.tau > kNegInf) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int x = c * kChunk + L::local(e, lane);
      if (x < p.V) z[e] = apply_proc(z[e], x, pr);
    }
  }
  float mx = z[0];
#pragma unroll
  for (int e = 1; e < 16; ++e) mx = fmaxf(mx, z[e]);
  const float mc = wave_max(mx);
  // exp2(a (z - mc)) = exp2(fma(z, a, -hi)) * exp2(-lo), a * mc = hi + lo exactly.
  const float a = ri.a;
  const float hi = a * mc;
  const float lo = __builtin_fmaf(a, mc, -hi);
  float sa = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) sa += exp2_acc(__builtin_fmaf(z[e], a, -hi));
  const float2 entry = make_float2(mc, mc > kNegInf ? wave_sum(sa) * exp2_acc(-lo) : 0.0f);
  if (lane == 0) p.chunk_tab[(int64_t)g * p.nc_stride + c] = entry;
}

// Flattened chunk ff of a slice: row lookup (cached) and statistics.
template <int DT>
__device__ __forceinline__ void process_chunk(const Params &p, int64_t ff, const u32x4 (&v)[Layout<DT>::kVec],
                                              RowInfo &cur, const RowInfo *rows, int g_first) {
  const int g = (int)(ff / p.NC);
  const int c = (int)(ff - (int64_t)g * p.NC);
  if (g != cur.g) cur = (g - g_first < kRowCache) ? rows[g - g_first] : row_info_of(p, lookup_req(p, g), g);
  if (cur.mode != kModeInvalid && cur.st < 0) chunk_stats<DT>(p, cur, c, v);
}

// Row state read back from LDS is the same in every lane: keep it in SGPRs.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float uni(float v) { return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v))); }
__device__ __forceinline__ RowInfo uniform_row(const RowInfo &x) {
  RowInfo y;
  y.g = uni(x.g);
  y.r = uni(x.r);
  y.i = uni(x.i);
  y.c0 = uni(x.c0);
  y.K = uni(x.K);
  y.g0 = uni(x.g0);
  y.mode = uni(x.mode);
  y.st = uni(x.st);
  y.a = uni(x.a);
  y.theta = uni(x.theta);
  y.tau = uni(x.tau);
  const uintptr_t c = (uintptr_t)x.counts;
  y.counts = (const int32_t *)(((uintptr_t)(uint32_t)uni((int)(uint32_t)c)) | ((uintptr_t)(uint32_t)uni((int)(uint32_t)(c >> 32)) << 32));
  return y;
}

struct StatsShared {
  RowInfo rows[kRowCache];
};

template <int DT>
__global__ __launch_bounds__(kThreads) void stats_kernel(Params p) {
  using L = Layout<DT>;
  constexpr int NV = L::kVec;
  __shared__ StatsShared sh;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t N = (int64_t)p.R * p.NC;
  const int64_t start = (int64_t)blockIdx.x * N / gridDim.x;
  const int64_t end = (int64_t)(blockIdx.x + 1) * N / gridDim.x;
  if (start >= end) return;
  const int g_first = (int)(start / p.NC), g_last = (int)((end - 1) / p.NC);
  const int nrows = g_last - g_first + 1;

  // Three chunks in flight per wave before anything else.
  u32x4 A[NV], Bv[NV], Cv[NV];
  int64_t f = start + wave;
  issue_chunk<DT>(p, f, end, A);
  issue_chunk<DT>(p, f + kWaves, end, Bv);
  issue_chunk<DT>(p, f + 2 * kWaves, end, Cv);

  // Request lookups for the first rows of the slice (overlapping the loads).
  if (wave < min(nrows, kRowCache)) {
    const int g = g_first + wave;
    const RowInfo ri = row_info_of(p, lookup_req(p, g), g);
    if (lane == 0) sh.rows[wave] = ri;
  }
  __syncthreads();

  RowInfo cur;
  cur.g = -1;
  for (; f < end; f += 3 * kWaves) {
    process_chunk<DT>(p, f, A, cur, sh.rows, g_first);
    issue_chunk<DT>(p, f + 3 * kWaves, end, A);
    if (f + kWaves >= end) break;
    process_chunk<DT>(p, f + kWaves, Bv, cur, sh.rows, g_first);
    issue_chunk<DT>(p, f + 4 * kWaves, end, Bv);
    if (f + 2 * kWaves >= end) break;
    process_chunk<DT>(p, f + 2 * kWaves, Cv, cur, sh.rows, g_first);
    issue_chunk<DT>(p, f + 5 * kWaves, end, Cv);
  }

}

// ---------------------------------------------------------------------------
// Fast streaming pass: aligned rows, V a multiple of the vector width, no
// penalty and no top-k (the common case, and the no-draft-probs workload).
// Same slices and tables as stats_kernel, with a loop the compiler
// can pipeline exactly: every wave issues one unconditional set of 16-byte
// loads per chunk (lanes past the row end read the row's first vector and are
// masked), tracks (row, chunk) in 32-bit, and keeps three chunks in flight.
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ void fast_load(const Params &p, int g, int c, u32x4 (&v)[Layout<DT>::kVec]) {
  using L = Layout<DT>;
  constexpr int kTok = 16 / L::kBytes;  // tokens per 16-byte vector
  const int lane = threadIdx.x & 63;
  // Uniform row base plus a 32-bit per-lane byte offset (SGPR-base addressing).
  const char *row = static_cast<const char *>(p.logits) + (int64_t)g * p.lstride * L::kBytes;
#pragma unroll
  for (int h = 0; h < L::kVec; ++h) {
    const int x = c * kChunk + L::local(h * kTok, lane);  // first token of this lane's vector h
    const uint32_t off = x + kTok <= p.V ? (uint32_t)x * L::kBytes : 0u;
    v[h] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(row + off));
  }
}

__device__ __forceinline__ void advance_chunk(int &g, int &c, int by, int NC) {
  c += by;
  while (c >= NC) {
    c -= NC;
    ++g;
  }
}

template <int DT>
__device__ __forceinline__ void fast_chunk(const Params &p, const RowInfo &ri, int c, const u32x4 (&v)[Layout<DT>::kVec]) {
  using L = Layout<DT>;
  const int lane = threadIdx.x & 63;
  float z[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) z[e] = L::elem(v, e);
  if ((c + 1) * kChunk > p.V) {  // row tail: tokens past V do not exist
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (c * kChunk + L::local(e, lane) >= p.V) z[e] = kNegInf;
  }
  float mx = z[0];
#pragma unroll
  for (int e = 1; e < 16; ++e) mx = fmaxf(mx, z[e]);
  const float mc = wave_max(mx);
  // exp2(a (z - mc)) = exp2(fma(z, a, -hi)) * exp2(-lo), a * mc = hi + lo
  // exactly; greedy rows carry a = 0 and only their maxima are used.
  const float a = ri.a;
  const float hi = a * mc;
  const float lo = __builtin_fmaf(a, mc, -hi);
  float sa = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) sa += exp2_acc(__builtin_fmaf(z[e], a, -hi));
  const float2 entry = make_float2(mc, mc > kNegInf ? wave_sum(sa) * exp2_acc(-lo) : 0.0f);
  if (lane == 0 && ri.mode != kModeInvalid) p.chunk_tab[(int64_t)ri.g * p.nc_stride + c] = entry;
}

template <int DT>
__global__ __launch_bounds__(kThreads) void stats_fast_kernel(Params p) {
  using L = Layout<DT>;
  constexpr int NV = L::kVec;
  __shared__ StatsShared sh;
  const int wave = uni((int)(threadIdx.x >> 6));
  const int N = p.R * p.NC;
  const int start = (int)((int64_t)blockIdx.x * N / gridDim.x);
  const int end = (int)((int64_t)(blockIdx.x + 1) * N / gridDim.x);
  if (start >= end) return;
  const int g_first = start / p.NC, g_last = (end - 1) / p.NC;
  const int nrows = g_last - g_first + 1;
  const int len = end - start;
  const int n = wave < len ? (len - wave + kWaves - 1) / kWaves : 0;

  int ga = (start + wave) / p.NC, ca = start + wave - ga * p.NC;
  int gb = ga, cb = ca, gc = ga, cc = ca;
  advance_chunk(gb, cb, kWaves, p.NC);
  advance_chunk(gc, cc, 2 * kWaves, p.NC);
  // The first three loads are unconditional (a wave with fewer chunks reads
  // the slice's first chunk instead), so that every path into the loop has the
  // same loads in flight and the waits stay three chunks deep.
  u32x4 A[NV], Bv[NV], Cv[NV];
  fast_load<DT>(p, n > 0 ? ga : g_first, n > 0 ? ca : 0, A);
  fast_load<DT>(p, n > 1 ? gb : g_first, n > 1 ? cb : 0, Bv);
  fast_load<DT>(p, n > 2 ? gc : g_first, n > 2 ? cc : 0, Cv);

  // Request lookups for the slice's rows (overlapping the loads); q(d) is
  // fetched here too so that the loop issues no dependent loads.
  if (wave < nrows) {
    const int g = g_first + wave;
    const RowInfo ri = row_info_of(p, lookup_req(p, g), g);
    if ((threadIdx.x & 63) == 0) sh.rows[wave] = ri;
  }
  __syncthreads();

  RowInfo cur = uniform_row(sh.rows[ga - g_first]);
  int k = 0;
  for (; k + 5 < n; k += 3) {
    if (ga != cur.g) cur = uniform_row(sh.rows[ga - g_first]);
    fast_chunk<DT>(p, cur, ca, A);
    advance_chunk(ga, ca, 3 * kWaves, p.NC);
    fast_load<DT>(p, ga, ca, A);
    if (gb != cur.g) cur = uniform_row(sh.rows[gb - g_first]);
    fast_chunk<DT>(p, cur, cb, Bv);
    advance_chunk(gb, cb, 3 * kWaves, p.NC);
    fast_load<DT>(p, gb, cb, Bv);
    if (gc != cur.g) cur = uniform_row(sh.rows[gc - g_first]);
    fast_chunk<DT>(p, cur, cc, Cv);
    advance_chunk(gc, cc, 3 * kWaves, p.NC);
    fast_load<DT>(p, gc, cc, Cv);
  }
  // Drain: at most 5 chunks left, loads only while in range.
#pragma unroll
  for (int t = 0; t < 6; ++t) {
    if (k + t >= n) break;
    if (t % 3 == 0) {
      if (ga != cur.g) cur = uniform_row(sh.rows[ga - g_first]);
      fast_chunk<DT>(p, cur, ca, A);
      if (k + t + 3 < n) {
        advance_chunk(ga, ca, 3 * kWaves, p.NC);
        fast_load<DT>(p, ga, ca, A);
      }
    } else if (t % 3 == 1) {
      if (gb != cur.g) cur = uniform_row(sh.rows[gb - g_first]);
      fast_chunk<DT>(p, cur, cb, Bv);
      if (k + t + 3 < n) {
        advance_chunk(gb, cb, 3 * kWaves, p.NC);
        fast_load<DT>(p, gb, cb, Bv);
      }
    } else {
      if (gc != cur.g) cur = uniform_row(sh.rows[gc - g_first]);
      fast_chunk<DT>(p, cur, cc, Cv);
      if (k + t + 3 < n) {
        advance_chunk(gc, cc, 3 * kWaves, p.NC);
        fast_load<DT>(p, gc, cc, Cv);
      }
    }
  }

}

// ---------------------------------------------------------------------------
// Residual pass (draft-probs mode, dense rows).  resid_kernel: chunk masses of
// w = max(0, p_j - q_j) for each rejected request (one workgroup per segment
// of cps chunks); resid_race_kernel: the race over them (one workgroup per
// request).  A request is active when its res_req entry carries this call's
// epoch.
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(kThreads) void resid_kernel(Params p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = blockIdx.x / p.nseg;
  const int seg = blockIdx.x - r * p.nseg;
  const int4 rq = p.res_req[r];
  if (rq.w != (int)p.epoch) return;
  const Req q = load_req(p, r);
  const int gs = rq.x, j = rq.y;
  const float4 ri = p.row_info[gs];
  const float m = ri.x, inv_s = 1.0f / ri.y, a = q.a;
  Proc pr = q.proc;
  if (__float_as_int(ri.w) == kRowThreshold) pr.tau = p.cand_tau[gs];
  const float *qrow = p.draft_probs + (int64_t)(q.c0 + j) * p.dstride;
  float *rt = p.res_tab + (int64_t)r * p.nc_stride;
  for (int c = seg * p.cps + wave; c < min(p.NC, (seg + 1) * p.cps); c += kWaves) {
    float acc = 0.0f;
    for (int t = lane; t < kChunk; t += 64) {
      const int x = c * kChunk + t;
      if (x < p.V) {
        const float px = exp2_acc(a * (apply_proc(load_logit(p, gs, x), x, pr) - m)) * inv_s;
        acc += fmaxf(px - qrow[x], 0.0f);
      }
    }
    const float Wc = wave_sum(acc);
    if (lane == 0) rt[c] = Wc;
  }
}

__global__ __launch_bounds__(kThreads) void resid_race_kernel(Params p) {
  __shared__ BlockScratch red;
  const int r = blockIdx.x;
  const int4 rq = p.res_req[r];
  if (rq.w != (int)p.epoch) return;
  const Req q = load_req(p, r);
  const int gs = rq.x, j = rq.y;
  const float4 ri = p.row_info[gs];
  const float m = ri.x, inv_s = 1.0f / ri.y, a = q.a;
  Proc pr = q.proc;
  if (__float_as_int(ri.w) == kRowThreshold) pr.tau = p.cand_tau[gs];
  const float *qrow = p.draft_probs + (int64_t)(q.c0 + j) * p.dstride;
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
      qx[k] = qrow[xc];
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
}

// Request epilogue kernel: one workgroup per request, after the stats pass.
__global__ __launch_bounds__(kThreads) void epilogue_kernel(Params p) {
  __shared__ EpiShared sh;
  request_epilogue(p, load_req(p, blockIdx.x), sh);
}

// ---------------------------------------------------------------------------
// Top-k pass: one workgroup per row.
// ---------------------------------------------------------------------------
constexpr int kBuf = 2048;   // LDS candidate buffer
constexpr int kTile = 1024;  // tokens appended per step at most

struct TopkShared {
  float bv[kBuf];
  int bi[kBuf];
  unsigned hist[256];
  int n;
  int sel, want;
  float theta;
};

// Order-preserving map float -> uint32 (larger float, larger key).
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float fval(uint32_t k) { return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k); }

// One MSD radix digit: among keys matching (prefix, mask), find the digit at
// `shift` holding the want-th largest; updates prefix/mask/want (uniform).
__device__ void radix_digit(TopkShared &sh, int shift, uint32_t &prefix, uint32_t &mask, int &want) {
  if (threadIdx.x == 0) {
    int acc = 0, sel = 0;
    for (int b = 255; b >= 0; --b) {
      const int h = (int)sh.hist[b];
      if (acc + h >= want) {
        sel = b;
        break;
      }
      acc += h;
    }
    sh.sel = sel;
    sh.want = want - acc;
  }
  __syncthreads();
  prefix |= (uint32_t)sh.sel << shift;
  mask |= 0xFFu << shift;
  want = sh.want;
  __syncthreads();
}

// k-th largest value among sh.bv[0..n) (1 <= k <= n).
__device__ float buffer_kth(TopkShared &sh, int n, int k) {
  uint32_t prefix = 0, mask = 0;
  int want = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    sh.hist[threadIdx.x] = 0;
    __syncthreads();
    for (int e = threadIdx.x; e < n; e += kThreads) {
      const uint32_t key = fkey(sh.bv[e]);
      if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 0xFFu], 1u);
    }
    __syncthreads();
    radix_digit(sh, shift, prefix, mask, want);
  }
  return fval(prefix);
}

// Keep the buffer entries >= t (order not preserved).
__device__ void buffer_keep(TopkShared &sh, int n, float t) {
  float kv[kBuf / kThreads];
  int ki[kBuf / kThreads];
  int nk = 0;
#pragma unroll
  for (int m = 0; m < kBuf / kThreads; ++m) {
    const int e = threadIdx.x + m * kThreads;
    if (e < n && sh.bv[e] >= t) {
      kv[nk] = sh.bv[e];
      ki[nk] = sh.bi[e];
      ++nk;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) sh.n = 0;
  __syncthreads();
  for (int m = 0; m < nk; ++m) {
    const int pos = atomicAdd(&sh.n, 1);
    sh.bv[pos] = kv[m];
    sh.bi[pos] = ki[m];
  }
  __syncthreads();
}

template <int DT>
__global__ __launch_bounds__(kThreads) void topk_kernel(Params p) {
  __shared__ TopkShared sh;
  const int g = blockIdx.x;
  const int r = find_request(p.cu, p.B, g);
  const Req q = load_req(p, r);
  const int k = p.top_k[r];
  const bool use = q.cu_ok && g >= q.g0 && g <= q.g0 + q.K && q.mode == kModeSample && k >= 1 && k < p.V;
  if (!use) {
    if (threadIdx.x == 0) {
      p.cand_n[g] = kRowDense;
      p.cand_tau[g] = kNegInf;
    }
    return;
  }
  const Proc pr = q.proc;  // penalty only

  if (threadIdx.x == 0) {
    sh.n = 0;
    sh.theta = kNegInf;
  }
  __syncthreads();
  bool overflow = k > kCandCap;
  if (!overflow) {
    for (int base = 0; base < p.V; base += kTile) {
      const float th = sh.theta;
#pragma unroll
      for (int t = 0; t < kTile / kThreads; ++t) {
        const int x = base + t * kThreads + (int)threadIdx.x;
        if (x < p.V) {
          const float z = apply_proc(load_logit(p, g, x), x, pr);
          if (z >= th && z > kNegInf) {
            const int pos = atomicAdd(&sh.n, 1);
            sh.bv[pos] = z;
            sh.bi[pos] = x;
          }
        }
      }
      __syncthreads();
      const int n = sh.n;
      if (n > kBuf - kTile) {
        const float t = buffer_kth(sh, n, k);
        buffer_keep(sh, n, t);
        if (threadIdx.x == 0) sh.theta = t;
        __syncthreads();
        if (sh.n > kBuf - kTile) {
          overflow = true;
          break;
        }
      }
    }
  }

  float tau;
  int ncand = -1;
  if (!overflow) {
    const int n = sh.n;
    if (n < k) {
      tau = kNegInf;  // fewer than k finite logits: nothing is removed
    } else {
      tau = buffer_kth(sh, n, k);
      buffer_keep(sh, n, tau);
      ncand = sh.n;
    }
  } else {
    // Exact tau by MSD radix select over the whole row (many ties).
    uint32_t prefix = 0, mask = 0;
    int want = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
      sh.hist[threadIdx.x] = 0;
      __syncthreads();
      for (int x = threadIdx.x; x < p.V; x += kThreads) {
        const uint32_t key = fkey(apply_proc(load_logit(p, g, x), x, pr));
        if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 0xFFu], 1u);
      }
      __syncthreads();
      radix_digit(sh, shift, prefix, mask, want);
    }
    tau = fval(prefix);
  }

  if (ncand < 0 || ncand > kCandCap) {
    if (threadIdx.x == 0) {
      p.cand_n[g] = (tau > kNegInf) ? kRowThreshold : kRowDense;
      p.cand_tau[g] = tau;
    }
    return;
  }

  // Sort the kept tokens by id (bitonic over kCandCap slots, padding = INT_MAX).
  for (int e = ncand + (int)threadIdx.x; e < kCandCap; e += kThreads) sh.bi[e] = 0x7FFFFFFF;
  __syncthreads();
  for (int size = 2; size <= kCandCap; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int pi = threadIdx.x; pi < kCandCap / 2; pi += kThreads) {
        const int i = 2 * stride * (pi / stride) + (pi % stride);
        const int jj = i + stride;
        const bool up = (i & size) == 0;
        const int a = sh.bi[i], b = sh.bi[jj];
        if ((a > b) == up) {
          sh.bi[i] = b;
          sh.bi[jj] = a;
          const float fa = sh.bv[i];
          sh.bv[i] = sh.bv[jj];
          sh.bv[jj] = fa;
        }
      }
      __syncthreads();
    }
  }
  for (int e = threadIdx.x; e < ncand; e += kThreads) {
    p.cand_val[(int64_t)g * kCandCap + e] = sh.bv[e];
    p.cand_idx[(int64_t)g * kCandCap + e] = sh.bi[e];
  }
  if (threadIdx.x == 0) {
    p.cand_n[g] = ncand;
    p.cand_tau[g] = tau;
  }
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

}  // namespace

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_topk(const Params &p, hipStream_t s) {
  if (p.dtype == 1)
    topk_kernel<1><<<dim3(p.R), dim3(kThreads), 0, s>>>(p);
  else
    topk_kernel<0><<<dim3(p.R), dim3(kThreads), 0, s>>>(p);
  return hipGetLastError();
}

// Launch with optional timing events: hipExtLaunchKernel stamps them from the
// dispatch packet itself, so their interval is the kernel's execution time.
hipError_t launch_timed(const void *fn, dim3 grid, const Params &p, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  Params arg = p;
  void *args[] = {&arg};
  return hipExtLaunchKernel(fn, grid, dim3(kThreads), args, 0, s, t0, t1, 0);
}

hipError_t launch_stats(const Params &p, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  const dim3 grid((unsigned)p.stats_grid);
  const void *fn = p.fast ? (p.dtype == 1 ? reinterpret_cast<const void *>(&stats_fast_kernel<1>)
                                          : reinterpret_cast<const void *>(&stats_fast_kernel<0>))
                          : (p.dtype == 1 ? reinterpret_cast<const void *>(&stats_kernel<1>)
                                          : reinterpret_cast<const void *>(&stats_kernel<0>));
  return launch_timed(fn, grid, p, s, t0, t1);
}

int stats_blocks_per_cu(int dtype, bool fast) {
  int n = 0;
  hipError_t e;
  if (fast)
    e = dtype == 1 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, stats_fast_kernel<1>, kThreads, 0)
                   : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, stats_fast_kernel<0>, kThreads, 0);
  else
    e = dtype == 1 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, stats_kernel<1>, kThreads, 0)
                   : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, stats_kernel<0>, kThreads, 0);
  return e == hipSuccess && n > 0 ? n : 1;
}

hipError_t launch_epilogue(const Params &p, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  return launch_timed(reinterpret_cast<const void *>(&epilogue_kernel), dim3((unsigned)p.B), p, s, t0, t1);
}

hipError_t launch_resid(const Params &p, hipStream_t s) {
  const dim3 grid((unsigned)(p.B * p.nseg));
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

hipError_t launch_post_update(const PostParams &p, hipStream_t s) {
  const int64_t total = (int64_t)p.B * p.tokens_stride;
  post_update_kernel<<<dim3((unsigned)((total + kThreads - 1) / kThreads)), dim3(kThreads), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace sv
