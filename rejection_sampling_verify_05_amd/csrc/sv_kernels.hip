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
  float top_p;       // nucleus mass in [1e-6, 1]; 1: off
  bool has_q;        // the drafts carry a distribution q (probabilities, or draft logits at T_q > 0)
  float aq;          // log2(e) / T_q (draft-logits mode)
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
  q.proc.freq = 0.0f;
  q.proc.pres = 0.0f;
  q.proc.tau = kNegInf;
  q.top_p = 1.0f;
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
  // Penalties: a valid setting other than the identity needs the request's
  // histogram slot.
  bool need_counts = false;
  if (p.rep_penalty != nullptr) {
    const float th = p.rep_penalty[r];
    if (!(th > 0.0f) || !__builtin_isfinite(th)) {
      q.mode = kModeInvalid;
      q.errbits |= SV_ERR_PENALTY;
    } else if (th != 1.0f) {
      q.proc.theta = th;
      need_counts = true;
    }
  }
  if (p.freq_penalty != nullptr) {
    const float f = p.freq_penalty[r];
    if (!__builtin_isfinite(f)) {
      q.mode = kModeInvalid;
      q.errbits |= SV_ERR_PENALTY;
    } else if (f != 0.0f) {
      q.proc.freq = f;
      need_counts = true;
    }
  }
  if (p.pres_penalty != nullptr) {
    const float f = p.pres_penalty[r];
    if (!__builtin_isfinite(f)) {
      q.mode = kModeInvalid;
      q.errbits |= SV_ERR_PENALTY;
    } else if (f != 0.0f) {
      q.proc.pres = f;
      need_counts = true;
    }
  }
  if (need_counts) {
    const int slot = p.idx_mapping[r];
    if (slot < 0 || slot >= p.num_slots) {
      q.mode = kModeInvalid;
      q.errbits |= SV_ERR_SLOT;
    } else {
      q.proc.counts = p.counts + (int64_t)slot * p.V;
    }
  }
  q.has_q = p.draft_probs != nullptr;
  q.aq = 0.0f;
  if (p.draft_logits != nullptr) {  // draft-logits mode; greedy drafts (T_q = 0) act as draft ids only
    const float tq = p.draft_temp[r];
    if (!(tq >= 0.0f) || !__builtin_isfinite(tq)) {
      q.mode = kModeInvalid;
      q.errbits |= SV_ERR_TEMPERATURE;
    } else if (tq > 0.0f) {
      q.has_q = true;
      q.aq = kLog2e / tq;
    }
  }
  if (p.top_p != nullptr) {
    const float tp = p.top_p[r];
    if (tp != tp) {
      q.mode = kModeInvalid;
      q.errbits |= SV_ERR_TOP_P;
    } else {
      q.top_p = tp < 1e-6f ? 1e-6f : (tp > 1.0f ? 1.0f : tp);
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

__device__ __forceinline__ int row_state(const Params &p, int g) { return p.cand_valid ? p.cand_n[g] : kRowDense; }

__device__ __forceinline__ float exp2_acc(float t) { return __builtin_amdgcn_exp2f(t); }

// q_i(x) of request q's draft row i: stored probability, or from the draft
// logits and the row's (m_q, s_q) (the draft-side sampler's formula).
__device__ __forceinline__ float draft_q_of(const Params &p, const Req &q, int i, int x) {
  const int64_t dr = q.c0 + i;
  if (p.draft_probs != nullptr) return p.draft_probs[dr * p.dstride + x];
  const float mq = p.draft_stats[2 * dr], inv_sq = 1.0f / p.draft_stats[2 * dr + 1];
  return exp2_acc(q.aq * (load_draft_logit(p, dr, x) - mq)) * inv_sq;
}


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
  float rcd[kWaves];         // 1/E of that chunk in the chunk race
  union {
    float2 tab[TC];  // dense rows: chunk tables of the request's rows
    CandBuf<CAND> cand;
  } u;
};
using EpiShared = EpiSharedT<kTabCache, true>;

// Block-level chunk race (all threads call it); thread t takes chunks t,
// t + 256, ...; W(c) >= 0.  Returns -1 if no chunk has positive weight.
template <class WF>
__device__ __forceinline__ int block_chunk_race(const Params &p, uint32_t g, int NC, WF W, BlockScratch &red,
                                                uint32_t tag = kTagChunk) {
  ArgMax best{-1.0f, 0x7FFFFFFF};
  for (int c = threadIdx.x; c < NC; c += kThreads) {
    const float Wc = W(c);
    if (Wc > 0.0f) {
      const uint4 w4 = rng_block(p, (uint32_t)c >> 2, g, tag);
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

// post_update of request r inside the verify call, once its tokens are final:
// the accepted drafts draft(0..j-1), then x (num_sampled = j + 1, num_rejected
// = K - j); the same updates as post_update_kernel.  All threads call it.
template <class DF>
__device__ __forceinline__ void fused_post_update(const Params &p, int r, int K, int j, int x, DF draft) {
  if (p.pu_idx_mapping == nullptr) return;
  const int s = p.pu_idx_mapping[r];
  if (s < 0 || s >= p.pu_num_slots) {
    if (threadIdx.x == 0) atomicOr(p.err, SV_ERR_SLOT);
    return;
  }
  for (int i = threadIdx.x; i <= j; i += blockDim.x) {  // each output counted once
    const int tok = i < j ? draft(i) : x;
    if (tok >= 0 && tok < p.V) atomicAdd(&p.pu_counts[(int64_t)s * p.V + tok], 1);
  }
  if (threadIdx.x == 0) {
    p.pu_last_sampled[s] = x;
    atomicAdd(&p.pu_num_computed[s], p.pu_query_len[r] - (K - j));
  }
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
// The dtype and alignment tests stay outside the loads so that they issue back
// to back: with aligned rows and V a multiple of 4, one 8-byte (bf16) or
// 16-byte (fp32) load per group of 4 tokens (a group at or past V reads group
// 0 and is masked later); otherwise 16 scalar loads.
__device__ __forceinline__ void load_chunk16_at(const void *base, int dtype, int64_t stride, bool vec, int V, int64_t g,
                                                int c, float (&z)[16]) {
  const int lane = threadIdx.x & 63;
  if (vec && (V & 3) == 0) {
    if (dtype == 1) {
      const uint2 *row = reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(base) + (int64_t)g * stride);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int x0 = c16_tok(c, 4 * t, lane);
        const uint2 w = row[x0 < V ? x0 >> 2 : 0];
        z[4 * t] = __uint_as_float(w.x << 16);
        z[4 * t + 1] = __uint_as_float(w.x & 0xFFFF0000u);
        z[4 * t + 2] = __uint_as_float(w.y << 16);
        z[4 * t + 3] = __uint_as_float(w.y & 0xFFFF0000u);
      }
    } else {
      const float4 *row = reinterpret_cast<const float4 *>(static_cast<const float *>(base) + (int64_t)g * stride);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int x0 = c16_tok(c, 4 * t, lane);
        const float4 w = row[x0 < V ? x0 >> 2 : 0];
        z[4 * t] = w.x;
        z[4 * t + 1] = w.y;
        z[4 * t + 2] = w.z;
        z[4 * t + 3] = w.w;
      }
    }
  } else if (dtype == 1) {
    const uint16_t *row = static_cast<const uint16_t *>(base) + (int64_t)g * stride;
#pragma unroll
    for (int e = 0; e < 16; ++e) z[e] = bf16_bits_to_f32(row[min(c16_tok(c, e, lane), V - 1)]);
  } else {
    const float *row = static_cast<const float *>(base) + (int64_t)g * stride;
#pragma unroll
    for (int e = 0; e < 16; ++e) z[e] = row[min(c16_tok(c, e, lane), V - 1)];
  }
}

__device__ __forceinline__ void load_chunk16(const Params &p, int g, int c, float (&z)[16]) {
  load_chunk16_at(p.logits, p.dtype, p.lstride, p.vec_ok, p.V, g, c, z);
}

// load_chunk16 with the row's penalties applied (those of apply_proc; the
// top-k threshold is left to the consumers): the counts of the chunk's tokens
// are loaded together with the logits, so penalties cost no extra round trip.
__device__ __forceinline__ void load_chunk16_pen(const Params &p, int g, int c, const Proc &pr, float (&z)[16]) {
  if (pr.counts == nullptr) {
    load_chunk16(p, g, c, z);
    return;
  }
  const int lane = threadIdx.x & 63;
  int cnt[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) cnt[e] = pr.counts[min(c16_tok(c, e, lane), p.V - 1)];
  load_chunk16(p, g, c, z);
#pragma unroll
  for (int e = 0; e < 16; ++e)
    if (cnt[e] > 0) z[e] = penalize(z[e], cnt[e], pr);
}

// The processing left for logits whose penalties are applied: the threshold.
__device__ __forceinline__ Proc proc_after_pen(const Proc &pr) {
  Proc id = pr;
  id.counts = nullptr;
  return id;
}

// Wave-level chunk race of row g over its chunk table (W_c = s_c exp2(a (r_c - m))),
// chunk `skip` left out.  Lane l draws the words of chunks 4l..4l+3.
// 1/E of the chunk race for a wave's first 256 chunks of row g: lane l holds
// chunks 4l..4l+3 (one Philox block).  Depends only on the row, so it can be
// computed while the chunk tables are still in flight.
struct ChunkNoise {
  float r[4];
};
__device__ __forceinline__ ChunkNoise chunk_noise(const Params &p, int g) {
  const int lane = threadIdx.x & 63;
  const uint4 w4 = rng_block(p, (uint32_t)lane, (uint32_t)g, kTagChunk);
  ChunkNoise n;
#pragma unroll
  for (int k = 0; k < 4; ++k) n.r[k] = __builtin_amdgcn_rcpf(exp_noise(pick(w4, k)));
  return n;
}

// Wave-level chunk race of row g over its chunk table (W_c = s_c exp2(a (r_c - m))),
// chunk `skip` left out; scores W_c / E_c = W_c * (1/E_c), with 1/E from cn for
// the first 256 chunks.  *rskip receives 1/E of chunk skip (if skip >= 0).
template <class EF>
__device__ __forceinline__ ArgMax wave_chunk_race(const Params &p, int g, EF ent, float a, float m, int skip,
                                                  const ChunkNoise &cn, float *rskip) {
  const int lane = threadIdx.x & 63;
  ArgMax best{-1.0f, 0x7FFFFFFF};
  float rs = 0.0f;
  for (int c0 = 4 * lane; c0 < p.NC; c0 += 256) {
    ChunkNoise n = cn;
    if (c0 >= 256) {  // chunks past the first 256: drawn here
      const uint4 w4 = rng_block(p, (uint32_t)c0 >> 2, (uint32_t)g, kTagChunk);
#pragma unroll
      for (int k = 0; k < 4; ++k) n.r[k] = __builtin_amdgcn_rcpf(exp_noise(pick(w4, k)));
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = c0 + k;
      if (c == skip) rs = n.r[k];
      if (c < p.NC && c != skip) {
        const float2 e = ent(c);
        if (e.x > kNegInf) {
          const float Wc = e.y * exp2_acc(a * (e.x - m));
          if (Wc > 0.0f) {
            ArgMax o{Wc * n.r[k], c};
            if (better(o, best)) best = o;
          }
        }
      }
    }
  }
  if (skip >= 0) *rskip = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rs), (skip >> 2) & 63));
  return wave_argmax(best);
}

// Token race over chunk c of row g whose raw logits are in LDS (zs, token
// order): weights exp2(fma(z', a, -hi)) on the processed z' (hi = a r_c; a
// factor common to the chunk cancels), token `skip` left out.  Thread t < 256
// takes tokens 4t..4t+3 (one Philox block); further threads of a larger
// workgroup only join the reduction.  All threads call it; -1 if no token has
// weight.
__device__ __forceinline__ int block_token_race(const Params &p, int g, int c, const float *zs, const Proc &pr,
                                                float a, float hi, int skip, BlockScratch &red,
                                                uint32_t tag = kTagToken) {
  ArgMax best{-1.0f, 0x7FFFFFFF};
  if (threadIdx.x < kThreads) {
    const int t4 = 4 * threadIdx.x;
    const int x0 = c * kChunk + t4;
    const uint4 w4 = rng_block(p, (uint32_t)x0 >> 2, (uint32_t)g, tag);
    const float4 z4 = *reinterpret_cast<const float4 *>(zs + t4);
    const float zz[4] = {z4.x, z4.y, z4.z, z4.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int x = x0 + k;
      const bool ok = x < p.V && x != skip;
      const float wx = ok ? exp2_acc(__builtin_fmaf(apply_proc(zz[k], min(x, p.V - 1), pr), a, -hi)) : 0.0f;
      const ArgMax o{race_score(wx, pick(w4, k)), x};
      if (wx > 0.0f && better(o, best)) best = o;
    }
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
  if (c1 >= 0) load_chunk16_pen(p, g, c1, pr, rs.zc);
  if (excl) load_chunk16_pen(p, g, rs.cd, pr, rs.zx);
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

// PLAIN: the call has no top-k, top-p, penalties or draft distributions and
// at most four rows per request; the settings they would read are then
// constants, and their paths compile away.
template <bool PLAIN, class SH>
__device__ __forceinline__ void request_epilogue(const Params &p, const Req &q_in, SH &sh) {
  constexpr int TC = SH::kCache;
  Req q = q_in;
  if (PLAIN) {
    q.proc.counts = nullptr;
    q.proc.theta = 1.0f;
    q.proc.freq = 0.0f;
    q.proc.pres = 0.0f;
    q.proc.tau = kNegInf;
    q.has_q = false;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = q.K, r = q.r, nrow = K + 1;

  if (!q.cu_ok || p.cu[0] != 0 || p.cu[p.B] != p.D) {
    if (tid == 0) raise_err(p, SV_ERR_CU);
    write_empty(p, r);
    return;
  }
  // The plain variant also runs only with at most four rows per request
  // (cu_ok bounds K by out_stride - 1): every row has a wave of its own.
  if (PLAIN) __builtin_assume(nrow <= kWaves);
  if (q.mode == kModeInvalid) {
    if (tid == 0) raise_err(p, q.errbits);
    write_empty(p, r);
    return;
  }
  const bool greedy = q.mode == kModeGreedy;

  // Row states (top-k pass results), draft ids and the chunk tables.
  for (int i = tid; i < nrow; i += kThreads) {
    const int g = q.g0 + i;
    const int st = PLAIN ? kRowDense : row_state(p, g);
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
    const int st = PLAIN ? kRowDense : sh.state[i];
    const int d = sh.d[i];
    auto ent = [&](int c) { return entry(i, c); };
    float m, s;
    int lc;
    row_stats(p, q, g, st, greedy, ent, m, s, lc);
    Proc pr = q.proc;
    pr.tau = PLAIN ? kNegInf : sh.tau[i];
    int am = 0x7FFFFFFF;
    float zd = kNegInf, qd = 1.0f, sx = 0.0f;
    const bool valid_d = i < K && d >= 0 && d < p.V;
    if (st < 0 && greedy) {
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
    if (lane == 0) {
      sh.m[i] = m;
      sh.s[i] = s;
      sh.amax[i] = am;
      sh.zd[i] = zd;
      sh.qd[i] = qd;
      sh.sx[i] = sx;
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
      if (p.synthetic) {
        // Synthetic acceptance: u * a_i <= a_{i+1} with a_0 = 1, exact in fp64.
        const double u = u_accept(rng_block(p, 0, (uint32_t)g, kTagAccept).x);
        const double prev = lane == 0 ? 1.0 : (double)p.syn[lane - 1];
        rej = !(d >= 0 && d < p.V && u * prev <= (double)p.syn[lane]);
        if (p.dbg_p_draft) {
          const bool valid = d >= 0 && d < p.V;
          p.dbg_p_draft[q.c0 + lane] = greedy ? -1.0f : (valid ? exp2_acc(q.a * (sh.zd[lane] - sh.m[lane])) / sh.s[lane] : 0.0f);
        }
      } else if (greedy) {
        rej = d != sh.amax[lane];
        if (p.dbg_p_draft) p.dbg_p_draft[q.c0 + lane] = -1.0f;
      } else {
        const bool valid = d >= 0 && d < p.V;
        float pd = 0.0f;
        double qd = q.has_q ? 0.0 : 1.0;
        if (valid) {
          pd = exp2_acc(q.a * (sh.zd[lane] - sh.m[lane])) / sh.s[lane];
          if (q.has_q) qd = (double)sh.qd[lane];
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
  pr.tau = PLAIN ? kNegInf : sh.tau[j];
  const int st = PLAIN ? kRowDense : sh.state[j];
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
  float a, theta, freq, pres, tau;
  const int32_t *counts;
};
// Rows a stats pass streams: dense rows, or on the second pass of a top-p
// call only the rows whose tables the top-p pass left to it.
__device__ __forceinline__ bool stream_state(const Params &p, int st) { return p.pass2 ? st == kRowTopPRedo : st < 0; }
constexpr int kRowCache = kSliceRows;  // rows of a slice looked up before streaming
// Chunks in flight per wave in the fast pass: bf16 rows 4 (with eight-wave
// workgroups, 2, 3, 5 and 6 measured 30.4, 28.5, 29.3 and 29.5 us against
// 28.0 on the 164 MB headline batch; 6 no longer fits 8 waves per SIMD),
// fp32 rows 3 (16 registers per chunk in flight instead of 8); 3 with penalties
// (at 4 the counts' registers leave one workgroup per CU instead of two).
template <int DT>
constexpr int kFastDepth = DT == 1 ? 4 : 3;
// Waves per workgroup of the fast pass: eight (two per SIMD) for bf16 rows
// without penalties, where halving the number of workgroups against four
// measured about 4 % faster; four otherwise (fp32 rows and the penalty variant
// measured about 1 % slower with eight).
template <int DT, bool PEN>
constexpr int kFastWaves = (DT == 1 && !PEN) ? 8 : 4;
template <int DT, bool PEN>
constexpr int kFastThreads = 64 * kFastWaves<DT, PEN>;
static_assert(kRowCache <= 4, "one wave looks up each row of a slice");

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
  ri.freq = q.proc.freq;
  ri.pres = q.proc.pres;
  ri.counts = q.proc.counts;
  ri.tau = (ok && row_has_tau(ri.st)) ? p.cand_tau[g] : kNegInf;
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
  pr.freq = ri.freq;
  pr.pres = ri.pres;
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
  if (cur.mode != kModeInvalid && stream_state(p, cur.st)) chunk_stats<DT>(p, cur, c, v);
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
  y.freq = uni(x.freq);
  y.pres = uni(x.pres);
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

  // Request lookups for the slice's rows first: rows that are not streamed
  // (invalid requests, compact top-k rows raced over their candidate lists)
  // issue no loads at all.
  if (wave < min(nrows, kRowCache)) {
    const int g = g_first + wave;
    const RowInfo ri = row_info_of(p, lookup_req(p, g), g);
    if (lane == 0) sh.rows[wave] = ri;
  }
  __syncthreads();
  auto streamed = [&](int64_t ff) {
    if (ff >= end) return false;
    const int gi = (int)(ff / p.NC) - g_first;
    return gi >= kRowCache || (sh.rows[gi].mode != kModeInvalid && stream_state(p, sh.rows[gi].st));
  };
  {
    bool any = false;
    for (int i = 0; i < min(nrows, kRowCache); ++i) any |= sh.rows[i].mode != kModeInvalid && stream_state(p, sh.rows[i].st);
    if (!any && nrows <= kRowCache) return;
  }

  // Three chunks in flight per wave.
  u32x4 A[NV], Bv[NV], Cv[NV];
  int64_t f = start + wave;
  issue_chunk<DT>(p, f, streamed(f) ? end : f, A);
  issue_chunk<DT>(p, f + kWaves, streamed(f + kWaves) ? end : f, Bv);
  issue_chunk<DT>(p, f + 2 * kWaves, streamed(f + 2 * kWaves) ? end : f, Cv);

  RowInfo cur;
  cur.g = -1;
  for (; f < end; f += 3 * kWaves) {
    process_chunk<DT>(p, f, A, cur, sh.rows, g_first);
    issue_chunk<DT>(p, f + 3 * kWaves, streamed(f + 3 * kWaves) ? end : f, A);
    if (f + kWaves >= end) break;
    process_chunk<DT>(p, f + kWaves, Bv, cur, sh.rows, g_first);
    issue_chunk<DT>(p, f + 4 * kWaves, streamed(f + 4 * kWaves) ? end : f, Bv);
    if (f + 2 * kWaves >= end) break;
    process_chunk<DT>(p, f + 2 * kWaves, Cv, cur, sh.rows, g_first);
    issue_chunk<DT>(p, f + 5 * kWaves, streamed(f + 5 * kWaves) ? end : f, Cv);
  }

}

// ---------------------------------------------------------------------------
// Fast streaming pass: aligned rows, V a multiple of the vector width, no
// top-k (the common case, and the no-draft-probs workload); the PEN variant
// also loads each token's output count with the logits (16-byte vectors of
// four counts) and applies the penalties.
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

// The counts of this lane's 16 tokens of chunk c (rows whose request has a
// penalty): four 16-byte vectors; vectors past V read the row start (masked).
template <int DT>
__device__ __forceinline__ void fast_load_counts(const Params &p, const int32_t *crow, int c, int4 (&cv)[4]) {
  using L = Layout<DT>;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int x = c * kChunk + L::local(4 * h, lane);  // tokens 4h .. 4h+3 of the lane are consecutive
    const uint32_t off = x + 4 <= p.V ? (uint32_t)x * 4u : 0u;
    cv[h] = *reinterpret_cast<const int4 *>(reinterpret_cast<const char *>(crow) + off);
  }
}

__device__ __forceinline__ void advance_chunk(int &g, int &c, int by, int NC) {
  c += by;
  while (c >= NC) {
    c -= NC;
    ++g;
  }
}

// Table entry of one chunk: (r, sum over its tokens of exp2(a (z - r))).  For
// a sampled row the reference r is the exact maximum of the first chunk of
// the row that this wave streamed (`ref`); later chunks then need only the
// sum, unless it reaches 2^20, in which case their exact maximum is taken and
// becomes the reference.  With m = max over the row's entries of r,
// a (z - m) <= 20 for every token, so every later use stays finite, and the
// exponent of each term is rounded with an absolute error of at most
// 20 * 2^-24.  Greedy rows (a = 0) always take the exact maximum: their
// argmax search needs it.
template <int DT, bool PEN>
__device__ __forceinline__ void fast_chunk(const Params &p, const RowInfo &ri, int c,
                                           const u32x4 (&v)[Layout<DT>::kVec], const int4 (&cv)[4], float &ref) {
  using L = Layout<DT>;
  const int lane = threadIdx.x & 63;
  float z[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) z[e] = L::elem(v, e);
  if (PEN && ri.counts != nullptr) {
    // Penalties of the tokens seen (count > 0), as apply_proc; the division
    // only when the repetition penalty is not 1.
    Proc pr;
    pr.theta = ri.theta;
    pr.freq = ri.freq;
    pr.pres = ri.pres;
    const bool rep = ri.theta != 1.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int4 q4 = cv[e >> 2];
      const int cnt = (e & 3) == 0 ? q4.x : (e & 3) == 1 ? q4.y : (e & 3) == 2 ? q4.z : q4.w;
      float zp = rep ? (z[e] > 0.0f ? z[e] / pr.theta : z[e] * pr.theta) : z[e];
      zp = zp - pr.freq * (float)cnt;
      zp = zp - pr.pres;
      z[e] = cnt > 0 ? zp : z[e];
    }
  }
  if ((c + 1) * kChunk > p.V) {  // row tail: tokens past V do not exist
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (c * kChunk + L::local(e, lane) >= p.V) z[e] = kNegInf;
  }
  const float a = ri.a;
  float2 entry;
  bool done = false;
  if (ref > kNegInf) {
    // exp2(a (z - r)) = exp2(fma(z, a, -hi)) * exp2(-lo), a * r = hi + lo exactly
    const float hi = a * ref, lo = __builtin_fmaf(a, ref, -hi);
    float sa = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) sa += exp2_acc(__builtin_fmaf(z[e], a, -hi));
    const float sr = wave_sum(sa);
    entry = make_float2(ref, sr * exp2_acc(-lo));
    done = sr < 0x1p20f;
  }
  if (!done) {
    float mx = z[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, z[e]);
    const float mc = wave_max(mx);
    const float hi = a * mc, lo = __builtin_fmaf(a, mc, -hi);
    float sa = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) sa += exp2_acc(__builtin_fmaf(z[e], a, -hi));
    entry = make_float2(mc, mc > kNegInf ? wave_sum(sa) * exp2_acc(-lo) : 0.0f);
    if (a > 0.0f) ref = mc;
  }
  if (lane == 0 && ri.mode != kModeInvalid) p.chunk_tab[(int64_t)ri.g * p.nc_stride + c] = entry;
}

template <int DT, bool PEN>
__global__ __launch_bounds__((kFastThreads<DT, PEN>)) void stats_fast_kernel(Params p) {
  constexpr int NW = kFastWaves<DT, PEN>;
  // Items in (request, chunk, row) order: the bf16 penalty variant (for fp32
  // rows its registers would cost a wave per SIMD).
  constexpr bool RQ = PEN && DT == 1;
  using L = Layout<DT>;
  constexpr int NV = L::kVec;
  constexpr int D = PEN ? 3 : kFastDepth<DT>;  // chunks in flight per wave (the counts take registers too)
  __shared__ StatsShared sh;
  const int wave = uni((int)(threadIdx.x >> 6));
  const int N = p.R * p.NC;
  const int start = (int)((int64_t)blockIdx.x * N / gridDim.x);
  const int end = (int)((int64_t)(blockIdx.x + 1) * N / gridDim.x);
  if (start >= end) return;
  const int g_first = start / p.NC, g_last = (end - 1) / p.NC;
  const int nrows = g_last - g_first + 1;
  const int len = end - start;
  const int n = wave < len ? (len - wave + NW - 1) / NW : 0;

  // The first D loads are unconditional (a wave with fewer chunks reads the
  // slice's first chunk instead), so that every path into the loop has the
  // same loads in flight and the waits stay D chunks deep.
  u32x4 buf[D][NV];
  int4 cb[D][4];
  int gs[D], cs[D];
  int xs[D], js[D];  // penalty variant: item index, and the slice row whose request holds it
  if (!RQ) {
    gs[0] = (start + wave) / p.NC;
    cs[0] = start + wave - gs[0] * p.NC;
#pragma unroll
    for (int s = 1; s < D; ++s) {
      gs[s] = gs[s - 1];
      cs[s] = cs[s - 1];
      advance_chunk(gs[s], cs[s], NW, p.NC);
    }
    if (!PEN) {
#pragma unroll
      for (int s = 0; s < D; ++s) fast_load<DT>(p, n > s ? gs[s] : g_first, n > s ? cs[s] : 0, buf[s]);
    }
  }

  // Request lookups for the slice's rows (overlapping the loads).
  if (wave < nrows) {
    const int g = g_first + wave;
    const RowInfo ri = row_info_of(p, lookup_req(p, g), g);
    if ((threadIdx.x & 63) == 0) sh.rows[wave] = ri;
  }
  __syncthreads();

  // Penalty variant: the counts rows of the slice's requests (a valid address
  // for rows without one), and the items in (request, chunk, row) order.  The
  // R NC items keep their ranges per request (request r owns [g0 NC,
  // (g0 + K + 1) NC) either way), but inside a request its rows' chunk c are
  // consecutive items: the waves of a workgroup stream chunk c of the
  // request's rows together, and the request's counts chunk c, the same for
  // each row, is fetched from memory once and found in L2 by the others.
  const int32_t *crow[kRowCache];
  int g0s[kRowCache], k1s[kRowCache];
  bool oks[kRowCache];
  if (PEN) {
#pragma unroll
    for (int i = 0; i < kRowCache; ++i) {
      const RowInfo x = uniform_row(sh.rows[i < nrows ? i : 0]);
      crow[i] = x.counts != nullptr ? x.counts : p.counts;
      g0s[i] = x.g0;
      k1s[i] = x.K + 1;
      oks[i] = x.mode != kModeInvalid;
    }
  }
  // Item x: row g, chunk c, and the slice row j whose request holds it (rows
  // of an invalid request keep the row order).
  auto place = [&](int x, int &g, int &c, int &j) {
    const int gr = uni(x / p.NC);
    j = gr - g_first;
    int g0 = g0s[0], k1 = k1s[0];
    bool ok = oks[0];  // (all uniform)
#pragma unroll
    for (int i = 1; i < kRowCache; ++i)
      if (j == i) {
        g0 = g0s[i];
        k1 = k1s[i];
        ok = oks[i];
      }
    if (!ok) {
      g = gr;
      c = x - gr * p.NC;
      return;
    }
    const int l = x - g0 * p.NC;
    c = uni(l / k1);
    g = uni(g0 + (l - c * k1));
  };
  auto load = [&](int s, int g, int c) {
    fast_load<DT>(p, g, c, buf[s]);
    if (PEN) {
      const int32_t *cr = crow[0];
#pragma unroll
      for (int i = 1; i < kRowCache; ++i) cr = (RQ ? js[s] : g - g_first) == i ? crow[i] : cr;
      fast_load_counts<DT>(p, cr, c, cb[s]);
    }
  };
  if (RQ) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      xs[s] = uni(start + wave + s * NW);
      if (n > s) {
        place(xs[s], gs[s], cs[s], js[s]);
      } else {
        gs[s] = g_first;
        cs[s] = 0;
        js[s] = 0;
      }
      load(s, gs[s], cs[s]);
    }
  } else if (PEN) {
#pragma unroll
    for (int s = 0; s < D; ++s) load(s, n > s ? gs[s] : g_first, n > s ? cs[s] : 0);
  }

  RowInfo cur = uniform_row(sh.rows[RQ ? js[0] : (n > 0 ? gs[0] - g_first : 0)]);  // a wave without chunks may start past the slice
  float ref = kNegInf;  // this wave's reference for row cur.g (uniform)
  // Penalty variant: a wave's references for up to four rows (its items move
  // between the rows of a request), slot g & 3.
  int rg[4] = {-1, -1, -1, -1};
  float rv[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
  auto chunk = [&](int s) {
    if (RQ) {
      cur = uniform_row(sh.rows[js[s]]);
      cur.g = gs[s];
      const int q = gs[s] & 3;
      ref = kNegInf;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (q == i && rg[i] == gs[s]) ref = rv[i];
      fast_chunk<DT, PEN>(p, cur, cs[s], buf[s], cb[s], ref);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (q == i) {
          rg[i] = gs[s];
          rv[i] = uni(ref);
        }
      return;
    }
    if (gs[s] != cur.g) {
      cur = uniform_row(sh.rows[gs[s] - g_first]);
      ref = kNegInf;
    }
    fast_chunk<DT, PEN>(p, cur, cs[s], buf[s], cb[s], ref);
  };
  auto advance = [&](int s) {
    if (RQ) {
      xs[s] = uni(xs[s] + D * NW);
      place(xs[s], gs[s], cs[s], js[s]);
    } else {
      advance_chunk(gs[s], cs[s], D * NW, p.NC);
    }
  };
  int k = 0;
  for (; k + 2 * D - 1 < n; k += D) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      chunk(s);
      advance(s);
      load(s, gs[s], cs[s]);
    }
  }
  // Drain: at most 2D - 1 chunks left, loads only while in range.
#pragma unroll
  for (int t = 0; t < 2 * D; ++t) {
    if (k + t >= n) break;
    const int s = t % D;
    chunk(s);
    if (k + t + D < n) {
      advance(s);
      load(s, gs[s], cs[s]);
    }
  }

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
template <bool PLAIN>
__global__ __launch_bounds__(kThreads) void epilogue_kernel(Params p) {
  __shared__ EpiShared sh;
  request_epilogue<PLAIN>(p, load_req(p, blockIdx.x), sh);
}

// ---------------------------------------------------------------------------
// Top-k pass: one workgroup per row.
// ---------------------------------------------------------------------------
constexpr int kBuf = 2048;   // LDS candidate buffer

struct TopkShared {
  float bv[kBuf];
  int bi[kBuf];
  unsigned hist[256];
  int n;
  int tile_n[2];  // passers of the current super-tile (by parity: one is reset while the other counts)
  int sel, want;
  float theta;
  BlockScratch red;
};
static_assert(kBuf >= 2 * kCandCap, "the id-ordered kept list is staged in the upper half of the buffer");

// Super-tile of the top-k filter: thread t holds kTopkPer tokens, as
// kTopkPer / VW vectors of VW tokens (VW = 4 fp32, 8 bf16) at
// base + (v kThreads + t) VW + w.
constexpr int kTopkPer = 16;
constexpr int kTopkTile = kTopkPer * kThreads;
template <int DT, int NT = kThreads>
__device__ __forceinline__ int topk_tok(int base, int e) {
  constexpr int VW = DT == 1 ? 8 : 4;
  return base + ((e / VW) * NT + (int)threadIdx.x) * VW + (e % VW);
}
template <int DT, int NPER = kTopkPer>
__device__ __forceinline__ void load_topk_tile(const Params &p, int g, int base, float (&z)[NPER]) {
  constexpr int VW = DT == 1 ? 8 : 4;
  static_assert(NPER % VW == 0, "whole vectors per thread");
  if (p.vec_ok) {
    const char *row = static_cast<const char *>(p.logits) + (int64_t)g * p.lstride * (DT == 1 ? 2 : 4);
#pragma unroll
    for (int v = 0; v < NPER / VW; ++v) {
      const int x0 = topk_tok<DT>(base, v * VW);
      const int xs = x0 + VW <= p.V ? x0 : 0;  // a vector past the row end reads the row start (masked)
      const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(row + (int64_t)xs * (DT == 1 ? 2 : 4)));
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < VW; ++i) {
        float val;
        if (DT == 1)
          val = (i & 1) ? __uint_as_float(ww[i >> 1] & 0xFFFF0000u) : __uint_as_float(ww[i >> 1] << 16);
        else
          val = __uint_as_float(ww[i]);
        z[v * VW + i] = x0 + VW <= p.V ? val : (x0 + i < p.V ? load_logit(p, g, x0 + i) : kNegInf);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < NPER; ++e) {
      const int x = topk_tok<DT>(base, e);
      z[e] = x < p.V ? load_logit(p, g, x) : kNegInf;
    }
  }
}

// Order-preserving map float -> uint32 (larger float, larger key).
__device__ __forceinline__ uint32_t ukey(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ukey_val(uint32_t k) { return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k); }

// One MSD radix digit: among keys matching (prefix, mask), find the digit at
// `shift` holding the want-th largest; updates prefix/mask/want (uniform).
__device__ __forceinline__ void radix_digit(TopkShared &sh, int shift, uint32_t &prefix, uint32_t &mask, int &want) {
  // Wave 0 finds the digit: lane l holds bins 255-4l .. 252-4l (descending),
  // an inclusive prefix sum over lanes gives the count of larger digits.
  if (threadIdx.x < 64) {
    const int l = threadIdx.x;
    const int h0 = (int)sh.hist[255 - 4 * l], h1 = (int)sh.hist[254 - 4 * l];
    const int h2 = (int)sh.hist[253 - 4 * l], h3 = (int)sh.hist[252 - 4 * l];
    const int own = h0 + h1 + h2 + h3;
    int incl = own;  // inclusive scan over lanes (Hillis-Steele with shuffles)
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      if (l >= d) incl += o;
    }
    const int before = incl - own;  // count in bins above this lane's four
    const bool here = before < want && incl >= want;
    if (here) {
      int acc = before, b = 255 - 4 * l;
      const int hh[4] = {h0, h1, h2, h3};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (acc + hh[i] >= want) {
          b = 255 - 4 * l - i;
          break;
        }
        acc += hh[i];
      }
      sh.sel = b;
      sh.want = want - acc;
    }
  }
  __syncthreads();
  prefix |= (uint32_t)sh.sel << shift;
  mask |= 0xFFu << shift;
  want = sh.want;
  __syncthreads();
}

// Pipelined form of the super-tile load for aligned rows: the raw 16-byte
// vectors are issued unconditionally (a vector not wholly inside [0, vfull)
// reads the row start) and decoded later; tokens in [vfull, V) are handled
// apart, after the loop.
template <int DT>
struct TopkRaw {
  static constexpr int VW = DT == 1 ? 8 : 4;
  u32x4 v[kTopkPer / VW];
};
template <int DT, int NT = kThreads>
__device__ __forceinline__ void topk_issue(const Params &p, int g, int base, int vfull, TopkRaw<DT> &r) {
  constexpr int VW = TopkRaw<DT>::VW;
  const char *row = static_cast<const char *>(p.logits) + (int64_t)g * p.lstride * (DT == 1 ? 2 : 4);
#pragma unroll
  for (int v = 0; v < kTopkPer / VW; ++v) {
    const int x0 = topk_tok<DT, NT>(base, v * VW);
    const uint32_t off = x0 + VW <= vfull ? (uint32_t)x0 * (DT == 1 ? 2u : 4u) : 0u;
    r.v[v] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(row + off));
  }
}
template <int DT, int NT = kThreads>
__device__ __forceinline__ void topk_decode(int base, int vfull, const TopkRaw<DT> &r, float (&z)[kTopkPer]) {
  constexpr int VW = TopkRaw<DT>::VW;
#pragma unroll
  for (int v = 0; v < kTopkPer / VW; ++v) {
    const int x0 = topk_tok<DT, NT>(base, v * VW);
    const uint32_t ww[4] = {r.v[v].x, r.v[v].y, r.v[v].z, r.v[v].w};
#pragma unroll
    for (int i = 0; i < VW; ++i) {
      const float val = DT == 1 ? ((i & 1) ? __uint_as_float(ww[i >> 1] & 0xFFFF0000u) : __uint_as_float(ww[i >> 1] << 16))
                                : __uint_as_float(ww[i]);
      z[v * VW + i] = x0 + VW <= vfull ? val : kNegInf;
    }
  }
}

// Repetition penalty on a whole super-tile held in z (raw logits): the counts
// of all its tokens are loaded together (one round trip per 8).
template <int DT, int NPER = kTopkPer>
__device__ __forceinline__ void penalize_tile(const Params &p, const Proc &pr, int base, float (&z)[NPER]) {
#pragma unroll
  for (int e0 = 0; e0 < NPER; e0 += 8) {
    int c[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) c[e] = pr.counts[min(topk_tok<DT>(base, e0 + e), p.V - 1)];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int x = topk_tok<DT>(base, e0 + e);
      if (x < p.V && c[e] > 0) z[e0 + e] = penalize(z[e0 + e], c[e], pr);
    }
  }
}

// Candidates appended with their raw logit (penalty still to apply) carry
// index | kUnresolved.  Applies the penalty to every such entry.
constexpr int kUnresolved = (int)0x80000000;
__device__ __forceinline__ void resolve_buffer(TopkShared &sh, int n, const Proc &pr) {
  for (int e = threadIdx.x; e < n; e += kThreads) {
    const int xi = sh.bi[e];
    if (xi & kUnresolved) {
      const int x = xi & 0x7FFFFFFF;
      float z = sh.bv[e];
      const int c = pr.counts[x];
      if (c > 0) z = penalize(z, c, pr);
      sh.bv[e] = z;
      sh.bi[e] = x;
    }
  }
  __syncthreads();
}

// k-th largest value among sh.bv[0..n) (1 <= k <= n).
__device__ __forceinline__ float buffer_kth(TopkShared &sh, int n, int k) {
  uint32_t prefix = 0, mask = 0;
  int want = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    sh.hist[threadIdx.x] = 0;
    __syncthreads();
    for (int e = threadIdx.x; e < n; e += kThreads) {
      const uint32_t key = ukey(sh.bv[e]);
      if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 0xFFu], 1u);
    }
    __syncthreads();
    radix_digit(sh, shift, prefix, mask, want);
  }
  return ukey_val(prefix);
}

// In-place compaction of the candidate buffer: keeps entry e < n when
// keep(value, index) holds, and sets sh.n.  Each thread reads its entries into
// registers (fixed slots, no dynamic indexing), then appends the kept ones.
template <class KEEP>
__device__ __forceinline__ void buffer_compact(TopkShared &sh, int n, KEEP keep) {
  float kv[kBuf / kThreads];
  int ki[kBuf / kThreads];
  bool kk[kBuf / kThreads];
#pragma unroll
  for (int m = 0; m < kBuf / kThreads; ++m) {
    const int e = threadIdx.x + m * kThreads;
    kv[m] = e < n ? sh.bv[e] : 0.0f;
    ki[m] = e < n ? sh.bi[e] : -1;
    kk[m] = e < n && keep(kv[m], ki[m]);
  }
  __syncthreads();
  if (threadIdx.x == 0) sh.n = 0;
  __syncthreads();
#pragma unroll
  for (int m = 0; m < kBuf / kThreads; ++m) {
    if (kk[m]) {
      const int pos = atomicAdd(&sh.n, 1);
      sh.bv[pos] = kv[m];
      sh.bi[pos] = ki[m];
    }
  }
  __syncthreads();
}
// Keep the buffer entries >= t (order not preserved).
__device__ __forceinline__ void buffer_keep(TopkShared &sh, int n, float t) {
  buffer_compact(sh, n, [t](float v, int) { return v >= t; });
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
    sh.tile_n[0] = sh.tile_n[1] = 0;
  }
  __syncthreads();
  // Streaming filter in super-tiles of kTopkTile tokens, kTopkPer per thread
  // (vector loads, all in flight together).  A token passes when its processed
  // logit is >= the running threshold theta (a lower bound of tau_k: the k-th
  // largest of a subset of the row).  With a repetition penalty >= 1 and
  // frequency and presence penalties >= 0 the penalties never raise a logit
  // (each step rounds monotonically), so later super-tiles test the raw logit and the counts
  // of the few passers are read only when a selection needs them.  Two barriers
  // per super-tile: one to count the passers (compacting the candidate buffer
  // first if they would not fit), one after they are appended.
  const bool pen = pr.counts != nullptr;
  const bool raw_first = !pen || (pr.theta >= 1.0f && pr.freq >= 0.0f && pr.pres >= 0.0f);
  bool overflow = k > kCandCap;
  constexpr int kFirstPer = kBuf / kThreads;  // the first kBuf tokens are all kept
  if (!overflow) {
    float z[kFirstPer];
    load_topk_tile<DT, kFirstPer>(p, g, 0, z);
    if (pen) penalize_tile<DT, kFirstPer>(p, pr, 0, z);
#pragma unroll
    for (int e = 0; e < kFirstPer; ++e) {
      const int x = topk_tok<DT>(0, e);
      sh.bv[threadIdx.x * kFirstPer + e] = z[e];
      sh.bi[threadIdx.x * kFirstPer + e] = x < p.V && z[e] > kNegInf ? x : -1;
    }
    __syncthreads();
    // compact the finite entries, then theta = their k-th largest
    buffer_compact(sh, kBuf, [](float, int x) { return x >= 0; });
    const int n = sh.n;
    if (n >= k) {
      const float t = buffer_kth(sh, n, k);
      buffer_keep(sh, n, t);
      if (threadIdx.x == 0) sh.theta = t;
    }
    __syncthreads();
  }
  // One super-tile: filter z (raw logits) against theta, count the passers,
  // make room if needed, append them.  All threads call it (barriers inside).
  auto tile_step = [&](int base, int par, float (&z)[kTopkPer]) {
    // sh.n and sh.theta last changed before the previous super-tile's final
    // barrier: every thread reads the same values here.
    const int n0 = sh.n;
    const float th = sh.theta;
    if (!raw_first) penalize_tile<DT>(p, pr, base, z);  // a penalty < 1 can raise logits: test processed ones
    int npass = 0;
#pragma unroll
    for (int e = 0; e < kTopkPer; ++e) {
      const int x = topk_tok<DT>(base, e);
      z[e] = (x < p.V && z[e] >= th && z[e] > kNegInf) ? z[e] : kNegInf;
      npass += z[e] > kNegInf ? 1 : 0;
    }
    if (npass) atomicAdd(&sh.tile_n[par], npass);
    __syncthreads();
    if (threadIdx.x == 0) sh.tile_n[par ^ 1] = 0;  // read last in the previous super-tile
    if (n0 + sh.tile_n[par] > kBuf) {
      // Not enough room: theta becomes the k-th largest kept candidate
      // (penalties applied first); this super-tile's passers are re-tested.
      if (n0 < k) {
        overflow = true;  // fewer than k finite logits so far and a full tile: exact radix select below
      } else {
        if (pen) resolve_buffer(sh, n0, pr);
        const float t = buffer_kth(sh, n0, k);
        buffer_keep(sh, n0, t);
        if (threadIdx.x == 0) {
          sh.theta = t;
          sh.tile_n[par] = 0;
        }
        __syncthreads();
        npass = 0;
#pragma unroll
        for (int e = 0; e < kTopkPer; ++e) {
          if (!(z[e] >= t)) z[e] = kNegInf;
          npass += z[e] > kNegInf ? 1 : 0;
        }
        if (npass) atomicAdd(&sh.tile_n[par], npass);
        __syncthreads();
        const bool full = sh.n + sh.tile_n[par] > kBuf;  // ties at theta: exact radix select below
        __syncthreads();  // every thread has read the counts before anyone appends
        overflow = full;
      }
    }
    if (overflow) return;
    const int flag = raw_first && pen ? kUnresolved : 0;  // raw logits: penalty applied at the next selection
#pragma unroll
    for (int e = 0; e < kTopkPer; ++e) {
      if (z[e] > kNegInf) {
        const int pos = atomicAdd(&sh.n, 1);
        sh.bv[pos] = z[e];
        sh.bi[pos] = topk_tok<DT>(base, e) | flag;
      }
    }
    __syncthreads();
  };
  if (p.vec_ok) {
    // Two super-tiles in flight: the next one's loads are issued before this
    // one is filtered.
    constexpr int VW = TopkRaw<DT>::VW;
    const int vfull = p.V - p.V % VW;
    TopkRaw<DT> ra, rb;
    int base = kBuf, par = 0;
    topk_issue<DT>(p, g, base, vfull, ra);
    topk_issue<DT>(p, g, base + kTopkTile, vfull, rb);
    while (base < vfull && !overflow) {
      float z[kTopkPer];
      topk_decode<DT>(base, vfull, ra, z);
      topk_issue<DT>(p, g, base + 2 * kTopkTile, vfull, ra);
      tile_step(base, par, z);
      base += kTopkTile;
      par ^= 1;
      if (base >= vfull || overflow) break;
      topk_decode<DT>(base, vfull, rb, z);
      topk_issue<DT>(p, g, base + 2 * kTopkTile, vfull, rb);
      tile_step(base, par, z);
      base += kTopkTile;
      par ^= 1;
    }
    if (!overflow && vfull < p.V) {  // the last V % VW tokens, penalty applied at once
      if (sh.n > kBuf - VW) {  // make room (n >= k here: k <= kCandCap < kBuf - VW)
        const int n = sh.n;
        if (pen) resolve_buffer(sh, n, pr);
        const float t = buffer_kth(sh, n, k);
        buffer_keep(sh, n, t);
        if (threadIdx.x == 0) sh.theta = t;
        __syncthreads();
      }
      const int x = vfull + (int)threadIdx.x;
      if (x < p.V) {
        const float z = apply_proc(load_logit(p, g, x), x, pr);
        if (z >= sh.theta && z > kNegInf) {
          const int pos = atomicAdd(&sh.n, 1);
          sh.bv[pos] = z;
          sh.bi[pos] = x;
        }
      }
      __syncthreads();
    }
  } else {
    for (int base = kBuf, par = 0; base < p.V && !overflow; base += kTopkTile, par ^= 1) {
      float z[kTopkPer];
      load_topk_tile<DT>(p, g, base, z);
      tile_step(base, par, z);
    }
  }
  if (pen && !overflow) resolve_buffer(sh, sh.n, pr);

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
        const uint32_t key = ukey(apply_proc(load_logit(p, g, x), x, pr));
        if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 0xFFu], 1u);
      }
      __syncthreads();
      radix_digit(sh, shift, prefix, mask, want);
    }
    tau = ukey_val(prefix);
  }

  if (ncand < 0 || ncand > kCandCap) {
    if (threadIdx.x == 0) {
      p.cand_n[g] = (tau > kNegInf) ? kRowThreshold : kRowDense;
      p.cand_tau[g] = tau;
    }
    return;
  }

  // The kept tokens in increasing id order, staged in the upper half of the
  // buffer: each one's position is the number of kept tokens with a smaller id
  // (ids are distinct).
  float *sv_ = sh.bv + kCandCap;
  int *si_ = sh.bi + kCandCap;
  for (int e = threadIdx.x; e < ncand; e += kThreads) {
    const int id = sh.bi[e];
    int rank = 0;
    for (int t = 0; t < ncand; ++t) rank += sh.bi[t] < id ? 1 : 0;
    sv_[rank] = sh.bv[e];
    si_[rank] = id;
  }
  __syncthreads();
  int nout = ncand;
  if (q.top_p < 1.0f) {
    // Top-p over the candidates, which hold the whole top-k distribution:
    // weights w = exp2(a (z - m)), S = sum w; token e stays iff the weight of
    // the tokens with a larger logit is below top_p * S.  Sums run in id order
    // (fixed, so the result replays bit for bit).  sh.bi[0..ncand) then holds
    // the kept flags.
    float lm = kNegInf;
    for (int e = threadIdx.x; e < ncand; e += kThreads) lm = fmaxf(lm, sv_[e]);
    const float m = block_max(lm, sh.red);
    const float a = q.a;
    float ls = 0.0f;
    for (int e = threadIdx.x; e < ncand; e += kThreads) ls += exp2_acc(a * (sv_[e] - m));
    const float bound = q.top_p * block_sum(ls, sh.red);
    for (int e = threadIdx.x; e < ncand; e += kThreads) {
      const float ze = sv_[e];
      float above = 0.0f;
      for (int t = 0; t < ncand; ++t)
        if (sv_[t] > ze) above += exp2_acc(a * (sv_[t] - m));
      sh.bi[e] = above < bound ? 1 : 0;
    }
    __syncthreads();
    // The kept set is every token with z >= the smallest kept logit, which is
    // also the row's new threshold for single-token lookups.
    float lt = __builtin_inff();
    for (int e = threadIdx.x; e < ncand; e += kThreads)
      if (sh.bi[e]) lt = fminf(lt, sv_[e]);
    tau = -block_max(-lt, sh.red);
    int pos = 0;
    for (int e = threadIdx.x; e < ncand; e += kThreads) {
      if (sh.bi[e]) {
        pos = 0;
        for (int t = 0; t < e; ++t) pos += sh.bi[t];
        p.cand_val[(int64_t)g * kCandCap + pos] = sv_[e];
        p.cand_idx[(int64_t)g * kCandCap + pos] = si_[e];
      }
    }
    int lk = 0;
    for (int e = threadIdx.x; e < ncand; e += kThreads) lk += sh.bi[e];
    nout = (int)block_sum((float)lk, sh.red);
  } else {
    for (int e = threadIdx.x; e < ncand; e += kThreads) {
      p.cand_val[(int64_t)g * kCandCap + e] = sv_[e];
      p.cand_idx[(int64_t)g * kCandCap + e] = si_[e];
    }
  }
  if (threadIdx.x == 0) {
    p.cand_n[g] = nout;
    p.cand_tau[g] = tau;
  }
}

// ---------------------------------------------------------------------------
// Top-p pass for dense rows (rows without a candidate list), after the first
// statistics pass.  One workgroup per row.  The kept set is every token whose
// strictly larger logits hold less than top_p of the mass: all z >= z* for a
// boundary logit z*, the row's threshold afterwards (cand_tau).
//
// Weights relative to the row scale m: w = 2^-t, t = a (m - z).  A token
// falls in sub-bucket j = floor(16 t) + 320 (clamped to [0, 1024)), of integer
// part k = j / 16 - 20, and one exp2 gives W = 2^(31 - (t - k)), an
// integer-valued float near 2^31: w = W 2^(-31-k) exactly, and sums of W
// within one sub-bucket are exact 64-bit integers (independent of order).
// Pass A: mass per sub-bucket; an fp64 scan in a fixed order finds the
// sub-bucket j* holding the boundary and the mass above it.  Pass B: the
// tokens of j* go to an LDS list, where a radix select on the order-preserving
// keys, weighted by W, finds z*; tokens before j* are summed per chunk, and
// the row's chunk table is rewritten as (m, kept mass): no further pass.  When
// j* holds more tokens than the list, the rows are not 16-byte aligned or the
// row has more chunks than the LDS tables, z* is selected straight from the
// row and the row is left to a second statistics pass (kRowTopPRedo).
// ---------------------------------------------------------------------------
constexpr int kToppSub = 1024;
constexpr int kToppSubOff = 320;  // sub-bucket of t = 0: t >= -20 is covered (a (z - m) <= 20)
constexpr int kToppList = 2048;
constexpr int kToppMaxNC = 512;   // chunks per row whose sums live in LDS (V <= 524288)
// Threads per row: eight waves when most rows are dense (one row per
// workgroup leaves few waves per CU, and the pass is bound by each
// workgroup's own arithmetic: eight waves measured 11 % faster per step on
// 640 dense bf16 rows); four with top-k on, where most rows have candidate
// lists and their workgroups return at once (eight measured 1 % slower there).
constexpr int kTpMaxWaves = 8;

struct ToppShared {
  unsigned long long mass[kToppSub];
  float lz[kToppList];
  int lx[kToppList];
  float part[kToppMaxNC * 4];            // per chunk, one slot per wave covering it
  unsigned long long lsum[kToppMaxNC];   // kept list weights per chunk (integer W)
  float tail[8];
  float wmax[kTpMaxWaves];
  unsigned long long need;
  int n, sel;
};

struct ToppW {
  int j, k;
  float W;  // 2^(31 - (t - k)): an integer-valued float below 2^32
};

// Sub-bucket and weight of logit z, branch-free: z = -inf (t = +inf) lands in
// the last sub-bucket with W = 0.  topp_j is the sub-bucket alone (the same
// operations), for tests that need no weight.
__device__ __forceinline__ int topp_j(float t) {
  const float u = fminf(fmaxf(__builtin_floorf(t * 16.0f), -(float)kToppSubOff), (float)(kToppSub - 1 - kToppSubOff));
  return (int)u + kToppSubOff;
}
__device__ __forceinline__ ToppW topp_w(float z, float m, float a) {
  const float t = (m - z) * a;
  const int j = topp_j(t);
  const int k = (j >> 4) - kToppSubOff / 16;
  return ToppW{j, k, exp2_acc(31.0f - (t - (float)k))};
}

// Calls fn(x, raw logit) for every token of row g (vector loads, two
// super-tiles in flight, when the rows are aligned).  All threads call it.
template <int DT, int NT, class F>
__device__ __forceinline__ void stream_row(const Params &p, int g, F fn) {
  if (p.vec_ok) {
    constexpr int VW = TopkRaw<DT>::VW;
    const int vfull = p.V - p.V % VW;
    TopkRaw<DT> ra, rb;
    int base = 0;
    topk_issue<DT, NT>(p, g, base, vfull, ra);
    topk_issue<DT, NT>(p, g, base + (kTopkPer * NT), vfull, rb);
    while (base < vfull) {
      float z[kTopkPer];
      topk_decode<DT, NT>(base, vfull, ra, z);
      topk_issue<DT, NT>(p, g, base + 2 * (kTopkPer * NT), vfull, ra);
#pragma unroll
      for (int e = 0; e < kTopkPer; ++e) {
        const int x = topk_tok<DT, NT>(base, e);
        if (x < vfull) fn(x, z[e]);
      }
      base += (kTopkPer * NT);
      if (base >= vfull) break;
      topk_decode<DT, NT>(base, vfull, rb, z);
      topk_issue<DT, NT>(p, g, base + 2 * (kTopkPer * NT), vfull, rb);
#pragma unroll
      for (int e = 0; e < kTopkPer; ++e) {
        const int x = topk_tok<DT, NT>(base, e);
        if (x < vfull) fn(x, z[e]);
      }
      base += (kTopkPer * NT);
    }
    for (int x = vfull + (int)threadIdx.x; x < p.V; x += NT) fn(x, load_logit(p, g, x));
  } else {
    for (int x = threadIdx.x; x < p.V; x += NT) fn(x, load_logit(p, g, x));
  }
}

// Calls tile(base, z[kTopkPer]) for every super-tile of an aligned row (two in
// flight); logits of tokens at or past vfull = V - V % VW read as -inf.
template <int DT, int NT, class F>
__device__ __forceinline__ void stream_tiles(const Params &p, int g, int vfull, F tile) {
  TopkRaw<DT> ra, rb;
  int base = 0;
  topk_issue<DT, NT>(p, g, base, vfull, ra);
  topk_issue<DT, NT>(p, g, base + (kTopkPer * NT), vfull, rb);
  while (base < vfull) {
    float z[kTopkPer];
    topk_decode<DT, NT>(base, vfull, ra, z);
    topk_issue<DT, NT>(p, g, base + 2 * (kTopkPer * NT), vfull, ra);
    tile(base, z);
    base += (kTopkPer * NT);
    if (base >= vfull) break;
    topk_decode<DT, NT>(base, vfull, rb, z);
    topk_issue<DT, NT>(p, g, base + 2 * (kTopkPer * NT), vfull, rb);
    tile(base, z);
    base += (kTopkPer * NT);
  }
}

// One MSD digit of the weighted select (wave 0 scans, all threads call):
// bins hold integer weights of the candidates matching the prefix; the digit
// is the largest whose bins above it hold less than `need` and whose own bin
// reaches it.  None reaches it only through rounding of the bound: the lowest
// non-empty digit (everything kept).  need is reduced by the bins above.
__device__ __forceinline__ int topp_digit(ToppShared &sh, unsigned long long &need) {
  if (threadIdx.x < 64) {
    const int l = threadIdx.x;
    unsigned long long h[4], own = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[i] = sh.mass[255 - 4 * l - i];
      own += h[i];
    }
    unsigned long long incl = own;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const unsigned long long o = __shfl_up(incl, d, 64);
      if (l >= d) incl += o;
    }
    const unsigned long long before = incl - own;
    const bool here = before < need && incl >= need;
    const unsigned long long any = __ballot(here);
    const unsigned long long nonempty = __ballot(own != 0);
    const int src = any ? __ffsll((long long)any) - 1 : 63 - __builtin_clzll(nonempty | 1ull);
    if (l == src) {
      unsigned long long acc = before;
      int sel = -1, low = 255 - 4 * l;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (h[i] == 0) continue;
        if (sel < 0 && acc + h[i] >= need) sel = 255 - 4 * l - i;
        if (sel < 0) acc += h[i];
        low = 255 - 4 * l - i;
      }
      if (sel < 0) {  // not reached: keep everything, descend into the lowest non-empty digit
        sel = low;
        acc -= h[255 - 4 * l - low];
      }
      sh.sel = sel;
      sh.need = need - acc;
    }
  }
  __syncthreads();
  const int sel = sh.sel;
  need = sh.need;
  __syncthreads();
  return sel;
}

// Weighted MSD radix select among the tokens `each` enumerates (each thread
// calls its callback with (z, W) for its share): the largest key whose
// strictly larger keys hold less than `need` integer weight units.
template <class EACH>
__device__ __forceinline__ float topp_select(ToppShared &sh, EACH each, unsigned long long need) {
  uint32_t prefix = 0, mask = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (threadIdx.x < 256) sh.mass[threadIdx.x] = 0;
    __syncthreads();
    each([&](float z, float W) {
      const uint32_t key = ukey(z);
      if ((key & mask) == prefix) atomicAdd(&sh.mass[(key >> shift) & 0xFFu], (unsigned long long)(uint32_t)W);
    });
    __syncthreads();
    prefix |= (uint32_t)topp_digit(sh, need) << shift;
    mask |= 0xFFu << shift;
  }
  return ukey_val(prefix);
}

template <int DT, int NT>
__global__ __launch_bounds__(NT) void topp_kernel(Params p) {
  static_assert(NT % 256 == 0 && NT / 64 <= kTpMaxWaves, "the selects' 256-bin histograms and the wave maxima");
  __shared__ ToppShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = blockIdx.x;
  const int r = find_request(p.cu, p.B, g);
  const Req q = load_req(p, r);
  const int st = p.has_topk ? p.cand_n[g] : kRowDense;
  const bool use = q.cu_ok && g >= q.g0 && g <= q.g0 + q.K && q.mode == kModeSample && q.top_p < 1.0f && st < 0;
  if (!use) {
    if (tid == 0 && !p.has_topk) p.cand_n[g] = kRowDense;  // later kernels read every row's state
    return;
  }
  Proc pr = q.proc;
  pr.tau = st == kRowThreshold ? p.cand_tau[g] : kNegInf;
  const float a = q.a, tau = pr.tau;

  // Row scale m from the first pass's chunk table.
  float2 *tab = p.chunk_tab + (int64_t)g * p.nc_stride;
  float lm = kNegInf;
  for (int c = tid; c < p.NC; c += NT) lm = fmaxf(lm, tab[c].x);
  lm = wave_max(lm);
  if (lane == 0) sh.wmax[wave] = lm;
  __syncthreads();
  float m = sh.wmax[0];
#pragma unroll
  for (int w = 1; w < (NT / 64); ++w) m = fmaxf(m, sh.wmax[w]);
  if (!(m > kNegInf)) {  // no finite logit: the epilogue flags the row
    if (tid == 0) p.cand_n[g] = st;
    return;
  }
  constexpr int VW = TopkRaw<DT>::VW;
  const int vfull = p.V - p.V % VW;
  // Aligned rows without a penalty take the branch-free tile loops.
  const bool tiles = p.vec_ok && pr.counts == nullptr;

  // Pass A: integer weight per sub-bucket.
  for (int j = tid; j < kToppSub; j += NT) sh.mass[j] = 0;
  __syncthreads();
  if (tiles) {
    stream_tiles<DT, NT>(p, g, vfull, [&](int, float (&z)[kTopkPer]) {
#pragma unroll
      for (int e = 0; e < kTopkPer; ++e) {
        const ToppW w = topp_w(z[e] < tau ? kNegInf : z[e], m, a);
        atomicAdd(&sh.mass[w.j], (unsigned long long)(uint32_t)w.W);
      }
    });
    if (vfull + tid < p.V) {
      const ToppW w = topp_w(apply_proc(load_logit(p, g, vfull + tid), vfull + tid, pr), m, a);
      atomicAdd(&sh.mass[w.j], (unsigned long long)(uint32_t)w.W);
    }
  } else {
    stream_row<DT, NT>(p, g, [&](int x, float raw) {
      const ToppW w = topp_w(apply_proc(raw, x, pr), m, a);
      atomicAdd(&sh.mass[w.j], (unsigned long long)(uint32_t)w.W);
    });
  }
  __syncthreads();
  // Scan (wave 0): lane l owns sub-buckets 16 l .. 16 l + 15, of integer part
  // k = l - 20; fp64 in a fixed order.
  if (wave == 0) {
    const int kl = lane - kToppSubOff / 16;
    double own = 0.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) own += __builtin_ldexp((double)sh.mass[16 * lane + i], -31 - kl);
    double incl = own;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const double o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    const double total = __shfl(incl, 63, 64);
    const double bound = (double)q.top_p * total;
    double acc = incl - own;
    int hit = -1;
    double hit_above = 0.0;
    for (int i = 0; i < 16; ++i) {
      const unsigned long long h = sh.mass[16 * lane + i];
      if (h == 0) continue;
      const double hm = __builtin_ldexp((double)h, -31 - kl);
      if (acc + hm >= bound) {
        hit = 16 * lane + i;
        hit_above = acc;
        break;
      }
      acc += hm;
    }
    const unsigned long long hits = __ballot(hit >= 0);
    // the first crossing; none only through rounding with top_p near 1: the last non-empty sub-bucket
    const unsigned long long nonempty = __ballot(own > 0.0);
    const int src = hits ? __ffsll((long long)hits) - 1 : 63 - __builtin_clzll(nonempty | 1ull);
    if (lane == src) {
      if (hit < 0) {
        for (int i = 15; i >= 0; --i)
          if (sh.mass[16 * lane + i]) {
            hit = 16 * lane + i;
            hit_above = incl - __builtin_ldexp((double)sh.mass[hit], -31 - kl);
            break;
          }
        if (hit < 0) hit = 16 * lane;
      }
      sh.sel = hit;
      // integer weight units of sub-bucket hit still needed to reach the bound
      const int kh = (hit >> 4) - kToppSubOff / 16;
      const double rest = __builtin_ceil(__builtin_ldexp(bound - hit_above, 31 + kh));
      sh.need = rest < 1.0 ? 1ull : (unsigned long long)rest;
      sh.n = 0;
    }
  }
  __syncthreads();
  const int jstar = sh.sel;
  const int kstar = (jstar >> 4) - kToppSubOff / 16;
  const unsigned long long need = sh.need;
  const bool direct = p.vec_ok && p.NC <= kToppMaxNC;

  // Pass B: the boundary sub-bucket into the list, the mass before it per chunk.
  bool redo = !direct;
  if (direct) {
    for (int c = tid; c < p.NC * 4; c += NT) sh.part[c] = 0.0f;
    for (int c = tid; c < p.NC; c += NT) sh.lsum[c] = 0;
    if (tid < 8) sh.tail[tid] = 0.0f;
    __syncthreads();
    constexpr int WPC = kChunk / (64 * VW);  // waves covering one chunk in a super-tile
    // Most tokens lie below the boundary sub-bucket: their weight is not
    // needed, and a wave whose tokens all do skips the rest.
    auto token = [&](int x, float z, float &acc) {
      if (topp_j((m - z) * a) > jstar) return;
      const ToppW w = topp_w(z, m, a);
      acc += w.j < jstar ? __builtin_ldexpf(w.W, -31 - w.k) : 0.0f;
      if (w.j == jstar && z > kNegInf) {
        const int pos = atomicAdd(&sh.n, 1);
        if (pos < kToppList) {
          sh.lz[pos] = z;
          sh.lx[pos] = x;
        }
      }
    };
    stream_tiles<DT, NT>(p, g, vfull, [&](int base, float (&z)[kTopkPer]) {
#pragma unroll
      for (int v = 0; v < kTopkPer / VW; ++v) {
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < VW; ++i) {
          const int e = v * VW + i;
          const int x = topk_tok<DT, NT>(base, e);
          float zz = z[e];
          if (!tiles && x < vfull) zz = apply_proc(zz, x, pr);  // penalty rows
          token(x, zz < tau ? kNegInf : zz, acc);
        }
        const float sum = wave_sum(acc);
        const int c = (base + (v * NT + wave * 64) * VW) / kChunk;
        if (lane == 0 && c < p.NC) sh.part[c * 4 + wave % WPC] = sum;
      }
    });
    if (vfull + tid < p.V) {  // the last V % VW tokens (one chunk)
      float acc = 0.0f;
      token(vfull + tid, apply_proc(load_logit(p, g, vfull + tid), vfull + tid, pr), acc);
      sh.tail[tid] = acc;
    }
    __syncthreads();
    redo = sh.n > kToppList;
  }

  float zstar;
  if (!redo) {
    const int n = sh.n;
    zstar = topp_select(
        sh, [&](auto fn) {
          for (int e = tid; e < n; e += NT) fn(sh.lz[e], topp_w(sh.lz[e], m, a).W);
        },
        need);
    // Kept list tokens into their chunks (integer sums), then the new table.
    for (int e = tid; e < n; e += NT)
      if (sh.lz[e] >= zstar)
        atomicAdd(&sh.lsum[sh.lx[e] / kChunk], (unsigned long long)(uint32_t)topp_w(sh.lz[e], m, a).W);
    __syncthreads();
    constexpr int WPC = kChunk / (64 * VW);
    const int clast = (p.V - 1) / kChunk;
    for (int c = tid; c < p.NC; c += NT) {
      float sc = 0.0f;
#pragma unroll
      for (int w = 0; w < WPC; ++w) sc += sh.part[c * 4 + w];
      if (c == clast) {
        float t = 0.0f;
        for (int i = 0; i < 8; ++i) t += sh.tail[i];
        sc += t;
      }
      sc += (float)__builtin_ldexp((double)sh.lsum[c], -31 - kstar);
      tab[c] = make_float2(m, sc);
    }
  } else {
    zstar = topp_select(
        sh, [&](auto fn) {
          stream_row<DT, NT>(p, g, [&](int x, float raw) {
            const float z = apply_proc(raw, x, pr);
            const ToppW w = topp_w(z, m, a);
            if (w.j == jstar && z > kNegInf) fn(z, w.W);
          });
        },
        need);
  }
  if (tid == 0) {
    p.cand_tau[g] = zstar;
    p.cand_n[g] = redo ? kRowTopPRedo : kRowTopP;
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

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Draft-side sampling, after a streaming pass over this step's draft rows (row
// r of the call = request r).  One workgroup per request: the row's scale m and
// mass s from its chunk table, then the two-level race on counter row
// cu[r] + step (the draft's row in the verify call) with the draft tags, or the
// argmax (lowest index) when T = 0; q(d) and (m, s) are recorded for the
// verifier.
// ---------------------------------------------------------------------------
struct DraftShared {
  BlockScratch red;
  float zs[kChunk];
};

__global__ __launch_bounds__(kThreads) void draft_race_kernel(Params p, DraftOut o) {
  __shared__ DraftShared sh;
  const int r = blockIdx.x, tid = threadIdx.x;
  const int K = o.cu[r + 1] - o.cu[r];
  const float T = p.temperature[r];
  const bool bad_t = !(T >= 0.0f) || !__builtin_isfinite(T);
  if (o.step >= K || bad_t) {  // no draft at this position, or an invalid temperature
    if (tid == 0) {
      if (bad_t && o.step < K) raise_err(p, SV_ERR_TEMPERATURE);
      o.tokens[r] = -1;
      if (o.q) o.q[r] = 0.0f;
    }
    return;
  }
  const uint32_t key = (uint32_t)(o.cu[r] + o.step);
  const float a = T > 0.0f ? kLog2e / T : 0.0f;
  const float2 *tab = p.chunk_tab + (int64_t)r * p.nc_stride;
  float lm = kNegInf;
  for (int c = tid; c < p.NC; c += kThreads) lm = fmaxf(lm, tab[c].x);
  const float m = block_max(lm, sh.red);
  if (!(m > kNegInf)) {
    if (tid == 0) {
      raise_err(p, SV_ERR_ROW);
      o.tokens[r] = -1;
      if (o.q) o.q[r] = 0.0f;
    }
    return;
  }
  float ls = 0.0f;
  for (int c = tid; c < p.NC; c += kThreads) {
    const float2 e = tab[c];
    if (e.x > kNegInf) ls += e.y * exp2_acc(a * (e.x - m));
  }
  const float s = block_sum(ls, sh.red);
  int cstar;
  if (T == 0.0f) {  // the lowest chunk holding the maximum (greedy tables hold exact chunk maxima)
    ArgMax best{-1.0f, 0x7FFFFFFF};
    for (int c = tid; c < p.NC; c += kThreads)
      if (tab[c].x == m && c < best.i) best = ArgMax{1.0f, c};
    cstar = block_argmax(best, sh.red).i;
  } else {
    cstar = block_chunk_race(p, key, p.NC, [&](int c) -> float {
      const float2 e = tab[c];
      return e.x > kNegInf ? e.y * exp2_acc(a * (e.x - m)) : 0.0f;
    }, sh.red, kTagDraftChunk);
  }
  int d = -1;
  if (cstar >= 0) {
    for (int t = tid; t < kChunk; t += kThreads) {
      const int x = cstar * kChunk + t;
      sh.zs[t] = x < p.V ? load_logit(p, r, x) : kNegInf;
    }
    __syncthreads();
    if (T == 0.0f) {  // first token of the chunk equal to the maximum
      ArgMax best{-1.0f, 0x7FFFFFFF};
      for (int t = tid; t < kChunk; t += kThreads)
        if (sh.zs[t] == m && t < best.i) best = ArgMax{1.0f, t};
      const ArgMax b = block_argmax(best, sh.red);
      d = b.s < 0.0f ? -1 : cstar * kChunk + b.i;
    } else {
      Proc pr;
      pr.counts = nullptr;
      pr.theta = 1.0f;
      pr.freq = pr.pres = 0.0f;
      pr.tau = kNegInf;
      d = block_token_race(p, (int)key, cstar, sh.zs, pr, a, a * m, -1, sh.red, kTagDraftToken);
    }
  }
  if (tid == 0) {
    o.tokens[r] = d;
    if (o.ids) o.ids[key] = d;
    o.stats[2 * (int64_t)key] = m;
    o.stats[2 * (int64_t)key + 1] = s;
    if (o.q) o.q[r] = d < 0 ? 0.0f : (T == 0.0f ? 1.0f : exp2_acc(a * (sh.zs[d - cstar * kChunk] - m)) / s);
  }
}

hipError_t launch_draft_race(const Params &p, const DraftOut &o, hipStream_t s) {
  draft_race_kernel<<<dim3((unsigned)p.B), dim3(kThreads), 0, s>>>(p, o);
  return hipGetLastError();
}


hipError_t launch_topp(const Params &p, hipStream_t s) {
  if (p.has_topk) {
    if (p.dtype == 1)
      topp_kernel<1, 256><<<dim3(p.R), dim3(256), 0, s>>>(p);
    else
      topp_kernel<0, 256><<<dim3(p.R), dim3(256), 0, s>>>(p);
  } else {
    if (p.dtype == 1)
      topp_kernel<1, 512><<<dim3(p.R), dim3(512), 0, s>>>(p);
    else
      topp_kernel<0, 512><<<dim3(p.R), dim3(512), 0, s>>>(p);
  }
  return hipGetLastError();
}

// Launch with optional timing events: hipExtLaunchKernel stamps them from the
// dispatch packet itself, so their interval is the kernel's execution time.
hipError_t launch_timed(const void *fn, dim3 grid, const Params &p, hipStream_t s, hipEvent_t t0, hipEvent_t t1,
                        int threads = kThreads) {
  Params arg = p;
  void *args[] = {&arg};
  return hipExtLaunchKernel(fn, grid, dim3(threads), args, 0, s, t0, t1, 0);
}

hipError_t launch_topk(const Params &p, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  const void *fn = p.dtype == 1 ? reinterpret_cast<const void *>(&topk_kernel<1>)
                                : reinterpret_cast<const void *>(&topk_kernel<0>);
  return launch_timed(fn, dim3((unsigned)p.R), p, s, t0, t1);
}

hipError_t launch_stats(const Params &p, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  const dim3 grid((unsigned)p.stats_grid);
  const void *fn = !p.fast ? (p.dtype == 1 ? reinterpret_cast<const void *>(&stats_kernel<1>)
                                           : reinterpret_cast<const void *>(&stats_kernel<0>))
                   : p.fast_pen ? (p.dtype == 1 ? reinterpret_cast<const void *>(&stats_fast_kernel<1, true>)
                                                : reinterpret_cast<const void *>(&stats_fast_kernel<0, true>))
                                : (p.dtype == 1 ? reinterpret_cast<const void *>(&stats_fast_kernel<1, false>)
                                                : reinterpret_cast<const void *>(&stats_fast_kernel<0, false>));
  const int threads = !p.fast ? kThreads
                      : p.fast_pen ? (p.dtype == 1 ? kFastThreads<1, true> : kFastThreads<0, true>)
                                   : (p.dtype == 1 ? kFastThreads<1, false> : kFastThreads<0, false>);
  return launch_timed(fn, grid, p, s, t0, t1, threads);
}

int stats_blocks_per_cu(int dtype, int kind) {
  int n = 0;
  hipError_t e;
  if (kind == 1)
    e = dtype == 1 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, stats_fast_kernel<1, false>, kFastThreads<1, false>, 0)
                   : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, stats_fast_kernel<0, false>, kFastThreads<0, false>, 0);
  else if (kind == 2)
    e = dtype == 1 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, stats_fast_kernel<1, true>, kFastThreads<1, true>, 0)
                   : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, stats_fast_kernel<0, true>, kFastThreads<0, true>, 0);
  else
    e = dtype == 1 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, stats_kernel<1>, kThreads, 0)
                   : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, stats_kernel<0>, kThreads, 0);
  return e == hipSuccess && n > 0 ? n : 1;
}

hipError_t launch_epilogue(const Params &p, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  const bool plain = plain_call(p);
  const void *fn = plain ? reinterpret_cast<const void *>(&epilogue_kernel<true>)
                         : reinterpret_cast<const void *>(&epilogue_kernel<false>);
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
