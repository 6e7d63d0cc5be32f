// sv_common.h -- device helpers shared by the verify kernels: per-request
// settings and row lookup, chunk decoding and loads, the two-level race, and
// the launch helper with timing events.
#pragma once
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
// A target row as the statistics passes see it, and one chunk's statistics.
// ---------------------------------------------------------------------------
struct RowInfo {
  int g, r, i, c0, K, g0, mode, st;  // mode kModeInvalid: row skipped
  float a, theta, freq, pres, tau;
  const int32_t *counts;
};

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

// ---------------------------------------------------------------------------
// Races.  RACE(w, g): chunk c* = argmax_c M_c / E(g, 1, c) over chunks with
// M_c > 0, then token x* = argmax_{x in c*} w_x / E(g, 2, x) over w_x > 0.
// Scores are fp32 (race_score); ties go to the lowest index.
// ---------------------------------------------------------------------------

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
      uint2 w[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int x0 = c16_tok(c, 4 * t, lane);
        w[t] = row[x0 < V ? x0 >> 2 : 0];
      }
      __builtin_amdgcn_sched_barrier(0);  // every load issued before the first use
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        z[4 * t] = __uint_as_float(w[t].x << 16);
        z[4 * t + 1] = __uint_as_float(w[t].x & 0xFFFF0000u);
        z[4 * t + 2] = __uint_as_float(w[t].y << 16);
        z[4 * t + 3] = __uint_as_float(w[t].y & 0xFFFF0000u);
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
    uint32_t h[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) h[e] = row[min(c16_tok(c, e, lane), V - 1)];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < 16; ++e) z[e] = bf16_bits_to_f32(h[e]);
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

// Chunks ca and cb of row g (the c16_tok layout) with every load of both
// issued before any value is used, so the pair costs one memory round trip
// (two chunk loads in a row would each wait for their data inside their dtype
// branch).  A negative chunk index reads chunk 0, whose values the caller
// ignores.
__device__ __forceinline__ void load_chunk16_pair(const Params &p, int g, int ca, int cb, float (&za)[16],
                                                  float (&zb)[16]) {
  const int lane = threadIdx.x & 63;
  const int V = p.V;
  ca = max(ca, 0);
  cb = max(cb, 0);
  if (p.vec_ok && (V & 3) == 0) {
    if (p.dtype == 1) {
      const uint2 *row = reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p.logits) + (int64_t)g * p.lstride);
      uint2 wa[4], wb[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int xa = c16_tok(ca, 4 * t, lane), xb = c16_tok(cb, 4 * t, lane);
        wa[t] = row[xa < V ? xa >> 2 : 0];
        wb[t] = row[xb < V ? xb >> 2 : 0];
      }
      __builtin_amdgcn_sched_barrier(0);  // every load issued before the first use
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        za[4 * t] = __uint_as_float(wa[t].x << 16);
        za[4 * t + 1] = __uint_as_float(wa[t].x & 0xFFFF0000u);
        za[4 * t + 2] = __uint_as_float(wa[t].y << 16);
        za[4 * t + 3] = __uint_as_float(wa[t].y & 0xFFFF0000u);
        zb[4 * t] = __uint_as_float(wb[t].x << 16);
        zb[4 * t + 1] = __uint_as_float(wb[t].x & 0xFFFF0000u);
        zb[4 * t + 2] = __uint_as_float(wb[t].y << 16);
        zb[4 * t + 3] = __uint_as_float(wb[t].y & 0xFFFF0000u);
      }
    } else {
      const float4 *row = reinterpret_cast<const float4 *>(static_cast<const float *>(p.logits) + (int64_t)g * p.lstride);
      float4 wa[4], wb[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int xa = c16_tok(ca, 4 * t, lane), xb = c16_tok(cb, 4 * t, lane);
        wa[t] = row[xa < V ? xa >> 2 : 0];
        wb[t] = row[xb < V ? xb >> 2 : 0];
      }
      __builtin_amdgcn_sched_barrier(0);  // every load issued before the first use
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        za[4 * t] = wa[t].x;
        za[4 * t + 1] = wa[t].y;
        za[4 * t + 2] = wa[t].z;
        za[4 * t + 3] = wa[t].w;
        zb[4 * t] = wb[t].x;
        zb[4 * t + 1] = wb[t].y;
        zb[4 * t + 2] = wb[t].z;
        zb[4 * t + 3] = wb[t].w;
      }
    }
  } else if (p.dtype == 1) {
    const uint16_t *row = static_cast<const uint16_t *>(p.logits) + (int64_t)g * p.lstride;
    uint32_t ha[16], hb[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      ha[e] = row[min(c16_tok(ca, e, lane), V - 1)];
      hb[e] = row[min(c16_tok(cb, e, lane), V - 1)];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      za[e] = bf16_bits_to_f32(ha[e]);
      zb[e] = bf16_bits_to_f32(hb[e]);
    }
  } else {
    const float *row = static_cast<const float *>(p.logits) + (int64_t)g * p.lstride;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      za[e] = row[min(c16_tok(ca, e, lane), V - 1)];
      zb[e] = row[min(c16_tok(cb, e, lane), V - 1)];
    }
  }
}

// load_chunk16_pair with the row's penalties applied (as load_chunk16_pen).
__device__ __forceinline__ void load_chunk16_pen_pair(const Params &p, int g, int ca, int cb, const Proc &pr,
                                                      float (&za)[16], float (&zb)[16]) {
  if (pr.counts == nullptr) {
    load_chunk16_pair(p, g, ca, cb, za, zb);
    return;
  }
  const int lane = threadIdx.x & 63;
  int na[16], nb[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    na[e] = pr.counts[min(c16_tok(max(ca, 0), e, lane), p.V - 1)];
    nb[e] = pr.counts[min(c16_tok(max(cb, 0), e, lane), p.V - 1)];
  }
  load_chunk16_pair(p, g, ca, cb, za, zb);
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    if (na[e] > 0) za[e] = penalize(za[e], na[e], pr);
    if (nb[e] > 0) zb[e] = penalize(zb[e], nb[e], pr);
  }
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

// Row statistics and chunk race of a dense stochastic row of at most 256
// chunks in one go: lane l holds the table entries of chunks 4l .. 4l + 3 in
// registers; m = the largest r_c, then W_c = s_c exp2(a (r_c - m)) once per
// chunk for both S = sum of W_c and the race (chunk `skip` left out, its 1/E
// to *rskip), the two wave reductions side by side.  Same results as the
// separate statistics and wave_chunk_race up to the summation order of S.
template <class EF>
__device__ __forceinline__ void row_stats_race(const Params &p, EF ent, float a, int skip, const ChunkNoise &cn,
                                               float &m, float &s, ArgMax &w1, float *rskip) {
  const int lane = threadIdx.x & 63;
  float2 e[4];
  float lm = kNegInf;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = 4 * lane + k;
    e[k] = c < p.NC ? ent(c) : make_float2(kNegInf, 0.0f);
    lm = fmaxf(lm, e[k].x);
  }
  m = wave_max(lm);
  float ls = 0.0f, rs = 0.0f;
  ArgMax best{-1.0f, 0x7FFFFFFF};
  if (m > kNegInf) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = 4 * lane + k;
      if (c == skip) rs = cn.r[k];
      if (e[k].x > kNegInf) {
        const float Wc = e[k].y * exp2_acc(a * (e[k].x - m));
        ls += Wc;
        if (c != skip && Wc > 0.0f) {
          const ArgMax o{Wc * cn.r[k], c};
          if (better(o, best)) best = o;
        }
      }
    }
  }
  s = wave_sum(ls);
  w1 = wave_argmax(best);
  if (skip >= 0) *rskip = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rs), (skip >> 2) & 63));
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

}  // namespace

// Launch with optional timing events: hipExtLaunchKernel stamps them from the
// dispatch packet itself, so their interval is the kernel's execution time.
inline hipError_t launch_timed(const void *fn, dim3 grid, const Params &p, hipStream_t s, hipEvent_t t0, hipEvent_t t1,
                        int threads = kThreads) {
  Params arg = p;
  void *args[] = {&arg};
  return hipExtLaunchKernel(fn, grid, dim3(threads), args, 0, s, t0, t1, 0);
}

}  // namespace sv
