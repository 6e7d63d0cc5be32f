// sv_kernels.hip -- gfx950 kernels of the speculative-decoding verify step.
//
// Data flow of one spec_verify_run (all on one stream):
//   topk_kernel   (only with top_k)      one workgroup per target row: exact
//                 k-th largest processed logit tau and, when at most
//                 kCandCap tokens reach tau, the kept tokens sorted by id.
//   stats_kernel  the streaming pass.  Workgroup (row g, segment) reads
//                 cps chunks of kChunk logits of row g once, and stores per
//                 chunk (max, sum exp2(a (z - max))) -- or (max, argmax) for
//                 greedy rows -- in the chunk table.  The last workgroup to
//                 finish a request (per-request arrival counter) runs the
//                 request epilogue: row softmax statistics from the chunk
//                 table, the accept tests, the first reject, and the
//                 bonus / recovered race.
//   resid_kernel  (draft-probs mode) residual max(0, p - q) chunk masses of
//                 each rejected request's row, then the race.
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

__device__ Req load_req(const Params &p, int r) {
  Req q;
  const int c0 = p.cu[r], c1 = p.cu[r + 1];
  q.r = r;
  q.c0 = c0;
  q.K = c1 - c0;
  q.g0 = c0 + r;
  q.cu_ok = c0 >= 0 && c0 <= c1 && c1 <= p.D && q.K <= p.out_stride - 1;
  q.errbits = 0;
  q.proc.counts = nullptr;
  q.proc.theta = 1.0f;
  q.proc.tau = kNegInf;
  const float T = p.temperature[r];
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
// Arrival protocol.  A counter holds (epoch << 32 | arrivals).  Each
// workgroup first raises the counter to (epoch << 32) -- a no-op once this
// call has started counting, a reset if it holds an older call's count --
// then adds one after its results are visible device-wide.  The last arrival
// resets the count so that replays with the same epoch also start from zero.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void arrive_begin(unsigned long long *ctr, uint32_t epoch) {
  if (threadIdx.x == 0)
    __hip_atomic_fetch_max(ctr, (unsigned long long)epoch << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Returns true (in every thread) if this workgroup is the last of `target`.
__device__ __forceinline__ bool arrive_end(unsigned long long *ctr, uint32_t epoch, unsigned target, int *sh_flag) {
  __threadfence();  // release this workgroup's table entries
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long old =
        __hip_atomic_fetch_add(ctr, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = (old >> 32) == epoch && (unsigned)(old & 0xFFFFFFFFu) + 1u == target;
    if (last) {
      __threadfence();  // acquire the other workgroups' entries
      __hip_atomic_store(ctr, (unsigned long long)epoch << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    *sh_flag = last ? 1 : 0;
  }
  __syncthreads();
  return *sh_flag != 0;
}

// ---------------------------------------------------------------------------
// Races.  RACE(w, g): chunk c* = argmax_c M_c / E(g, 1, c) over chunks with
// M_c > 0, then token x* = argmax_{x in c*} w_x / E(g, 2, x) over w_x > 0.
// Scores are compared in fp64; ties go to the lowest index.
// ---------------------------------------------------------------------------
struct EpiShared {
  BlockScratch red;
  float m[kMaxDrafts + 1];
  float s[kMaxDrafts + 1];
  int amax[kMaxDrafts + 1];
  int state[kMaxDrafts + 1];
  float tau[kMaxDrafts + 1];
  int j;
  int bad;
  int flag;
  float cw[kCandCap];  // compact rows: candidate weights
  int ci[kCandCap];    // compact rows: candidate token ids
};

// Chunk race with weights from a functor W(c) (fp32, >= 0).
template <class WF>
__device__ int chunk_race(const Params &p, uint32_t g, int NC, WF W, BlockScratch &red) {
  ArgMax best{-1.0, 0x7FFFFFFF};
  for (int base = 0; base < NC; base += 4 * kThreads) {
    const int c0 = base + 4 * (int)threadIdx.x;
    if (c0 < NC) {
      const uint4 w4 = rng_block(p, (uint32_t)c0 >> 2, g, kTagChunk);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int c = c0 + k;
        if (c < NC) {
          const float Wc = W(c);
          if (Wc > 0.0f) {
            ArgMax o{(double)Wc / exp_noise(pick(w4, k)), c};
            if (better(o, best)) best = o;
          }
        }
      }
    }
  }
  const ArgMax b = block_argmax(best, red);
  return b.s < 0.0 ? -1 : b.i;
}

// Token race inside chunk c (0 <= c < NC) with weights from a functor w(x)
// (x < V).  Returns -1 if no token of the chunk has positive weight.
template <class TF>
__device__ int token_race(const Params &p, uint32_t g, int c, TF w, BlockScratch &red) {
  ArgMax best{-1.0, 0x7FFFFFFF};
  const int x0 = c * kChunk + 4 * (int)threadIdx.x;
  const uint4 w4 = rng_block(p, (uint32_t)x0 >> 2, g, kTagToken);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int x = x0 + k;
    if (x < p.V) {
      const float wx = w(x);
      if (wx > 0.0f) {
        ArgMax o{(double)wx / exp_noise(pick(w4, k)), x};
        if (better(o, best)) best = o;
      }
    }
  }
  const ArgMax b = block_argmax(best, red);
  return b.s < 0.0 ? -1 : b.i;
}

// Race over a compact candidate list (token ids ascending in sh.ci, weights in
// sh.cw, n entries).  Same law and random words as the dense race: chunk
// masses are the sums over the candidates of each chunk.
__device__ int compact_race(const Params &p, uint32_t g, int n, EpiShared &sh) {
  __syncthreads();
  ArgMax best{-1.0, 0x7FFFFFFF};
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const int c = sh.ci[i] / kChunk;
    if (i > 0 && sh.ci[i - 1] / kChunk == c) continue;  // not the first candidate of its chunk
    float M = 0.0f;
    for (int t = i; t < n && sh.ci[t] / kChunk == c; ++t) M += sh.cw[t];
    if (M > 0.0f) {
      const uint4 w4 = rng_block(p, (uint32_t)c >> 2, g, kTagChunk);
      ArgMax o{(double)M / exp_noise(pick(w4, c & 3)), c};
      if (better(o, best)) best = o;
    }
  }
  const ArgMax cb = block_argmax(best, sh.red);
  if (cb.s < 0.0) return -1;
  const int cstar = cb.i;
  ArgMax tb{-1.0, 0x7FFFFFFF};
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const int x = sh.ci[i];
    if (x / kChunk != cstar || !(sh.cw[i] > 0.0f)) continue;
    const uint4 w4 = rng_block(p, (uint32_t)x >> 2, g, kTagToken);
    ArgMax o{(double)sh.cw[i] / exp_noise(pick(w4, x & 3)), x};
    if (better(o, tb)) tb = o;
  }
  const ArgMax b = block_argmax(tb, sh.red);
  return b.s < 0.0 ? -1 : b.i;
}

__device__ void write_empty(const Params &p, int r) {
  for (int t = threadIdx.x; t < p.out_stride; t += kThreads) p.out_tokens[(int64_t)r * p.out_stride + t] = -1;
  if (threadIdx.x == 0) {
    p.out_ns[r] = 0;
    p.out_nr[r] = 0;
  }
}

// ---------------------------------------------------------------------------
// Request epilogue (run by the last stats workgroup of request q.r).
// ---------------------------------------------------------------------------
__device__ void request_epilogue(const Params &p, const Req &q, EpiShared &sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = q.K, r = q.r;

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

  // Row statistics: one wave per row.
  for (int i = wave; i <= K; i += kWaves) {
    const int g = q.g0 + i;
    const int st = row_state(p, g);
    float m, s = 0.0f;
    int am = 0x7FFFFFFF;
    if (st >= 0) {
      const float *cv = p.cand_val + (int64_t)g * kCandCap;
      float lm = kNegInf;
      for (int t = lane; t < st; t += 64) lm = fmaxf(lm, cv[t]);
      m = wave_max(lm);
      float ls = 0.0f;
      for (int t = lane; t < st; t += 64) ls += exp2_acc(q.a * (cv[t] - m));
      s = wave_sum(ls);
    } else {
      const float2 *tab = p.chunk_tab + (int64_t)g * p.nc_stride;
      float lm = kNegInf;
      for (int c = lane; c < p.NC; c += 64) lm = fmaxf(lm, tab[c].x);
      m = wave_max(lm);
      if (greedy) {
        int li = 0x7FFFFFFF;
        for (int c = lane; c < p.NC; c += 64) {
          const float2 e = tab[c];
          if (e.x == m) li = min(li, __float_as_int(e.y));
        }
        am = wave_min_i(li);
      } else if (m > kNegInf) {
        float ls = 0.0f;
        for (int c = lane; c < p.NC; c += 64) {
          const float2 e = tab[c];
          if (e.x > kNegInf) ls += e.y * exp2_acc(q.a * (e.x - m));
        }
        s = wave_sum(ls);
      }
    }
    if (lane == 0) {
      sh.m[i] = m;
      sh.s[i] = s;
      sh.amax[i] = am;
      sh.state[i] = st;
      sh.tau[i] = (st == kRowDense) ? kNegInf : p.cand_tau[g];
      p.row_info[g] = make_float4(m, s, __int_as_float(am), __int_as_float(st));
    }
  }
  __syncthreads();
  if (tid == 0) {
    int bad = 0;
    for (int i = 0; i <= K; ++i) bad |= !__builtin_isfinite(sh.m[i]);
    sh.bad = bad;
  }
  __syncthreads();
  if (sh.bad) {
    if (tid == 0) raise_err(p, SV_ERR_ROW);
    write_empty(p, r);
    return;
  }

  // Accept tests: lane i of wave 0 takes draft position i.
  if (wave == 0) {
    bool rej = false;
    if (lane < K) {
      const int d = p.draft_ids[q.c0 + lane];
      const int g = q.g0 + lane;
      if (greedy) {
        rej = d != sh.amax[lane];
        if (p.dbg_p_draft) p.dbg_p_draft[q.c0 + lane] = -1.0f;
      } else {
        const bool valid = d >= 0 && d < p.V;
        float pd = 0.0f;
        if (valid) {
          Proc pr = q.proc;
          pr.tau = sh.tau[lane];
          const float z = apply_proc(load_logit(p, g, d), d, pr);
          pd = exp2_acc(q.a * (z - sh.m[lane])) / sh.s[lane];
        }
        double qd = 1.0;
        if (p.draft_probs) qd = valid ? (double)p.draft_probs[(int64_t)(q.c0 + lane) * p.dstride + d] : 0.0;
        const double u = u_accept(rng_block(p, 0, (uint32_t)g, kTagAccept).x);
        rej = !(valid && qd > 0.0 && (double)pd >= u * qd);
        if (p.dbg_p_draft) p.dbg_p_draft[q.c0 + lane] = pd;
      }
    }
    const unsigned long long mask = __ballot(rej);
    if (lane == 0) sh.j = mask ? (__ffsll((long long)mask) - 1) : K;
  }
  __syncthreads();
  const int j = sh.j;

  // Accepted prefix, padding and counts.
  for (int t = tid; t < p.out_stride; t += kThreads) {
    int v = -1;
    if (t < j) v = p.draft_ids[q.c0 + t];
    if (t != j) p.out_tokens[(int64_t)r * p.out_stride + t] = v;
  }
  if (tid == 0) {
    p.out_ns[r] = j + 1;
    p.out_nr[r] = K - j;
  }
  int64_t out_j = (int64_t)r * p.out_stride + j;

  if (greedy) {
    if (tid == 0) p.out_tokens[out_j] = sh.amax[j];
    return;
  }

  const int gs = q.g0 + j;
  const bool rejected = j < K;
  const int dj = rejected ? p.draft_ids[q.c0 + j] : -1;
  const float m = sh.m[j], s = sh.s[j];
  Proc pr = q.proc;
  pr.tau = sh.tau[j];
  const int st = sh.state[j];

  if (st >= 0) {
    // Compact top-k row: the race runs over the kept tokens only.
    const float *cv = p.cand_val + (int64_t)gs * kCandCap;
    const int32_t *cix = p.cand_idx + (int64_t)gs * kCandCap;
    const float *qrow = (rejected && p.draft_probs) ? p.draft_probs + (int64_t)(q.c0 + j) * p.dstride : nullptr;
    float part = 0.0f;
    for (int t = tid; t < st; t += kThreads) {
      const int x = cix[t];
      const float pxv = exp2_acc(q.a * (cv[t] - m)) / s;
      float w = pxv;
      if (rejected) {
        if (qrow)
          w = fmaxf(pxv - qrow[x], 0.0f);
        else if (x == dj)
          w = 0.0f;
      }
      sh.ci[t] = x;
      sh.cw[t] = w;
      part += w;
    }
    const float total = block_sum(part, sh.red);
    if (!(total > 0.0f)) {  // residual empty by rounding: race over p
      for (int t = tid; t < st; t += kThreads) sh.cw[t] = exp2_acc(q.a * (cv[t] - m)) / s;
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
  // Chunk weights come from the chunk table, W_c = s_c exp2(a (m_c - m)); the
  // token weights inside a chunk use the streaming pass's own per-element
  // formula exp2(fma(z, a, -hi_c)) (a common factor per chunk cancels in the
  // token race), so a chunk with positive weight always has a token with one.
  const float2 *tab = p.chunk_tab + (int64_t)gs * p.nc_stride;
  const float a = q.a;
  bool excl = rejected && dj >= 0 && dj < p.V;
  const int cd = excl ? dj / kChunk : -1;
  float Wd = 0.0f;
  if (excl) {
    const float2 e = tab[cd];
    const float hi = a * e.x, lo = __builtin_fmaf(a, e.x, -hi);
    float part = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int x = cd * kChunk + 4 * tid + k;
      if (x < p.V && x != dj) part += exp2_acc(__builtin_fmaf(apply_proc(load_logit(p, gs, x), x, pr), a, -hi));
    }
    Wd = e.x > kNegInf ? block_sum(part, sh.red) * exp2_acc(-lo) * exp2_acc(a * (e.x - m)) : 0.0f;
  }
  auto chunk_w = [&](int c) -> float {
    if (excl && c == cd) return Wd;
    const float2 e = tab[c];
    return e.x > kNegInf ? e.y * exp2_acc(a * (e.x - m)) : 0.0f;
  };
  int cstar = chunk_race(p, (uint32_t)gs, p.NC, chunk_w, sh.red);
  if (cstar < 0 && excl) {  // nothing left once d_j is removed (rounding): race over p_j
    excl = false;
    cstar = chunk_race(p, (uint32_t)gs, p.NC, chunk_w, sh.red);
  }
  int x = -1;
  if (cstar >= 0) {
    const float hi = a * tab[cstar].x;
    x = token_race(
        p, (uint32_t)gs, cstar,
        [&](int xx) -> float {
          if (excl && xx == dj) return 0.0f;
          return exp2_acc(__builtin_fmaf(apply_proc(load_logit(p, gs, xx), xx, pr), a, -hi));
        },
        sh.red);
  }
  if (tid == 0) p.out_tokens[out_j] = x;
}

// ---------------------------------------------------------------------------
// Streaming statistics pass.
// ---------------------------------------------------------------------------
template <int DT, int CPW>
__global__ __launch_bounds__(kThreads) void stats_kernel(Params p) {
  using L = Layout<DT>;
  constexpr int NV = L::kVec;
  __shared__ EpiShared sh;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = blockIdx.x / p.nseg;
  const int seg = blockIdx.x - g * p.nseg;
  const int cbase = seg * p.cps + wave;

  // Issue this wave's streaming loads before anything else.
  const char *rowp = static_cast<const char *>(p.logits) + (int64_t)g * p.lstride * L::kBytes;
  u32x4 raw[CPW][NV];
#pragma unroll
  for (int k = 0; k < CPW; ++k) {
    const int c = cbase + kWaves * k;
    if (p.vec_ok && c < p.NC && (c + 1) * kChunk <= p.V) {
      const u32x4 *v = reinterpret_cast<const u32x4 *>(rowp + (int64_t)c * kChunk * L::kBytes);
#pragma unroll
      for (int h = 0; h < NV; ++h) raw[k][h] = __builtin_nontemporal_load(&v[h * 64 + lane]);
    }
  }

  const int r = find_request(p.cu, p.B, g);
  arrive_begin(p.req_ctr + r, p.epoch);
  const Req q = load_req(p, r);
  const bool row_ok = q.cu_ok && g >= q.g0 && g <= q.g0 + q.K && q.mode != kModeInvalid;
  const int st = row_state(p, g);

  if (row_ok && st < 0) {
    Proc pr = q.proc;
    if (st == kRowThreshold) pr.tau = p.cand_tau[g];
    const bool plain = pr.counts == nullptr && !(pr.tau > kNegInf);
    const bool greedy = q.mode == kModeGreedy;
    const float a = q.a;
    float2 *tab = p.chunk_tab + (int64_t)g * p.nc_stride;
#pragma unroll
    for (int k = 0; k < CPW; ++k) {
      const int c = cbase + kWaves * k;
      if (c >= p.NC) break;
      float z[16];
      if (p.vec_ok && (c + 1) * kChunk <= p.V) {
#pragma unroll
        for (int e = 0; e < 16; ++e) z[e] = L::elem(raw[k], e);
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int x = c * kChunk + L::local(e, lane);
          z[e] = x < p.V ? load_logit(p, g, x) : kNegInf;
        }
      }
      if (!plain) {
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
      float2 entry;
      if (greedy) {
        int li = 0x7FFFFFFF;
#pragma unroll
        for (int e = 15; e >= 0; --e)
          if (z[e] == mc) li = L::local(e, lane);
        entry = make_float2(mc, __int_as_float(c * kChunk + wave_min_i(li)));
      } else if (mc > kNegInf) {
        // exp2(a (z - mc)) = exp2(fma(z, a, -hi)) * exp2(-lo), a * mc = hi + lo exactly.
        const float hi = a * mc;
        const float lo = __builtin_fmaf(a, mc, -hi);
        float sacc = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc += exp2_acc(__builtin_fmaf(z[e], a, -hi));
        entry = make_float2(mc, wave_sum(sacc) * exp2_acc(-lo));
      } else {
        entry = make_float2(kNegInf, 0.0f);
      }
      if (lane == 0) tab[c] = entry;
    }
  }

  if (!arrive_end(p.req_ctr + r, p.epoch, (unsigned)((q.cu_ok ? q.K + 1 : 1) * p.nseg), &sh.flag)) return;
  request_epilogue(p, q, sh);
}

// ---------------------------------------------------------------------------
// Residual pass (draft-probs mode, dense rows): chunk masses of
// w = max(0, p_j - q_j) for each rejected request, then the race.
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(kThreads) void resid_kernel(Params p) {
  __shared__ EpiShared sh;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = blockIdx.x / p.nseg;
  const int seg = blockIdx.x - r * p.nseg;
  const int4 rq = p.res_req[r];
  if (rq.w != (int)p.epoch) return;
  arrive_begin(p.res_ctr + r, p.epoch);
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

  if (!arrive_end(p.res_ctr + r, p.epoch, (unsigned)p.nseg, &sh.flag)) return;

  float part = 0.0f;
  for (int c = threadIdx.x; c < p.NC; c += kThreads) part += rt[c];
  const bool fallback = !(block_sum(part, sh.red) > 0.0f);
  const float2 *tab = p.chunk_tab + (int64_t)gs * p.nc_stride;
  const int cstar = chunk_race(
      p, (uint32_t)gs, p.NC,
      [&](int c) -> float {
        if (!fallback) return rt[c];
        const float2 e = tab[c];
        return e.x > kNegInf ? e.y * exp2_acc(a * (e.x - m)) : 0.0f;
      },
      sh.red);
  int x = -1;
  if (cstar >= 0)
    x = token_race(
        p, (uint32_t)gs, cstar,
        [&](int xx) -> float {
          const float px = exp2_acc(a * (apply_proc(load_logit(p, gs, xx), xx, pr) - m)) * inv_s;
          return fallback ? px : fmaxf(px - qrow[xx], 0.0f);
        },
        sh.red);
  if (threadIdx.x == 0) p.out_tokens[(int64_t)r * p.out_stride + j] = x;
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
__global__ __launch_bounds__(kThreads) void post_update_kernel(PostParams p) {
  const int r = blockIdx.x * kThreads + threadIdx.x;
  if (r >= p.B) return;
  int n = p.num_sampled[r];
  if (n <= 0) return;
  const int s = p.idx_mapping[r];
  if (s < 0 || s >= p.num_slots) {
    atomicOr(p.err, SV_ERR_SLOT);
    return;
  }
  n = min(n, p.tokens_stride);
  const int32_t *tok = p.tokens + (int64_t)r * p.tokens_stride;
  for (int i = 0; i < n; ++i) {
    const int t = tok[i];
    if (t >= 0 && t < p.V) atomicAdd(&p.counts[(int64_t)s * p.V + t], 1);
  }
  p.last_sampled[s] = tok[n - 1];
  atomicAdd(&p.num_computed[s], p.query_len[r] - p.num_rejected[r]);
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

hipError_t launch_stats(const Params &p, hipStream_t s) {
  const dim3 grid((unsigned)(p.R * p.nseg));
  if (p.dtype == 1)
    stats_kernel<1, kStatsCPW><<<grid, dim3(kThreads), 0, s>>>(p);
  else
    stats_kernel<0, kStatsCPW><<<grid, dim3(kThreads), 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_resid(const Params &p, hipStream_t s) {
  const dim3 grid((unsigned)(p.B * p.nseg));
  if (p.dtype == 1)
    resid_kernel<1><<<grid, dim3(kThreads), 0, s>>>(p);
  else
    resid_kernel<0><<<grid, dim3(kThreads), 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_dbg_probs(const Params &p, hipStream_t s) {
  const dim3 grid((unsigned)((p.V + kThreads - 1) / kThreads), (unsigned)p.R);
  dbg_kernel<<<grid, dim3(kThreads), 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_post_update(const PostParams &p, hipStream_t s) {
  post_update_kernel<<<dim3((unsigned)((p.B + kThreads - 1) / kThreads)), dim3(kThreads), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace sv
