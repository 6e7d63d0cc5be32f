// sv_topk.hip -- the top-k pass: per target row, the exact k-th largest processed logit and the kept tokens.
#include <stdint.h>

#include "sv_common.h"
#include "sv_tiles.h"

namespace sv {

namespace {

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
  // barrier-free path: each wave's histogram, count, threshold; overflow flag
  unsigned whist[kWaves][256];
  int wn[kWaves];
  float wth[kWaves];
  int wflag;
};
static_assert(kBuf >= 2 * kCandCap, "the id-ordered kept list is staged in the upper half of the buffer");


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

// Candidates appended with their raw logit (penalty still to apply) carry
// index | kUnresolved.
constexpr int kUnresolved = (int)0x80000000;

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

// Resolves (applies the penalty to) the unresolved entries whose value is >=
// t; returns, the same in every thread, whether any value changed.  The
// counts of a thread's entries are loaded four at a time.
__device__ __forceinline__ bool resolve_at_least(TopkShared &sh, int n, float t, const Proc &pr) {
  constexpr int M = 4;  // entries per batch (two batches: the registers of the tiles in flight stay free)
  bool changed = false;
#pragma unroll
  for (int h = 0; h < kBuf / kThreads; h += M) {
    int xs[M], c[M];
    float vs[M];
    bool need[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int e = threadIdx.x + (h + m) * kThreads;
      xs[m] = e < n ? sh.bi[e] : 0;
      vs[m] = e < n ? sh.bv[e] : kNegInf;
      need[m] = e < n && (xs[m] & kUnresolved) && vs[m] >= t;
    }
#pragma unroll
    for (int m = 0; m < M; ++m) c[m] = need[m] ? pr.counts[xs[m] & 0x7FFFFFFF] : 0;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      if (need[m]) {
        const int e = threadIdx.x + (h + m) * kThreads;
        const float z = c[m] > 0 ? penalize(vs[m], c[m], pr) : vs[m];
        changed |= z != vs[m];
        sh.bv[e] = z;
        sh.bi[e] = xs[m] & 0x7FFFFFFF;
      }
    }
  }
  return __syncthreads_or(changed) != 0;
}

// The k-th largest processed value among the n buffer entries (k <= n), where
// unresolved entries hold raw logits that are never below their processed
// value (penalties that cannot raise a logit).  Only entries that can reach
// the k-th largest are resolved: take t = the k-th largest current value,
// resolve the unresolved entries >= t, and repeat while that changed a value.
// At the end every entry >= t holds its processed value and every other entry
// is below t, so t is exact.
__device__ __forceinline__ float select_tau(TopkShared &sh, int n, int k, const Proc &pr) {
  for (;;) {
    const float t = buffer_kth(sh, n, k);
    if (pr.counts == nullptr || !resolve_at_least(sh, n, t, pr)) return t;
  }
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

// Offsets of this thread's passers within a super-tile: an exclusive prefix
// over the wave, and one LDS atomic per wave (on tile_n[par]) for the wave's
// base.  Returns the wave's base; excl receives the thread's offset in the wave.
__device__ __forceinline__ int wave_offsets(TopkShared &sh, int npass, int par, int &excl) {
  const int lane = threadIdx.x & 63;
  int incl = npass;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  excl = incl - npass;
  const int wtot = __shfl(incl, 63, 64);
  int wb = 0;
  if (lane == 63 && wtot > 0) wb = atomicAdd(&sh.tile_n[par], wtot);
  return __shfl(wb, 63, 64);
}

// ---------------------------------------------------------------------------
// Barrier-free filter, for k <= kWaveTopk on aligned rows.  Each wave keeps
// its own candidates, in its own kSeg-entry segment of the buffer, with its own
// threshold, and selects within the segment (wave-level steps, no workgroup
// barrier) when it fills.  A wave's k-th largest never exceeds the row's, so
// the union of the segments holds every token of the row's top k; they are
// merged once at the end, where the exact selection of the two-barrier path
// takes over.  (Two barriers per super-tile cost that path about a quarter of
// its time on 608 KB rows.)
// ---------------------------------------------------------------------------
constexpr int kSeg = kBuf / kWaves;
constexpr int kWaveTopk = 128;

// Exclusive prefix of npass over the wave, and the wave's total (uniform).
__device__ __forceinline__ void wave_scan(int npass, int &excl, int &wtot) {
  const int lane = threadIdx.x & 63;
  int incl = npass;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  excl = incl - npass;
  wtot = __builtin_amdgcn_readfirstlane(__shfl(incl, 63, 64));
}

// k-th largest value among the n entries of segment s (1 <= k <= n): MSD radix
// select over order-preserving keys with the wave's own 256-bin histogram.
__device__ __forceinline__ float wave_kth(TopkShared &sh, int s, int n, int k) {
  const int lane = threadIdx.x & 63;
  unsigned *h = sh.whist[s];
  const float *bv = sh.bv + s * kSeg;
  uint32_t prefix = 0, mask = 0;
  int want = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) h[lane + 64 * i] = 0;
    for (int e = lane; e < n; e += 64) {
      const uint32_t key = ukey(bv[e]);
      if ((key & mask) == prefix) atomicAdd(&h[(key >> shift) & 0xFFu], 1u);
    }
    // lane l holds bins 255 - 4l .. 252 - 4l (descending): the lane whose
    // bins the want-th largest falls in picks the digit
    int hh[4], own = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hh[i] = (int)h[255 - 4 * lane - i];
      own += hh[i];
    }
    int incl = own;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    const int before = incl - own;
    const unsigned long long here = __ballot(before < want && incl >= want);
    const int src = __ffsll((long long)here) - 1;  // one lane: the matching keys number at least want
    int sel = 0, nwant = want;
    if (lane == src) {
      int acc = before;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (acc + hh[i] >= want) {
          sel = 255 - 4 * lane - i;
          nwant = want - acc;
          break;
        }
        acc += hh[i];
      }
    }
    sel = __builtin_amdgcn_readlane(sel, src);
    want = __builtin_amdgcn_readlane(nwant, src);
    prefix |= (uint32_t)sel << shift;
    mask |= 0xFFu << shift;
  }
  return ukey_val(prefix);
}

// Applies the penalty to the unresolved entries of segment s that are >= t;
// whether any value changed (uniform).
__device__ __forceinline__ bool wave_resolve(TopkShared &sh, int s, int n, float t, const Proc &pr) {
  const int lane = threadIdx.x & 63;
  float *bv = sh.bv + s * kSeg;
  int *bi = sh.bi + s * kSeg;
  bool changed = false;
#pragma unroll
  for (int h = 0; h < kSeg / 64; h += 4) {
    int xs[4], c[4];
    float vs[4];
    bool need[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int e = lane + 64 * (h + m);
      xs[m] = e < n ? bi[e] : 0;
      vs[m] = e < n ? bv[e] : kNegInf;
      need[m] = e < n && (xs[m] & kUnresolved) && vs[m] >= t;
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) c[m] = need[m] ? pr.counts[xs[m] & 0x7FFFFFFF] : 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (need[m]) {
        const int e = lane + 64 * (h + m);
        const float z = c[m] > 0 ? penalize(vs[m], c[m], pr) : vs[m];
        changed |= z != vs[m];
        bv[e] = z;
        bi[e] = xs[m] & 0x7FFFFFFF;
      }
    }
  }
  return __ballot(changed) != 0;
}

// select_tau within segment s.
__device__ __forceinline__ float wave_select_tau(TopkShared &sh, int s, int n, int k, const Proc &pr) {
  for (;;) {
    const float t = wave_kth(sh, s, n, k);
    if (pr.counts == nullptr || !wave_resolve(sh, s, n, t, pr)) return t;
  }
}

// Keeps the entries of segment s that are >= t, compacted in order (every
// entry is read before any is written); the new count (uniform).
__device__ __forceinline__ int wave_keep(TopkShared &sh, int s, int n, float t) {
  const int lane = threadIdx.x & 63;
  constexpr int M = kSeg / 64;
  float *bv = sh.bv + s * kSeg;
  int *bi = sh.bi + s * kSeg;
  float v[M];
  int x[M];
  bool keep[M];
#pragma unroll
  for (int i = 0; i < M; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < n ? bv[e] : kNegInf;
    x[i] = e < n ? bi[e] : 0;
    keep[i] = e < n && v[i] >= t;
  }
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < M; ++i) {
    const unsigned long long b = __ballot(keep[i]);
    if (keep[i]) {
      const int pos = cnt + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
      bv[pos] = v[i];
      bi[pos] = x[i];
    }
    cnt += __popcll(b);
  }
  return cnt;
}

template <int DT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void topk_kernel(Params p) {
  __shared__ TopkShared sh;
  const int g = blockIdx.x;
  constexpr int kFirstPer = kBuf / kThreads;  // the first kBuf tokens: kFirstPer per thread
  constexpr int VW = TopkRaw<DT>::VW;
  const int vfull = p.V - p.V % VW;
  // Aligned rows: the row's first loads (its first kBuf tokens and the first
  // two streaming super-tiles) do not depend on its request and are issued
  // before the lookup; the last V % VW tokens are taken apart at the end.
  TopkRaw<DT, kFirstPer> r0;
  TopkRaw<DT> ra, rb;
  if (p.vec_ok) {
    topk_issue<DT, kThreads, kFirstPer>(p, g, 0, vfull, r0);
    topk_issue<DT>(p, g, kBuf, vfull, ra);
    topk_issue<DT>(p, g, kBuf + kTopkTile, vfull, rb);
  }
  const Req q = lookup_req(p, g);  // one wide load in the common case
  const int r = q.r;
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
    sh.wflag = 0;
  }
  __syncthreads();
  // Streaming filter in super-tiles of kTopkTile tokens, kTopkPer per thread
  // (vector loads, all in flight together).  A token passes when its processed
  // logit is >= the running threshold theta (a lower bound of tau_k: the k-th
  // largest of a subset of the row).  With a repetition penalty >= 1 and
  // frequency and presence penalties >= 0 the penalties never raise a logit
  // (each step rounds monotonically), so later super-tiles test the raw logit and the counts
  // of the few passers are read only when a selection needs them.  Two barriers
  // per super-tile: one to count the passers (one LDS atomic per wave; the
  // candidate buffer is compacted first if they would not fit), one after they
  // are appended.
  const bool pen = pr.counts != nullptr;
  const bool raw_first = !pen || (pr.theta >= 1.0f && pr.freq >= 0.0f && pr.pres >= 0.0f);
  bool overflow = k > kCandCap;
  const bool wpath = p.vec_ok && k <= kWaveTopk;  // the barrier-free filter
  int wn0 = 0;  // its first passers in this wave's segment
  if (!overflow && k <= kThreads) {
    // First threshold: the k-th largest of the threads' maxima over the first
    // kBuf tokens (k distinct tokens reach it, so it is a lower bound of
    // tau_k), found by wave 0 alone; then the first tokens that reach it are
    // appended.  Values and counts are loaded together.
    float z[kFirstPer];
    int cnt[kFirstPer];
    if (pen) {
#pragma unroll
      for (int e = 0; e < kFirstPer; ++e) cnt[e] = pr.counts[min(topk_tok<DT>(0, e), p.V - 1)];
    }
    if (p.vec_ok)
      topk_decode<DT, kThreads, kFirstPer>(0, vfull, r0, z);
    else
      load_topk_tile<DT, kFirstPer>(p, g, 0, z);
    float tmax = kNegInf;
#pragma unroll
    for (int e = 0; e < kFirstPer; ++e) {
      if (pen && topk_tok<DT>(0, e) < p.V && cnt[e] > 0) z[e] = penalize(z[e], cnt[e], pr);
      if (z[e] > kNegInf) tmax = fmaxf(tmax, z[e]);
    }
    sh.bv[threadIdx.x] = tmax;
    __syncthreads();
    if (threadIdx.x < 64) {
      // MSD bitwise select of the k-th largest of 256 keys, four per lane.
      const int lane = threadIdx.x;
      uint32_t key[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) key[i] = ukey(sh.bv[4 * lane + i]);
      uint32_t prefix = 0;
      int want = k;
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t hi = bit == 31 ? 0u : ~0u << (bit + 1);
        int ones = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) ones += __popcll(__ballot((key[i] & hi) == prefix && ((key[i] >> bit) & 1u)));
        if (ones >= want)
          prefix |= 1u << bit;
        else
          want -= ones;
      }
      if (lane == 0) sh.theta = ukey_val(prefix);
    }
    __syncthreads();
    const float th = sh.theta;
    int npass = 0;
#pragma unroll
    for (int e = 0; e < kFirstPer; ++e) {
      if (!(z[e] >= th && z[e] > kNegInf)) z[e] = kNegInf;
      npass += z[e] > kNegInf ? 1 : 0;
    }
    int excl;
    if (wpath) {  // into this wave's segment (kFirstPer per lane: it fits)
      int wtot;
      wave_scan(npass, excl, wtot);
      int pos = (int)(threadIdx.x >> 6) * kSeg + excl;
#pragma unroll
      for (int e = 0; e < kFirstPer; ++e) {
        if (z[e] > kNegInf) {
          sh.bv[pos] = z[e];
          sh.bi[pos] = topk_tok<DT>(0, e);
          ++pos;
        }
      }
      wn0 = wtot;
    } else {
      const int wb = wave_offsets(sh, npass, 0, excl);
      __syncthreads();
      const int n = sh.tile_n[0];
      int pos = wb + excl;
#pragma unroll
      for (int e = 0; e < kFirstPer; ++e) {
        if (z[e] > kNegInf) {
          sh.bv[pos] = z[e];
          sh.bi[pos] = topk_tok<DT>(0, e);
          ++pos;
        }
      }
      __syncthreads();  // every thread has read tile_n[0]
      if (threadIdx.x == 0) {
        sh.n = n;
        sh.tile_n[0] = 0;
      }
      __syncthreads();
    }
  } else if (!overflow) {
    // k above the thread count: theta = the exact k-th largest of the first
    // kBuf tokens.
    float z[kFirstPer];
    if (p.vec_ok)
      topk_decode<DT, kThreads, kFirstPer>(0, vfull, r0, z);
    else
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
    int n0 = sh.n;
    const float th = sh.theta;
    if (!raw_first) penalize_tile<DT>(p, pr, base, z);  // a penalty < 1 can raise logits: test processed ones
    int npass = 0;
#pragma unroll
    for (int e = 0; e < kTopkPer; ++e) {
      const int x = topk_tok<DT>(base, e);
      z[e] = (x < p.V && z[e] >= th && z[e] > kNegInf) ? z[e] : kNegInf;
      npass += z[e] > kNegInf ? 1 : 0;
    }
    int excl;
    int wb = wave_offsets(sh, npass, par, excl);
    __syncthreads();
    if (threadIdx.x == 0) sh.tile_n[par ^ 1] = 0;  // read last in the previous super-tile
    int tot = sh.tile_n[par];
    if (n0 + tot > kBuf) {
      // Not enough room: theta becomes the k-th largest kept candidate
      // (penalties applied first); this super-tile's passers are re-tested.
      if (n0 < k) {
        overflow = true;  // fewer than k finite logits so far and a full tile: exact radix select below
      } else {
        const float t = select_tau(sh, n0, k, pr);
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
        wb = wave_offsets(sh, npass, par, excl);
        __syncthreads();
        n0 = sh.n;
        tot = sh.tile_n[par];
        overflow = n0 + tot > kBuf;  // ties at theta: exact radix select below
        __syncthreads();  // every thread has read the counts before sh.n changes
      }
    }
    if (overflow) return;
    // Every thread has read n0 (before the barrier above): sh.n can move on.
    if (threadIdx.x == 0) sh.n = n0 + tot;
    const int flag = raw_first && pen ? kUnresolved : 0;  // raw logits: penalty applied at the next selection
    int pos = n0 + wb + excl;
#pragma unroll
    for (int e = 0; e < kTopkPer; ++e) {
      if (z[e] > kNegInf) {
        sh.bv[pos] = z[e];
        sh.bi[pos] = topk_tok<DT>(base, e) | flag;
        ++pos;
      }
    }
    __syncthreads();
  };
  if (p.vec_ok && wpath) {
    // Barrier-free: each wave filters its own tokens into its own segment,
    // two super-tiles in flight as below.
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int wn = wn0;
    float wth = sh.theta;
    bool wover = false;
    const int flag = raw_first && pen ? kUnresolved : 0;
    auto wave_tile = [&](int base, float (&z)[kTopkPer]) {
      if (!raw_first) penalize_tile<DT>(p, pr, base, z);  // a penalty < 1 can raise logits: test processed ones
      // One comparison per token (-inf never passes; tokens past the row
      // decode as -inf), and nothing more when no token of the wave passes:
      // the common case once the threshold has risen.
      const float th = fmaxf(wth, -__FLT_MAX__);
      int npass = 0;
#pragma unroll
      for (int e = 0; e < kTopkPer; ++e) npass += z[e] >= th ? 1 : 0;
      if (__ballot(npass != 0) == 0) return;
#pragma unroll
      for (int e = 0; e < kTopkPer; ++e)
        if (!(z[e] >= th)) z[e] = kNegInf;
      int excl, wtot;
      wave_scan(npass, excl, wtot);
      if (wn + wtot > kSeg) {
        // Full: the wave's threshold becomes the k-th largest of its
        // candidates (penalties applied first), then this super-tile's passers
        // are tested again.  Fewer than k candidates or still no room: the
        // exact radix select below.
        if (wn < k) {
          wover = true;
          return;
        }
        const float t = wave_select_tau(sh, wv, wn, k, pr);
        wn = wave_keep(sh, wv, wn, t);
        wth = t;
        npass = 0;
#pragma unroll
        for (int e = 0; e < kTopkPer; ++e) {
          if (!(z[e] >= t)) z[e] = kNegInf;
          npass += z[e] > kNegInf ? 1 : 0;
        }
        wave_scan(npass, excl, wtot);
        if (wn + wtot > kSeg) {
          wover = true;
          return;
        }
      }
      int pos = wv * kSeg + wn + excl;
#pragma unroll
      for (int e = 0; e < kTopkPer; ++e) {
        if (z[e] > kNegInf) {
          sh.bv[pos] = z[e];
          sh.bi[pos] = topk_tok<DT>(base, e) | flag;
          ++pos;
        }
      }
      wn += wtot;
    };
    int base = kBuf;
    while (base < vfull && !wover) {
      float z[kTopkPer];
      topk_decode<DT>(base, vfull, ra, z);
      topk_issue<DT>(p, g, base + 2 * kTopkTile, vfull, ra);
      wave_tile(base, z);
      base += kTopkTile;
      if (base >= vfull || wover) break;
      topk_decode<DT>(base, vfull, rb, z);
      topk_issue<DT>(p, g, base + 2 * kTopkTile, vfull, rb);
      wave_tile(base, z);
      base += kTopkTile;
    }
    if (lane == 0) {
      sh.wn[wv] = wn;
      sh.wth[wv] = wth;
      if (wover) atomicOr(&sh.wflag, 1);
    }
    __syncthreads();
    overflow = sh.wflag != 0;
    if (!overflow) {
      // Merge the segments into buffer[0, n): every entry read, then written.
      constexpr int M = kSeg / 64;
      float mv[M];
      int mi[M];
#pragma unroll
      for (int i = 0; i < M; ++i) {
        const int e = lane + 64 * i;
        mv[i] = e < wn ? sh.bv[wv * kSeg + e] : 0.0f;
        mi[i] = e < wn ? sh.bi[wv * kSeg + e] : 0;
      }
      int off = 0, tot = 0;
      float th = kNegInf;  // each wave's threshold is a lower bound of tau_k: the largest one
#pragma unroll
      for (int v = 0; v < kWaves; ++v) {
        if (v < wv) off += sh.wn[v];
        tot += sh.wn[v];
        th = fmaxf(th, sh.wth[v]);
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < M; ++i) {
        const int e = lane + 64 * i;
        if (e < wn) {
          sh.bv[off + e] = mv[i];
          sh.bi[off + e] = mi[i];
        }
      }
      if (threadIdx.x == 0) {
        sh.n = tot;
        sh.theta = th;
      }
      __syncthreads();
    }
  }
  if (p.vec_ok) {
    // Two super-tiles in flight: the next one's loads are issued before this
    // one is filtered (the first two at the start, above).
    int base = kBuf, par = 0;
    while (!wpath && base < vfull && !overflow) {
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
        const float t = select_tau(sh, n, k, pr);
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
  float tau;
  int ncand = -1;
  if (!overflow) {
    const int n = sh.n;
    if (n < k) {
      tau = kNegInf;  // fewer than k finite logits: nothing is removed
    } else {
      // exact tau; the kept entries (>= tau) all hold processed values
      tau = select_tau(sh, n, k, pr);
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

}  // namespace

hipError_t launch_topk(const Params &p, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  const void *fn = p.dtype == 1 ? reinterpret_cast<const void *>(&topk_kernel<1>)
                                : reinterpret_cast<const void *>(&topk_kernel<0>);
  return launch_timed(fn, dim3((unsigned)p.R), p, s, t0, t1);
}

}  // namespace sv
