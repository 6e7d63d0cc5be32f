// sv_topp.hip -- the top-p pass over dense rows.
#include <stdint.h>

#include "sv_common.h"
#include "sv_tiles.h"

namespace sv {

namespace {

// ---------------------------------------------------------------------------
// Top-p pass for dense rows (rows without a candidate list), after the first
// statistics pass.  One workgroup per row.  The kept set is every token whose
// strictly larger logits hold less than top_p of the mass: all z >= z* for a
// boundary logit z*, the row's threshold afterwards (cand_tau).
//
// Weights relative to the row scale m: E = 2^(a (z - m)), below 2^21.  The
// bucket of a weight is its float exponent and top four mantissa bits
// (monotone in E); its units are its 24-bit significand, so the weights of one
// bucket are integer multiples of one power of two and sum exactly, in any
// order.  The row mass S comes from the chunk tables.  Tokens lighter than
// E_skip = (1 - top_p) S / (2 V) weigh less than (1 - top_p) S / 2 together,
// so the boundary lies among the heavier ones: both passes below test most
// tokens with one comparison against a logit bound.
// Pass A: units per bucket of the tokens not below E_skip; an fp64 scan from
// the heaviest bucket finds the bucket b* where the mass above reaches
// top_p S.  Pass B: the tokens of b* go to an LDS list, where a radix select
// on the order-preserving keys, weighted by the units, finds z*; heavier
// tokens are summed per chunk, and the row's chunk table is rewritten as
// (m, kept mass): no further pass.  When b* holds more tokens than the list,
// the rows are not 16-byte aligned or the row has more chunks than the LDS
// tables, z* is selected straight from the row and the row is left to a
// second statistics pass (kRowTopPRedo).
// ---------------------------------------------------------------------------
// The statistics pass's chunk references leave a (z - m) <= 20 (its maxima
// are exact only where a chunk's sum reaches 2^20), so weights reach 2^20:
// the buckets start at 2^21 and run down to 2^-43, below which a token's
// weight is dropped (at most V 2^-43 of a row whose heaviest token weighs 1).
constexpr int kToppBuckets = 1024;                  // buckets kept, the heaviest first
constexpr int kToppTop = ((127 + 21) << 23) >> 19;  // bucket of E = 2^21
constexpr int kToppList = 2048;
constexpr int kToppMaxNC = 512;   // chunks per row whose sums live in LDS (V <= 524288)
// Threads per row: eight waves when most rows are dense (one row per
// workgroup leaves few waves per CU); four with top-k on, where most rows have
// candidate lists and their workgroups return at once.
constexpr int kTpMaxWaves = 8;

struct ToppShared {
  unsigned long long mass[kToppBuckets];  // units per bucket, index kToppTop - bucket
  float lz[kToppList];
  int lx[kToppList];
  float part[kToppMaxNC * 4];            // kept weight per chunk, one slot per wave covering it
  unsigned long long lsum[kToppMaxNC];   // kept list units per chunk
  float tail[8];
  float wmax[kTpMaxWaves];
  double wsum[kTpMaxWaves];
  unsigned long long need;
  int n, sel;
};

// Weight, bucket and units of a (processed) logit; z = -inf weighs 0, whose
// bucket lies below every kept one.  The weight is the epilogue's
// 2^(a (z - m)), with the same roundings, so the kept masses written to the
// chunk table normalise exactly the probabilities it computes.
__device__ __forceinline__ float tp_weight(float z, float a, float m) { return exp2_acc(a * (z - m)); }
__device__ __forceinline__ int tp_bucket(float E) { return (int)(__float_as_uint(E) >> 19); }
__device__ __forceinline__ unsigned long long tp_units(float E) { return (__float_as_uint(E) & 0x7FFFFFu) | 0x800000u; }
// Binary exponent of one unit of bucket b.
__device__ __forceinline__ int tp_unit_exp(int b) { return (b >> 4) - 150; }
// Smallest logit whose weight can reach E (a conservative bound: 0.01 below in
// log2 units, far beyond the rounding of the weight).
__device__ __forceinline__ float tp_logit_bound(float E, float m, float a) { return m + (__log2f(E) - 0.01f) / a; }

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

// Super-tiles in flight per workgroup in the top-p passes.
template <int DT>
constexpr int kToppDepth = 2;

// Calls tile(base, z[kTopkPer]) for every super-tile of an aligned row
// (kToppDepth in flight); logits of tokens at or past vfull = V - V % VW read
// as -inf.
template <int DT, int NT, class F>
__device__ __forceinline__ void stream_tiles(const Params &p, int g, int vfull, F tile) {
  constexpr int D = kToppDepth<DT>;
  constexpr int T = kTopkPer * NT;
  TopkRaw<DT> r[D];
#pragma unroll
  for (int i = 0; i < D; ++i) topk_issue<DT, NT>(p, g, i * T, vfull, r[i]);
  for (int base = 0; base < vfull; base += D * T) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const int b = base + i * T;
      if (b >= vfull) break;
      float z[kTopkPer];
      topk_decode<DT, NT>(b, vfull, r[i], z);
      topk_issue<DT, NT>(p, g, b + D * T, vfull, r[i]);
      tile(b, z);
    }
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
// calls its callback with (z, units) for its share): the largest key whose
// strictly larger keys hold less than `need` units.
template <class EACH>
__device__ __forceinline__ float topp_select(ToppShared &sh, EACH each, unsigned long long need) {
  uint32_t prefix = 0, mask = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (threadIdx.x < 256) sh.mass[threadIdx.x] = 0;
    __syncthreads();
    each([&](float z, unsigned long long w) {
      const uint32_t key = ukey(z);
      if ((key & mask) == prefix) atomicAdd(&sh.mass[(key >> shift) & 0xFFu], w);
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
  const Req q = lookup_req(p, g);
  const int st = p.has_topk ? p.cand_n[g] : kRowDense;
  const bool use = q.cu_ok && g >= q.g0 && g <= q.g0 + q.K && q.mode == kModeSample && q.top_p < 1.0f && st < 0;
  if (!use) {
    if (tid == 0 && !p.has_topk) p.cand_n[g] = kRowDense;  // later kernels read every row's state
    return;
  }
  Proc pr = q.proc;
  pr.tau = st == kRowThreshold ? p.cand_tau[g] : kNegInf;
  const float a = q.a, tau = pr.tau;

  // Row scale m and mass S (relative to 2^(a m)) from the first pass's chunk table.
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
  double ls = 0.0;
  for (int c = tid; c < p.NC; c += NT) {
    const float2 e = tab[c];
    if (e.x > kNegInf) ls += (double)(e.y * exp2_acc(a * (e.x - m)));
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) ls += __shfl_xor(ls, d, 64);
  if (lane == 0) sh.wsum[wave] = ls;
  __syncthreads();
  double S = 0.0;
#pragma unroll
  for (int w = 0; w < (NT / 64); ++w) S += sh.wsum[w];
  const double bound = (double)q.top_p * S;
  const float zskip = tp_logit_bound((float)((1.0 - (double)q.top_p) * S / (2.0 * p.V)), m, a);

  constexpr int VW = TopkRaw<DT>::VW;
  const int vfull = p.V - p.V % VW;
  // Aligned rows without a penalty take the branch-free tile loops.
  const bool tiles = p.vec_ok && pr.counts == nullptr;

  // Pass A: units per bucket of the tokens not below E_skip.
  for (int j = tid; j < kToppBuckets; j += NT) sh.mass[j] = 0;
  __syncthreads();
  auto count = [&](float z) {
    const float E = tp_weight(z, a, m);
    const int i = max(kToppTop - tp_bucket(E), 0);  // never clamped: E < 2^21
    if (i < kToppBuckets) atomicAdd(&sh.mass[i], tp_units(E));
  };
  // Aligned rows: whole super-tiles (penalties applied per token); the last
  // V % VW tokens, and unaligned rows, one token per thread.
  if (p.vec_ok) {
    stream_tiles<DT, NT>(p, g, vfull, [&](int base, float (&z)[kTopkPer]) {
#pragma unroll
      for (int e = 0; e < kTopkPer; ++e) {
        const int x = topk_tok<DT, NT>(base, e);
        float zz = z[e];
        if (!tiles && x < vfull) zz = apply_proc(zz, x, pr);  // penalty rows
        zz = zz < tau ? kNegInf : zz;
        if (zz >= zskip) count(zz);
      }
    });
    if (vfull + tid < p.V) {
      const float z = apply_proc(load_logit(p, g, vfull + tid), vfull + tid, pr);
      if (z >= zskip) count(z);
    }
  } else {
    stream_row<DT, NT>(p, g, [&](int x, float raw) {
      const float z = apply_proc(raw, x, pr);
      if (z >= zskip) count(z);
    });
  }
  __syncthreads();
  // Scan (wave 0): lane l owns buckets 16 l .. 16 l + 15 (heaviest first); fp64
  // in a fixed order.
  if (wave == 0) {
    double own = 0.0;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      own += __builtin_ldexp((double)sh.mass[16 * lane + i], tp_unit_exp(kToppTop - (16 * lane + i)));
    double incl = own;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const double o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    double acc = incl - own;
    int hit = -1;
    double hit_above = 0.0;
    for (int i = 0; i < 16; ++i) {
      const unsigned long long h = sh.mass[16 * lane + i];
      if (h == 0) continue;
      const double hm = __builtin_ldexp((double)h, tp_unit_exp(kToppTop - (16 * lane + i)));
      if (acc + hm >= bound) {
        hit = 16 * lane + i;
        hit_above = acc;
        break;
      }
      acc += hm;
    }
    const unsigned long long hits = __ballot(hit >= 0);
    // the first crossing; none only through rounding (S from the tables, top_p
    // near 1): the lightest non-empty bucket
    const unsigned long long nonempty = __ballot(own > 0.0);
    const int src = hits ? __ffsll((long long)hits) - 1 : 63 - __builtin_clzll(nonempty | 1ull);
    if (lane == src) {
      if (hit < 0) {
        for (int i = 15; i >= 0; --i)
          if (sh.mass[16 * lane + i]) {
            hit = 16 * lane + i;
            hit_above = incl - __builtin_ldexp((double)sh.mass[hit], tp_unit_exp(kToppTop - hit));
            break;
          }
        if (hit < 0) hit = 16 * lane;
      }
      sh.sel = kToppTop - hit;
      // units of bucket b* still needed to reach the bound
      const double rest = __builtin_ceil(__builtin_ldexp(bound - hit_above, -tp_unit_exp(kToppTop - hit)));
      sh.need = rest < 1.0 ? 1ull : (unsigned long long)rest;
      sh.n = 0;
    }
  }
  __syncthreads();
  const int bstar = sh.sel;
  const int ustar = tp_unit_exp(bstar);
  const unsigned long long need = sh.need;
  // every token of bucket b* or heavier is at or above this logit
  const float zb = tp_logit_bound(__uint_as_float((uint32_t)bstar << 19), m, a);
  const bool direct = p.vec_ok && p.NC <= kToppMaxNC;

  // Pass B: bucket b* into the list, the heavier tokens' weight per chunk
  // (per vector, one wave sum into a slot of its own: a fixed order).
  bool redo = !direct;
  if (direct) {
    for (int c = tid; c < p.NC * 4; c += NT) sh.part[c] = 0.0f;
    for (int c = tid; c < p.NC; c += NT) sh.lsum[c] = 0;
    if (tid < 8) sh.tail[tid] = 0.0f;
    __syncthreads();
    constexpr int WPC = kChunk / (64 * VW);  // waves covering one chunk in a super-tile
    auto token = [&](int x, float z, float &acc) {
      if (!(z >= zb)) return;  // most tokens: lighter than bucket b*
      const float E = tp_weight(z, a, m);
      const int b = tp_bucket(E);
      if (b > bstar) acc += E;
      if (b == bstar) {
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
        const float sum = __ballot(acc != 0.0f) ? wave_sum(acc) : 0.0f;
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
          for (int e = tid; e < n; e += NT) fn(sh.lz[e], tp_units(tp_weight(sh.lz[e], a, m)));
        },
        need);
    // Kept list tokens into their chunks (units), then the new table.
    for (int e = tid; e < n; e += NT)
      if (sh.lz[e] >= zstar) atomicAdd(&sh.lsum[sh.lx[e] / kChunk], tp_units(tp_weight(sh.lz[e], a, m)));
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
      sc += (float)__builtin_ldexp((double)sh.lsum[c], ustar);
      tab[c] = make_float2(m, sc);
    }
  } else {
    zstar = topp_select(
        sh, [&](auto fn) {
          stream_row<DT, NT>(p, g, [&](int x, float raw) {
            const float z = apply_proc(raw, x, pr);
            if (z >= zb) {
              const float E = tp_weight(z, a, m);
              if (tp_bucket(E) == bstar) fn(z, tp_units(E));
            }
          });
        },
        need);
  }
  if (tid == 0) {
    p.cand_tau[g] = zstar;
    p.cand_n[g] = redo ? kRowTopPRedo : kRowTopP;
  }
}

}  // namespace

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

}  // namespace sv
