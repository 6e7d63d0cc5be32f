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
// Waves per row: up to sixteen (the register-resident pass below); the
// two-pass kernel takes eight when most rows are dense (one row per workgroup
// leaves few waves per CU), four with top-k on, where most rows have
// candidate lists and their workgroups return at once.
constexpr int kTpMaxWaves = 16;

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

// Boundary bucket (wave 0 scans, all threads call; a barrier follows): with
// sh.mass holding each bucket's units, lane l owns buckets 16 l .. 16 l + 15
// (heaviest first) and an fp64 scan in a fixed order finds the first bucket
// b* where the mass above reaches `bound`.  Sets sh.sel = b*, sh.need = the
// units of b* still needed to reach the bound, sh.n = 0.  It runs once per
// row on one wave; its loops stay rolled so that it needs few registers
// beside a row held in them.
__device__ __forceinline__ void topp_scan(ToppShared &sh, double bound) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    double own = 0.0;
#pragma unroll 1
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
#pragma unroll 1
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
    // the first crossing; none only through the rounding of S against the
    // bucket sums (top_p near 1): the lightest non-empty bucket
    const unsigned long long nonempty = __ballot(own > 0.0);
    const int src = hits ? __ffsll((long long)hits) - 1 : 63 - __builtin_clzll(nonempty | 1ull);
    if (lane == src) {
      if (hit < 0) {
#pragma unroll 1
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
  topp_scan(sh, bound);
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

// ---------------------------------------------------------------------------
// Top-p call over rows held in registers.  For aligned bf16 rows of at most
// kResidentMaxChunks chunks, without top-k or penalties, one workgroup of
// kResidentThreads threads takes one target row: wave w loads chunks w,
// w + 16, ... once, in the streaming pass's layout (two 16-byte vectors per
// lane and chunk; 64 registers hold the row), and every step runs from those
// registers, so the call reads each row once and needs no streaming pass.
// Rows without a nucleus (greedy requests, top_p = 1) get the streaming
// pass's chunk statistics.  Nucleus rows: the row scale m, the row mass S as
// a sum of the weights 2^(a (z - m)) (fp32 over each lane's 16 tokens of a
// chunk, fp64 beyond), then the boundary.  Without penalties all tokens of
// one bf16 value weigh the same, so counting the tokens of each value near
// the top (one LDS increment per token, no weight) gives exact masses, and a
// scan over the values finds z* itself; the kept mass per chunk then takes one
// more pass.  When the nucleus reaches below that window of values, the
// bucket steps of the two-pass kernel above run on the registers instead
// (histogram of units, boundary bucket, list and weighted select).
// The pass is bound by the VALU and LDS work per token rather than by HBM:
// while a workgroup computes, its CU has no loads in flight.
// ---------------------------------------------------------------------------
constexpr int kResWaves = kResidentThreads / 64;
constexpr int kResSlots = kResidentMaxChunks / kResWaves;  // chunks per wave
static_assert(kResidentThreads == kToppBuckets && kResWaves <= kTpMaxWaves, "one bucket per thread to clear");
static_assert(kResidentMaxChunks <= kToppMaxNC, "chunk sums in LDS");

// An empty asm statement that "rewrites" one chunk's registers: placed before
// each use of a chunk in each pass, so that the compiler decodes the logits
// and computes the weights there (a few instructions each) instead of keeping
// those of many chunks live at once, which would not fit the 128 registers a
// lane has.
__device__ __forceinline__ void res_fence(u32x4 (&w)[2]) { asm volatile("" : "+v"(w[0]), "+v"(w[1])); }

// Order-preserving 16-bit key of a bf16 bit pattern (larger value, larger key)
// and back.
__device__ __forceinline__ uint32_t res_key(uint32_t b) { return b ^ ((b & 0x8000u) ? 0xFFFFu : 0x8000u); }
__device__ __forceinline__ float res_val(uint32_t k) { return __uint_as_float((k ^ ((k & 0x8000u) ? 0x8000u : 0xFFFFu)) << 16); }
// bf16 bit pattern of element e of a chunk in the layout of Layout<1>.
__device__ __forceinline__ uint32_t res_bits(const u32x4 (&w)[2], int e) {
  const u32x4 x = w[e >> 3];
  const int k = e & 7;
  const uint32_t u = (k >> 1) == 0 ? x.x : (k >> 1) == 1 ? x.y : (k >> 1) == 2 ? x.z : x.w;
  return (k & 1) ? (u >> 16) : (u & 0xFFFFu);
}

constexpr int kResValueBins = 4096;  // bf16 values below the row maximum counted one by one
struct ResShared {
  ToppShared t;
  unsigned cnt[kResValueBins];
  int wmin[kResWaves];
};

__global__ __launch_bounds__(kResidentThreads) void topp_resident_kernel(Params p) {
  using L = Layout<1>;
  __shared__ ResShared rs;
  ToppShared &sh = rs.t;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = blockIdx.x;
  // The row first.  Vector h of chunk c = wave + 16 j holds tokens
  // c C + 512 h + 8 lane .. + 7; vectors at or past V (a multiple of 8) and
  // chunks past the row read as -inf.
  u32x4 v[kResSlots][2];
  {
    const u32x4 *row = reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(p.logits) + (int64_t)g * p.lstride);
    const u32x4 ninf = {0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u};
#pragma unroll
    for (int j = 0; j < kResSlots; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int x0 = (wave + kResWaves * j) * kChunk + 512 * h + 8 * lane;
        v[j][h] = x0 < p.V ? __builtin_nontemporal_load(&row[x0 >> 3]) : ninf;
      }
  }
  const Req q = lookup_req(p, g);
  const RowInfo ri = row_info_of(p, q, g);
  if (ri.mode == kModeInvalid) {  // no table; the epilogue flags the request
    if (tid == 0) p.cand_n[g] = kRowDense;
    return;
  }
  if (ri.mode != kModeSample || !(q.top_p < 1.0f)) {
#pragma unroll
    for (int j = 0; j < kResSlots; ++j) {
      res_fence(v[j]);
      const int c = wave + kResWaves * j;
      if (c < p.NC) chunk_stats<1>(p, ri, c, v[j]);
    }
    if (tid == 0) p.cand_n[g] = kRowDense;
    return;
  }

  const float a = q.a;
  float2 *tab = p.chunk_tab + (int64_t)g * p.nc_stride;
  sh.mass[tid] = 0;
  if (tid < kResidentMaxChunks) sh.lsum[tid] = 0;
#pragma unroll
  for (int i = 0; i < kResValueBins / kResidentThreads; ++i) rs.cnt[tid + i * kResidentThreads] = 0;
  // Row scale m and row mass S in one pass.  Each lane takes as its
  // reference r the largest of its tokens in its first chunk and sums the
  // weights 2^(a (z - r)) of every later chunk in the same sweep that takes
  // their maximum (fp32 over a chunk's 16 tokens, fp64 beyond; each weight
  // 2^(fma(z, a, -hi)) 2^(-lo) with a r = hi + lo exactly).  Weights above 1
  // are fine up to 2^64; a chunk whose maximum lies further above r moves r
  // up to it, rescales the sum and sums that chunk again (rare).  Then m is the
  // largest token and S the sum of the lane sums scaled to m.
  float lr, lmax;  // the lane's reference and its largest token so far
  double ls = 0.0;
  float hi = 0.0f, sl = 1.0f;  // a lr = hi + lo, sl = 2^(-lo); hi = 0 while lr = -inf
  {
    res_fence(v[0]);
    float cm = kNegInf;
#pragma unroll
    for (int e = 0; e < 16; ++e) cm = fmaxf(cm, L::elem(v[0], e));
    lr = lmax = cm;
    if (lr > kNegInf) {
      hi = a * lr;
      sl = exp2_acc(-__builtin_fmaf(a, lr, -hi));
    }
    res_fence(v[0]);  // decode again rather than hold 16 decoded values across the maximum
    float cs = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) cs += exp2_acc(__builtin_fmaf(L::elem(v[0], e), a, -hi));
    ls = (double)cs * (double)sl;  // 0 for a lane of padding only (its z are -inf)
  }
#pragma unroll
  for (int j = 1; j < kResSlots; ++j) {
    res_fence(v[j]);
    float cm = kNegInf, cs = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float z = L::elem(v[j], e);
      cm = fmaxf(cm, z);
      cs += exp2_acc(__builtin_fmaf(z, a, -hi));
    }
    lmax = fmaxf(lmax, cm);
    if (cm > lr && (lr == kNegInf || a * (cm - lr) > 64.0f)) {
      ls *= lr > kNegInf ? (double)tp_weight(lr, a, cm) : 0.0;
      lr = cm;
      hi = a * lr;
      sl = exp2_acc(-__builtin_fmaf(a, lr, -hi));
      res_fence(v[j]);
      cs = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) cs += exp2_acc(__builtin_fmaf(L::elem(v[j], e), a, -hi));
    }
    ls += (double)cs * (double)sl;
  }
  const float wm = wave_max(lmax);
  if (lane == 0) sh.wmax[wave] = wm;
  __syncthreads();
  float m = sh.wmax[0];
#pragma unroll
  for (int w = 1; w < kResWaves; ++w) m = fmaxf(m, sh.wmax[w]);
  if (!(m > kNegInf)) {  // no finite logit: the streaming pass's entries; the epilogue flags the row
    for (int c = tid; c < p.NC; c += kResidentThreads) tab[c] = make_float2(kNegInf, 0.0f);
    if (tid == 0) p.cand_n[g] = kRowDense;
    return;
  }
  if (lr > kNegInf) ls *= (double)tp_weight(lr, a, m);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) ls += __shfl_xor(ls, d, 64);
  if (lane == 0) sh.wsum[wave] = ls;
  __syncthreads();
  double S = 0.0;
#pragma unroll
  for (int w = 0; w < kResWaves; ++w) S += sh.wsum[w];
  const double bound = (double)q.top_p * S;
  const float zskip = tp_logit_bound((float)((1.0 - (double)q.top_p) * S / (2.0 * p.V)), m, a);

  // Exact boundary from counts of bf16 values.  Without penalties all tokens
  // of one bf16 value weigh the same, so a value's mass is its count times one
  // weight.  The tokens whose keys lie in the kResValueBins keys up to the row
  // maximum's (and not below E_skip's) are counted; a block scan over those
  // values from the top finds z*, the smallest value whose strictly larger
  // values hold less than top_p S.  When the whole window holds less than
  // top_p S the boundary lies below it and the bucket path takes over.
  {
    const uint32_t khi = res_key(__float_as_uint(m) >> 16);
    const uint32_t k0 = khi >= (uint32_t)(kResValueBins - 1) ? khi - (uint32_t)(kResValueBins - 1) : 0u;
    const uint32_t kcut = max(k0, res_key(__float_as_uint(zskip) >> 16));
#pragma unroll
    for (int j = 0; j < kResSlots; ++j) {
      res_fence(v[j]);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t key = res_key(res_bits(v[j], e));
        // (a NaN's key lies above the window: clamped, so the index stays in it)
        if (key >= kcut) atomicAdd(&rs.cnt[min(key - k0, (uint32_t)(kResValueBins - 1))], 1u);
      }
    }
    __syncthreads();
    // Thread t holds keys khi - 4 t .. khi - 4 t - 3 (the heaviest first); an
    // fp64 scan in a fixed order gives each key the mass strictly above it.
    constexpr int PER = kResValueBins / kResidentThreads;
    auto mass_of = [&](int i) {  // mass of this thread's i-th key (recomputed where needed)
      const int kk = (int)khi - (PER * tid + i);
      const unsigned c = kk >= (int)kcut ? rs.cnt[kk - (int)k0] : 0u;
      return c ? (double)c * (double)tp_weight(res_val((uint32_t)kk), a, m) : 0.0;
    };
    double own = 0.0;
#pragma unroll
    for (int i = 0; i < PER; ++i) own += mass_of(i);
    double incl = own;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const double o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    if (lane == 63) sh.wsum[wave] = incl;
    __syncthreads();
    double before = incl - own, total = 0.0;
#pragma unroll
    for (int w = 0; w < kResWaves; ++w) {
      const double sw = sh.wsum[w];
      if (w < wave) before += sw;
      total += sw;
    }
    if (total >= bound) {  // uniform: the boundary is inside the window
      int kmin = 0x7FFFFFFF;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int kk = (int)khi - (PER * tid + i);
        if (kk >= (int)kcut && before < bound) kmin = kk;
        before += mass_of(i);
      }
      kmin = wave_min_i(kmin);
      if (lane == 0) rs.wmin[wave] = kmin;
      __syncthreads();
      int ks = rs.wmin[0];
#pragma unroll
      for (int w = 1; w < kResWaves; ++w) ks = min(ks, rs.wmin[w]);
      const float zstar = res_val((uint32_t)ks);
      // Kept mass per chunk: one wave sum, written by the chunk's wave (the
      // weights in the same hi / lo form as above).
      const float hm = a * m, lm = __builtin_fmaf(a, m, -hm), sm = exp2_acc(-lm);
#pragma unroll
      for (int j = 0; j < kResSlots; ++j) {
        res_fence(v[j]);
        float acc = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float z = L::elem(v[j], e);
          if (z >= zstar) acc += exp2_acc(__builtin_fmaf(z, a, -hm));
        }
        const int c = wave + kResWaves * j;
        const float sum = wave_sum(acc) * sm;
        if (lane == 0 && c < p.NC) tab[c] = make_float2(m, sum);
      }
      if (tid == 0) {
        p.cand_tau[g] = zstar;
        p.cand_n[g] = kRowTopP;
      }
      return;
    }
  }

  // Pass A: units per bucket of the tokens not below E_skip.
#pragma unroll
  for (int j = 0; j < kResSlots; ++j) {
    res_fence(v[j]);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float z = L::elem(v[j], e);
      if (z >= zskip) {
        const float E = tp_weight(z, a, m);
        const int i = max(kToppTop - tp_bucket(E), 0);  // never clamped: E <= 1
        if (i < kToppBuckets) atomicAdd(&sh.mass[i], tp_units(E));
      }
    }
  }
  __syncthreads();
  topp_scan(sh, bound);
  const int bstar = sh.sel;
  const int ustar = tp_unit_exp(bstar);
  const unsigned long long need = sh.need;
  const float zb = tp_logit_bound(__uint_as_float((uint32_t)bstar << 19), m, a);

  // Every token of bucket b* lies in [zb, zt]: the logit bounds of b* and of
  // the next bucket, each 0.01 log2 units beyond the weight's rounding.
  const float zt = m + (__log2f(__uint_as_float((uint32_t)(bstar + 1) << 19)) + 0.01f) / a;
  // Pass B: per chunk the weight of the tokens heavier than bucket b* (one
  // wave sum: a fixed order).
#pragma unroll
  for (int j = 0; j < kResSlots; ++j) {
    res_fence(v[j]);
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float z = L::elem(v[j], e);
      if (z >= zb) {
        const float E = tp_weight(z, a, m);
        if (tp_bucket(E) > bstar) acc += E;
      }
    }
    const int c = wave + kResWaves * j;
    const float sum = __ballot(acc != 0.0f) ? wave_sum(acc) : 0.0f;
    if (lane == 0 && c < p.NC) sh.part[c] = sum;
  }
  // Bucket b*'s tokens into the list (few: one atomic per wave and hit).
#pragma unroll
  for (int j = 0; j < kResSlots; ++j) {
    res_fence(v[j]);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float z = L::elem(v[j], e);
      bool in = z >= zb && z <= zt;
      if (__ballot(in) == 0) continue;
      in = in && tp_bucket(tp_weight(z, a, m)) == bstar;
      const unsigned long long hit = __ballot(in);
      if (hit == 0) continue;
      int base = 0;
      if (lane == 0) base = atomicAdd(&sh.n, __popcll(hit));
      base = __shfl(base, 0, 64);
      const int pos =
          base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(hit >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)hit, 0u));
      if (in && pos < kToppList) {
        sh.lz[pos] = z;
        sh.lx[pos] = (wave + kResWaves * j) * kChunk + L::local(e, lane);
      }
    }
  }
  __syncthreads();
  const int n = sh.n;
  float zstar;
  if (n <= kToppList) {
    zstar = topp_select(
        sh, [&](auto fn) {
          for (int e = tid; e < n; e += kResidentThreads) fn(sh.lz[e], tp_units(tp_weight(sh.lz[e], a, m)));
        },
        need);
    for (int e = tid; e < n; e += kResidentThreads)
      if (sh.lz[e] >= zstar) atomicAdd(&sh.lsum[sh.lx[e] / kChunk], tp_units(tp_weight(sh.lz[e], a, m)));
  } else {  // b* holds more tokens than the list: from the registers again
    zstar = topp_select(
        sh, [&](auto fn) {
#pragma unroll
          for (int j = 0; j < kResSlots; ++j) {
            res_fence(v[j]);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const float z = L::elem(v[j], e);
              if (z >= zb && z <= zt) {
                const float E = tp_weight(z, a, m);
                if (tp_bucket(E) == bstar) fn(z, tp_units(E));
              }
            }
          }
        },
        need);
#pragma unroll
    for (int j = 0; j < kResSlots; ++j) {
      res_fence(v[j]);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float z = L::elem(v[j], e);
        if (z >= zb && z <= zt && z >= zstar) {
          const float E = tp_weight(z, a, m);
          if (tp_bucket(E) == bstar) atomicAdd(&sh.lsum[wave + kResWaves * j], tp_units(E));
        }
      }
    }
  }
  __syncthreads();
  for (int c = tid; c < p.NC; c += kResidentThreads)
    tab[c] = make_float2(m, sh.part[c] + (float)__builtin_ldexp((double)sh.lsum[c], ustar));
  if (tid == 0) {
    p.cand_tau[g] = zstar;
    p.cand_n[g] = kRowTopP;
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

hipError_t launch_topp_resident(const Params &p, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  return launch_timed(reinterpret_cast<const void *>(&topp_resident_kernel), dim3((unsigned)p.R), p, s, t0, t1,
                      kResidentThreads);
}

}  // namespace sv
