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
