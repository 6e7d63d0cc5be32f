// sv_stats.hip -- the streaming softmax-statistics pass (general and fast variants).
#include <stdint.h>

#include "sv_common.h"

namespace sv {

namespace {

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
// Waves per workgroup of the fast pass: eight for bf16 rows, where halving
// the number of workgroups against four measured about 4 % faster without
// penalties and, with two chunks in flight, 3 % with them; four for fp32
// rows (about 1 % slower with eight).
template <int DT, bool PEN>
constexpr int kFastWaves = DT == 1 ? 8 : 4;
template <int DT, bool PEN>
constexpr int kFastThreads = 64 * kFastWaves<DT, PEN>;
static_assert(kRowCache <= 4, "one wave looks up each row of a slice");

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
    // Counts are sparse (a request's output so far): a group of four
    // tokens per lane whose counts are zero in every lane of the wave is
    // skipped (a uniform branch).
    const bool rep = ri.theta != 1.0f;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int4 q4 = cv[h];
      if (!__ballot((q4.x | q4.y | q4.z | q4.w) != 0)) continue;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int e = 4 * h + k;
        const int cnt = k == 0 ? q4.x : k == 1 ? q4.y : k == 2 ? q4.z : q4.w;
        float zp = rep ? (z[e] > 0.0f ? z[e] / pr.theta : z[e] * pr.theta) : z[e];
        zp = zp - pr.freq * (float)cnt;
        zp = zp - pr.pres;
        z[e] = cnt > 0 ? zp : z[e];
      }
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
  // Chunks in flight per wave (the counts take registers too): with penalties
  // two for bf16 rows (78 VGPRs, eight-wave workgroups; three with four-wave
  // workgroups measured 3 % slower), three for fp32 rows.
  constexpr int D = PEN ? (DT == 1 ? 2 : 3) : kFastDepth<DT>;
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

}  // namespace

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

}  // namespace sv
