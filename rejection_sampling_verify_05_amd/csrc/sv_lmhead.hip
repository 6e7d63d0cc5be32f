// sv_lmhead.hip -- gfx950 kernels of the verify step on LM-head logits.
//
// The target logits are z = W h_g: the target rows' hidden states h_g [d]
// times the LM-head weight W [V, d], both bf16 ("【vllm】DeepSeekMTP、eagle":
// compute_logits is the LM head applied to the hidden states of the logit
// positions).  lm_gemm_kernel computes them on the bf16 matrix cores tile by
// tile (256 tokens x 128 rows) and reduces each tile in its epilogue to what
// the verify step needs ("speculative decoding in vLLM", 7.4: the statistics
// pass takes max, argmax and sum of exp over the target logits): per (row,
// tile) the maximum logit, sum exp2(a (z - max)), the sampling race's best
// token with its key, and for a draft row the draft token's logit and the
// race's best token without it.  The logits never reach memory.
// lm_request_kernel then takes each request's decisions from those records:
// the accept tests, the first reject, the recovered or bonus token (8.3 of
// "vLLM 投机解码（Eagle / MTP）实现与运行流程", no-draft-probs mode).
//
// Sampling is the one-level exponential race argmax_x w_x / E_x of the
// NO_DRAFT_PROBS Q&A, compared as keys a (z_x - m) - log2(E_x) (a = log2(e) /
// T): E_x is drawn for every token of every sampled row in the epilogue, so
// whichever row a request samples, its winner is already known.
#include <stdint.h>

#include "sv_device.h"

namespace sv {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr float kLog2eL = 1.4426950408889634f;
constexpr float kNegInfL = -__builtin_inff();
constexpr int kIntMax = 0x7FFFFFFF;

// Main loop: a workgroup (4 waves, one per SIMD; two workgroups per CU, so
// that one's epilogue overlaps the other's matrix work) owns a tile of kLmTok
// = 256 tokens x kLmRows = 128 target rows; wave w computes tokens 64 w .. + 64
// of all 128 rows as 2 x 4 MFMA 32x32x16 tiles (128 fp32 accumulators per
// lane).  The hidden dimension advances kLmK = 32 elements per step; each
// step's W slice (256 rows x 64 bytes) and hidden slice (128 rows x 64 bytes)
// are copied to LDS by the loads themselves (global_load_lds, no registers)
// into a ring of kStages stages, kStages - 1 steps ahead of the MFMAs.
constexpr int kStages = 3;
constexpr int kRowBytes = kLmK * 2;                    // 64 bytes of one row per step
constexpr int kWPart = kLmTok * kRowBytes;             // W part of a stage: 16 KB
constexpr int kHPart = kLmRows * kRowBytes;            // hidden part: 8 KB
constexpr int kStage = kWPart + kHPart;
constexpr int kDmaW = kWPart / (kThreads * 16);        // 16-byte loads per thread per stage: W (4)
constexpr int kDmaH = kHPart / (kThreads * 16);        // ... and hidden (2)

// Rows are stored densely (64 bytes); the 16-byte chunk c of row r sits at
// position c ^ ((r >> 2) & 3), so that the fragment reads of 16 consecutive
// rows (one LDS cycle of 16-byte reads) hit 16 distinct bank groups.
__device__ __forceinline__ int chunk_pos(int r, int c) { return c ^ ((r >> 2) & 3); }

struct LmRed {  // per (wave, row) partial results of the epilogue
  float m[kWaves][kLmRows], s[kWaves][kLmRows], k1[kWaves][kLmRows], k2[kWaves][kLmRows], zd[kWaves][kLmRows];
  int x1[kWaves][kLmRows], x2[kWaves][kLmRows], xg[kWaves][kLmRows], hd[kWaves][kLmRows];
};

struct LmShared {
  union alignas(16) {
    unsigned char ring[kStages][kStage];
    LmRed red;
  } u;
  float a[kLmRows];  // log2(e) / T of each row's request (0: greedy or invalid)
  int d[kLmRows];    // draft token of the row (-1: bonus row or no valid draft slot)
};
static_assert(sizeof(LmRed) <= kStages * kStage, "epilogue partials reuse the ring");

__device__ __forceinline__ bool key_better(float k, int x, float bk, int bx) { return k > bk || (k == bk && x < bx); }

// One 16-byte load per lane from global memory straight into LDS: lane i
// writes bytes lds + 16 i .. + 16 (lds is the wave's 1 KB destination).  The
// waits for these loads are explicit (s_waitcnt vmcnt in the main loop).
__device__ __forceinline__ void dma16(const void *g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(__builtin_amdgcn_readfirstlane(lds)),
               "v"(g)
               : "memory", "m0");
}

// Per-lane source rows of the stage copies: wave w's load i of a part fills
// the part's bytes (n_w + i) KB .. + 1 KB, i.e. rows 16 (n_w + i) + (lane >> 2),
// stored chunk lane & 3, which holds chunk chunk_pos(row, lane & 3) of the
// row's 64 bytes (n_w = kDmaW w for W, kDmaH w for the hidden part).
struct DmaSrc {
  const uint16_t *w[kDmaW];  // W rows (+ chunk offset), step 0
  const uint16_t *h[kDmaH];  // hidden rows (+ chunk offset), step 0
};

__device__ __forceinline__ void issue_stage(const DmaSrc &src, uint32_t stage_lds, int kb) {
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < kDmaW; ++i) dma16(src.w[i] + (int64_t)kb * kLmK, stage_lds + (kDmaW * wave + i) * 1024);
#pragma unroll
  for (int i = 0; i < kDmaH; ++i)
    dma16(src.h[i] + (int64_t)kb * kLmK, stage_lds + kWPart + (kDmaH * wave + i) * 1024);
}

// Waits until at most `ahead` steps of this wave's stage copies are in flight.
__device__ __forceinline__ void wait_stages(int ahead) {
  static_assert(kDmaW + kDmaH == 6 && kStages == 3, "vmcnt immediates below assume 6 loads per step");
  if (ahead >= 1)
    asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// MFMAs of one step on stage S: MFMA k index 8 (l >> 5) + e of sub-step j is
// hidden element 16 j + 8 (l >> 5) + e of the step, i.e. chunk 2 j + (l >> 5).
__device__ __forceinline__ void compute_stage(const unsigned char *stage, f32x16 (&acc)[2][4]) {
  const int lane = threadIdx.x & 63, l32 = lane & 31, half = lane >> 5, wave = threadIdx.x >> 6;
  bf16x8 wf[2][2], hf[2][4];  // both sub-steps' fragments are read first
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = 2 * j + half;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int rw = 64 * wave + 32 * t + l32;
      wf[j][t] = *reinterpret_cast<const bf16x8 *>(stage + rw * kRowBytes + 16 * chunk_pos(rw, c));
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int rh = 32 * t + l32;
      hf[j][t] = *reinterpret_cast<const bf16x8 *>(stage + kWPart + rh * kRowBytes + 16 * chunk_pos(rh, c));
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
      for (int tn = 0; tn < 4; ++tn)
        acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j][tm], hf[j][tn], acc[tm][tn], 0, 0, 0);
}

// Step kb on ring slot S: wait for its copies (this wave's, then everybody's
// through the barrier, which also retires every wave's reads of the slot the
// next copy overwrites), start the copy of step kb + kStages - 1, compute.
template <int S>
__device__ __forceinline__ void main_step(LmShared &sh, const DmaSrc &src, uint32_t ring_lds, f32x16 (&acc)[2][4],
                                          int kb, int nk) {
  wait_stages(min(nk - 1 - kb, kStages - 2));
  __builtin_amdgcn_s_barrier();
  if (kb + kStages - 1 < nk) issue_stage(src, ring_lds + ((S + kStages - 1) % kStages) * kStage, kb + kStages - 1);
  compute_stage(sh.u.ring[S], acc);
}

__device__ __forceinline__ float shfl32f(float v) { return __shfl_xor(v, 32); }
__device__ __forceinline__ int shfl32i(int v) { return __shfl_xor(v, 32); }

// Epilogue of row subtile TN: lane l holds the logits of row 32 TN + (l & 31)
// for tokens tok0 + 64 wave + 32 tm + 8 (q >> 2) + 4 (l >> 5) + (q & 3),
// tm < 2, q < 16; lanes l and l ^ 32 together hold the wave's 64 tokens.
template <int TN>
__device__ __forceinline__ void epilogue_rows(const LmParams &p, LmShared &sh, const f32x16 (&acc)[2][4], int tok0,
                                              int row0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, rl = 32 * TN + (lane & 31);
  const int g = row0 + rl;
  const float a = sh.a[rl];
  const int dd = sh.d[rl];
  const int xb = tok0 + 64 * wave + 4 * half;
  auto tok = [&](int tm, int q) { return xb + 32 * tm + 8 * (q >> 2) + (q & 3); };

  float m = kNegInfL;
  int bad = 0;
#pragma unroll
  for (int tm = 0; tm < 2; ++tm)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const float z = acc[tm][TN][q];
      if (tok(tm, q) < p.V) {
        m = fmaxf(m, z);
        bad |= !__builtin_isfinite(z);
      }
    }
  if (p.dbg_logits != nullptr && g < p.R) {
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
      for (int q = 0; q < 16; ++q)
        if (tok(tm, q) < p.V) p.dbg_logits[(int64_t)g * p.V + tok(tm, q)] = acc[tm][TN][q];
  }
  m = fmaxf(m, shfl32f(m));
  bad |= shfl32i(bad);

  float s = 0.0f, zd = 0.0f, k1 = kNegInfL, k2 = kNegInfL;
  int x1 = kIntMax, x2 = kIntMax, xg = kIntMax, hd = 0;
  if (a > 0.0f) {
    // Tokens are visited in increasing order, so a strictly larger key is
    // needed to replace the best (ties keep the lowest token).
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int x0 = tok(tm, 4 * qq);
        const uint4 w4 = philox10(make_uint4((uint32_t)x0 >> 2, (uint32_t)g, kTagToken, p.offset), p.seed_lo, p.seed_hi);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int x = x0 + e;
          const float z = acc[tm][TN][4 * qq + e];
          if (x < p.V) {
            const float t = a * (z - m);
            s += __builtin_amdgcn_exp2f(t);
            const float key = t - __builtin_amdgcn_logf(exp_noise(pick(w4, e)));
            if (key > k1) {
              k1 = key;
              x1 = x;
            }
            if (x != dd && key > k2) {
              k2 = key;
              x2 = x;
            }
            if (x == dd) {
              zd = z;
              hd = 1;
            }
          }
        }
      }
  } else {
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
      for (int q = 0; q < 16; ++q)
        if (tok(tm, q) < p.V && acc[tm][TN][q] == m) xg = min(xg, tok(tm, q));
  }
  // Combine with the partner lane (the other 32 tokens of the wave).
  s += shfl32f(s);
  {
    const float pk = shfl32f(k1);
    const int px = shfl32i(x1);
    if (key_better(pk, px, k1, x1)) k1 = pk, x1 = px;
  }
  {
    const float pk = shfl32f(k2);
    const int px = shfl32i(x2);
    if (key_better(pk, px, k2, x2)) k2 = pk, x2 = px;
  }
  xg = min(xg, shfl32i(xg));
  {
    const float pz = shfl32f(zd);
    const int ph = shfl32i(hd);
    if (ph) zd = pz;
    hd |= ph;
  }
  if (half == 0) {
    LmRed &r = sh.u.red;
    r.m[wave][rl] = bad ? __builtin_nanf("") : m;
    r.s[wave][rl] = s;
    r.k1[wave][rl] = k1;
    r.x1[wave][rl] = x1;
    r.k2[wave][rl] = k2;
    r.x2[wave][rl] = x2;
    r.xg[wave][rl] = xg;
    r.zd[wave][rl] = zd;
    r.hd[wave][rl] = hd;
  }
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void lm_gemm_kernel(LmParams p) {
  __shared__ LmShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // Tile order: workgroup b runs on XCD b mod 8; the tiles are renumbered so
  // that each XCD takes a contiguous run in which the row blocks of one token
  // tile are adjacent, and those workgroups share the tile's W rows in the
  // XCD's L2.
  const int total = p.NT * p.RB;
  const int b = blockIdx.x, per = total >> 3, rem = total & 7, xcd = b & 7, loc = b >> 3;
  const int idx = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + loc;
  const int tt = idx / p.RB, rb = idx - tt * p.RB;
  const int tok0 = tt * kLmTok, row0 = rb * kLmRows;

  // Request settings of the tile's rows.
  if (tid < kLmRows) {
    const int g = row0 + tid;
    float a = 0.0f;
    int d = -1;
    if (g < p.R) {
      const int r = find_request(p.cu, p.B, g);
      const int c0 = p.cu[r], c1 = p.cu[r + 1];
      const int i = g - (c0 + r);
      const float T = p.temperature[r];
      if (T > 0.0f && __builtin_isfinite(T)) a = kLog2eL / T;
      if (i >= 0 && i < c1 - c0) {
        const int di = c0 + i;
        if (di >= 0 && di < p.D) d = p.draft_ids[di];
      }
    }
    sh.a[tid] = a;
    sh.d[tid] = d;
  }

  // Copy sources: tokens past V read row V - 1, rows past R read row R - 1
  // (their results are masked in the epilogue).
  DmaSrc src;
#pragma unroll
  for (int i = 0; i < kDmaW; ++i) {
    const int r = 16 * (kDmaW * wave + i) + (lane >> 2);
    src.w[i] = p.W + (int64_t)min(tok0 + r, p.V - 1) * p.wstride + 8 * chunk_pos(r, lane & 3);
  }
#pragma unroll
  for (int i = 0; i < kDmaH; ++i) {
    const int r = 16 * (kDmaH * wave + i) + (lane >> 2);
    src.h[i] = p.H + (int64_t)min(row0 + r, p.R - 1) * p.hstride + 8 * chunk_pos(r, lane & 3);
  }
  // LDS byte address of the ring (an address-space-3 pointer is the offset itself).
  const uint32_t ring_lds =
      (uint32_t)(uintptr_t)((__attribute__((address_space(3))) unsigned char *)(&sh.u.ring[0][0]));

  f32x16 acc[2][4];
#pragma unroll
  for (int tm = 0; tm < 2; ++tm)
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[tm][tn][q] = 0.0f;

  const int nk = p.d / kLmK;
  __syncthreads();  // sh.a / sh.d written; nothing in flight
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s)
    if (s < nk) issue_stage(src, ring_lds + s * kStage, s);
  for (int kb = 0; kb < nk; kb += kStages) {
    main_step<0>(sh, src, ring_lds, acc, kb, nk);
    if (kb + 1 < nk) main_step<1>(sh, src, ring_lds, acc, kb + 1, nk);
    if (kb + 2 < nk) main_step<2>(sh, src, ring_lds, acc, kb + 2, nk);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();  // every wave done with the ring: it now holds the epilogue partials

  epilogue_rows<0>(p, sh, acc, tok0, row0);
  epilogue_rows<1>(p, sh, acc, tok0, row0);
  epilogue_rows<2>(p, sh, acc, tok0, row0);
  epilogue_rows<3>(p, sh, acc, tok0, row0);
  __syncthreads();

  // One thread per row merges the four waves (in token order) into the tile record.
  if (tid < kLmRows) {
    const int g = row0 + tid;
    if (g < p.R) {
      const LmRed &r = sh.u.red;
      const float a = sh.a[tid];
      const int dd = sh.d[tid];
      float mc = kNegInfL;
      int bad = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = r.m[w][tid];
        if (mw != mw)
          bad = 1;
        else
          mc = fmaxf(mc, mw);
      }
      float4 out;
      if (a > 0.0f) {
        float sc = 0.0f, kc = kNegInfL, k2c = kNegInfL, zdc = 0.0f;
        int xc = kIntMax, x2c = kIntMax, hdc = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float mw = r.m[w][tid];
          if (mw > kNegInfL) {  // the wave held valid tokens
            const float sh_ = a * (mw - mc);
            sc += r.s[w][tid] * __builtin_amdgcn_exp2f(sh_);
            const float ka = r.k1[w][tid] + sh_, kb = r.k2[w][tid] + sh_;
            if (key_better(ka, r.x1[w][tid], kc, xc)) kc = ka, xc = r.x1[w][tid];
            if (key_better(kb, r.x2[w][tid], k2c, x2c)) k2c = kb, x2c = r.x2[w][tid];
          }
          if (r.hd[w][tid]) {
            zdc = r.zd[w][tid];
            hdc = 1;
          }
        }
        out = make_float4(bad ? __builtin_nanf("") : mc, sc, kc, __int_as_float(xc));
        if (hdc && dd >= 0) p.drec[g] = make_float4(zdc, k2c, __int_as_float(x2c), 0.0f);
      } else {
        int xg = kIntMax;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
          if (r.m[w][tid] == mc) xg = min(xg, r.xg[w][tid]);
        out = make_float4(bad ? __builtin_nanf("") : mc, 0.0f, 0.0f, __int_as_float(xg));
      }
      p.rec[(int64_t)g * p.NT + tt] = out;
    }
  }
}

// ---------------------------------------------------------------------------
// Request kernel: one workgroup per request; wave w reduces rows w, w + 4, ...
// ---------------------------------------------------------------------------
struct LmReqShared {
  float m[kMaxDrafts + 1], s[kMaxDrafts + 1], zd[kMaxDrafts + 1];
  int amax[kMaxDrafts + 1], xw[kMaxDrafts + 1], d[kMaxDrafts + 1], bad[kMaxDrafts + 1];
  int j;
};

__device__ __forceinline__ void lm_write_empty(const LmParams &p, int r) {
  for (int t = threadIdx.x; t < p.out_stride; t += kThreads) p.out_tokens[(int64_t)r * p.out_stride + t] = -1;
  if (threadIdx.x == 0) {
    p.out_ns[r] = 0;
    p.out_nr[r] = 0;
  }
}

__global__ __launch_bounds__(kThreads) void lm_request_kernel(LmParams p) {
  __shared__ LmReqShared sh;
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c0 = p.cu[r], c1 = p.cu[r + 1], K = c1 - c0, g0 = c0 + r;
  const bool cu_ok = c0 >= 0 && c0 <= c1 && c1 <= p.D && K <= p.out_stride - 1 && p.cu[0] == 0 && p.cu[p.B] == p.D;
  if (!cu_ok) {
    if (tid == 0) atomicOr(p.err, SV_ERR_CU);
    lm_write_empty(p, r);
    return;
  }
  const float T = p.temperature[r];
  if (!(T >= 0.0f) || !__builtin_isfinite(T)) {
    if (tid == 0) atomicOr(p.err, SV_ERR_TEMPERATURE);
    lm_write_empty(p, r);
    return;
  }
  const bool greedy = T == 0.0f;
  const float a = greedy ? 0.0f : kLog2eL / T;
  const int nrow = K + 1;

  for (int i = wave; i < nrow; i += kWaves) {
    const int g = g0 + i;
    const int d = i < K ? p.draft_ids[c0 + i] : -1;
    const bool vd = i < K && d >= 0 && d < p.V;
    const float4 *rr = p.rec + (int64_t)g * p.NT;
    float lm = kNegInfL;
    int lbad = 0;
    for (int c = lane; c < p.NT; c += 64) {
      const float x = rr[c].x;
      if (x != x)
        lbad = 1;
      else
        lm = fmaxf(lm, x);
    }
    const float m = wave_max(lm);
    const int bad = wave_max_i(lbad);
    float s = 0.0f, zd = 0.0f;
    int am = -1, xw = -1;
    if (greedy) {
      int lc = kIntMax;
      for (int c = lane; c < p.NT; c += 64)
        if (rr[c].x == m) lc = min(lc, c);
      lc = wave_min_i(lc);
      if (lc < p.NT) am = __float_as_int(rr[lc].w);
    } else {
      const int cd = vd ? d / kLmTok : -1;
      const float4 dr = vd ? p.drec[g] : make_float4(0.0f, kNegInfL, __int_as_float(kIntMax), 0.0f);
      float ls = 0.0f;
      ArgMax bi{kNegInfL, kIntMax}, bx{kNegInfL, kIntMax};
      for (int c = lane; c < p.NT; c += 64) {
        const float4 e = rr[c];
        const float sh_ = a * (e.x - m);
        ls += e.y * __builtin_amdgcn_exp2f(sh_);
        const ArgMax ci{e.z + sh_, __float_as_int(e.w)};
        if (better(ci, bi)) bi = ci;
        const ArgMax cx = c == cd ? ArgMax{dr.y + sh_, __float_as_int(dr.z)} : ci;
        if (better(cx, bx)) bx = cx;
      }
      s = wave_sum(ls);
      bi = wave_argmax(bi);
      bx = wave_argmax(bx);
      // Without d_j nothing may be left (a one-token vocabulary): race over p_j.
      xw = (vd && bx.i < p.V) ? bx.i : bi.i;
      if (vd) zd = dr.x;
    }
    if (lane == 0) {
      sh.m[i] = m;
      sh.s[i] = s;
      sh.zd[i] = zd;
      sh.amax[i] = am;
      sh.xw[i] = xw;
      sh.d[i] = d;
      sh.bad[i] = bad;
    }
  }
  __syncthreads();
  if (tid == 0) {
    int bad = 0;
    for (int i = 0; i < nrow; ++i) bad |= sh.bad[i];
    sh.bad[0] = bad;
  }
  // Accept tests: lane i of wave 0 takes draft position i.
  if (wave == 0) {
    bool rej = false;
    if (lane < K) {
      const int d = sh.d[lane];
      const int g = g0 + lane;
      if (greedy) {
        rej = d != sh.amax[lane];
        if (p.dbg_p_draft) p.dbg_p_draft[c0 + lane] = -1.0f;
      } else {
        const bool valid = d >= 0 && d < p.V;
        const float pd = valid ? __builtin_amdgcn_exp2f(a * (sh.zd[lane] - sh.m[lane])) / sh.s[lane] : 0.0f;
        const uint4 w4 = philox10(make_uint4(0u, (uint32_t)g, kTagAccept, p.offset), p.seed_lo, p.seed_hi);
        rej = !(valid && (double)pd >= u_accept(w4.x));
        if (p.dbg_p_draft) p.dbg_p_draft[c0 + lane] = pd;
      }
    }
    const unsigned long long mask = __ballot(rej);
    if (lane == 0) sh.j = mask ? (__ffsll((long long)mask) - 1) : K;
  }
  __syncthreads();
  if (sh.bad[0]) {
    if (tid == 0) atomicOr(p.err, SV_ERR_ROW);
    lm_write_empty(p, r);
    return;
  }
  const int j = sh.j;
  for (int t = tid; t < p.out_stride; t += kThreads) {
    int v = -1;
    if (t < j) v = sh.d[t];
    if (t == j) v = greedy ? sh.amax[j] : sh.xw[j];
    p.out_tokens[(int64_t)r * p.out_stride + t] = v;
  }
  if (tid == 0) {
    p.out_ns[r] = j + 1;
    p.out_nr[r] = K - j;
  }
}

}  // namespace

hipError_t launch_lm_head(const LmParams &p, hipStream_t s, const hipEvent_t *ev) {
  LmParams arg = p;
  void *args[] = {&arg};
  const dim3 grid((unsigned)(p.NT * p.RB));
  hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void *>(&lm_gemm_kernel), grid, dim3(kThreads), args, 0, s,
                                    ev ? ev[0] : nullptr, ev ? ev[1] : nullptr, 0);
  if (e != hipSuccess) return e;
  return hipExtLaunchKernel(reinterpret_cast<const void *>(&lm_request_kernel), dim3((unsigned)p.B), dim3(kThreads),
                            args, 0, s, ev ? ev[2] : nullptr, ev ? ev[3] : nullptr, 0);
}

}  // namespace sv
