// sv_tiles.h -- row tiles of the top-k and top-p passes: 16 tokens per thread,
// loaded as raw words first and decoded after, with the row's penalties.
#pragma once
#include "sv_common.h"

namespace sv {

namespace {

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

// Pipelined form of the super-tile load for aligned rows: the raw 16-byte
// vectors are issued unconditionally (a vector not wholly inside [0, vfull)
// reads the row start) and decoded later; tokens in [vfull, V) are handled
// apart, after the loop.
template <int DT, int NPER = kTopkPer>
struct TopkRaw {
  static constexpr int VW = DT == 1 ? 8 : 4;
  u32x4 v[NPER / VW];
};
template <int DT, int NT = kThreads, int NPER = kTopkPer>
__device__ __forceinline__ void topk_issue(const Params &p, int g, int base, int vfull, TopkRaw<DT, NPER> &r) {
  constexpr int VW = TopkRaw<DT, NPER>::VW;
  const char *row = static_cast<const char *>(p.logits) + (int64_t)g * p.lstride * (DT == 1 ? 2 : 4);
#pragma unroll
  for (int v = 0; v < NPER / VW; ++v) {
    const int x0 = topk_tok<DT, NT>(base, v * VW);
    const uint32_t off = x0 + VW <= vfull ? (uint32_t)x0 * (DT == 1 ? 2u : 4u) : 0u;
    r.v[v] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(row + off));
  }
}
template <int DT, int NT = kThreads, int NPER = kTopkPer>
__device__ __forceinline__ void topk_decode(int base, int vfull, const TopkRaw<DT, NPER> &r, float (&z)[NPER]) {
  constexpr int VW = TopkRaw<DT, NPER>::VW;
#pragma unroll
  for (int v = 0; v < NPER / VW; ++v) {
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


// Order-preserving map float -> uint32 (larger float, larger key).
__device__ __forceinline__ uint32_t ukey(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ukey_val(uint32_t k) { return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k); }

}  // namespace

}  // namespace sv
