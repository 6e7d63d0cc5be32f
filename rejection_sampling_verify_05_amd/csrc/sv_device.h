// sv_device.h -- gfx950 device helpers for the verify kernels: the Philox
// counter stream, wave64 reductions built on DPP row operations, block
// reductions through LDS, and logit-row access.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "sv_internal.h"

namespace sv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two 32x32
// multiplies whose high halves are xored with the other counter words and the
// round key; the key advances by the golden-ratio Weyl increments.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint4 philox10(uint4 ctr, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint32_t m0 = 0xD2511F53u, m1 = 0xCD9E8D57u;
    uint32_t hi0 = __umulhi(m0, ctr.x), lo0 = m0 * ctr.x;
    uint32_t hi1 = __umulhi(m1, ctr.z), lo1 = m1 * ctr.z;
    ctr = make_uint4(hi1 ^ ctr.y ^ k0, lo1, hi0 ^ ctr.w ^ k1, lo0);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return ctr;
}

enum : uint32_t { kTagAccept = 0, kTagChunk = 1, kTagToken = 2 };

// Four consecutive words idx = 4*blk .. 4*blk+3 of stream (g, tag).
__device__ __forceinline__ uint4 rng_block(const Params &p, uint32_t blk, uint32_t g, uint32_t tag) {
  return philox10(make_uint4(blk, g, tag, p.offset), p.seed_lo, p.seed_hi);
}

__device__ __forceinline__ uint32_t pick(uint4 w, int k) {
  return k == 0 ? w.x : k == 1 ? w.y : k == 2 ? w.z : w.w;
}

// Accept uniform ((w>>8)+1) 2^-24 in (0,1]; exact in fp64.
__device__ __forceinline__ double u_accept(uint32_t w) { return (double)((w >> 8) + 1u) * 0x1p-24; }

// Exp(1) noise E = -ln U from the race uniform U = (w>>8) 2^-24 in [0,1);
// U = 0 gives +inf.  Short straight-line code (it runs once per raced chunk
// and token, in unrolled loops):
//  - U < 1/2: E = -ln2 log2(U) with the hardware log2 (U is exact in fp32 and
//    |log2 U| >= 1, so about one ulp relative);
//  - U >= 1/2: with v = 1 - U (exact) and y = v / (2 - v) <= 1/3,
//    E = -ln(1 - v) = ln((1 + y)/(1 - y)) = 2 (y + y^3/3 + ... + y^15/15),
//    so small E (the likely race winners) keep full relative precision.
// The relative error is below 4e-7 over the whole grid; race scores are
// compared in fp32, so decisions can differ from exact arithmetic only where
// two scores are within a few 1e-7 of each other.
__device__ __forceinline__ float exp_noise(uint32_t w) {
  const uint32_t k = w >> 8;
  const float lg = -0.69314718055994531f * __builtin_amdgcn_logf((float)k * 0x1p-24f);
  const float v = (float)((1u << 24) - k) * 0x1p-24f;
  const float y = v * __builtin_amdgcn_rcpf(2.0f - v);
  const float y2 = y * y;
  float t = 1.0f / 15.0f;
  t = __builtin_fmaf(t, y2, 1.0f / 13.0f);
  t = __builtin_fmaf(t, y2, 1.0f / 11.0f);
  t = __builtin_fmaf(t, y2, 1.0f / 9.0f);
  t = __builtin_fmaf(t, y2, 1.0f / 7.0f);
  t = __builtin_fmaf(t, y2, 1.0f / 5.0f);
  t = __builtin_fmaf(t, y2, 1.0f / 3.0f);
  t = __builtin_fmaf(t, y2, 1.0f);
  const float E = k < (1u << 23) ? lg : 2.0f * y * t;  // both computed: no divergent branch
  return k == 0 ? __builtin_inff() : E;
}

// Race score w / E for the word w of a race position (0 when U = 0).
__device__ __forceinline__ float race_score(float weight, uint32_t w) {
  return weight * __builtin_amdgcn_rcpf(exp_noise(w));
}

// ---------------------------------------------------------------------------
// wave64 reductions.  Within a 16-lane row: quad_perm swaps and the two
// mirrors leave the row total in every lane; the four row totals are then
// combined through readlane (uniform result).
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
constexpr int kQuad1032 = 0xB1, kQuad2301 = 0x4E, kHalfMirror = 0x141, kMirror = 0x140;

__device__ __forceinline__ float rd(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<kQuad1032>(v));
  v = fmaxf(v, dpp_f<kQuad2301>(v));
  v = fmaxf(v, dpp_f<kHalfMirror>(v));
  v = fmaxf(v, dpp_f<kMirror>(v));
  return fmaxf(fmaxf(rd(v, 0), rd(v, 16)), fmaxf(rd(v, 32), rd(v, 48)));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<kQuad1032>(v);
  v += dpp_f<kQuad2301>(v);
  v += dpp_f<kHalfMirror>(v);
  v += dpp_f<kMirror>(v);
  return (rd(v, 0) + rd(v, 16)) + (rd(v, 32) + rd(v, 48));
}

__device__ __forceinline__ int wave_min_i(int v) {
  v = min(v, dpp_i<kQuad1032>(v));
  v = min(v, dpp_i<kQuad2301>(v));
  v = min(v, dpp_i<kHalfMirror>(v));
  v = min(v, dpp_i<kMirror>(v));
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// (score, index) arg-max with the lowest index winning ties; non-candidates
// carry score -1 (real scores are >= 0).
struct ArgMax {
  float s;
  int i;
};
__device__ __forceinline__ bool better(ArgMax a, ArgMax b) { return a.s > b.s || (a.s == b.s && a.i < b.i); }

template <int CTRL>
__device__ __forceinline__ ArgMax argmax_dpp(ArgMax a) {
  ArgMax o{dpp_f<CTRL>(a.s), dpp_i<CTRL>(a.i)};
  return better(o, a) ? o : a;
}
// Wave-wide arg-max with DPP row steps; uniform result.
__device__ __forceinline__ ArgMax wave_argmax(ArgMax a) {
  a = argmax_dpp<kQuad1032>(a);
  a = argmax_dpp<kQuad2301>(a);
  a = argmax_dpp<kHalfMirror>(a);
  a = argmax_dpp<kMirror>(a);
  ArgMax b{rd(a.s, 0), __builtin_amdgcn_readlane(a.i, 0)};
#pragma unroll
  for (int row = 16; row < 64; row += 16) {
    ArgMax o{rd(a.s, row), __builtin_amdgcn_readlane(a.i, row)};
    if (better(o, b)) b = o;
  }
  return b;
}

// ---------------------------------------------------------------------------
// Publication between workgroups of one launch.  Entries are written with
// agent-scope stores (written through to the device-coherent level, not held
// in one XCD's L2), the writer waits for its stores to be acknowledged, and
// only then bumps an agent-scope counter; the reader observes the counter and
// then reads the entries with agent-scope loads.  No L2 write-back or
// invalidate of unrelated lines is needed.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void publish_f2(float2 *addr, float2 v) {
  __hip_atomic_store(reinterpret_cast<unsigned long long *>(addr), __builtin_bit_cast(unsigned long long, v),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 fetch_f2(const float2 *addr) {
  return __builtin_bit_cast(float2, __hip_atomic_load(reinterpret_cast<const unsigned long long *>(addr),
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void publish_f(float *addr, float v) {
  __hip_atomic_store(addr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float fetch_f(const float *addr) {
  return __hip_atomic_load(addr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory operation this wave issued has completed.
__device__ __forceinline__ void wait_memory() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Block-wide (256 threads) reductions; every thread gets the result.
struct BlockScratch {
  float s[kWaves];
  int i[kWaves];
  float f[kWaves];
};

__device__ __forceinline__ ArgMax block_argmax(ArgMax a, BlockScratch &sh) {
  a = wave_argmax(a);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    sh.s[w] = a.s;
    sh.i[w] = a.i;
  }
  __syncthreads();
  ArgMax b{sh.s[0], sh.i[0]};
#pragma unroll
  for (int k = 1; k < kWaves; ++k) {
    ArgMax o{sh.s[k], sh.i[k]};
    if (better(o, b)) b = o;
  }
  return b;
}

__device__ __forceinline__ float block_sum(float v, BlockScratch &sh) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh.f[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) t += sh.f[k];
  return t;
}

__device__ __forceinline__ float block_max(float v, BlockScratch &sh) {
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh.f[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = sh.f[0];
#pragma unroll
  for (int k = 1; k < kWaves; ++k) t = fmaxf(t, sh.f[k]);
  return t;
}

// ---------------------------------------------------------------------------
// Logit access
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ float load_logit(const Params &p, int64_t row, int x) {
  if (p.dtype == 1) {
    const uint16_t *b = static_cast<const uint16_t *>(p.logits);
    return bf16_bits_to_f32(b[row * p.lstride + x]);
  }
  return static_cast<const float *>(p.logits)[row * p.lstride + x];
}

// Per-request logit processing (penalty, then the top-k threshold).
struct Proc {
  const int32_t *counts; // counts row or nullptr (no penalty)
  float theta;
  float tau;             // -inf: no threshold
};

__device__ __forceinline__ float apply_proc(float z, int x, const Proc &pr) {
  if (pr.counts != nullptr && pr.counts[x] > 0) z = z > 0.0f ? z / pr.theta : z * pr.theta;
  return z < pr.tau ? -__builtin_inff() : z;
}

// Largest r in [0, B) with cu[r] + r <= g (cu nondecreasing => cu[r] + r
// strictly increasing).  With a corrupt cu it still returns some r in range.
__device__ __forceinline__ int find_request(const int32_t *__restrict__ cu, int B, int g) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] + mid <= g)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ void raise_err(const Params &p, unsigned bits) { atomicOr(p.err, bits); }

}  // namespace sv
