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
// Each 32x32 -> 64-bit product is one v_mad_u64_u32 (high and low halves at once).
__device__ __forceinline__ uint4 philox10(uint4 ctr, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * ctr.x, p1 = (uint64_t)0xCD9E8D57u * ctr.z;
    ctr = make_uint4((uint32_t)(p1 >> 32) ^ ctr.y ^ k0, (uint32_t)p1, (uint32_t)(p0 >> 32) ^ ctr.w ^ k1, (uint32_t)p0);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return ctr;
}

enum : uint32_t { kTagAccept = 0, kTagChunk = 1, kTagToken = 2, kTagDraftChunk = 3, kTagDraftToken = 4 };

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
// mirrors leave the row total in every lane; row_bcast:15 then folds rows 0
// and 2 into rows 1 and 3, row_bcast:31 folds row 1 into row 3, and lane 63
// holds the wave total (read out once: uniform result).  Maxima are taken on
// order-preserving integer keys of the floats, so each step is one integer
// max with its DPP operand (a float max would first canonicalise it).
// ---------------------------------------------------------------------------
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp_f(float v, float old = 0.0f) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old), __builtin_bit_cast(int, v),
                                                               CTRL, ROWS, 0xF, false));
}
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ int dpp_i(int v, int old = 0) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, 0xF, false);
}
constexpr int kQuad1032 = 0xB1, kQuad2301 = 0x4E, kHalfMirror = 0x141, kMirror = 0x140;
constexpr int kBcast15 = 0x142, kBcast31 = 0x143;

__device__ __forceinline__ float rd(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Order-preserving map float -> int32 (its own inverse): negative floats get
// their magnitude bits flipped.
__device__ __forceinline__ int fkey(float f) {
  const int b = __builtin_bit_cast(int, f);
  return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float fkey_inv(int k) { return __builtin_bit_cast(float, k ^ ((k >> 31) & 0x7FFFFFFF)); }

__device__ __forceinline__ int wave_max_i(int v) {
  v = max(v, dpp_i<kQuad1032>(v));
  v = max(v, dpp_i<kQuad2301>(v));
  v = max(v, dpp_i<kHalfMirror>(v));
  v = max(v, dpp_i<kMirror>(v));
  v = max(v, dpp_i<kBcast15, 0xA>(v, (int)0x80000000));
  v = max(v, dpp_i<kBcast31, 0xC>(v, (int)0x80000000));
  return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ float wave_max(float v) { return fkey_inv(wave_max_i(fkey(v))); }

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<kQuad1032>(v);
  v += dpp_f<kQuad2301>(v);
  v += dpp_f<kHalfMirror>(v);
  v += dpp_f<kMirror>(v);
  v += dpp_f<kBcast15, 0xA>(v);
  v += dpp_f<kBcast31, 0xC>(v);
  return rd(v, 63);
}

__device__ __forceinline__ int wave_min_i(int v) { return -wave_max_i(-v); }

// (score, index) arg-max with the lowest index winning ties; non-candidates
// carry score -1 (real scores are >= 0).
struct ArgMax {
  float s;
  int i;
};
__device__ __forceinline__ bool better(ArgMax a, ArgMax b) { return a.s > b.s || (a.s == b.s && a.i < b.i); }

template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ ArgMax argmax_dpp(ArgMax a) {
  // rows outside ROWS read back their own pair (the DPP "old" operand)
  ArgMax o{dpp_f<CTRL, ROWS>(a.s, a.s), dpp_i<CTRL, ROWS>(a.i, a.i)};
  return better(o, a) ? o : a;
}
// Wave-wide arg-max with the same DPP steps as the reductions; uniform result.
__device__ __forceinline__ ArgMax wave_argmax(ArgMax a) {
  a = argmax_dpp<kQuad1032>(a);
  a = argmax_dpp<kQuad2301>(a);
  a = argmax_dpp<kHalfMirror>(a);
  a = argmax_dpp<kMirror>(a);
  a = argmax_dpp<kBcast15, 0xA>(a);
  a = argmax_dpp<kBcast31, 0xC>(a);
  return ArgMax{rd(a.s, 63), __builtin_amdgcn_readlane(a.i, 63)};
}

// Block-wide reductions over every wave of the workgroup (up to kMaxBlockWaves);
// every thread gets the result.
constexpr int kMaxBlockWaves = 16;
struct BlockScratch {
  float s[kMaxBlockWaves];
  int i[kMaxBlockWaves];
  float f[kMaxBlockWaves];
};
__device__ __forceinline__ int block_waves() { return (int)(blockDim.x >> 6); }

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
  for (int k = 1; k < block_waves(); ++k) {
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
  for (int k = 0; k < block_waves(); ++k) t += sh.f[k];
  return t;
}

__device__ __forceinline__ float block_max(float v, BlockScratch &sh) {
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh.f[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = sh.f[0];
  for (int k = 1; k < block_waves(); ++k) t = fmaxf(t, sh.f[k]);
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

__device__ __forceinline__ float load_draft_logit(const Params &p, int64_t row, int x) {
  if (p.ddtype == 1) {
    const uint16_t *b = static_cast<const uint16_t *>(p.draft_logits);
    return bf16_bits_to_f32(b[row * p.dlstride + x]);
  }
  return static_cast<const float *>(p.draft_logits)[row * p.dlstride + x];
}

// Per-request logit processing (penalty, then the top-k threshold).
struct Proc {
  const int32_t *counts; // counts row or nullptr (no penalty)
  float theta;           // repetition penalty (1: none)
  float freq, pres;      // frequency and presence penalties (0: none)
  float tau;             // -inf: no threshold
};

// Penalties of a token seen c > 0 times, in this order and each rounded to
// fp32: repetition (z / theta for z > 0, z * theta otherwise), frequency
// (z - freq * c), presence (z - pres).  With theta = 1 and zero penalties
// every step is exact, so the identity settings need no test.
__device__ __forceinline__ float penalize(float z, int c, const Proc &pr) {
  z = z > 0.0f ? z / pr.theta : z * pr.theta;
  z = z - pr.freq * (float)c;
  return z - pr.pres;
}

__device__ __forceinline__ float apply_proc(float z, int x, const Proc &pr) {
  if (pr.counts != nullptr) {
    const int c = pr.counts[x];
    if (c > 0) z = penalize(z, c, pr);
  }
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
