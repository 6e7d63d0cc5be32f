// sv_lmhead.hip -- gfx950 kernels of the verify step on LM-head logits.
//
// The target logits are z = W h_g: the target rows' hidden states h_g [d]
// times the LM-head weight W [V, d], both bf16 ("【vllm】DeepSeekMTP、eagle":
// compute_logits is the LM head applied to the hidden states of the logit
// positions).  lm_gemm_kernel computes them on the bf16 matrix cores tile by
// tile (256 tokens x 256 rows) and reduces them in its epilogue to what the
// verify step needs ("speculative decoding in vLLM", 7.4: the statistics pass
// takes max, argmax and sum of exp over the target logits): per row and chunk
// of kLmChunk = 64 tokens the maximum logit, sum exp2(a (z - max)) and the
// lowest argmax, and for a draft row the draft token's logit and its chunk's
// mass without it.  The logits never reach memory.
//
// lm_request_kernel then takes each request's decisions from those records:
// the accept tests, the first reject, and the recovered or bonus token (8.3 of
// "vLLM 投机解码（Eagle / MTP）实现与运行流程", no-draft-probs mode) by the
// two-level exponential race of the NO_DRAFT_PROBS Q&A: a chunk by its mass,
// then a token of that chunk, whose 64 logits it recomputes from W and h (a
// 512 KB read per sampled request at d = 4096, instead of keeping any logits).
#include <stdint.h>

#include "sv_device.h"

namespace sv {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr float kLog2eL = 1.4426950408889634f;
constexpr float kNegInfL = -__builtin_inff();
constexpr int kIntMax = 0x7FFFFFFF;

// Main loop: one workgroup per CU (8 waves, two per SIMD) owns a tile of
// kLmTok = 256 tokens x kLmRows = 256 target rows; wave w computes the 64
// tokens of chunk (w & 3) of the tile for rows 128 (w >> 2) .. + 128 as 2 x 4
// MFMA 32x32x16 tiles (128 fp32 accumulators per lane).  The hidden dimension
// advances kLmK = 64 elements per step, so that each row's slice of a step is
// one whole 128-byte line: with half lines per step every line was requested
// twice (the second half a step later, after the L1 had dropped it) and the
// loop ran about 6 % slower.  A step's W and hidden slices (256 rows x 128
// bytes each, the step's two parts) are copied to LDS by the loads themselves
// (global_load_lds, no registers) into a ring of kSlots = 5 part slots: while
// step k computes from its two parts, the three parts after them are in flight
// (96 KB; the ring is the whole 160 KB of LDS).
constexpr int kSlots = 5;
constexpr int kRowBytes = kLmK * 2;                    // 128 bytes of one row per step
constexpr int kPart = kLmTok * kRowBytes;              // one part (W or hidden) of a step: 32 KB
constexpr int kDmaPart = kPart / (kLmThreads * 16);    // 16-byte loads per thread per part (4)
static_assert(kLmTok == kLmRows, "W and hidden parts have the same size");
static_assert(kLmTok == 4 * kLmChunk, "four chunks per token tile, one per wave column");
static_assert(kLmChunk % (8 * kWaves) == 0, "the recompute takes tokens in blocks of 8 per wave");
static_assert(kDmaPart == 4, "vmcnt immediates below assume 4 loads per part");

// Rows are stored densely (128 bytes); the 16-byte chunk c of row r sits at
// position c ^ ((r >> 1) & 7), so that the fragment reads of 16 consecutive
// rows (one LDS cycle of 16-byte reads over 64 banks) hit 16 distinct bank
// groups: rows of one parity take 8 distinct positions, and the two parities
// fall in the two halves of the banks.
__device__ __forceinline__ int chunk_pos(int r, int c) { return c ^ ((r >> 1) & 7); }

union LmShared {
  alignas(16) unsigned char ring[kSlots][kPart];
  struct {
    float a[kLmRows];  // log2(e) / T of each row's request (0: greedy or invalid)
    int d[kLmRows];    // draft token of the row (-1: bonus row or no valid draft slot)
  } rq;                // written once the ring is no longer read
};

// One 16-byte load per lane from global memory straight into LDS: lane i
// writes bytes lds + 16 i .. + 16 (lds is the wave's 1 KB destination).  The
// waits for these loads are explicit (s_waitcnt vmcnt in the main loop); the
// compiler's own form of this load makes it wait for every copy before any
// LDS read, which serialises the ring.  hipcc warns that m0 is a reserved
// register in the clobber list: nothing else in this file's kernels uses m0
// (the generated code sets it only in these statements), so no value of the
// compiler's lives in it across them.
__device__ __forceinline__ void dma16(const void *g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(__builtin_amdgcn_readfirstlane(lds)),
               "v"(g)
               : "memory", "m0");
}

// Per-lane source rows of the part copies: wave w's load i of a part fills the
// part's bytes (4 w + i) KB .. + 1 KB, i.e. rows 8 (4 w + i) + (lane >> 3),
// stored chunk lane & 7, which holds chunk chunk_pos(row, lane & 7) of the
// row's 128 bytes (the XOR is its own inverse).
struct DmaSrc {
  const uint16_t *w[kDmaPart];  // W rows (+ chunk offset), step 0
  const uint16_t *h[kDmaPart];  // hidden rows (+ chunk offset), step 0
};

// Part 2 k + e of the copy sequence: e = 0 the W part of step k, e = 1 its hidden part.
__device__ __forceinline__ void issue_part(const DmaSrc &src, uint32_t slot_lds, int k, int e) {
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < kDmaPart; ++i)
    dma16((e == 0 ? src.w[i] : src.h[i]) + (int64_t)k * kLmK, slot_lds + (kDmaPart * wave + i) * 1024);
}

// MFMAs of one step from its W and hidden parts: MFMA k index 8 (l >> 5) + e
// of sub-step j is hidden element 16 j + 8 (l >> 5) + e of the step, i.e.
// chunk 2 j + (l >> 5).  Only the wave's first NTN row subtiles hold target
// rows (the others lie past R in the last row block) and only those are read
// and multiplied.
template <int NTN>
struct StepFrags {
  bf16x8 wf[4][2], hf[4][NTN > 0 ? NTN : 1];
};

// Fragment reads of sub-steps j0, j0 + 1.
template <int NTN>
__device__ __forceinline__ void read_frags(const unsigned char *wpart, const unsigned char *hpart, StepFrags<NTN> &f,
                                           int j0) {
  const int lane = threadIdx.x & 63, l32 = lane & 31, half = lane >> 5, wave = threadIdx.x >> 6;
  const int tq = wave & 3, wr = wave >> 2;
#pragma unroll
  for (int j = j0; j < j0 + 2; ++j) {
    const int c = 2 * j + half;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int rw = 64 * tq + 32 * t + l32;
      f.wf[j][t] = *reinterpret_cast<const bf16x8 *>(wpart + rw * kRowBytes + 16 * chunk_pos(rw, c));
    }
#pragma unroll
    for (int t = 0; t < NTN; ++t) {
      const int rh = 128 * wr + 32 * t + l32;
      f.hf[j][t] = *reinterpret_cast<const bf16x8 *>(hpart + rh * kRowBytes + 16 * chunk_pos(rh, c));
    }
  }
}

// Step k, with S = k mod 5: its parts 2 k and 2 k + 1 sit in slots 2 S mod 5
// and (2 S + 1) mod 5.  Wait for them (this wave's copies: everything but part
// 2 k + 2, the last one issued; then everybody's through the barrier, which
// also retires every wave's reads of step k - 1), read the fragments of
// sub-steps 0 and 1, copy parts 2 k + 3 and 2 k + 4 into step k - 1's slots,
// then the MFMAs of sub-steps 0 and 1 with the reads of sub-steps 2 and 3
// between them (one after each MFMA: their LDS latency is hidden by matrix
// work), then the MFMAs of 2 and 3.
template <int S, int NTN>
__device__ __forceinline__ void main_step(LmShared &sh, const DmaSrc &src, uint32_t ring_lds, f32x16 (&acc)[2][4],
                                          int k, int nk) {
  if (k + 1 < nk)
    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  constexpr int s3 = (2 * S + 3) % kSlots, s4 = (2 * S + 4) % kSlots;
  const unsigned char *wpart = sh.ring[(2 * S) % kSlots], *hpart = sh.ring[(2 * S + 1) % kSlots];
  StepFrags<NTN> f;
  if (NTN > 0) read_frags<NTN>(wpart, hpart, f, 0);
  if (k + 1 < nk) issue_part(src, ring_lds + s3 * kPart, k + 1, 1);
  if (k + 2 < nk) issue_part(src, ring_lds + s4 * kPart, k + 2, 0);
  if (NTN > 0) {
    read_frags<NTN>(wpart, hpart, f, 2);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int tm = 0; tm < 2; ++tm)
#pragma unroll
        for (int tn = 0; tn < NTN; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.wf[j][tm], f.hf[j][tn], acc[tm][tn], 0, 0, 0);
    constexpr int kReads2 = 2 * (2 + NTN);  // reads of two sub-steps
    constexpr int kMfma2 = 2 * 2 * NTN;     // MFMAs of two sub-steps
#pragma unroll
    for (int i = 0; i < kReads2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * kMfma2 - kReads2, 0);
  }
}

// The whole hidden dimension for a wave with NTN row subtiles (every wave of
// the workgroup runs the same copies and barriers).
template <int NTN>
__device__ __forceinline__ void main_loop(LmShared &sh, const DmaSrc &src, uint32_t ring_lds, f32x16 (&acc)[2][4],
                                          int nk) {
  for (int k = 0; k < nk; k += kSlots) {
    main_step<0, NTN>(sh, src, ring_lds, acc, k, nk);
    if (k + 1 < nk) main_step<1, NTN>(sh, src, ring_lds, acc, k + 1, nk);
    if (k + 2 < nk) main_step<2, NTN>(sh, src, ring_lds, acc, k + 2, nk);
    if (k + 3 < nk) main_step<3, NTN>(sh, src, ring_lds, acc, k + 3, nk);
    if (k + 4 < nk) main_step<4, NTN>(sh, src, ring_lds, acc, k + 4, nk);
  }
}

__device__ __forceinline__ float shfl32f(float v) { return __shfl_xor(v, 32); }
__device__ __forceinline__ int shfl32i(int v) { return __shfl_xor(v, 32); }

// Epilogue of row subtile TN: lane l holds the logits of row
// 128 wr + 32 TN + (l & 31) for tokens tok0 + 64 tq + 32 tm + 8 (q >> 2) +
// 4 (l >> 5) + (q & 3), tm < 2, q < 16; lanes l and l ^ 32 together hold the
// wave's chunk of 64 tokens.  Lane l < 32 writes the (row, chunk) record.
template <int TN>
__device__ __forceinline__ void epilogue_rows(const LmParams &p, const LmShared &sh, const f32x16 (&acc)[2][4],
                                              int tok0, int row0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tq = wave & 3, wr = wave >> 2;
  const int half = lane >> 5, rl = 128 * wr + 32 * TN + (lane & 31);
  const int g = row0 + rl;
  const int c = tok0 / kLmChunk + tq;
  const float a = sh.rq.a[rl];
  const int dd = sh.rq.d[rl];
  const int xb = tok0 + kLmChunk * tq + 4 * half;
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

  float s = 0.0f, sx = 0.0f, zd = 0.0f;
  int xg = kIntMax, hd = 0;
  if (a > 0.0f) {
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int x = tok(tm, q);
        const float z = acc[tm][TN][q];
        const float w = x < p.V ? __builtin_amdgcn_exp2f(a * (z - m)) : 0.0f;
        s += w;
        if (x == dd) {
          zd = z;
          hd = 1;
        } else {
          sx += w;
        }
      }
  } else {
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
      for (int q = 0; q < 16; ++q)
        if (tok(tm, q) < p.V && acc[tm][TN][q] == m) xg = min(xg, tok(tm, q));
  }
  s += shfl32f(s);
  sx += shfl32f(sx);
  xg = min(xg, shfl32i(xg));
  {
    const float pz = shfl32f(zd);
    const int ph = shfl32i(hd);
    if (ph) zd = pz;
    hd |= ph;
  }
  if (half == 0 && g < p.R && c < p.NC) {
    p.rec[(int64_t)g * p.NC + c] = make_float4(bad ? __builtin_nanf("") : m, s, __int_as_float(xg), 0.0f);
    if (hd) p.drec[g] = make_float4(zd, sx, 0.0f, 0.0f);
  }
}

__global__ __launch_bounds__(kLmThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void lm_gemm_kernel(LmParams p) {
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

  // Request settings of the tile's rows (kept in registers until the ring is free).
  float row_a = 0.0f;
  int row_d = -1;
  if (tid < kLmRows) {
    const int g = row0 + tid;
    if (g < p.R) {
      const int r = find_request(p.cu, p.B, g);
      const int c0 = p.cu[r], c1 = p.cu[r + 1];
      const int i = g - (c0 + r);
      const float T = p.temperature[r];
      if (T > 0.0f && __builtin_isfinite(T)) row_a = kLog2eL / T;
      if (i >= 0 && i < c1 - c0) {
        const int di = c0 + i;
        if (di >= 0 && di < p.D) row_d = p.draft_ids[di];
      }
    }
  }

  // Copy sources: tokens past V read row V - 1, rows past R read row R - 1
  // (their results are never written).
  DmaSrc src;
#pragma unroll
  for (int i = 0; i < kDmaPart; ++i) {
    const int r = 8 * (kDmaPart * wave + i) + (lane >> 3);
    src.w[i] = p.W + (int64_t)min(tok0 + r, p.V - 1) * p.wstride + 8 * chunk_pos(r, lane & 7);
    src.h[i] = p.H + (int64_t)min(row0 + r, p.R - 1) * p.hstride + 8 * chunk_pos(r, lane & 7);
  }
  // LDS byte address of the ring (an address-space-3 pointer is the offset itself).
  const uint32_t ring_lds = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) unsigned char *)(&sh.ring[0][0]));

  f32x16 acc[2][4];
#pragma unroll
  for (int tm = 0; tm < 2; ++tm)
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[tm][tn][q] = 0.0f;

  // Parts 0, 1 and 2 (step 0, W of step 1) into slots 0, 1, 2.
  const int nk = p.d / kLmK;
  issue_part(src, ring_lds, 0, 0);
  issue_part(src, ring_lds + kPart, 0, 1);
  if (nk > 1) issue_part(src, ring_lds + 2 * kPart, 1, 0);
  // Row subtiles of this wave that hold target rows (4 except in the last row block).
  const int ntn = __builtin_amdgcn_readfirstlane(max(0, min(4, (p.R - row0 - 128 * (wave >> 2) + 31) / 32)));
  if (ntn == 4)
    main_loop<4>(sh, src, ring_lds, acc, nk);
  else if (ntn == 3)
    main_loop<3>(sh, src, ring_lds, acc, nk);
  else if (ntn == 2)
    main_loop<2>(sh, src, ring_lds, acc, nk);
  else if (ntn == 1)
    main_loop<1>(sh, src, ring_lds, acc, nk);
  else
    main_loop<0>(sh, src, ring_lds, acc, nk);
  __syncthreads();  // every wave is done with the ring (its last step waited for all its copies)
  if (tid < kLmRows) {
    sh.rq.a[tid] = row_a;
    sh.rq.d[tid] = row_d;
  }
  __syncthreads();

  if (ntn > 0) epilogue_rows<0>(p, sh, acc, tok0, row0);
  if (ntn > 1) epilogue_rows<1>(p, sh, acc, tok0, row0);
  if (ntn > 2) epilogue_rows<2>(p, sh, acc, tok0, row0);
  if (ntn > 3) epilogue_rows<3>(p, sh, acc, tok0, row0);
}

// ---------------------------------------------------------------------------
// Request kernel: one workgroup (256 threads) per request.
// ---------------------------------------------------------------------------
struct LmReqShared {
  float m[kMaxDrafts + 1], s[kMaxDrafts + 1], zd[kMaxDrafts + 1], sxd[kMaxDrafts + 1];
  int amax[kMaxDrafts + 1], d[kMaxDrafts + 1], bad[kMaxDrafts + 1];
  int j, xw;          // first reject; the sampled token
  float z[kLmChunk];  // recomputed logits of the winning chunk
  BlockScratch red;
};

__device__ __forceinline__ void lm_write_empty(const LmParams &p, int r) {
  for (int t = threadIdx.x; t < p.out_stride; t += kThreads) p.out_tokens[(int64_t)r * p.out_stride + t] = -1;
  if (threadIdx.x == 0) {
    p.out_ns[r] = 0;
    p.out_nr[r] = 0;
  }
}

// post_update of request r once its tokens are final (the accepted drafts
// sh.d[0..j-1], then x): the updates of spec_post_update.  All threads call it.
__device__ __forceinline__ void lm_post_update(const LmParams &p, const LmReqShared &sh, int r, int K, int j, int x) {
  if (p.pu_idx_mapping == nullptr) return;
  const int s = p.pu_idx_mapping[r];
  if (s < 0 || s >= p.pu_num_slots) {
    if (threadIdx.x == 0) atomicOr(p.err, SV_ERR_SLOT);
    return;
  }
  for (int i = threadIdx.x; i <= j; i += kThreads) {
    const int tok = i < j ? sh.d[i] : x;
    if (tok >= 0 && tok < p.V) atomicAdd(&p.pu_counts[(int64_t)s * p.V + tok], 1);
  }
  if (threadIdx.x == 0) {
    p.pu_last_sampled[s] = x;
    atomicAdd(&p.pu_num_computed[s], p.pu_query_len[r] - (K - j));
  }
}

// Race noise 1/E of position idx of stream (g, tag) (one position).
__device__ __forceinline__ float inv_noise(const LmParams &p, uint32_t idx, uint32_t g, uint32_t tag) {
  const uint4 w4 = philox10(make_uint4(idx >> 2, g, tag, p.offset), p.seed_lo, p.seed_hi);
  return __builtin_amdgcn_rcpf(exp_noise(pick(w4, (int)(idx & 3))));
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

  // Row statistics from the chunk records: wave w takes rows w, w + 4, ...
  for (int i = wave; i < nrow; i += kWaves) {
    const int g = g0 + i;
    const int d = i < K ? p.draft_ids[c0 + i] : -1;
    const bool vd = i < K && d >= 0 && d < p.V;
    const float4 *rr = p.rec + (int64_t)g * p.NC;
    // One pass over the records with 8 loads in flight per lane; a lane keeps
    // (max, mass relative to it), rescaled when the max grows (greedy rows: the
    // max and the first chunk holding it; chunks are visited in order).
    float lm = kNegInfL, ls = 0.0f;
    int lbad = 0, lc = kIntMax;
    for (int cb = lane; cb < p.NC; cb += 64 * 8) {
      float4 e[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = cb + 64 * u;
        e[u] = c < p.NC ? rr[c] : make_float4(kNegInfL, 0.0f, 0.0f, 0.0f);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float x = e[u].x;
        if (x != x) {
          lbad = 1;
        } else if (x > lm) {
          ls = greedy ? 0.0f : ls * __builtin_amdgcn_exp2f(a * (lm - x)) + e[u].y;
          lm = x;
          lc = cb + 64 * u;
        } else if (!greedy && x > kNegInfL) {
          ls += e[u].y * __builtin_amdgcn_exp2f(a * (x - lm));
        }
      }
    }
    const float m = wave_max(lm);
    const int bad = wave_max_i(lbad);
    float s = 0.0f;
    int am = -1;
    if (greedy) {
      lc = wave_min_i(lm == m ? lc : kIntMax);
      if (lc < p.NC) am = __float_as_int(rr[lc].z);
    } else {
      s = wave_sum(lm > kNegInfL ? ls * __builtin_amdgcn_exp2f(a * (lm - m)) : 0.0f);
    }
    if (lane == 0) {
      const float4 dr = vd && !greedy ? p.drec[g] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      sh.m[i] = m;
      sh.s[i] = s;
      sh.zd[i] = dr.x;
      sh.sxd[i] = dr.y;
      sh.amax[i] = am;
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
    if (t == j && greedy) v = sh.amax[j];
    if (t != j || greedy) p.out_tokens[(int64_t)r * p.out_stride + t] = v;
  }
  if (tid == 0) {
    p.out_ns[r] = j + 1;
    p.out_nr[r] = K - j;
  }
  if (greedy) {
    lm_post_update(p, sh, r, K, j, sh.amax[j]);
    return;
  }

  // Sampled row j: chunk race over the chunk masses (the draft token's chunk
  // with its mass without d when j is a rejected draft), then the token race
  // inside the winner on its recomputed logits.
  const int gs = g0 + j;
  const int dj = j < K ? sh.d[j] : -1;
  const int cd = (dj >= 0 && dj < p.V) ? dj / kLmChunk : -1;
  const float m = sh.m[j];
  const float4 *rr = p.rec + (int64_t)gs * p.NC;
  ArgMax best{-1.0f, kIntMax}, bestf{-1.0f, kIntMax};  // without d_j / over p_j
  for (int c4 = 4 * tid; c4 < p.NC; c4 += 4 * kThreads) {  // one Philox block per 4 chunks
    const uint4 w4 = philox10(make_uint4((uint32_t)c4 >> 2, (uint32_t)gs, kTagChunk, p.offset), p.seed_lo, p.seed_hi);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = c4 + k;
      if (c < p.NC) {
        const float4 e = rr[c];
        const float sc = __builtin_amdgcn_exp2f(a * (e.x - m));
        const float rn = __builtin_amdgcn_rcpf(exp_noise(pick(w4, k)));
        const float wf = e.y * sc, wx = c == cd ? sh.sxd[j] * sc : wf;
        if (wf > 0.0f && better(ArgMax{wf * rn, c}, bestf)) bestf = ArgMax{wf * rn, c};
        if (wx > 0.0f && better(ArgMax{wx * rn, c}, best)) best = ArgMax{wx * rn, c};
      }
    }
  }
  best = block_argmax(best, sh.red);
  bestf = block_argmax(bestf, sh.red);
  const bool excl = cd >= 0 && best.s >= 0.0f;  // without d nothing left (rounding): race over p_j
  const ArgMax win = excl ? best : bestf;
  if (win.s < 0.0f) {
    if (tid == 0) p.out_tokens[(int64_t)r * p.out_stride + j] = -1;
    lm_post_update(p, sh, r, K, j, -1);
    return;
  }
  const int cs = win.i;

  // Logits of chunk cs of row gs: wave w takes tokens 16 w .. 16 w + 15 of the
  // chunk, eight at a time; lane l reads the 16-byte pieces l, l + 64, ... of
  // the W rows and of h (whole-wave 1 KB reads, 4 pieces of each row in flight),
  // fp32 FMAs, then a wave sum per token.
  {
    constexpr int kTB = 8;  // tokens per block
    const uint4 *hrow = reinterpret_cast<const uint4 *>(p.H + (int64_t)gs * p.hstride);
    const int n8 = p.d / 8;
    for (int tb = 0; tb < kLmChunk / kWaves; tb += kTB) {
      const int tk0 = (kLmChunk / kWaves) * wave + tb;
      const uint4 *wr[kTB];
#pragma unroll
      for (int t = 0; t < kTB; ++t)
        wr[t] = reinterpret_cast<const uint4 *>(p.W + (int64_t)min(cs * kLmChunk + tk0 + t, p.V - 1) * p.wstride);
      float acc[kTB];
#pragma unroll
      for (int t = 0; t < kTB; ++t) acc[t] = 0.0f;
      for (int kb8 = lane; kb8 < n8; kb8 += 64 * 4) {
        uint4 hv[4], wv[kTB][4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int k8 = min(kb8 + 64 * u, n8 - 1);
          hv[u] = hrow[k8];
#pragma unroll
          for (int t = 0; t < kTB; ++t) wv[t][u] = wr[t][k8];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (kb8 + 64 * u >= n8) break;
          const uint32_t hh[4] = {hv[u].x, hv[u].y, hv[u].z, hv[u].w};
#pragma unroll
          for (int t = 0; t < kTB; ++t) {
            const uint32_t ww[4] = {wv[t][u].x, wv[t][u].y, wv[t][u].z, wv[t][u].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              acc[t] = __builtin_fmaf(__uint_as_float(ww[e] << 16), __uint_as_float(hh[e] << 16), acc[t]);
              acc[t] = __builtin_fmaf(__uint_as_float(ww[e] & 0xFFFF0000u), __uint_as_float(hh[e] & 0xFFFF0000u),
                                      acc[t]);
            }
          }
        }
      }
#pragma unroll
      for (int t = 0; t < kTB; ++t) {
        const float z = wave_sum(acc[t]);
        if (lane == 0) sh.z[tk0 + t] = z;
      }
    }
  }
  __syncthreads();
  if (wave == 0) {
    const int x = cs * kLmChunk + lane;
    const bool ok = x < p.V && !(excl && x == dj);
    const float zc = ok ? sh.z[lane] : kNegInfL;
    const float hi = wave_max(zc);
    const float w = ok ? __builtin_amdgcn_exp2f(a * (zc - hi)) : 0.0f;
    ArgMax o{-1.0f, kIntMax};
    if (w > 0.0f) o = ArgMax{w * inv_noise(p, (uint32_t)x, (uint32_t)gs, kTagToken), x};
    o = wave_argmax(o);
    if (lane == 0) {
      const int x = o.s < 0.0f ? -1 : o.i;
      p.out_tokens[(int64_t)r * p.out_stride + j] = x;
      sh.xw = x;
    }
  }
  __syncthreads();
  lm_post_update(p, sh, r, K, j, sh.xw);
}

}  // namespace

hipError_t launch_lm_head(const LmParams &p, hipStream_t s, const hipEvent_t *ev) {
  LmParams arg = p;
  void *args[] = {&arg};
  const dim3 grid((unsigned)(p.NT * p.RB));
  hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void *>(&lm_gemm_kernel), grid, dim3(kLmThreads), args, 0,
                                    s, ev ? ev[0] : nullptr, ev ? ev[1] : nullptr, 0);
  if (e != hipSuccess) return e;
  return hipExtLaunchKernel(reinterpret_cast<const void *>(&lm_request_kernel), dim3((unsigned)p.B), dim3(kThreads),
                            args, 0, s, ev ? ev[2] : nullptr, ev ? ev[3] : nullptr, 0);
}

}  // namespace sv
