// sv_internal.h -- launch parameters shared by the host API and the gfx950
// kernels of the verify step.  Not part of the public ABI.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "specverify.h"

namespace sv {

constexpr int kChunk = 1024;      // tokens per race chunk (SV_RACE_CHUNK)
constexpr int kThreads = 256;     // threads per workgroup (4 wave64)
constexpr int kWaves = kThreads / 64;
constexpr int kMaxDrafts = 64;    // SV_MAX_DRAFTS: one lane per draft position
constexpr int kCandCap = 1024;    // SV_TOPK_CANDIDATES
constexpr int kResidCPS = 8;      // chunks per residual-pass workgroup

// Per-row candidate state written by the top-k pass.
constexpr int kRowDense = -2;     // no top-k on this row: dense stats
constexpr int kRowThreshold = -1; // top-k kept too many tokens: dense stats with z < tau masked
constexpr int kRowTopP = -3;      // top-p threshold on a dense row, its chunk table rewritten under it
constexpr int kRowTopPRedo = -4;  // top-p threshold on a dense row, chunk table from a second stats pass
__host__ __device__ constexpr bool row_has_tau(int st) {
  return st == kRowThreshold || st == kRowTopP || st == kRowTopPRedo;
}

// Request-level modes.
enum : int { kModeSample = 0, kModeGreedy = 1, kModeInvalid = 2 };

struct Params {
  // inputs
  const void *logits;
  const float *draft_probs;
  const int32_t *draft_ids;
  const int32_t *cu;
  const float *temperature;
  const int32_t *top_k;
  const float *rep_penalty;
  const int32_t *idx_mapping;
  const int32_t *counts;
  const float *freq_penalty;
  const float *pres_penalty;
  const float *top_p;
  // draft-logits mode: q_i(x) = exp2(aq (zq_x - m_q)) / s_q from the draft row
  // and its (m_q, s_q) pair; aq = log2(e) / draft temperature
  const void *draft_logits;
  const float *draft_stats;   // [2 D]
  const float *draft_temp;    // [B]
  // outputs
  int32_t *out_tokens;
  int32_t *out_ns;
  int32_t *out_nr;
  float *dbg_p_draft;
  float *dbg_probs;
  float *dbg_margin;
  // scratch
  float2 *chunk_tab;           // [max_rows, nc_stride]: (r_c, s_c)
  float4 *row_info;            // [max_rows]: (m, s, argmax bits, state bits)
  int4 *res_req;               // [max_reqs]: (row g*, position j, draft d_j, epoch)
  float *res_tab;              // [max_reqs, nc_stride] residual chunk masses
  int *res_list;               // [max_reqs + 1]: count of rejected draft-probs requests, then their ids (count zero between calls)
  int32_t resid_grid;          // persistent residual-pass workgroups
  float *cand_val;             // [max_rows, kCandCap]
  int32_t *cand_idx;           // [max_rows, kCandCap]
  int32_t *cand_n;             // [max_rows]
  float *cand_tau;             // [max_rows]
  unsigned int *err;           // device error word
  // sizes and scalars
  int64_t lstride;
  int64_t dstride;
  int64_t dlstride;  // draft-logits row stride (elements)
  int32_t ddtype;    // draft-logits dtype
  int32_t dvec_ok;   // draft-logit rows and base 16-byte aligned
  int32_t dtype;
  int32_t R, B, D, V;
  int32_t NC;        // ceil(V / kChunk)
  int32_t nc_stride; // chunk-table row length (>= NC)
  int32_t cps;       // chunks per residual-pass workgroup
  int32_t nseg;      // residual-pass workgroups per row
  int32_t stats_grid; // stats workgroups (persistent grid; slices span <= kRowCache rows)
  int32_t fast;       // use the fast streaming pass
  int32_t fast_pen;   // ... its variant that applies penalties (counts loaded as vectors)
  int32_t out_stride;
  int32_t num_slots;
  int32_t vec_ok;    // rows and base 16-byte aligned: vector loads allowed
  int32_t has_topk;
  int32_t has_topp;
  int32_t cand_valid; // cand_n holds this call's row states (after the top-k or top-p pass)
  int32_t pass2;      // stats pass over the rows the top-p pass left to it (kRowTopPRedo) only
  uint32_t seed_lo, seed_hi, offset;
  uint32_t epoch;
  // post_update applied inside the call (pu_idx_mapping null: not requested)
  const int32_t *pu_idx_mapping, *pu_query_len;
  int32_t *pu_last_sampled, *pu_counts, *pu_num_computed;
  int32_t pu_num_slots;
  int32_t synthetic;  // synthetic acceptance with the rates below
  float syn[kMaxDrafts]; // unconditional acceptance rates of draft positions 1..
};

// Draft-side sampling: outputs of one spec_draft_sample call.
struct DraftOut {
  const int32_t *cu;     // [B + 1] prefix sums of the verify call
  int32_t step;
  int32_t *tokens;       // [B]
  float *q;              // [B] or null
  float *stats;          // [2 D]
  int32_t *ids;          // [D] or null
};

// LM-head path: the logits of target row g are z = W h_g (W [V, d], h_g [d],
// bf16), computed tile by tile and reduced in the tile's epilogue; they are
// never stored (except to dbg_logits).
constexpr int kLmTok = 256;     // tokens per workgroup tile
constexpr int kLmRows = 256;    // target rows per workgroup tile
constexpr int kLmK = 64;        // hidden elements per main-loop step (d must be a multiple)
constexpr int kLmChunk = 64;    // tokens per race chunk (SV_LM_HEAD_CHUNK; one record per row and chunk)
constexpr int kLmThreads = 512; // threads of the GEMM workgroup (8 waves)
static_assert(kLmChunk == SV_LM_HEAD_CHUNK, "the ABI names the LM-head race chunk");

struct LmParams {
  const uint16_t *H;          // [R, hstride] hidden states (bf16 bits)
  const uint16_t *W;          // [V, wstride] LM-head weight (bf16 bits)
  int64_t hstride, wstride;   // elements between rows
  int32_t d;                  // hidden size
  const int32_t *draft_ids;   // [D]
  const int32_t *cu;          // [B + 1]
  const float *temperature;   // [B]
  int32_t *out_tokens, *out_ns, *out_nr;
  float *dbg_p_draft;         // [D] or null
  float *dbg_logits;          // [R, V] or null
  float4 *rec;                // [R, NC]: per (row, chunk) (max z, sum exp2(a (z - max)), lowest argmax bits, 0)
  float4 *drec;               // [R]: the draft token's chunk, (z_d, its mass without d, 0, 0)
  unsigned int *err;
  int32_t R, B, D, V;
  int32_t NC;                 // chunks ceil(V / kLmChunk)
  int32_t NT;                 // token tiles ceil(V / kLmTok)
  int32_t RB;                 // row blocks ceil(R / kLmRows)
  int32_t out_stride;
  uint32_t seed_lo, seed_hi, offset;
  // post_update applied inside the call (pu_idx_mapping null: not requested)
  const int32_t *pu_idx_mapping, *pu_query_len;
  int32_t *pu_last_sampled, *pu_counts, *pu_num_computed;
  int32_t pu_num_slots;
};

// ev: null, or four events stamped around the GEMM and the request kernel.
hipError_t launch_lm_head(const LmParams &p, hipStream_t s, const hipEvent_t *ev);

struct PostParams {
  const int32_t *idx_mapping, *query_len, *tokens, *num_sampled, *num_rejected;
  int32_t *last_sampled, *counts, *num_computed;
  int32_t B, tokens_stride, V, num_slots;
  unsigned int *err;
};

// Launchers (sv_stats.hip, sv_topk.hip, sv_topp.hip, sv_epilogue.hip,
// sv_draft.hip).  Return the hipError_t of the last launch.
hipError_t launch_topk(const Params &p, hipStream_t s, hipEvent_t t0, hipEvent_t t1);
hipError_t launch_topp(const Params &p, hipStream_t s);
// Top-p call with every row held in registers (aligned bf16 rows of at most
// kResidentMaxChunks chunks, no top-k, no penalties): replaces the streaming
// pass and the two-pass top-p kernel; the first two events bracket it.
constexpr int kResidentThreads = 1024;
constexpr int kResidentMaxChunks = 128;
hipError_t launch_topp_resident(const Params &p, hipStream_t s, hipEvent_t t0, hipEvent_t t1);
// t0, t1: optional events stamped at the kernel's start and end (may be null).
hipError_t launch_stats(const Params &p, hipStream_t s, hipEvent_t t0, hipEvent_t t1);
hipError_t launch_epilogue(const Params &p, hipStream_t s, hipEvent_t t0, hipEvent_t t1);
// Rows of at most kInlineResidNC chunks: a rejected request's residual
// max(0, p - q) and its race are taken in the epilogue's own workgroup (its
// four waves load two chunks each at once: one round trip), and the residual
// kernels are not launched.  Past that the workgroup needs one more round trip
// per eight chunks: at 32 chunks (V = 32000) it was slower than the residual
// kernels.
constexpr int kInlineResidNC = 8;
hipError_t launch_resid(const Params &p, hipStream_t s);
// Zeroes the residual-request count (after a call that stopped before the residual race).
hipError_t launch_zero_count(int *count, hipStream_t s);
hipError_t launch_dbg_probs(const Params &p, hipStream_t s);
hipError_t launch_dbg_margin(const Params &p, hipStream_t s);
hipError_t launch_draft_race(const Params &p, const DraftOut &o, hipStream_t s);
hipError_t launch_post_update(const PostParams &p, hipStream_t s);
// Debug: Philox blocks of n counters (uint4 each) under one key; Exp(1) noise of n words.
hipError_t launch_dbg_philox(const uint32_t *ctr, int64_t n, uint64_t key, uint32_t *out, hipStream_t s);
hipError_t launch_dbg_noise(const uint32_t *words, int64_t n, float *out, hipStream_t s);
// Resident stats workgroups per CU (occupancy query); kind 0 general pass,
// 1 fast pass, 2 fast pass with penalties.
int stats_blocks_per_cu(int dtype, int kind);
inline bool pen_call(const Params &p) {
  return p.rep_penalty != nullptr || p.freq_penalty != nullptr || p.pres_penalty != nullptr;
}
// Calls the lean request epilogue serves: no top-k; top-p and penalties
// (at most four rows per request), or draft distributions without either (any
// number of rows), in instantiations of their own.
inline bool plain_call(const Params &p) {
  const bool qd = p.draft_probs != nullptr || p.draft_logits != nullptr;
  return !p.has_topk && (qd ? !(p.has_topp || pen_call(p)) : p.out_stride <= kWaves);
}
constexpr int kSliceRows = 4;  // rows a stats slice may span (kRowCache)

}  // namespace sv
