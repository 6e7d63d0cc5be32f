// sv_api.hip -- C ABI of the verify library (declared in include/specverify.h):
// context and scratch ownership, host-side argument checks, launch sequencing.
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <new>

#include <hip/hip_runtime.h>

#include "specverify.h"
#include "sv_internal.h"

struct sv_ctx {
  int device;
  int32_t max_rows, max_reqs, max_k, max_vocab;
  uint32_t flags;
  int32_t nc_stride;
  uint32_t epoch;
  int32_t resident[2][3];  // resident stats workgroups: [dtype][general, fast, fast with penalties]
  int32_t ncu;             // compute units
  float2 *chunk_tab;
  float4 *row_info;
  int4 *res_req;
  float *res_tab;
  int *res_list;
  bool res_dirty;  // a call listed residual requests but did not reach the residual race
  float *cand_val;
  int32_t *cand_idx;
  int32_t *cand_n;
  float *cand_tau;
  int32_t *zeros;    // [max_reqs + 1] zero prefix sums (draft-side sampling: row r is request r)
  float4 *lm_rec;    // [max_rows, ceil(max_vocab / 64)] LM-head chunk records (SV_CREATE_LM_HEAD)
  float4 *lm_drec;   // [max_rows] LM-head draft-token records
  unsigned int *err;
  hipEvent_t *ev;   // measurement: 4 events per recorded call
  int32_t ev_cap, ev_n;
};

namespace {

void free_events(sv_ctx *c) {
  if (c->ev) {
    for (int32_t i = 0; i < 4 * c->ev_cap; ++i)
      if (c->ev[i]) (void)hipEventDestroy(c->ev[i]);
    delete[] c->ev;
  }
  c->ev = nullptr;
  c->ev_cap = c->ev_n = 0;
}

void free_ctx(sv_ctx *c) {
  free_events(c);
  void *ptrs[] = {c->chunk_tab, c->row_info, c->res_req, c->res_tab, c->res_list, c->cand_val, c->cand_idx,
                  c->cand_n,    c->cand_tau, c->zeros,   c->lm_rec,  c->lm_drec,   c->err};
  for (void *p : ptrs)
    if (p) (void)hipFree(p);
  delete c;
}

template <class T>
bool dev_alloc(T **p, size_t count) {
  *p = nullptr;
  if (count == 0) count = 1;
  return hipMalloc(reinterpret_cast<void **>(p), sizeof(T) * count) == hipSuccess;
}

}  // namespace

extern "C" int spec_verify_create(sv_ctx **out, int32_t max_rows, int32_t max_reqs, int32_t max_k,
                                  int32_t max_vocab, uint32_t flags) {
  if (!out) return SV_EINVAL;
  *out = nullptr;
  if (max_rows <= 0 || max_reqs <= 0 || max_k < 0 || max_vocab <= 0) return SV_EINVAL;
  if (max_k > SV_MAX_DRAFTS || max_rows > (1 << 30) / 2) return SV_ECAPACITY;
  if ((flags & ~(uint32_t)(SV_CREATE_TOPK | SV_CREATE_LM_HEAD)) != 0) return SV_EINVAL;
  sv_ctx *c = new (std::nothrow) sv_ctx();
  if (!c) return SV_EHIP;
  if (hipGetDevice(&c->device) != hipSuccess) {
    delete c;
    return SV_EHIP;
  }
  c->max_rows = max_rows;
  c->max_reqs = max_reqs;
  c->max_k = max_k;
  c->max_vocab = max_vocab;
  c->flags = flags;
  c->nc_stride = (max_vocab + sv::kChunk - 1) / sv::kChunk;
  c->epoch = 0;
  const size_t rows = (size_t)max_rows, reqs = (size_t)max_reqs, ncs = (size_t)c->nc_stride;
  bool ok = dev_alloc(&c->chunk_tab, rows * ncs) && dev_alloc(&c->row_info, rows) &&
            dev_alloc(&c->res_req, reqs) &&
            dev_alloc(&c->res_tab, reqs * ncs) && dev_alloc(&c->res_list, reqs + 1) && dev_alloc(&c->err, 1);
  // Row states and thresholds (top-k and top-p); candidate lists only for top-k.
  if (ok) ok = dev_alloc(&c->cand_n, rows) && dev_alloc(&c->cand_tau, rows);
  if (ok) ok = dev_alloc(&c->zeros, reqs + 1);
  if (ok && (flags & SV_CREATE_TOPK))
    ok = dev_alloc(&c->cand_val, rows * sv::kCandCap) && dev_alloc(&c->cand_idx, rows * sv::kCandCap);
  if (ok && (flags & SV_CREATE_LM_HEAD))
    ok = dev_alloc(&c->lm_rec, rows * (size_t)((max_vocab + sv::kLmChunk - 1) / sv::kLmChunk)) &&
         dev_alloc(&c->lm_drec, rows);
  if (ok)
    ok = hipMemset(c->res_req, 0, reqs * sizeof(int4)) == hipSuccess &&
         hipMemset(c->zeros, 0, (reqs + 1) * sizeof(int32_t)) == hipSuccess &&
         hipMemset(c->res_list, 0, sizeof(int)) == hipSuccess &&
         hipMemset(c->err, 0, sizeof(unsigned int)) == hipSuccess &&
         hipDeviceSynchronize() == hipSuccess;
  int ncu = 0;
  if (ok) ok = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, c->device) == hipSuccess;
  if (!ok) {
    free_ctx(c);
    return SV_EHIP;
  }
  for (int dt = 0; dt < 2; ++dt)
    for (int f = 0; f < 3; ++f) c->resident[dt][f] = ncu * sv::stats_blocks_per_cu(dt, f);
  c->ncu = ncu > 0 ? ncu : 1;
  *out = c;
  return SV_OK;
}

extern "C" void spec_verify_destroy(sv_ctx *ctx) {
  if (!ctx) return;
  (void)hipDeviceSynchronize();
  free_ctx(ctx);
}

namespace {
int verify_on(sv_ctx *ctx, const sv_verify_args *a, hipStream_t stream);
}  // namespace

extern "C" int spec_verify_run(sv_ctx *ctx, const sv_verify_args *a, hipStream_t stream) {
  if (!ctx || !a) return SV_EINVAL;
  return verify_on(ctx, a, stream);
}

namespace {
// The verify step on ctx's scratch (a context, or the fixed array of
// spec_verify_run_noalloc described as one).
int verify_on(sv_ctx *ctx, const sv_verify_args *a, hipStream_t stream) {
  if (!ctx || !a) return SV_EINVAL;
  if (a->logits_dtype != SV_F32 && a->logits_dtype != SV_BF16) return SV_EDTYPE;
  if (a->num_reqs < 0 || a->vocab_size <= 0 || a->num_rows < a->num_reqs) return SV_EINVAL;
  if (a->num_reqs == 0) return SV_OK;
  if (a->num_rows > ctx->max_rows || a->num_reqs > ctx->max_reqs || a->vocab_size > ctx->max_vocab)
    return SV_ECAPACITY;
  if (a->out_stride < 1) return SV_EINVAL;
  if (a->out_stride > ctx->max_k + 1) return SV_ECAPACITY;
  const int32_t D = a->num_rows - a->num_reqs;
  if (!a->target_logits || !a->cu_num_draft || !a->temperature || !a->out_tokens || !a->out_num_sampled ||
      !a->out_num_rejected)
    return SV_EINVAL;
  if (D > 0 && !a->draft_ids) return SV_EINVAL;
  if (a->logits_row_stride < a->vocab_size) return SV_EINVAL;
  if (a->draft_probs && a->draft_row_stride < a->vocab_size) return SV_EINVAL;
  if (a->draft_logits || a->draft_stats || a->draft_temperature) {  // draft-logits mode: all three
    if (!a->draft_logits || !a->draft_stats || !a->draft_temperature || a->draft_probs) return SV_EINVAL;
    if (a->draft_logits_stride < a->vocab_size) return SV_EINVAL;
    if (a->draft_logits_dtype != SV_F32 && a->draft_logits_dtype != SV_BF16) return SV_EDTYPE;
  }
  if (a->offset >> 32) return SV_EINVAL;
  const bool penalty = a->rep_penalty || a->frequency_penalty || a->presence_penalty;
  if (penalty && (!a->idx_mapping || !a->output_bin_counts || a->num_slots < 1)) return SV_EINVAL;
  if (a->top_k && !(ctx->flags & SV_CREATE_TOPK)) return SV_ECAPACITY;
  // Synthetic acceptance: unconditional rates of positions 1..out_stride-1, in
  // [0, 1] and non-increasing (host array, checked here).
  if (a->synthetic_rates) {
    float prev = 1.0f;
    for (int32_t i = 0; i + 1 < a->out_stride; ++i) {
      const float v = a->synthetic_rates[i];
      if (!(v >= 0.0f && v <= prev)) return SV_EINVAL;
      prev = v;
    }
  }

  sv::Params p;
  memset(&p, 0, sizeof p);
  p.logits = a->target_logits;
  p.draft_probs = a->draft_probs;
  p.draft_ids = a->draft_ids;
  p.cu = a->cu_num_draft;
  p.temperature = a->temperature;
  p.top_k = a->top_k;
  p.rep_penalty = a->rep_penalty;
  p.idx_mapping = a->idx_mapping;
  p.counts = a->output_bin_counts;
  p.draft_logits = a->draft_logits;
  p.draft_stats = a->draft_stats;
  p.draft_temp = a->draft_temperature;
  p.dlstride = a->draft_logits ? a->draft_logits_stride : 0;
  p.ddtype = a->draft_logits_dtype;
  p.dvec_ok = a->draft_logits && ((uintptr_t)a->draft_logits % 16 == 0) &&
              ((a->draft_logits_stride * (a->draft_logits_dtype == SV_BF16 ? 2 : 4)) % 16 == 0);
  p.freq_penalty = a->frequency_penalty;
  p.pres_penalty = a->presence_penalty;
  p.top_p = a->top_p;
  p.out_tokens = a->out_tokens;
  p.out_ns = a->out_num_sampled;
  p.out_nr = a->out_num_rejected;
  p.dbg_p_draft = a->dbg_p_draft;
  p.dbg_probs = a->dbg_probs;
  p.dbg_margin = a->dbg_margin;
  if (a->post_update) {  // post_update inside the call
    const sv_post_update_args *u = a->post_update;
    if (a->dbg_probs || a->dbg_margin || u->num_reqs != a->num_reqs || u->vocab_size != a->vocab_size || u->num_slots < 1 ||
        !u->idx_mapping || !u->query_len || !u->last_sampled || !u->output_bin_counts || !u->num_computed_tokens)
      return SV_EINVAL;
    p.pu_idx_mapping = u->idx_mapping;
    p.pu_query_len = u->query_len;
    p.pu_last_sampled = u->last_sampled;
    p.pu_counts = u->output_bin_counts;
    p.pu_num_computed = u->num_computed_tokens;
    p.pu_num_slots = u->num_slots;
  }
  p.chunk_tab = ctx->chunk_tab;
  p.row_info = ctx->row_info;
  p.res_req = ctx->res_req;
  p.res_tab = ctx->res_tab;
  p.res_list = ctx->res_list;
  p.cand_val = ctx->cand_val;
  p.cand_idx = ctx->cand_idx;
  p.cand_n = ctx->cand_n;
  p.cand_tau = ctx->cand_tau;
  p.err = ctx->err;
  p.lstride = a->logits_row_stride;
  p.dstride = a->draft_probs ? a->draft_row_stride : 0;
  p.dtype = a->logits_dtype;
  p.R = a->num_rows;
  p.B = a->num_reqs;
  p.D = D;
  p.V = a->vocab_size;
  p.NC = (a->vocab_size + sv::kChunk - 1) / sv::kChunk;
  p.nc_stride = ctx->nc_stride;
  p.cps = sv::kResidCPS;
  p.nseg = (p.NC + p.cps - 1) / p.cps;
  {
    const int64_t items = (int64_t)a->num_reqs * p.nseg;  // upper bound of (request, segment) items
    const int64_t cap = (int64_t)ctx->ncu * 8;
    p.resid_grid = (int32_t)(items < cap ? items : cap);
  }
  {
    // Fast pass: aligned rows whose length is whole 16-byte vectors, no top-k.
    // Grid: every resident workgroup, but enough workgroups that a slice of the
    // R * NC chunks spans at most kSliceRows rows.
    const int esize_ = a->logits_dtype == SV_BF16 ? 2 : 4;
    const bool aligned = ((uintptr_t)a->target_logits % 16 == 0) && ((a->logits_row_stride * esize_) % 16 == 0);
    // With a penalty the counts rows are read as 16-byte vectors too.
    const bool counts_ok = !penalty || ((uintptr_t)a->output_bin_counts % 16 == 0 && a->vocab_size % 4 == 0);
    p.fast = aligned && a->vocab_size % (16 / esize_) == 0 && counts_ok && !a->top_k;
    p.fast_pen = p.fast && penalty;
    const int64_t chunks = (int64_t)a->num_rows * p.NC;
    if (chunks > 0x7FFFFFFF) return SV_ECAPACITY;
    const int64_t per = (int64_t)(sv::kSliceRows - 1) * p.NC + 1;  // longest slice allowed
    int64_t grid = ctx->resident[a->logits_dtype][p.fast ? (p.fast_pen ? 2 : 1) : 0];
    if (grid * per < chunks) grid = (chunks + per - 1) / per;
    if (grid > chunks) grid = chunks;
    p.stats_grid = (int32_t)grid;
  }
  p.out_stride = a->out_stride;
  p.num_slots = penalty ? a->num_slots : 0;
  const int esize = a->logits_dtype == SV_BF16 ? 2 : 4;
  p.vec_ok = ((uintptr_t)a->target_logits % 16 == 0) && ((a->logits_row_stride * esize) % 16 == 0);
  p.has_topk = a->top_k ? 1 : 0;
  p.has_topp = a->top_p ? 1 : 0;
  p.cand_valid = p.has_topk;
  if (a->synthetic_rates) {
    p.synthetic = 1;
    for (int32_t i = 0; i + 1 < a->out_stride; ++i) p.syn[i] = a->synthetic_rates[i];
  }
  p.seed_lo = (uint32_t)(a->seed & 0xFFFFFFFFu);
  p.seed_hi = (uint32_t)(a->seed >> 32);
  p.offset = (uint32_t)a->offset;
  ctx->epoch = ctx->epoch == 0xFFFFFFFFu ? 1u : ctx->epoch + 1u;
  p.epoch = ctx->epoch;

  if ((int64_t)p.B * p.nseg > 0x7FFFFFFF) return SV_ECAPACITY;

  hipEvent_t *ev = (ctx->ev && ctx->ev_n < ctx->ev_cap) ? ctx->ev + 4 * ctx->ev_n++ : nullptr;
  if (ctx->res_dirty) {
    if (sv::launch_zero_count(ctx->res_list, stream) != hipSuccess) return SV_EHIP;
    ctx->res_dirty = false;
  }
  // Measurement: the first pass over the rows carries the first two events --
  // the top-k pass when top-k is on (the statistics pass then skips the rows
  // it reduced to candidate lists), else the statistics pass.
  hipEvent_t e0 = ev ? ev[0] : nullptr, e1 = ev ? ev[1] : nullptr;
  if (p.has_topk && sv::launch_topk(p, stream, e0, e1) != hipSuccess) return SV_EHIP;
  if (p.has_topk) e0 = e1 = nullptr;
  // Residual kernels: draft distributions given and rows of more chunks than
  // the epilogue takes on itself.
  const bool resid = (p.draft_probs != nullptr || p.draft_logits != nullptr) && p.NC > sv::kInlineResidNC;
  ctx->res_dirty = resid;  // until the residual race has zeroed the count
  // Top-p on aligned bf16 rows that fit the registers of one workgroup, with
  // no top-k or penalty: a single pass that holds each row and does the
  // statistics and the nucleus from it.
  const bool resident = p.has_topp && !p.has_topk && !penalty && p.dtype == SV_BF16 && p.fast &&
                        p.NC <= sv::kResidentMaxChunks;
  if (resident) {
    if (sv::launch_topp_resident(p, stream, e0, e1) != hipSuccess) return SV_EHIP;
    p.cand_valid = 1;
  } else if (sv::launch_stats(p, stream, e0, e1) != hipSuccess) {
    return SV_EHIP;
  }
  if (p.has_topp && !resident) {
    // Top-p on dense rows, then their statistics again under the threshold
    // (general pass, only the marked rows).
    if (sv::launch_topp(p, stream) != hipSuccess) return SV_EHIP;
    p.cand_valid = 1;
    sv::Params p2 = p;
    p2.pass2 = 1;
    p2.fast = 0;
    const int64_t chunks = (int64_t)p.R * p.NC;
    const int64_t per = (int64_t)(sv::kSliceRows - 1) * p.NC + 1;
    int64_t grid = ctx->resident[a->logits_dtype][0];
    if (grid * per < chunks) grid = (chunks + per - 1) / per;
    if (grid > chunks) grid = chunks;
    p2.stats_grid = (int32_t)grid;
    if (sv::launch_stats(p2, stream, nullptr, nullptr) != hipSuccess) return SV_EHIP;
  }
  if (sv::launch_epilogue(p, stream, ev ? ev[2] : nullptr, ev ? ev[3] : nullptr) != hipSuccess) return SV_EHIP;
  if (resid) {
    if (sv::launch_resid(p, stream) != hipSuccess) return SV_EHIP;
    ctx->res_dirty = false;
  }
  if (p.dbg_probs && sv::launch_dbg_probs(p, stream) != hipSuccess) return SV_EHIP;
  if (p.dbg_margin && p.R > 0 && sv::launch_dbg_margin(p, stream) != hipSuccess) return SV_EHIP;
  return SV_OK;
}
}  // namespace

extern "C" int spec_draft_sample(sv_ctx *ctx, const sv_draft_args *a, hipStream_t stream) {
  if (!ctx || !a) return SV_EINVAL;
  if (a->logits_dtype != SV_F32 && a->logits_dtype != SV_BF16) return SV_EDTYPE;
  if (a->num_reqs < 0 || a->vocab_size <= 0 || a->step < 0) return SV_EINVAL;
  if (a->num_reqs == 0) return SV_OK;
  if (a->num_reqs > ctx->max_reqs || a->num_reqs > ctx->max_rows || a->vocab_size > ctx->max_vocab)
    return SV_ECAPACITY;
  if (!a->draft_logits || !a->temperature || !a->cu_num_draft || !a->out_tokens || !a->draft_stats)
    return SV_EINVAL;
  if (a->logits_row_stride < a->vocab_size || (a->offset >> 32)) return SV_EINVAL;

  // A streaming pass over the draft rows (row r = request r), then the race.
  sv::Params p;
  memset(&p, 0, sizeof p);
  p.logits = a->draft_logits;
  p.cu = ctx->zeros;
  p.temperature = a->temperature;
  p.chunk_tab = ctx->chunk_tab;
  p.row_info = ctx->row_info;
  p.res_req = ctx->res_req;
  p.res_tab = ctx->res_tab;
  p.res_list = ctx->res_list;
  p.cand_val = ctx->cand_val;
  p.cand_idx = ctx->cand_idx;
  p.cand_n = ctx->cand_n;
  p.cand_tau = ctx->cand_tau;
  p.err = ctx->err;
  p.lstride = a->logits_row_stride;
  p.dtype = a->logits_dtype;
  p.R = a->num_reqs;
  p.B = a->num_reqs;
  p.D = 0;
  p.V = a->vocab_size;
  p.NC = (a->vocab_size + sv::kChunk - 1) / sv::kChunk;
  p.nc_stride = ctx->nc_stride;
  p.cps = sv::kResidCPS;
  p.nseg = (p.NC + p.cps - 1) / p.cps;
  p.resid_grid = 1;
  const int esize = a->logits_dtype == SV_BF16 ? 2 : 4;
  p.vec_ok = ((uintptr_t)a->draft_logits % 16 == 0) && ((a->logits_row_stride * esize) % 16 == 0);
  p.fast = p.vec_ok && a->vocab_size % (16 / esize) == 0;
  {
    const int64_t chunks = (int64_t)p.R * p.NC;
    if (chunks > 0x7FFFFFFF) return SV_ECAPACITY;
    const int64_t per = (int64_t)(sv::kSliceRows - 1) * p.NC + 1;
    int64_t grid = ctx->resident[a->logits_dtype][p.fast ? 1 : 0];
    if (grid * per < chunks) grid = (chunks + per - 1) / per;
    if (grid > chunks) grid = chunks;
    p.stats_grid = (int32_t)grid;
  }
  p.out_stride = 1;  // each row a request without drafts (its lookups take K = 0)
  p.seed_lo = (uint32_t)(a->seed & 0xFFFFFFFFu);
  p.seed_hi = (uint32_t)(a->seed >> 32);
  p.offset = (uint32_t)a->offset;

  sv::DraftOut o;
  o.cu = a->cu_num_draft;
  o.step = a->step;
  o.tokens = a->out_tokens;
  o.q = a->out_q;
  o.stats = a->draft_stats;
  o.ids = a->draft_ids;
  if (sv::launch_stats(p, stream, nullptr, nullptr) != hipSuccess) return SV_EHIP;
  if (sv::launch_draft_race(p, o, stream) != hipSuccess) return SV_EHIP;
  return SV_OK;
}

extern "C" int spec_verify_synthetic_rates(float mean_length, int32_t k, float *rates) {
  if (k < 0 || (k > 0 && !rates)) return SV_EINVAL;
  const double L = (double)mean_length;
  if (!(L >= 1.0) || !(L <= (double)k + 1.0)) return SV_EINVAL;
  // The accepted count takes floor(L - 1) or that + 1: P(N >= i) is 1, then
  // the fractional part, then 0.
  const double n0 = __builtin_floor(L - 1.0), frac = (L - 1.0) - n0;
  for (int32_t i = 1; i <= k; ++i) rates[i - 1] = (float)((double)i <= n0 ? 1.0 : ((double)i == n0 + 1.0 ? frac : 0.0));
  return SV_OK;
}

extern "C" int spec_post_update(sv_ctx *ctx, const sv_post_update_args *a, hipStream_t stream) {
  if (!ctx || !a) return SV_EINVAL;
  if (a->num_reqs < 0 || a->tokens_stride < 1 || a->vocab_size <= 0 || a->num_slots < 1) return SV_EINVAL;
  if (a->num_reqs == 0) return SV_OK;
  if (!a->idx_mapping || !a->query_len || !a->tokens || !a->num_sampled || !a->num_rejected ||
      !a->last_sampled || !a->output_bin_counts || !a->num_computed_tokens)
    return SV_EINVAL;
  sv::PostParams p;
  p.idx_mapping = a->idx_mapping;
  p.query_len = a->query_len;
  p.tokens = a->tokens;
  p.num_sampled = a->num_sampled;
  p.num_rejected = a->num_rejected;
  p.last_sampled = a->last_sampled;
  p.counts = a->output_bin_counts;
  p.num_computed = a->num_computed_tokens;
  p.B = a->num_reqs;
  p.tokens_stride = a->tokens_stride;
  p.V = a->vocab_size;
  p.num_slots = a->num_slots;
  p.err = ctx->err;
  return sv::launch_post_update(p, stream) == hipSuccess ? SV_OK : SV_EHIP;
}

extern "C" const char *spec_verify_strerror(int status) {
  switch (status) {
    case SV_OK:
      return "ok";
    case SV_EINVAL:
      return "invalid argument";
    case SV_ECAPACITY:
      return "exceeds context capacity";
    case SV_EDTYPE:
      return "unsupported logits dtype";
    case SV_EHIP:
      return "HIP runtime error";
    case SV_EINPUT:
      return "device-side input check failed";
    default:
      return "unknown status";
  }
}

extern "C" int spec_verify_read_error(sv_ctx *ctx, uint32_t *host_flags, hipStream_t stream) {
  if (!ctx || !host_flags) return SV_EINVAL;
  unsigned int h = 0;
  if (hipStreamSynchronize(stream) != hipSuccess) return SV_EHIP;
  if (hipMemcpy(&h, ctx->err, sizeof h, hipMemcpyDeviceToHost) != hipSuccess) return SV_EHIP;
  if (hipMemset(ctx->err, 0, sizeof h) != hipSuccess) return SV_EHIP;
  *host_flags = h;
  return h ? SV_EINPUT : SV_OK;
}

extern "C" int spec_verify_lm_head(sv_ctx *ctx, const sv_lm_head_args *a, hipStream_t stream) {
  if (!ctx || !a) return SV_EINVAL;
  if (a->num_reqs < 0 || a->vocab_size <= 0 || a->num_rows < a->num_reqs) return SV_EINVAL;
  if (a->num_reqs == 0) return SV_OK;
  if (!(ctx->flags & SV_CREATE_LM_HEAD)) return SV_ECAPACITY;
  if (a->num_rows > ctx->max_rows || a->num_reqs > ctx->max_reqs || a->vocab_size > ctx->max_vocab)
    return SV_ECAPACITY;
  if (a->out_stride < 1) return SV_EINVAL;
  if (a->out_stride > ctx->max_k + 1) return SV_ECAPACITY;
  const int32_t D = a->num_rows - a->num_reqs;
  if (!a->hidden || !a->lm_head || !a->cu_num_draft || !a->temperature || !a->out_tokens || !a->out_num_sampled ||
      !a->out_num_rejected || (D > 0 && !a->draft_ids))
    return SV_EINVAL;
  // The main loop copies 16-byte pieces: aligned bases and strides, d a multiple of 64.
  if (a->hidden_size <= 0 || a->hidden_size % sv::kLmK != 0) return SV_EINVAL;
  if (a->hidden_row_stride < a->hidden_size || a->lm_head_row_stride < a->hidden_size) return SV_EINVAL;
  if (a->hidden_row_stride % 8 != 0 || a->lm_head_row_stride % 8 != 0) return SV_EINVAL;
  if ((uintptr_t)a->hidden % 16 != 0 || (uintptr_t)a->lm_head % 16 != 0) return SV_EINVAL;
  if (a->offset >> 32) return SV_EINVAL;
  const int32_t NT = (a->vocab_size + sv::kLmTok - 1) / sv::kLmTok;
  const int32_t RB = (a->num_rows + sv::kLmRows - 1) / sv::kLmRows;
  if ((int64_t)NT * RB > 0x7FFFFFFF) return SV_ECAPACITY;

  sv::LmParams p;
  memset(&p, 0, sizeof p);
  p.H = static_cast<const uint16_t *>(a->hidden);
  p.W = static_cast<const uint16_t *>(a->lm_head);
  p.hstride = a->hidden_row_stride;
  p.wstride = a->lm_head_row_stride;
  p.d = a->hidden_size;
  p.draft_ids = a->draft_ids;
  p.cu = a->cu_num_draft;
  p.temperature = a->temperature;
  p.out_tokens = a->out_tokens;
  p.out_ns = a->out_num_sampled;
  p.out_nr = a->out_num_rejected;
  p.dbg_p_draft = a->dbg_p_draft;
  p.dbg_logits = a->dbg_logits;
  p.rec = ctx->lm_rec;
  p.drec = ctx->lm_drec;
  p.err = ctx->err;
  p.R = a->num_rows;
  p.B = a->num_reqs;
  p.D = D;
  p.V = a->vocab_size;
  p.NT = NT;
  p.NC = (a->vocab_size + sv::kLmChunk - 1) / sv::kLmChunk;
  p.RB = RB;
  p.out_stride = a->out_stride;
  p.seed_lo = (uint32_t)(a->seed & 0xFFFFFFFFu);
  p.seed_hi = (uint32_t)(a->seed >> 32);
  p.offset = (uint32_t)a->offset;
  if (a->post_update) {  // post_update inside the call
    const sv_post_update_args *u = a->post_update;
    if (u->num_reqs != a->num_reqs || u->vocab_size != a->vocab_size || u->num_slots < 1 || !u->idx_mapping ||
        !u->query_len || !u->last_sampled || !u->output_bin_counts || !u->num_computed_tokens)
      return SV_EINVAL;
    p.pu_idx_mapping = u->idx_mapping;
    p.pu_query_len = u->query_len;
    p.pu_last_sampled = u->last_sampled;
    p.pu_counts = u->output_bin_counts;
    p.pu_num_computed = u->num_computed_tokens;
    p.pu_num_slots = u->num_slots;
  }
  hipEvent_t *ev = (ctx->ev && ctx->ev_n < ctx->ev_cap) ? ctx->ev + 4 * ctx->ev_n++ : nullptr;
  return sv::launch_lm_head(p, stream, ev) == hipSuccess ? SV_OK : SV_EHIP;
}

extern "C" int spec_verify_profile_start(sv_ctx *ctx, int32_t max_calls) {
  if (!ctx || max_calls < 1 || max_calls > 65536) return SV_EINVAL;
  free_events(ctx);
  ctx->ev = new (std::nothrow) hipEvent_t[4 * (size_t)max_calls]();
  if (!ctx->ev) return SV_EHIP;
  ctx->ev_cap = max_calls;
  // Timing-only events: without the system-scope fence, recording them adds no
  // cache writeback or invalidation to the kernels they bracket.
  for (int32_t i = 0; i < 4 * max_calls; ++i)
    if (hipEventCreateWithFlags(&ctx->ev[i], hipEventDisableSystemFence) != hipSuccess) {
      free_events(ctx);
      return SV_EHIP;
    }
  return SV_OK;
}

extern "C" int spec_verify_profile_read(sv_ctx *ctx, float *stream_ms, float *epilogue_ms, int32_t *n_calls) {
  if (!ctx || !n_calls || !ctx->ev) return SV_EINVAL;
  const int32_t n = ctx->ev_n;
  int st = SV_OK;
  for (int32_t i = 0; i < n && st == SV_OK; ++i) {
    hipEvent_t *e = ctx->ev + 4 * i;
    if (hipEventSynchronize(e[3]) != hipSuccess) {
      st = SV_EHIP;
      break;
    }
    float a = 0.0f, b = 0.0f;
    if (hipEventElapsedTime(&a, e[0], e[1]) != hipSuccess || hipEventElapsedTime(&b, e[2], e[3]) != hipSuccess)
      st = SV_EHIP;
    if (stream_ms) stream_ms[i] = a;
    if (epilogue_ms) epilogue_ms[i] = b;
  }
  *n_calls = st == SV_OK ? n : 0;
  free_events(ctx);
  return st;
}

extern "C" int spec_verify_debug_philox(const uint32_t *counters, int64_t n, uint64_t key, uint32_t *out,
                                        hipStream_t stream) {
  if (n < 0) return SV_EINVAL;
  if (n == 0) return SV_OK;
  if (!counters || !out || (uintptr_t)counters % 16 != 0 || (uintptr_t)out % 16 != 0) return SV_EINVAL;
  return sv::launch_dbg_philox(counters, n, key, out, stream) == hipSuccess ? SV_OK : SV_EHIP;
}

extern "C" int spec_verify_debug_exp_noise(const uint32_t *words, int64_t n, float *out, hipStream_t stream) {
  if (n < 0) return SV_EINVAL;
  if (n == 0) return SV_OK;
  if (!words || !out) return SV_EINVAL;
  return sv::launch_dbg_noise(words, n, out, stream) == hipSuccess ? SV_OK : SV_EHIP;
}

// ---------------------------------------------------------------------------
// spec_verify_run without a context: the scratch of a context carved from one
// fixed device array, looked up once per device.
// ---------------------------------------------------------------------------
namespace {
constexpr size_t kNoallocTab = (size_t)SV_NOALLOC_MAX_CHUNKS * sizeof(float2);
constexpr size_t kNoallocRowInfo = (size_t)SV_NOALLOC_MAX_ROWS * sizeof(float4);
constexpr size_t kNoallocResReq = (size_t)SV_NOALLOC_MAX_REQS * sizeof(int4);
constexpr size_t kNoallocResTab = (size_t)SV_NOALLOC_MAX_RESID * sizeof(float);
constexpr size_t kNoallocResList = ((size_t)SV_NOALLOC_MAX_REQS + 1) * sizeof(int) + 252;  // kept 256-aligned
constexpr size_t kNoallocCandN = (size_t)SV_NOALLOC_MAX_ROWS * sizeof(int32_t);
constexpr size_t kNoallocCandTau = (size_t)SV_NOALLOC_MAX_ROWS * sizeof(float);
constexpr size_t kNoallocBytes =
    kNoallocTab + kNoallocRowInfo + kNoallocResReq + kNoallocResTab + kNoallocResList + kNoallocCandN + kNoallocCandTau;
static_assert(kNoallocResList % 256 == 0, "regions stay 256-byte aligned");

// Zero-initialised at load, which every region relies on only for the
// residual-request count (res_list[0]) and the residual descriptors' epoch tags
// (res_req[].w); everything else is written before it is read within a call.
static __device__ __align__(256) unsigned char scratch[kNoallocBytes];

constexpr int kMaxDevices = 64;
struct NoallocDevice {
  std::mutex mu;
  bool ready = false;
  unsigned char *base = nullptr;  // this device's copy of `scratch` (never the host-side name)
  int32_t resident[2][3] = {};
  int32_t ncu = 1;
  uint32_t epoch = 0;
  bool res_dirty = false;
};
NoallocDevice g_noalloc[kMaxDevices];

int noalloc_setup(int dev, NoallocDevice &nd) {
  if (nd.ready) return SV_OK;
  void *ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return SV_EHIP;
  int ncu = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return SV_EHIP;
  nd.ncu = ncu > 0 ? ncu : 1;
  for (int dt = 0; dt < 2; ++dt)
    for (int f = 0; f < 3; ++f) nd.resident[dt][f] = nd.ncu * sv::stats_blocks_per_cu(dt, f);
  nd.base = static_cast<unsigned char *>(ptr);
  nd.ready = true;
  return SV_OK;
}
}  // namespace

extern "C" int spec_verify_run_noalloc(const sv_verify_args *a, uint32_t *device_errors, hipStream_t stream) {
  if (!a || !device_errors) return SV_EINVAL;
  if (a->top_k) return SV_ECAPACITY;
  if (a->vocab_size <= 0 || a->num_reqs < 0) return SV_EINVAL;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SV_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return SV_ECAPACITY;
  NoallocDevice &nd = g_noalloc[dev];
  std::lock_guard<std::mutex> lock(nd.mu);
  const int st = noalloc_setup(dev, nd);
  if (st != SV_OK) return st;
  const int32_t nc = (a->vocab_size + sv::kChunk - 1) / sv::kChunk;
  sv_ctx c{};  // a context over the fixed array: capacities from its sizes for this vocabulary
  c.device = dev;
  c.max_vocab = a->vocab_size;
  c.nc_stride = nc;
  c.max_rows = (int32_t)(SV_NOALLOC_MAX_ROWS < SV_NOALLOC_MAX_CHUNKS / nc ? SV_NOALLOC_MAX_ROWS : SV_NOALLOC_MAX_CHUNKS / nc);
  c.max_reqs = (int32_t)(SV_NOALLOC_MAX_REQS < SV_NOALLOC_MAX_RESID / nc ? SV_NOALLOC_MAX_REQS : SV_NOALLOC_MAX_RESID / nc);
  c.max_k = SV_MAX_DRAFTS;
  c.flags = 0;
  c.epoch = nd.epoch;
  c.res_dirty = nd.res_dirty;
  for (int dt = 0; dt < 2; ++dt)
    for (int f = 0; f < 3; ++f) c.resident[dt][f] = nd.resident[dt][f];
  c.ncu = nd.ncu;
  unsigned char *q = nd.base;
  c.chunk_tab = reinterpret_cast<float2 *>(q);
  q += kNoallocTab;
  c.row_info = reinterpret_cast<float4 *>(q);
  q += kNoallocRowInfo;
  c.res_req = reinterpret_cast<int4 *>(q);
  q += kNoallocResReq;
  c.res_tab = reinterpret_cast<float *>(q);
  q += kNoallocResTab;
  c.res_list = reinterpret_cast<int *>(q);
  q += kNoallocResList;
  c.cand_n = reinterpret_cast<int32_t *>(q);
  q += kNoallocCandN;
  c.cand_tau = reinterpret_cast<float *>(q);
  c.err = device_errors;
  const int rc = verify_on(&c, a, stream);
  nd.epoch = c.epoch;
  nd.res_dirty = c.res_dirty;
  return rc;
}
