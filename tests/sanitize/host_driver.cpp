// Host-side logic of the C ABI (rejection_sampling_verify_05_amd/csrc/sv_api.hip)
// under AddressSanitizer and UndefinedBehaviorSanitizer, with no GPU.
//
// This file includes sv_api.hip itself, so that a context can be built by hand
// with fake device pointers, and it stubs the kernel launchers so that nothing
// reaches the device.  Each stub records the launch parameters it was given.
// The driver then runs the argument checks, the scalar and capacity
// validation, the choice between the fast and general passes and the
// epilogue variants, and the grid sizing, and checks the parameters that would have been launched.
#include "sv_api.hip"

#include <cstdio>
#include <cstdlib>

namespace sv {
namespace {
Params g_last;
LmParams g_lm;
PostParams g_post;
int g_n[14];
}  // namespace
enum { kTopk, kTopp, kStats, kEpi, kResid, kZero, kDbg, kDraft, kPost, kPhilox, kNoise, kLm, kRes, kMargin };
hipError_t launch_topk(const Params &p, hipStream_t, hipEvent_t, hipEvent_t) { g_last = p; ++g_n[kTopk]; return hipSuccess; }
hipError_t launch_topp(const Params &p, hipStream_t) { g_last = p; ++g_n[kTopp]; return hipSuccess; }
hipError_t launch_topp_resident(const Params &p, hipStream_t, hipEvent_t, hipEvent_t) { g_last = p; ++g_n[kRes]; return hipSuccess; }
hipError_t launch_stats(const Params &p, hipStream_t, hipEvent_t, hipEvent_t) { g_last = p; ++g_n[kStats]; return hipSuccess; }
hipError_t launch_epilogue(const Params &p, hipStream_t, hipEvent_t, hipEvent_t) { g_last = p; ++g_n[kEpi]; return hipSuccess; }
hipError_t launch_resid(const Params &p, hipStream_t) { g_last = p; ++g_n[kResid]; return hipSuccess; }
hipError_t launch_zero_count(int *, hipStream_t) { ++g_n[kZero]; return hipSuccess; }
hipError_t launch_dbg_probs(const Params &p, hipStream_t) { g_last = p; ++g_n[kDbg]; return hipSuccess; }
hipError_t launch_dbg_margin(const Params &p, hipStream_t) { g_last = p; ++g_n[kMargin]; return hipSuccess; }
hipError_t launch_draft_race(const Params &p, const DraftOut &, hipStream_t) { g_last = p; ++g_n[kDraft]; return hipSuccess; }
hipError_t launch_post_update(const PostParams &p, hipStream_t) { g_post = p; ++g_n[kPost]; return hipSuccess; }
hipError_t launch_dbg_philox(const uint32_t *, int64_t, uint64_t, uint32_t *, hipStream_t) { ++g_n[kPhilox]; return hipSuccess; }
hipError_t launch_dbg_noise(const uint32_t *, int64_t, float *, hipStream_t) { ++g_n[kNoise]; return hipSuccess; }
hipError_t launch_lm_head(const LmParams &p, hipStream_t, const hipEvent_t *) { g_lm = p; ++g_n[kLm]; return hipSuccess; }
int stats_blocks_per_cu(int, int kind) { return kind == 1 ? 3 : 8; }
}  // namespace sv

#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      std::exit(2);                                                \
    }                                                              \
  } while (0)

alignas(16) static char g_fake[1 << 16];  // stands in for device buffers (never dereferenced)

static sv_ctx make_ctx(int32_t rows, int32_t reqs, int32_t k, int32_t vocab, uint32_t flags) {
  sv_ctx c{};
  c.max_rows = rows;
  c.max_reqs = reqs;
  c.max_k = k;
  c.max_vocab = vocab;
  c.flags = flags;
  c.nc_stride = (vocab + sv::kChunk - 1) / sv::kChunk;
  for (int dt = 0; dt < 2; ++dt)
    for (int f = 0; f < 3; ++f) c.resident[dt][f] = 256 * sv::stats_blocks_per_cu(dt, f);
  c.ncu = 256;
  void *f = g_fake;
  c.chunk_tab = (float2 *)f;
  c.row_info = (float4 *)f;
  c.res_req = (int4 *)f;
  c.res_tab = (float *)f;
  c.res_list = (int *)f;
  c.cand_n = (int32_t *)f;
  c.cand_tau = (float *)f;
  c.zeros = (int32_t *)f;
  c.err = (unsigned int *)f;
  return c;
}

static sv_verify_args plain_args(int32_t B, int32_t R, int32_t V, int32_t dtype, int32_t out_stride) {
  sv_verify_args a{};
  a.target_logits = g_fake;
  a.logits_dtype = dtype;
  a.logits_row_stride = V;
  a.draft_ids = (const int32_t *)g_fake;
  a.cu_num_draft = (const int32_t *)g_fake;
  a.num_reqs = B;
  a.num_rows = R;
  a.vocab_size = V;
  a.temperature = (const float *)g_fake;
  a.out_tokens = (int32_t *)g_fake;
  a.out_num_sampled = (int32_t *)g_fake;
  a.out_num_rejected = (int32_t *)g_fake;
  a.out_stride = out_stride;
  a.seed = 0x123456789ABCDEFull;
  a.offset = 7;
  return a;
}

int main() {
  using namespace sv;
  sv_ctx *out = nullptr;
  CHECK(spec_verify_create(nullptr, 1, 1, 1, 1, 0) == SV_EINVAL);
  CHECK(spec_verify_create(&out, 1, 1, SV_MAX_DRAFTS + 1, 1, 0) == SV_ECAPACITY);
  CHECK(spec_verify_create(&out, 1, 1, 1, 1, 0x80) == SV_EINVAL);
  CHECK(spec_verify_strerror(SV_EINPUT) != nullptr && spec_verify_strerror(99) != nullptr);

  // The headline shape: the fast pass and the plain epilogue, slices of at most four rows.
  sv_ctx c = make_ctx(1100, 256, 3, 128256, 0);
  sv_verify_args a = plain_args(256, 650, 128256, SV_BF16, 4);
  CHECK(spec_verify_run(&c, &a, nullptr) == SV_OK);
  CHECK(g_n[kStats] == 1 && g_n[kEpi] == 1 && g_last.fast == 1 && sv::plain_call(g_last) && !sv::pen_call(g_last));
  CHECK(g_last.NC == 126 && g_last.D == 394 && g_last.epoch == 1);
  {
    const int64_t chunks = (int64_t)650 * 126, per = 3 * 126 + 1;
    CHECK(g_last.stats_grid >= 1 && g_last.stats_grid <= chunks && (int64_t)g_last.stats_grid * per >= chunks);
    CHECK(g_last.stats_grid == 256 * 3);  // every resident workgroup
  }
  // fp32 rows, unaligned rows, a vocabulary that is not whole 16-byte vectors.
  sv_verify_args af = a;
  af.logits_dtype = SV_F32;
  CHECK(spec_verify_run(&c, &af, nullptr) == SV_OK && g_last.fast == 1);
  sv_verify_args au = a;
  au.target_logits = g_fake + 2;
  CHECK(spec_verify_run(&c, &au, nullptr) == SV_OK && g_last.fast == 0);
  sv_verify_args av = a;
  av.vocab_size = av.logits_row_stride = 128250;
  CHECK(spec_verify_run(&c, &av, nullptr) == SV_OK && g_last.fast == 0 && g_last.NC == 126);

  // Settings that leave the plain path: penalties, top-k, top-p, draft probabilities.
  sv_verify_args ap = a;
  ap.rep_penalty = (const float *)g_fake;
  CHECK(spec_verify_run(&c, &ap, nullptr) == SV_EINVAL);  // no histogram
  ap.idx_mapping = (const int32_t *)g_fake;
  ap.output_bin_counts = (const int32_t *)g_fake;
  ap.num_slots = 300;
  // (penalties alone keep the lean epilogue, in its penalty instantiation)
  CHECK(spec_verify_run(&c, &ap, nullptr) == SV_OK && g_last.fast_pen == 1 && sv::plain_call(g_last) && sv::pen_call(g_last));
  sv_verify_args ak = a;
  ak.top_k = (const int32_t *)g_fake;
  CHECK(spec_verify_run(&c, &ak, nullptr) == SV_ECAPACITY);  // context without top-k storage
  sv_ctx ct = make_ctx(1100, 256, 3, 128256, SV_CREATE_TOPK);
  ct.cand_val = (float *)g_fake;
  ct.cand_idx = (int32_t *)g_fake;
  const int nt = g_n[kTopk];
  CHECK(spec_verify_run(&ct, &ak, nullptr) == SV_OK && g_n[kTopk] == nt + 1 && g_last.fast == 0);
  sv_verify_args aq = a;
  aq.top_p = (const float *)g_fake;
  // Aligned bf16 rows of at most 128 chunks: the register-resident pass alone.
  int np = g_n[kTopp], ns_ = g_n[kStats], nres = g_n[kRes];
  CHECK(spec_verify_run(&c, &aq, nullptr) == SV_OK && g_n[kRes] == nres + 1 && g_n[kTopp] == np &&
        g_n[kStats] == ns_ && g_last.cand_valid == 1);
  CHECK(sv::plain_call(g_last) && g_last.has_topp == 1 && !sv::pen_call(g_last));  // the lean epilogue with thresholds
  // Larger vocabularies, fp32 rows or penalties: the two-pass kernel between two statistics passes.
  sv_verify_args aq2 = aq;
  aq2.logits_dtype = SV_F32;
  np = g_n[kTopp], ns_ = g_n[kStats], nres = g_n[kRes];
  CHECK(spec_verify_run(&c, &aq2, nullptr) == SV_OK && g_n[kTopp] == np + 1 && g_n[kStats] == ns_ + 2 && g_n[kRes] == nres);
  aq2 = aq;
  aq2.frequency_penalty = (const float *)g_fake;
  aq2.idx_mapping = (const int32_t *)g_fake;
  aq2.output_bin_counts = (const int32_t *)g_fake;
  aq2.num_slots = 300;
  np = g_n[kTopp], ns_ = g_n[kStats], nres = g_n[kRes];
  CHECK(spec_verify_run(&c, &aq2, nullptr) == SV_OK && g_n[kTopp] == np + 1 && g_n[kStats] == ns_ + 2 && g_n[kRes] == nres);
  sv_verify_args ad = a;
  ad.draft_probs = (const float *)g_fake;
  ad.draft_row_stride = a.vocab_size;
  const int nr = g_n[kResid];
  // (draft distributions alone keep the lean epilogue; with top-p or penalties, the general one)
  CHECK(spec_verify_run(&c, &ad, nullptr) == SV_OK && g_n[kResid] == nr + 1 && sv::plain_call(g_last));
  {
    sv_verify_args adq = ad;
    adq.top_p = (const float *)g_fake;
    CHECK(spec_verify_run(&c, &adq, nullptr) == SV_OK && !sv::plain_call(g_last));
  }
  ad.draft_row_stride = a.vocab_size - 1;
  CHECK(spec_verify_run(&c, &ad, nullptr) == SV_EINVAL);
  // Debug margins: one more launch, after the epilogue's.
  sv_verify_args am = a;
  am.dbg_margin = (float *)g_fake;
  const int nm = g_n[kMargin];
  CHECK(spec_verify_run(&c, &am, nullptr) == SV_OK && g_n[kMargin] == nm + 1 && g_last.dbg_margin == am.dbg_margin);
  CHECK(spec_verify_run(&c, &a, nullptr) == SV_OK && g_n[kMargin] == nm + 1);

  // Scalar and capacity checks (nothing launched).
  const int before = g_n[kStats];
  sv_verify_args e = a;
  e.offset = 1ull << 32;
  CHECK(spec_verify_run(&c, &e, nullptr) == SV_EINVAL);
  e = a;
  e.out_stride = 5;
  CHECK(spec_verify_run(&c, &e, nullptr) == SV_ECAPACITY);
  e = a;
  e.num_rows = 1101;
  CHECK(spec_verify_run(&c, &e, nullptr) == SV_ECAPACITY);
  e = a;
  e.vocab_size = 128257;
  CHECK(spec_verify_run(&c, &e, nullptr) == SV_ECAPACITY);
  e = a;
  e.logits_row_stride = 100;
  CHECK(spec_verify_run(&c, &e, nullptr) == SV_EINVAL);
  e = a;
  e.logits_dtype = 3;
  CHECK(spec_verify_run(&c, &e, nullptr) == SV_EDTYPE);
  e = a;
  e.temperature = nullptr;
  CHECK(spec_verify_run(&c, &e, nullptr) == SV_EINVAL);
  e = a;
  e.draft_logits = g_fake;
  CHECK(spec_verify_run(&c, &e, nullptr) == SV_EINVAL);  // draft-logits mode needs all three arrays
  float rates[SV_MAX_DRAFTS] = {0.9f, 0.95f};
  e = a;
  e.synthetic_rates = rates;
  CHECK(spec_verify_run(&c, &e, nullptr) == SV_EINVAL);  // increasing rates
  CHECK(g_n[kStats] == before);
  rates[1] = 0.5f;
  rates[2] = 0.25f;
  CHECK(spec_verify_run(&c, &e, nullptr) == SV_OK && g_last.synthetic == 1 && g_last.syn[2] == 0.25f);
  // The widest draft count: 64 synthetic rates copied, none beyond.
  sv_ctx c64 = make_ctx(70, 1, SV_MAX_DRAFTS, 3000, 0);
  sv_verify_args a64 = plain_args(1, 65, 3000, SV_F32, SV_MAX_DRAFTS + 1);
  for (int i = 0; i < SV_MAX_DRAFTS; ++i) rates[i] = 1.0f / (float)(i + 1);
  a64.synthetic_rates = rates;
  CHECK(spec_verify_run(&c64, &a64, nullptr) == SV_OK && g_last.syn[SV_MAX_DRAFTS - 1] == rates[SV_MAX_DRAFTS - 1]);
  // post_update inside the call: mismatched sizes are rejected.
  sv_post_update_args pu{};
  pu.idx_mapping = pu.query_len = (const int32_t *)g_fake;
  pu.last_sampled = pu.output_bin_counts = pu.num_computed_tokens = (int32_t *)g_fake;
  pu.num_reqs = 256;
  pu.vocab_size = 128256;
  pu.num_slots = 300;
  pu.tokens_stride = 4;
  e = a;
  e.post_update = &pu;
  CHECK(spec_verify_run(&c, &e, nullptr) == SV_OK && g_last.pu_idx_mapping != nullptr);
  e.dbg_margin = (float *)g_fake;  // debug margins read the penalties' counts: not with post_update
  CHECK(spec_verify_run(&c, &e, nullptr) == SV_EINVAL);
  e.dbg_margin = nullptr;
  pu.num_reqs = 255;
  CHECK(spec_verify_run(&c, &e, nullptr) == SV_EINVAL);
  // Epochs advance per call and skip 0 on wrap.
  c.epoch = 0xFFFFFFFFu;
  CHECK(spec_verify_run(&c, &a, nullptr) == SV_OK && g_last.epoch == 1);

  // post_update, draft-side sampling, LM head, debug entry points.
  sv_post_update_args pa = pu;
  pa.num_reqs = 256;
  pa.tokens = pa.num_sampled = pa.num_rejected = (const int32_t *)g_fake;
  CHECK(spec_post_update(&c, &pa, nullptr) == SV_OK && g_n[kPost] == 1 && g_post.B == 256);
  pa.tokens_stride = 0;
  CHECK(spec_post_update(&c, &pa, nullptr) == SV_EINVAL);
  sv_draft_args da{};
  da.draft_logits = g_fake;
  da.logits_dtype = SV_BF16;
  da.logits_row_stride = 128256;
  da.temperature = (const float *)g_fake;
  da.cu_num_draft = (const int32_t *)g_fake;
  da.out_tokens = (int32_t *)g_fake;
  da.draft_stats = (float *)g_fake;
  da.num_reqs = 256;
  da.vocab_size = 128256;
  da.step = 2;
  CHECK(spec_draft_sample(&c, &da, nullptr) == SV_OK && g_n[kDraft] == 1 && g_last.R == 256);
  sv_ctx cl = make_ctx(1100, 256, 3, 128256, SV_CREATE_LM_HEAD);
  sv_lm_head_args la{};
  la.hidden = la.lm_head = g_fake;
  la.hidden_row_stride = la.lm_head_row_stride = la.hidden_size = 4096;
  la.draft_ids = la.cu_num_draft = (const int32_t *)g_fake;
  la.temperature = (const float *)g_fake;
  la.out_tokens = la.out_num_sampled = la.out_num_rejected = (int32_t *)g_fake;
  la.num_reqs = 256;
  la.num_rows = 650;
  la.vocab_size = 128256;
  la.out_stride = 4;
  CHECK(spec_verify_lm_head(&cl, &la, nullptr) == SV_OK && g_lm.NT == 501 && g_lm.RB == 3 && g_lm.NC == 2004);
  CHECK(spec_verify_lm_head(&c, &la, nullptr) == SV_ECAPACITY);
  la.hidden_size = 4000;
  CHECK(spec_verify_lm_head(&cl, &la, nullptr) == SV_EINVAL);
  CHECK(spec_verify_debug_philox((const uint32_t *)g_fake, 4, 1, (uint32_t *)(g_fake + 8), nullptr) == SV_EINVAL);
  CHECK(spec_verify_debug_philox((const uint32_t *)g_fake, 4, 1, (uint32_t *)(g_fake + 16), nullptr) == SV_OK);
  CHECK(spec_verify_debug_exp_noise((const uint32_t *)g_fake, 8, (float *)g_fake, nullptr) == SV_OK);
  // The entry point without a context: argument checks before any HIP call.
  uint32_t *dev_err = (uint32_t *)g_fake;
  CHECK(spec_verify_run_noalloc(nullptr, dev_err, nullptr) == SV_EINVAL);
  CHECK(spec_verify_run_noalloc(&a, nullptr, nullptr) == SV_EINVAL);
  CHECK(spec_verify_run_noalloc(&ak, dev_err, nullptr) == SV_ECAPACITY);
  CHECK(spec_verify_run_noalloc(&a, dev_err, nullptr) == SV_EHIP);  // no device here
  float r3[3];
  CHECK(spec_verify_synthetic_rates(2.5f, 3, r3) == SV_OK && r3[0] == 1.0f && r3[1] == 0.5f && r3[2] == 0.0f);
  CHECK(spec_verify_synthetic_rates(5.0f, 3, r3) == SV_EINVAL);
  std::printf("ok\n");
  return 0;
}
