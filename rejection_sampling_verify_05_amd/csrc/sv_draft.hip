// sv_draft.hip -- draft-side sampling after a streaming pass over the draft rows.
#include <stdint.h>

#include "sv_common.h"

namespace sv {

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Draft-side sampling, after a streaming pass over this step's draft rows (row
// r of the call = request r).  One workgroup per request: the row's scale m and
// mass s from its chunk table, then the two-level race on counter row
// cu[r] + step (the draft's row in the verify call) with the draft tags, or the
// argmax (lowest index) when T = 0; q(d) and (m, s) are recorded for the
// verifier.
// ---------------------------------------------------------------------------
struct DraftShared {
  BlockScratch red;
  float zs[kChunk];
};

__global__ __launch_bounds__(kThreads) void draft_race_kernel(Params p, DraftOut o) {
  __shared__ DraftShared sh;
  const int r = blockIdx.x, tid = threadIdx.x;
  const int K = o.cu[r + 1] - o.cu[r];
  const float T = p.temperature[r];
  const bool bad_t = !(T >= 0.0f) || !__builtin_isfinite(T);
  if (o.step >= K || bad_t) {  // no draft at this position, or an invalid temperature
    if (tid == 0) {
      if (bad_t && o.step < K) raise_err(p, SV_ERR_TEMPERATURE);
      o.tokens[r] = -1;
      if (o.q) o.q[r] = 0.0f;
    }
    return;
  }
  const uint32_t key = (uint32_t)(o.cu[r] + o.step);
  const float a = T > 0.0f ? kLog2e / T : 0.0f;
  const float2 *tab = p.chunk_tab + (int64_t)r * p.nc_stride;
  float lm = kNegInf;
  for (int c = tid; c < p.NC; c += kThreads) lm = fmaxf(lm, tab[c].x);
  const float m = block_max(lm, sh.red);
  if (!(m > kNegInf)) {
    if (tid == 0) {
      raise_err(p, SV_ERR_ROW);
      o.tokens[r] = -1;
      if (o.q) o.q[r] = 0.0f;
    }
    return;
  }
  float ls = 0.0f;
  for (int c = tid; c < p.NC; c += kThreads) {
    const float2 e = tab[c];
    if (e.x > kNegInf) ls += e.y * exp2_acc(a * (e.x - m));
  }
  const float s = block_sum(ls, sh.red);
  int cstar;
  if (T == 0.0f) {  // the lowest chunk holding the maximum (greedy tables hold exact chunk maxima)
    ArgMax best{-1.0f, 0x7FFFFFFF};
    for (int c = tid; c < p.NC; c += kThreads)
      if (tab[c].x == m && c < best.i) best = ArgMax{1.0f, c};
    cstar = block_argmax(best, sh.red).i;
  } else {
    cstar = block_chunk_race(p, key, p.NC, [&](int c) -> float {
      const float2 e = tab[c];
      return e.x > kNegInf ? e.y * exp2_acc(a * (e.x - m)) : 0.0f;
    }, sh.red, kTagDraftChunk);
  }
  int d = -1;
  if (cstar >= 0) {
    for (int t = tid; t < kChunk; t += kThreads) {
      const int x = cstar * kChunk + t;
      sh.zs[t] = x < p.V ? load_logit(p, r, x) : kNegInf;
    }
    __syncthreads();
    if (T == 0.0f) {  // first token of the chunk equal to the maximum
      ArgMax best{-1.0f, 0x7FFFFFFF};
      for (int t = tid; t < kChunk; t += kThreads)
        if (sh.zs[t] == m && t < best.i) best = ArgMax{1.0f, t};
      const ArgMax b = block_argmax(best, sh.red);
      d = b.s < 0.0f ? -1 : cstar * kChunk + b.i;
    } else {
      Proc pr;
      pr.counts = nullptr;
      pr.theta = 1.0f;
      pr.freq = pr.pres = 0.0f;
      pr.tau = kNegInf;
      d = block_token_race(p, (int)key, cstar, sh.zs, pr, a, a * m, -1, sh.red, kTagDraftToken);
    }
  }
  if (tid == 0) {
    o.tokens[r] = d;
    if (o.ids) o.ids[key] = d;
    o.stats[2 * (int64_t)key] = m;
    o.stats[2 * (int64_t)key + 1] = s;
    if (o.q) o.q[r] = d < 0 ? 0.0f : (T == 0.0f ? 1.0f : exp2_acc(a * (sh.zs[d - cstar * kChunk] - m)) / s);
  }
}

hipError_t launch_draft_race(const Params &p, const DraftOut &o, hipStream_t s) {
  draft_race_kernel<<<dim3((unsigned)p.B), dim3(kThreads), 0, s>>>(p, o);
  return hipGetLastError();
}

}  // namespace sv
