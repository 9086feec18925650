// One speculative-decoding round of a draft and a target model, on the
// device (gfx950).
//
// [P2] "LLM推論の高速化｜KVキャッシュと投機的デコーディングを自作で実測" section
// 投機的デコーディングとは (the round's listing and flowchart): the draft
// proposes gamma tokens, each drawn from its distribution q_j; the target is
// called once over [last committed token] + proposals; the accept tests, the
// residual or bonus draw and the emitted tokens are spec_reject_sample's; the
// sequence grows by the accepted proposals and the drawn token, the target
// cache is cut back to base + 1 + n and the draft cache likewise.
//
// Draft side.  A sequence of L committed tokens keeps the draft cache at
// L - 2 tokens on entry: the draft's first call of a round runs over the last
// two committed tokens at positions L-2, L-1 (re-running the second-to-last
// one, whose K/V the cache may or may not hold: when every proposal of the
// previous round was accepted, the draft never ran the last of them), then one
// call per proposal.  Every sequence thus feeds the same number of tokens per
// call, and after the round the draft cache is cut to L' - 2 with the same
// length reset as the target's (+1 + n).  Each proposal is the inverse-CDF
// draw of softmax(z / T) at its uniform (the convention of the final draw);
// at T = 0 it is the argmax.
//
// The only kernel here commits tokens and lengths.  The forwards are the
// verify forward's, taking their tokens and positions from the sequence
// buffer and the proposals (TokenSource) and making the draft's draws
// (DrawSpec); the verification is spec_reject_sample.
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "model_internal.h"
#include "spec_common.h"
#include "spec_verify.h"

namespace specv {

// Commit: append the n+1 emitted tokens, and advance the sequence, target
// and draft lengths by n + 1.  A negative n (a sampler error) changes
// nothing; so does a sequence whose tokens would not fit, and it is reported
// as n_accepted = -1.
__global__ __launch_bounds__(256) void round_commit(int32_t* __restrict__ seq, int32_t* __restrict__ seq_len,
                                                   int max_len, int32_t* __restrict__ target_len,
                                                   int32_t* __restrict__ draft_len,
                                                   int32_t* __restrict__ n_accepted,
                                                   const int32_t* __restrict__ out_tokens, int gamma, int B) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int n = n_accepted[b];
  if (n < 0 || n > gamma) return;
  const int L = seq_len[b];
  if (L < 0 || (long)L + n + 1 > (long)max_len) {
    n_accepted[b] = -1;
    return;
  }
  for (int i = 0; i <= n; ++i) seq[(size_t)b * max_len + L + i] = out_tokens[(size_t)b * (gamma + 1) + i];
  seq_len[b] = L + n + 1;
  target_len[b] += n + 1;
  draft_len[b] += n + 1;
}

struct RoundPlan {
  size_t off_fwd, fwd_bytes, off_rs, rs_bytes, off_pos, off_step, off_dl, off_xs, off_tl, total;
};

static inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

static bool round_plan(const spec_model_t* t, const spec_model_t* d, int B, int gamma, int hint, RoundPlan* p) {
  const int V = t->V;
  size_t fwd = spec_verify_forward_workspace_size(t, B, gamma + 1, std::max(0, hint - 1));
  const size_t f0 = spec_verify_forward_workspace_size(d, B, 2, std::max(0, hint - 2));
  const size_t f1 = spec_verify_forward_workspace_size(d, B, 1, hint + gamma - 2);
  if (fwd == 0 || f0 == 0 || f1 == 0) return false;
  fwd = std::max(fwd, std::max(f0, f1));
  const size_t rs = spec_reject_sample_workspace_size(B, gamma, V, SPEC_F32);
  if (rs == 0) return false;
  RoundPlan r{};
  size_t off = 0;
  r.off_fwd = off;
  r.fwd_bytes = fwd;
  off = align256(off + fwd);
  r.off_rs = off;
  r.rs_bytes = rs;
  off = align256(off + rs);
  r.off_pos = off;
  off = align256(off + sizeof(int32_t) * (size_t)B);
  r.off_step = off;
  off = align256(off + sizeof(float) * 2 * (size_t)B * V);
  r.off_dl = off;
  off = align256(off + sizeof(float) * (size_t)B * gamma * V);
  r.off_xs = off;
  off = align256(off + sizeof(int32_t) * (size_t)B * gamma);
  r.off_tl = off;
  off = align256(off + sizeof(float) * (size_t)B * (gamma + 1) * V);
  r.total = off;
  *p = r;
  return true;
}

}  // namespace specv

using namespace specv;

extern "C" size_t spec_speculative_round_workspace_size(const spec_model_t* target, const spec_model_t* draft, int B,
                                                        int gamma, int max_len_hint) {
  if (!target || !draft || B < 1 || gamma < 1 || gamma > 15 || max_len_hint < 2) return 0;
  if (target->V != draft->V) return 0;
  RoundPlan p;
  return round_plan(target, draft, B, gamma, max_len_hint, &p) ? p.total : 0;
}

extern "C" spec_status_t spec_speculative_round(
    const spec_model_t* target, const float* target_params, const spec_model_t* draft, const float* draft_params,
    int32_t* seq, int32_t* seq_len, int max_len, float* target_kv, int32_t* target_len, int target_max_T,
    float* draft_kv, int32_t* draft_len, int draft_max_T, const double* u_draft, const double* u_verify, int B,
    int gamma, float temperature, int max_len_hint, int32_t* n_accepted, int32_t* out_tokens, void* workspace,
    size_t workspace_bytes, hipStream_t stream) {
  if (!target || !draft || !target_params || !draft_params || !seq || !seq_len || !target_kv || !target_len ||
      !draft_kv || !draft_len || !n_accepted || !out_tokens || !workspace)
    return SPEC_ERR_ARG;
  const bool greedy = temperature == 0.f;
  if (!greedy && (!u_draft || !u_verify || !(temperature > 0.f) || !isfinite(temperature))) return SPEC_ERR_ARG;
  if (B < 1 || gamma < 1 || max_len_hint < 2 || max_len < 1) return SPEC_ERR_ARG;
  if (target->V != draft->V || spec_model_param_count(target) == 0 || spec_model_param_count(draft) == 0)
    return SPEC_ERR_ARG;
  if (gamma > 15) return SPEC_ERR_UNSUPPORTED;  // the verify call runs gamma + 1 <= 16 tokens
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return SPEC_ERR_ARG;
  // room for the round: gamma + 1 more tokens, caches and positions
  if ((long)max_len_hint + gamma + 1 > (long)max_len) return SPEC_ERR_OVERFLOW;
  if ((long)max_len_hint + gamma > (long)target_max_T || (long)max_len_hint + gamma > (long)target->T)
    return SPEC_ERR_OVERFLOW;
  if ((long)max_len_hint + gamma - 1 > (long)draft_max_T || (long)max_len_hint + gamma - 1 > (long)draft->T)
    return SPEC_ERR_OVERFLOW;
  RoundPlan p;
  if (!round_plan(target, draft, B, gamma, max_len_hint, &p)) return SPEC_ERR_UNSUPPORTED;
  if (workspace_bytes < p.total) return SPEC_ERR_ARG;

  char* ws = static_cast<char*>(workspace);
  void* fws = ws + p.off_fwd;
  void* rws = ws + p.off_rs;
  int32_t* pos = reinterpret_cast<int32_t*>(ws + p.off_pos);
  float* step = reinterpret_cast<float*>(ws + p.off_step);
  float* dlog = reinterpret_cast<float*>(ws + p.off_dl);
  int32_t* xs = reinterpret_cast<int32_t*>(ws + p.off_xs);
  float* tlog = reinterpret_cast<float*>(ws + p.off_tl);
  const int V = target->V;
  const float c32 = greedy ? 0.f : (float)(1.4426950408889634 / (double)temperature);  // 2^(z c) = e^(z/T)
  const unsigned gB = (unsigned)((B + 255) / 256);

  // The forwards read their tokens and positions from the sequence buffer
  // and the proposals themselves (TokenSource), in their first launch.
  TokenSource src{};
  src.seq = seq;
  src.seq_len = seq_len;
  src.max_len = max_len;
  src.xs = xs;
  src.gamma = gamma;
  for (int j = 0; j < gamma; ++j) {
    const int n = j == 0 ? 2 : 1;
    src.mode = SRC_DRAFT_STEP;
    src.base_len = draft_len;
    src.pos_out = pos;
    src.j = j;
    const int hint = j == 0 ? max_len_hint - 2 : max_len_hint + j - 1;
    DrawSpec dr{};
    dr.u = u_draft;
    dr.draft_logits = dlog;
    dr.xs = xs;
    dr.gamma = gamma;
    dr.j = j;
    dr.greedy = greedy ? 1 : 0;
    dr.c32 = c32;
    spec_status_t st = verify_forward(draft, draft_params, src, draft_kv, draft_max_T, step, B, n, hint, fws,
                                      p.fwd_bytes, stream, &dr);
    if (st != SPEC_OK) return st;
  }
  src.mode = SRC_VERIFY;
  src.cache_len = target_len;
  spec_status_t st = verify_forward(target, target_params, src, target_kv, target_max_T, tlog, B, gamma + 1,
                                    max_len_hint - 1, fws, p.fwd_bytes, stream);
  if (st != SPEC_OK) return st;
  st = spec_reject_sample(tlog, greedy ? nullptr : dlog, xs, greedy ? nullptr : u_verify, B, gamma, V, temperature,
                          SPEC_F32, n_accepted, out_tokens, nullptr, nullptr, rws, p.rs_bytes, stream);
  if (st != SPEC_OK) return st;
  hipLaunchKernelGGL(round_commit, dim3(gB), dim3(256), 0, stream, seq, seq_len, max_len, target_len, draft_len,
                     n_accepted, out_tokens, gamma, B);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_LAUNCH;
}
