// Library-internal entry to the verify forward: where its input tokens and
// positions come from.  spec_verify_forward takes them from caller arrays;
// a speculative round derives them on the GPU from its sequence buffer, in
// the forward's first launch.
#pragma once
#include <stdint.h>

#include "spec_verify.h"

namespace specv {

enum { SRC_ARRAYS = 0, SRC_DRAFT_STEP = 1, SRC_VERIFY = 2 };

struct TokenSource {
  int mode;
  // SRC_ARRAYS: tokens [B][n], cache_len [B] (the positions start there).
  const int32_t* tokens;
  const int32_t* cache_len;
  // SRC_DRAFT_STEP j (n = 2 at j = 0, else 1) and SRC_VERIFY (n = gamma + 1),
  // from a round's committed tokens seq [B][max_len] (seq_len [B]) and its
  // proposals xs [B][gamma]:
  //   draft step 0: seq[L-2], seq[L-1] at positions base_len[b], +1;
  //   draft step j: xs[j-1] at position base_len[b] + j + 1;
  //   verify:       seq[L-1], xs[0..gamma) from position cache_len[b].
  // A sequence length out of range gives token -1 (NaN rows for that
  // sequence only).  A draft step writes its cache lengths to pos_out [B],
  // which the step's attention then reads.
  const int32_t* seq;
  const int32_t* seq_len;
  const int32_t* base_len;
  const int32_t* xs;
  int32_t* pos_out;
  int max_len, gamma, j;
};

// A draw from the last logit row of each sequence, made by the forward as
// soon as that row exists: the row is copied to draft_logits[b][j] and
// proposal xs[b][j] is drawn at u[b][j] from softmax(z / T) (c32 = log2(e)/T),
// or is the row's argmax when greedy.
struct DrawSpec {
  const double* u;     // [B][gamma]
  float* draft_logits;  // [B][gamma][V]
  int32_t* xs;          // [B][gamma]
  int gamma, j, greedy;
  float c32;
};

spec_status_t verify_forward(const spec_model_t* model, const float* params, const TokenSource& src,
                             float* kv_cache, int max_T, float* logits, int B, int n, int max_len_hint,
                             void* workspace, size_t workspace_bytes, hipStream_t stream,
                             const DrawSpec* draw = nullptr);

}  // namespace specv
