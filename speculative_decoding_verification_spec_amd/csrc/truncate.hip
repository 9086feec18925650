// KV length reset after a verification round (gfx950).
//
// [P2] "LLM推論の高速化｜KVキャッシュと投機的デコーディングを自作で実測":
// section numpyで小さなTransformerを自作する (KVCache.truncate only moves the
// length) and section 投機的デコーディングとは (the target cache is cut back to
// base + 1 + n_accepted after the round).  The rows of rejected drafts stay in
// memory but lie past the length, where nothing reads them.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "spec_verify.h"

namespace specv {

__global__ __launch_bounds__(256) void kv_truncate_kernel(int32_t* __restrict__ len, const int32_t* __restrict__ nacc,
                                                          int B, int n_q) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int n = nacc[b];
  if (n < 0) return;  // the sampler flagged this sequence; keep its length
  len[b] += 1 + min(n, n_q - 1);
}

}  // namespace specv

extern "C" spec_status_t spec_kv_truncate(int32_t* cache_len, const int32_t* n_accepted, int B, int n_q,
                                          hipStream_t stream) {
  if (!cache_len || !n_accepted || B < 1 || n_q < 1) return SPEC_ERR_ARG;
  hipLaunchKernelGGL(specv::kv_truncate_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, cache_len, n_accepted,
                     B, n_q);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_LAUNCH;
}
