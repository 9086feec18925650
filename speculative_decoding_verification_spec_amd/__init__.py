"""Speculative-decoding verification step on AMD MI355X (gfx950).

The step is three calls into the C-ABI library libspecverify.so, bound here
with ctypes (see include/spec_verify.h for the contract of each):

  spec_verify_attention  KV append + causal multi-query verify attention (GQA)
  spec_verify_attention_paged  the same over a paged cache (block tables)
  spec_verify_attention_int8   the same over an int8 cache with fp16 row scales
  spec_reject_sample     modified rejection sampling over the vocabulary
                         (greedy verification at temperature 0)
  spec_kv_truncate       length reset after the round
  spec_verify_forward    the cached verify forward of a GPT-2-type decoder
                         (embeddings, blocks with the verify attention, logits)
  spec_speculative_round one whole round on the device: draft proposals, the
                         target's verify forward, the sampler, the commit

PyTorch supplies device memory and streams; all arithmetic runs in the HIP
kernels.  Importing this package does not load the library; the first call
does, and raises if the library has not been built.
"""

from ._lib import (  # noqa: F401
    EXPORTED,
    LIB_PATH,
    SpecError,
    SpecModel,
    Workspace,
    load,
    model_param_count,
    model_param_layout,
    reject_sample_workspace_size,
    spec_kv_truncate,
    spec_reject_sample,
    spec_speculative_round,
    spec_verify_attention,
    spec_verify_attention_int8,
    spec_verify_attention_paged,
    spec_verify_forward,
    verify_attention_workspace_size,
    version,
)
