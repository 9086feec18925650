"""CPU oracle for the speculative-decoding verification step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product (the HIP library and its
Python binding) imports, links or runs anything here.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
use this package.

The oracle is a plain, slow, obviously-correct numpy implementation in fp64
of what the verification step computes.  It shares no code with the GPU path.
Each function cites the passage of the source pages it follows.  The pages are
cited by title and section:

  [P1] "投機的デコーディングとドラフトモデル" (tech-tldr.com)
  [P2] "LLM推論の高速化｜KVキャッシュと投機的デコーディングを自作で実測" (r-jc.jp)
  [P3] "Speculative Decoding（投機的デコーディング）とは？仕組みと速くなる条件、
        LM Studio・llama.cpp・vLLMでの設定" (issoh.co.jp)

Modules:
  sampler    -- modified rejection sampling (accept test, first rejection,
                residual / bonus inverse-CDF draw, emitted tokens)
  greedy     -- temperature-0 verification (accept while the draft is the
                target's argmax, then the target's argmax)
  attention  -- KV append and causal multi-query verify attention, plus the
                uncached full-sequence recompute it must agree with
  paged      -- verify attention over a paged cache (block tables), and the
                allocation-waste count of paging
  quant      -- verify attention over an int8 cache with per-row float16
                scales (quantise, convert back, attend)
  truncate   -- the KV length reset after verification
  model      -- the verify forward of the pages' GPT-2-type decoder (cached,
                and the uncached full-sequence forward it must agree with)
  round      -- one speculative round of a draft and a target model: draft
                proposals, one verify call, the draw, both cache truncations
  formulas   -- closed forms: acceptance rate, expected committed tokens,
                speed-up estimate, KV-cache bytes
  bf16       -- exact decoding of bfloat16 bit patterns to fp64

Parity status: every function here is pinned by ``-m "not gpu"`` tests against
printed values of the pages, closed forms, library routines or brute force.
That includes the margin helpers that decide which decisions fall inside the
1e-6 threshold band (tests/test_oracle_band.py: a margin below eps is exactly
a decision that a shift of eps would change) and the band probability that
bounds how many sequences a comparison may leave out.  Nothing is "parity
unpinned" except the mapping of the decisions inside that band: those draws
are counted and bounded, not compared.
"""

from . import attention, bf16, formulas, greedy, model, paged, quant, round, sampler, truncate  # noqa: F401
