/* spec_verify.h -- C ABI of the speculative-decoding verification step on
 * AMD Instinct MI355X (gfx950).
 *
 * Source pages (cited by title and section):
 *   [P1] "投機的デコーディングとドラフトモデル" (tech-tldr.com)
 *   [P2] "LLM推論の高速化｜KVキャッシュと投機的デコーディングを自作で実測" (r-jc.jp)
 *   [P3] "Speculative Decoding（投機的デコーディング）とは？仕組みと速くなる条件、
 *         LM Studio・llama.cpp・vLLMでの設定" (issoh.co.jp)
 *
 * One verification round of speculative decoding for a batch of B sequences:
 *   1. spec_verify_attention: the target's single call over [last committed
 *      token] + gamma drafts appends those n_q = gamma+1 tokens' K/V to each
 *      sequence's cache and runs causal multi-query attention of the n_q rows
 *      against it ([P2] numpyで小さなTransformerを自作する; 投機的デコーディングとは).
 *   2. spec_reject_sample: modified rejection sampling over the vocabulary
 *      ([P1] 受理判定の数理：修正版棄却サンプリング; [P2] 投機的デコーディングとは;
 *      [P3] 受理・棄却の規則と出力分布が変わらない理由).
 *   3. spec_kv_truncate: the length reset that drops the rejected drafts' K/V
 *      ([P2] numpyで小さなTransformerを自作する, KVCache.truncate).
 *
 * Conventions for every entry point:
 *   - Pointers named as device pointers must point to device memory (e.g. the
 *     data of PyTorch CUDA/HIP tensors); the caller owns all of them.
 *   - Arrays are dense, row-major (C order), in the layouts stated below.
 *   - All work is enqueued on `stream` (0 = the null stream); no call
 *     synchronises, allocates device memory or keeps state across calls other
 *     than what lives in the caller's workspace.
 *   - Host-side argument checks run before any launch; a failed check returns
 *     an error code and launches nothing.  Nothing throws across the ABI.
 *   - Outputs must not alias inputs.  Calls that share a workspace must not
 *     run concurrently.
 *   - Workspaces need no initialisation: every call writes each workspace
 *     word before reading it, so one buffer may serve calls of any sizes (up
 *     to its capacity) one after another on a stream.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPEC_OK = 0,
  SPEC_ERR_ARG = 1,         /* bad pointer, size, alignment or workspace size   */
  SPEC_ERR_OVERFLOW = 2,    /* cache too small: max_len_hint + n_q > max_T      */
  SPEC_ERR_UNSUPPORTED = 3, /* valid request outside what the library supports */
  SPEC_ERR_LAUNCH = 4,      /* the HIP runtime refused a kernel launch          */
  SPEC_ERR_SCRATCH = 5      /* more than a no-allocation call's fixed scratch    */
} spec_status_t;

/* Element type of the tensors a call reads and writes: fp32, bf16, or IEEE
 * half (SPEC_F16: the verify attention entry points only; the sampler takes
 * SPEC_F32 and SPEC_BF16 logits). */
typedef enum { SPEC_F32 = 0, SPEC_BF16 = 1, SPEC_F16 = 2 } spec_dtype_t;

/* Library version, e.g. "specverify 0.1.0 gfx950". Static string. */
const char* spec_version(void);

/* Human-readable name of a status code. Static string. */
const char* spec_status_string(spec_status_t s);

/* ------------------------------------------------------------------------- */
/* Verify attention                                                           */
/* ------------------------------------------------------------------------- */

/* Workspace bytes spec_verify_attention needs for these sizes.  A workspace
 * sized for max_len_hint h serves every call with the same other sizes and a
 * hint <= h.  Returns 0 for invalid sizes. */
size_t spec_verify_attention_workspace_size(int B, int Hq, int Hkv, int n_q, int D, int max_len_hint,
                                            spec_dtype_t dtype);

/* Causal multi-query verify attention with KV append.
 *
 * Defined by [P2] section numpyで小さなTransformerを自作する (the forward_cached
 * listing): with p0 = the cache length before the call, the n new tokens' K/V
 * go to cache rows [p0, p0+n); the i-th new query attends to rows [0, p0+i];
 * scores are scaled by 1/sqrt(D) and soft-maxed.  Grouped-query sharing
 * ([P2] section GQA・MQAでKVキャッシュを減らす): query head h reads KV head
 * h / (Hq / Hkv) (contiguous groups).
 *
 *   q        device, [B][Hq][n_q][D]        dtype       queries of the n_q rows
 *   k_new    device, [B][Hkv][n_q][D]       dtype       K of [last committed] + drafts
 *   v_new    device, [B][Hkv][n_q][D]       dtype
 *   k_cache  device, [B][Hkv][max_T][D]     dtype, in/out
 *   v_cache  device, [B][Hkv][max_T][D]     dtype, in/out
 *            rows [cache_len[b], cache_len[b] + n_q) are overwritten with
 *            k_new / v_new; no other row is written; rows >= cache_len[b] are
 *            never read (their contents may be anything, NaN included).
 *   cache_len device, [B] int32, committed length L_b before the call (read only;
 *            spec_kv_truncate commits the new length).
 *   out      device, [B][Hq][n_q][D]        dtype       attention output
 *   scale    score scale; the pages' value is 1/sqrt(D).
 *   max_len_hint  host upper bound on max_b cache_len[b]; it sizes the launch.
 *   workspace device, >= spec_verify_attention_workspace_size(...) bytes.
 * Arithmetic: scores, softmax and accumulation in fp32; bf16 and fp16 inputs
 * are consumed exactly, the probabilities are rounded to the input type for
 * the PV product, and the output is rounded to nearest-even.
 * Supported: dtype SPEC_BF16 with D in {64, 128}; SPEC_F16 (the fp16 cache of
 * [P2] section PagedAttentionとKVキャッシュの量子化) with D in {64, 128} and
 * B <= 1024; SPEC_F32 with D in {24, 32, 64, 128}; 1 <= n_q <= 16;
 * Hq % Hkv == 0; Hq/Hkv * n_q <= 256.
 * Errors: SPEC_ERR_ARG for null pointers, non-positive sizes, Hq % Hkv != 0,
 * pointers not 16-byte aligned, or a small workspace; SPEC_ERR_OVERFLOW if
 * max_len_hint + n_q > max_T; SPEC_ERR_UNSUPPORTED outside the supported set.
 * A sequence whose device-side cache_len[b] is negative or exceeds
 * max_len_hint is not processed: nothing is written to its cache rows and its
 * output rows are set to NaN. */
spec_status_t spec_verify_attention(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                    void* v_cache, const int32_t* cache_len, void* out, int B, int Hq, int Hkv,
                                    int n_q, int D, int max_T, int max_len_hint, float scale, spec_dtype_t dtype,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Verify attention with KV append over a paged cache.
 *
 * Defined by [P2] section PagedAttentionとKVキャッシュの量子化 (paging): a
 * sequence's cache positions are held in fixed blocks of page_size positions,
 * and a block table lists the page of each of its blocks; the attention is
 * that of spec_verify_attention on the sequence's positions in table order.
 *
 *   k_pages, v_pages device, [Hkv][num_pages][page_size][D] dtype, in/out:
 *            position j of sequence b, KV head g, is
 *            pages[g][block_table[b][j / page_size]][j % page_size].  The new
 *            rows go to positions [cache_len[b], cache_len[b] + n_q); no other
 *            position is written, positions >= cache_len[b] are never read.
 *            Pages may be shared by several sequences for reading; the pages
 *            receiving new rows must not be.
 *   block_table device, [B][max_blocks] int32: entries for the blocks that hold
 *            positions [0, cache_len[b] + n_q) must lie in [0, num_pages).
 *   page_size 16 or 32.
 *   The other arguments are those of spec_verify_attention; the workspace size
 *   is spec_verify_attention_workspace_size(...) for the same sizes.
 * Supported: dtype SPEC_BF16 or SPEC_F16, D in {64, 128}, B <= 1024, and the
 * limits of spec_verify_attention.
 * Errors: as spec_verify_attention, with max_T = max_blocks * page_size;
 * SPEC_ERR_ARG for a null block_table, num_pages < 1 or max_blocks < 1;
 * SPEC_ERR_UNSUPPORTED for another page size, dtype, or B > 1024.  A sequence
 * with a table entry outside [0, num_pages) gets NaN output rows and nothing is
 * written through that entry; a negative cache_len[b] or one above
 * max_len_hint is handled as in spec_verify_attention. */
spec_status_t spec_verify_attention_paged(const void* q, const void* k_new, const void* v_new, void* k_pages,
                                          void* v_pages, const int32_t* block_table, const int32_t* cache_len,
                                          void* out, int B, int Hq, int Hkv, int n_q, int D, int page_size,
                                          int num_pages, int max_blocks, int max_len_hint, float scale,
                                          spec_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                          hipStream_t stream);

/* Workspace bytes spec_verify_attention_int8 needs (a workspace sized for a
 * hint serves smaller hints).  Returns 0 for invalid or unsupported sizes. */
size_t spec_verify_attention_int8_workspace_size(int B, int Hq, int Hkv, int n_q, int D, int max_len_hint);

/* Verify attention with KV append over an int8 cache.
 *
 * Defined by [P2] section PagedAttentionとKVキャッシュの量子化 (quantisation):
 * every cached row -- one KV head at one position -- holds int8 values q and a
 * float16 scale s, and stands for q * s; the attention is that of
 * spec_verify_attention on those values.  The n_q new rows are quantised on
 * append: s = max|x| / 127, q = round-half-even(x / s) clipped to +-127, both
 * in fp32 (a zero row gives s = 0, q = 0), the stored scale fp16(s) rounded to
 * nearest-even; the call attends to the new rows' quantised values too.
 *
 *   q, k_new, v_new, out  as spec_verify_attention, dtype bf16.
 *   k_cache, v_cache device, [B][Hkv][max_T][D] int8, in/out.
 *   k_scale, v_scale device, [B][Hkv][max_T] float16 (bits), in/out.
 *            Rows [cache_len[b], cache_len[b] + n_q) of both are overwritten
 *            with the quantised new rows; no other row is written; rows >=
 *            cache_len[b] are never used.
 *   workspace device, >= spec_verify_attention_int8_workspace_size(...) bytes.
 * Arithmetic: scores from the f16 MFMA with fp32 accumulation, the int8
 * values widened to f16 exactly and the bf16 query converted to f16 (exact
 * down to 2^-14 in magnitude, a few low bits lost below), times the key's
 * scale in fp32; V rows dequantised to bf16(q s) for the bf16 PV product.
 * Probabilities are taken against a fixed per-row reference (the row's
 * largest score in its first key block).  A group of rows sharing a KV head
 * is computed again on an exact fp32 path with the usual running-maximum
 * rescale when one of its rows sums to more than 2^64 against that reference
 * or to a value that is not finite, or when one of its query elements is
 * beyond f16's range (|x| > 65504, inf or NaN).
 * Supported: D in {64, 128}, B <= 1024, and the limits of
 * spec_verify_attention.
 * Errors: as spec_verify_attention (dtype fixed to bf16 activations), and
 * SPEC_ERR_ARG if max_T is not a multiple of 8 or a pointer is not 16-byte
 * aligned; SPEC_ERR_UNSUPPORTED outside the supported set. */
spec_status_t spec_verify_attention_int8(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                         void* k_scale, void* v_cache, void* v_scale, const int32_t* cache_len,
                                         void* out, int B, int Hq, int Hkv, int n_q, int D, int max_T,
                                         int max_len_hint, float scale, void* workspace, size_t workspace_bytes,
                                         hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* Modified rejection sampler                                                 */
/* ------------------------------------------------------------------------- */

/* Workspace bytes spec_reject_sample needs.  Returns 0 for invalid sizes. */
size_t spec_reject_sample_workspace_size(int B, int gamma, int V, spec_dtype_t dtype);

/* Modified rejection sampling for one round.
 *
 * Defined by [P1] section 受理判定の数理：修正版棄却サンプリング, [P2] section
 * 投機的デコーディングとは (the verify listing) and [P3] section
 * 受理・棄却の規則と出力分布が変わらない理由 (the five steps):
 *   p_i = softmax(target_logits[b][i] / T), i = 0..gamma
 *   q_i = softmax(draft_logits[b][i] / T),  i = 0..gamma-1
 *   position i is accepted iff uniforms[b][i] < min(1, p_i(x_i) / q_i(x_i));
 *   n = the number of leading accepted positions (the scan stops at the first
 *   rejection);
 *   if n < gamma the final token is drawn from normalize(max(0, p_n - q_n))
 *   (if that mass is exactly zero, from p_n); if n == gamma it is the bonus
 *   token drawn from p_gamma; the draw is inverse-CDF with uniforms[b][gamma]:
 *   the smallest j with C_j / C_{V-1} > u, C the prefix sum of the weights.
 *
 * T == 0 is greedy verification, [P2] section 投機的デコーディングとは (the
 * listing omits its temperature-0 branch; the results after it say that the
 * test then checks whether the draft token is the target's most likely token,
 * and that the output is then the target's own greedy decoding):
 *   position i is accepted iff argmax target_logits[b][i] == x_i; n as above;
 *   the final token is argmax target_logits[b][n].  argmax is the first index
 *   of the largest value (values compared exactly; -0 == +0; NaN is largest).
 *   draft_logits and uniforms are not read and may be NULL; p_draft[i] is 1.0
 *   when x_i is the argmax, else 0.0; q_draft is written as NaN.
 *
 *   target_logits device, [B][gamma+1][V] dtype
 *   draft_logits  device, [B][gamma][V]   dtype (NULL allowed when T == 0)
 *   draft_tokens  device, [B][gamma] int32, x_i, each in [0, V)
 *   uniforms      device, [B][gamma+1] double in [0, 1): [i < gamma] the accept
 *                 test at i, [gamma] the final draw (residual or bonus); NULL
 *                 allowed when T == 0
 *   temperature   T > 0 applied to both target and draft logits, or 0 (greedy)
 *   n_accepted    device out, [B] int32 in 0..gamma (-1: a draft token of this
 *                 sequence was outside [0, V); its out_tokens are all -1)
 *   out_tokens    device out, [B][gamma+1] int32: x_0..x_{n-1}, the final token,
 *                 then -1
 *   p_draft, q_draft  device out or NULL, [B][gamma] float: p_i(x_i), q_i(x_i)
 *   workspace     device, >= spec_reject_sample_workspace_size(...) bytes
 * Arithmetic: logits are read exactly; per-element exponentials and the
 * residual weights in fp32; row sums and all prefix sums in fp64; the accept
 * comparison in fp64.  Distributions are never assumed to sum to 1.
 * Errors: SPEC_ERR_ARG for null required pointers, B < 1, gamma < 1,
 * gamma > 31, V < 1, T < 0 or not finite, or a small workspace;
 * SPEC_ERR_UNSUPPORTED when a row holds more than 1024 segments of the
 * kernels' tiling (V above about 2 million). */
spec_status_t spec_reject_sample(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                                 const double* uniforms, int B, int gamma, int V, float temperature,
                                 spec_dtype_t dtype, int32_t* n_accepted, int32_t* out_tokens, float* p_draft,
                                 float* q_draft, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* spec_reject_sample without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments and results, minus the
 * workspace.  Its scratch is a fixed 16 MiB array in device memory that each
 * GPU the library runs on holds from the first load of the library's code
 * until the process ends; the call allocates nothing (no hipMalloc, no
 * library routine that does).  Every call on a GPU uses that GPU's one
 * array, so calls that overlap in time on one GPU (different streams, or
 * other threads) race and must be ordered by the caller.  A request whose
 * spec_reject_sample_workspace_size(B, gamma, V, dtype) exceeds 16 MiB
 * returns SPEC_ERR_SCRATCH (about B * (2 gamma + 1) * ceil(V / 2048) * 16
 * bytes for bf16: 256 sequences of gamma = 8 over 128,256 tokens need 4.6
 * MiB); other errors as spec_reject_sample, SPEC_ERR_LAUNCH if the scratch's
 * device address cannot be found. */
spec_status_t spec_reject_sample_noalloc(const void* target_logits, const void* draft_logits,
                                         const int32_t* draft_tokens, const double* uniforms, int B, int gamma, int V,
                                         float temperature, spec_dtype_t dtype, int32_t* n_accepted,
                                         int32_t* out_tokens, float* p_draft, float* q_draft, hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* KV length reset                                                            */
/* ------------------------------------------------------------------------- */

/* cache_len[b] <- cache_len[b] + 1 + n_accepted[b].
 *
 * Defined by [P2] section 投機的デコーディングとは: after the round the target
 * cache is cut back to base + 1 + n_accepted -- the last committed token and
 * the accepted drafts keep their K/V, the rejected drafts' rows become dead
 * (they are simply past the length).  The final (corrected or bonus) token has
 * no K/V yet; it is the first input of the next round.
 *   cache_len   device, [B] int32, in/out
 *   n_accepted  device, [B] int32; values above n_q-1 are clamped to n_q-1;
 *               negative values (a sampler error) leave cache_len[b] unchanged
 * Errors: SPEC_ERR_ARG for null pointers, B < 1 or n_q < 1. */
spec_status_t spec_kv_truncate(int32_t* cache_len, const int32_t* n_accepted, int B, int n_q, hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* Verify forward of a GPT-2-type decoder                                     */
/* ------------------------------------------------------------------------- */

/* Shape of a decoder-only model as in [P2] section
 * numpyで小さなTransformerを自作する: pre-LayerNorm blocks, learned token and
 * position embeddings, GELU MLP of width 4C; head dimension D = C / H.  The
 * section's parameter counts (513,600 for V=96 C=96 L=4 H=4 T=512; 61,968 for
 * the draft V=96 C=48 L=1 H=2 T=512) fix the parameter set below. */
typedef struct {
  int V; /* vocabulary */
  int C; /* width (C % H == 0) */
  int L; /* layers */
  int H; /* heads */
  int T; /* positions: rows of the position embedding */
} spec_model_t;

/* Floats in the packed fp32 parameter array of `model` (0 for an invalid
 * shape).  The array holds, in this order and each row-major:
 *   token embedding E_tok [V][C], position embedding E_pos [T][C],
 *   per block: norm1 gain [C], norm1 bias [C], attention-in W_in [C][3C],
 *              attention-out W_out [C][C], norm2 gain [C], norm2 bias [C],
 *              MLP up W_up [C][4C], up bias [4C], MLP down W_down [4C][C],
 *              down bias [C],
 *   final norm gain [C], final norm bias [C], unembedding W_vocab [C][V].
 * W_in's columns are q, then k, then v; within each third, head h owns the
 * columns [h D, (h+1) D). */
size_t spec_model_param_count(const spec_model_t* model);

size_t spec_verify_forward_workspace_size(const spec_model_t* model, int B, int n, int max_len_hint);

/* Logits of the n new tokens of each of B sequences, appending their K/V to
 * every layer's cache: the cached forward of [P2] section
 * numpyで小さなTransformerを自作する (for the verify call, the n = gamma+1
 * tokens [last committed token] + drafts, [P2] section 投機的デコーディングとは).
 * For sequence b with p0 = cache_len[b]:
 *   x_i = E_tok[tokens[b][i]] + E_pos[p0 + i]
 *   per block: h = norm1(x); q, k, v = h W_in (split in thirds, then by
 *     head); the K/V rows go to positions [p0, p0+n) of the layer's cache;
 *     new row i attends to positions [0, p0+i] with scores scaled by
 *     1/sqrt(D); x += (heads concatenated) W_out;
 *     x += gelu(norm2(x) W_up + up bias) W_down + down bias
 *   logits = final_norm(x) W_vocab
 * LayerNorm: (x - mean) / sqrt(var + 1e-5) * g + b over C (population
 * variance); gelu(v) = v/2 (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))).  All
 * arithmetic is fp32 (the attention as spec_verify_attention with SPEC_F32).
 *
 *   model      host, the model's shape; the head dimension C/H must be one
 *              spec_verify_attention supports for SPEC_F32 (24, 32, 64, 128)
 *   params     device, spec_model_param_count(model) floats (layout above)
 *   tokens     device, [B][n] int32; a token outside [0, V) gives NaN logits
 *              for its sequence's affected rows
 *   cache_len  device, [B] int32, p0 of each sequence; not modified (commit
 *              the accepted length with spec_kv_truncate)
 *   kv_cache   device, [L][2][B][H][max_T][D] float (layer, K then V,
 *              sequence, head, position, dim); rows [p0, p0+n) of every
 *              layer are written, rows below p0 are read, others untouched
 *   logits     device out, [B][n][V] float
 *   n          new tokens per sequence, 1..16
 *   max_len_hint  host upper bound on max_b cache_len[b]
 *   workspace  device, >= spec_verify_forward_workspace_size(...) bytes,
 *              256-byte aligned
 * Errors: SPEC_ERR_ARG for an invalid shape, null pointers, non-positive
 * sizes, a small or unaligned workspace; SPEC_ERR_OVERFLOW when
 * max_len_hint + n exceeds max_T or T; SPEC_ERR_UNSUPPORTED for a head
 * dimension the attention does not support, n > 16, or a width C above 144
 * or not a multiple of 16. */
spec_status_t spec_verify_forward(const spec_model_t* model, const float* params, const int32_t* tokens,
                                  const int32_t* cache_len, float* kv_cache, int max_T, float* logits, int B, int n,
                                  int max_len_hint, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* One speculative round: draft proposals, verify, draw, commit               */
/* ------------------------------------------------------------------------- */

size_t spec_speculative_round_workspace_size(const spec_model_t* target, const spec_model_t* draft, int B,
                                             int gamma, int max_len_hint);

/* One round of speculative decoding for B sequences, all on `stream`
 * ([P2] section 投機的デコーディングとは: the round's listing and flowchart):
 *   1. the draft proposes gamma tokens: its first call runs over the last two
 *      committed tokens (positions L-2, L-1), then one call per proposal;
 *      proposal j is the inverse-CDF draw of softmax(z_j / T) at
 *      u_draft[b][j] (the smallest index whose prefix of the weights exceeds
 *      u times their sum), or argmax z_j at T = 0;
 *   2. the target runs once over [last committed token] + the proposals
 *      (spec_verify_forward, n = gamma + 1);
 *   3. spec_reject_sample decides n_accepted and the emitted tokens from the
 *      target's and the draft's logits and u_verify (greedy at T = 0);
 *   4. the n + 1 emitted tokens are appended to seq[b]; seq_len, target_len
 *      and draft_len each grow by n + 1 (the pages' truncate of both caches).
 * State on entry, for each sequence with L = seq_len[b] committed tokens:
 * target_len[b] = L - 1 (the target cache holds seq[b][0 .. L-2]) and
 * draft_len[b] = L - 2 (the draft cache holds at least seq[b][0 .. L-3]);
 * every call leaves this so.  Start a sequence by prefilling both caches
 * (spec_verify_forward over the prompt, 16 tokens per call).
 *
 *   target, draft   host, model shapes with the same V; params as for
 *                   spec_verify_forward
 *   seq             device, [B][max_len] int32 committed tokens, in/out
 *   seq_len         device, [B] int32 L >= 2, in/out
 *   target_kv, draft_kv  device, [L][2][B][H][max_T][D] caches of each model
 *   target_len, draft_len  device, [B] int32, in/out (see above)
 *   u_draft         device, [B][gamma] double in [0, 1) (NULL at T = 0)
 *   u_verify        device, [B][gamma+1] double in [0, 1), as for
 *                   spec_reject_sample (NULL at T = 0)
 *   max_len_hint    host upper bound on max_b seq_len[b] (>= 2)
 *   n_accepted      device out, [B]: as spec_reject_sample's; -1 also when a
 *                   sequence's tokens would not fit in max_len (nothing is
 *                   committed for it)
 *   out_tokens      device out, [B][gamma+1]: the emitted tokens, then -1
 *   workspace       device, >= spec_speculative_round_workspace_size(...)
 *                   bytes, 256-byte aligned
 * Errors: SPEC_ERR_ARG for null pointers, different vocabularies, a bad
 * shape, T < 0, max_len_hint < 2 or a small workspace; SPEC_ERR_OVERFLOW when
 * max_len_hint + gamma + 1 exceeds max_len, max_len_hint + gamma exceeds the
 * target's max_T or T, or max_len_hint + gamma - 1 the draft's;
 * SPEC_ERR_UNSUPPORTED for gamma > 15 or what spec_verify_forward or
 * spec_reject_sample does not support. */
spec_status_t spec_speculative_round(const spec_model_t* target, const float* target_params,
                                     const spec_model_t* draft, const float* draft_params, int32_t* seq,
                                     int32_t* seq_len, int max_len, float* target_kv, int32_t* target_len,
                                     int target_max_T, float* draft_kv, int32_t* draft_len, int draft_max_T,
                                     const double* u_draft, const double* u_verify, int B, int gamma,
                                     float temperature, int max_len_hint, int32_t* n_accepted, int32_t* out_tokens,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
