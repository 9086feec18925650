// The verify forward of a GPT-2-type decoder (gfx950, fp32).
//
// [P2] "LLM推論の高速化｜KVキャッシュと投機的デコーディングを自作で実測" section
// numpyで小さなTransformerを自作する: the cached forward takes the n new tokens
// of a sequence, adds token and position embeddings (positions p0 .. p0+n-1,
// p0 = the cache length) and runs pre-LayerNorm blocks -- fused q/k/v
// projection, the K/V append and causal attention over the cache, the output
// projection and residual, a second LayerNorm and a GELU MLP with residual --
// then a final LayerNorm and the vocabulary projection.  The same section's
// parameter counts (513,600 for the 4-layer width-96 model, 61,968 for the
// 1-layer width-48 draft) fix MLP width 4C, biases on the MLP only.  The
// listing leaves LayerNorm and GELU undefined: GPT-2's readings are taken
// (population variance, eps 1e-5; GELU in its tanh form).
//
// Launches, for the M = B*n new rows, 16 rows per workgroup with every
// intermediate of a row block in LDS:
//   embed_qkv              x = tok_emb[token] + pos_emb[position]; then layer 0's
//                          q | k_new | v_new = LN1(x) w_in, written head-major
//                          ([B][H][n][D]) for the attention
// and per layer:
//   spec_verify_attention  appends k_new, v_new at [p0, p0+n) of the layer's
//                          cache and attends (the library's fp32 kernels)
//   block_mlp              x += O w_out (reading O [B][H][n][D] as [M][C]);
//                          x += gelu(LN2(x) w_up + b_up) w_down + b_down; then the next
//                          layer's q | k_new | v_new, or after the last layer
//                          logits = LNf(x) w_vocab (a launch of its own, gemm,
//                          above kFusedVocabMax tokens)
// The products are fp32 matrix-core tiles (v_mfma_f32_16x16x4_f32: exact
// fp32 products, fp32 sums); the LayerNorms, biases, GELU, residual adds and
// the head-major q/k/v scatter are fused around them.
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "model_internal.h"
#include "spec_common.h"
#include "spec_verify.h"

namespace specv {

constexpr float kLnEps = 1e-5f;

// Offsets (in floats) of the parameters in the packed array, in the order
// tok_emb, pos_emb, per layer (n1_gain, n1_bias, w_in, w_out, n2_gain, n2_bias, w_up, b_up, w_down, b_down),
// nf_gain, nf_bias, w_vocab.
struct ModelLayout {
  int V, C, L, H, T, F, D;
  size_t tok_emb, pos_emb, nf_gain, nf_bias, w_vocab, total;
  size_t layer0, layer_stride;  // first layer's n1_gain; floats per layer
  // offsets inside a layer
  size_t n1_gain, n1_bias, w_in, w_out, n2_gain, n2_bias, w_up, b_up, w_down, b_down;
};

static bool model_layout(const spec_model_t* m, ModelLayout* o) {
  if (!m || m->V < 1 || m->C < 1 || m->L < 1 || m->H < 1 || m->T < 1 || m->C % m->H != 0) return false;
  ModelLayout l{};
  l.V = m->V;
  l.C = m->C;
  l.L = m->L;
  l.H = m->H;
  l.T = m->T;
  l.F = 4 * m->C;
  l.D = m->C / m->H;
  const size_t C = l.C, F = l.F, V = l.V, T = l.T;
  size_t off = 0;
  l.tok_emb = off;
  off += V * C;
  l.pos_emb = off;
  off += T * C;
  l.layer0 = off;
  size_t in = 0;
  l.n1_gain = in;
  in += C;
  l.n1_bias = in;
  in += C;
  l.w_in = in;
  in += 3 * C * C;
  l.w_out = in;
  in += C * C;
  l.n2_gain = in;
  in += C;
  l.n2_bias = in;
  in += C;
  l.w_up = in;
  in += C * F;
  l.b_up = in;
  in += F;
  l.w_down = in;
  in += F * C;
  l.b_down = in;
  in += C;
  l.layer_stride = in;
  off += in * (size_t)l.L;
  l.nf_gain = off;
  off += C;
  l.nf_bias = off;
  off += C;
  l.w_vocab = off;
  off += C * V;
  l.total = off;
  *o = l;
  return true;
}

// x[b n + i][:] = tok_emb[tok[b][i]][:] + pos_emb[lens[b] + i][:]; an out-of-range
// token or position writes NaN rows (which then reach the logits).
constexpr int kBM = 32, kBN = 32;    // output tile: 4 waves, 16 x 16 each
constexpr int kFusedVocabMax = 1024;  // vocabularies projected inside the last layer's launch
constexpr int kPad = 4;              // floats of padding per staged A row (LDS banks)
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct GemmArgs {
  const float* A;      // [M][K]
  const float* W;      // [K][N]
  const float* n_gain;   // LN gain / bias over K
  const float* n_bias;
  float* out;          // [M][N]
  int M, N, K;
};

__device__ __forceinline__ float gelu_tanh(float v) {
  const float u = 0.7978845608028654f * (v + 0.044715f * v * v * v);  // sqrt(2/pi) (v + 0.044715 v^3)
  return 0.5f * v * (1.f + tanhf(u));
}

// One 16 x 16 tile on v_mfma_f32_16x16x4_f32: the 16 rows of A (in LDS, row
// stride KP floats) times columns col of W ([K][N], row-major, through the
// buffer resource wrs).  The instruction takes A[l % 16][l / 16] and
// B[l / 16][l % 16] from lane l and leaves C[4 (l / 16) + i][l % 16] in its
// i-th result; here lane group l / 16 walks its own contiguous quarter of K
// (K a multiple of 16), so its A values are 16-byte LDS reads and its W
// values coalesce across the 16 columns.  W comes through buffer loads from a
// scalar base, issued without branches four steps ahead (a column past N or a
// step past the last reads a valid element whose product is discarded), so
// the compiler waits for the oldest only.
constexpr int kWRing = 4;  // steps of W loads in flight per lane group

__device__ __forceinline__ __amdgpu_buffer_rsrc_t w_rsrc(const float* W, int K, int N) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(W), 0, (int)((long)K * N * sizeof(float)), 0x00020000);
}

__device__ __forceinline__ f32x4 mfma_tile16(const float* A, int KP, int K, __amdgpu_buffer_rsrc_t wrs, int N, int col,
                                             bool col_ok, int lr, int lgp) {
  const int K4 = K / 4;
  const float* Ar = A + lr * KP + lgp * K4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  constexpr int kRing = kWRing;
  const int NIT = K4 / 4;
  const uint32_t cbase = (uint32_t)(lgp * K4) * (uint32_t)N + (uint32_t)(col_ok ? col : 0);
  float w[kRing][4];
  auto load_it = [&](int it, float (&r)[4]) {
    const int it_c = min(it, NIT - 1);
#pragma unroll
    for (int t = 0; t < 4; ++t)
      r[t] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(wrs, (cbase + (uint32_t)(4 * it_c + t) * (uint32_t)N) * 4u, 0, 0));
  };
#pragma unroll
  for (int q = 0; q < kRing; ++q) load_it(q, w[q]);
  for (int it0 = 0; it0 < NIT; it0 += kRing) {
#pragma unroll
    for (int q = 0; q < kRing; ++q) {
      const int it = it0 + q;
      if (it < NIT) {  // uniform
        const float4 a4 = *reinterpret_cast<const float4*>(Ar + 4 * it);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.x, w[q][0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.y, w[q][1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.z, w[q][2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.w, w[q][3], acc, 0, 0, 0);
      }
      load_it(it + kRing, w[q]);
    }
  }
  return acc;
}

// Output tile [m0, m0+32) x [n0, n0+32) (exact fp32 products, fp32
// accumulation).  The 32 A rows are staged in LDS whole (K floats each, rows
// padded by kPad floats), and LayerNorm-ed in place.  Wave w owns the
// 16 x 16 sub-tile (rows 16 (w / 2), columns 16 (w % 2)), computed by
// mfma_tile16; W is read from L2 (it is small and shared by every row tile).
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  extern __shared__ float As[];  // [kBM][K + kPad]
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int m0 = blockIdx.y * kBM, n0 = blockIdx.x * kBN;
  const int K = g.K, KP = K + kPad;

  // stage the A rows
  for (int e = threadIdx.x; e < kBM * K; e += blockDim.x) {
    const int r = e / K, k = e - r * K;
    const int m = m0 + r;
    As[r * KP + k] = m < g.M ? g.A[(size_t)m * K + k] : 0.f;
  }
  __syncthreads();
  // each wave normalises 8 rows: mean, then the variance about it
  for (int r = wave * 8; r < wave * 8 + 8; ++r) {
    float s = 0.f;
    for (int k = lane; k < K; k += kWave) s += As[r * KP + k];
    const float mu = wave_sum(s) / (float)K;
    float v = 0.f;
    for (int k = lane; k < K; k += kWave) {
      const float d = As[r * KP + k] - mu;
      v += d * d;
    }
    const float rstd = 1.f / sqrtf(wave_sum(v) / (float)K + kLnEps);
    for (int k = lane; k < K; k += kWave) As[r * KP + k] = (As[r * KP + k] - mu) * rstd * g.n_gain[k] + g.n_bias[k];
  }
  __syncthreads();

  const int lr = lane & 15, lgp = lane >> 4;
  const int wr = wave >> 1, wc = wave & 1;
  const int col = n0 + 16 * wc + lr;
  const bool col_ok = col < g.N;
  const f32x4 acc = mfma_tile16(As + 16 * wr * KP, KP, K, w_rsrc(g.W, K, g.N), g.N, col, col_ok, lr, lgp);
  if (!col_ok) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + 16 * wr + 4 * lgp + i;
    if (m >= g.M) break;
    g.out[(size_t)m * g.N + col] = acc[i];
  }
}

static hipError_t gemm(const GemmArgs& g, hipStream_t s) {
  const dim3 grid((unsigned)((g.N + kBN - 1) / kBN), (unsigned)((g.M + kBM - 1) / kBM));
  hipLaunchKernelGGL(gemm_kernel, grid, dim3(256),
                     sizeof(float) * kBM * (g.K + kPad), s, g);
  return hipGetLastError();
}

// Ordered key of a logit for the argmax: a larger value gives a larger key,
// -0 equals +0, a NaN is above every number.
__device__ __forceinline__ uint32_t logit_key(float v) {
  if (v != v) return 0xffffffffu;
  const uint32_t u = (v == 0.f) ? 0u : __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One wave, for sequence b whose last logit row is z: copies the row into
// draft_logits[b][j] and draws proposal j: at T > 0 the smallest index whose
// fp64 prefix of w = 2^((z - max) c) exceeds u * sum(w) (the last positive
// weight if rounding leaves none); at T = 0 the first index of the largest
// logit.
__device__ __forceinline__ void draw_row(const DrawSpec& dr, const float* z, int V, int b, int lane) {
  const int gamma = dr.gamma, j = dr.j;
  const float c32 = dr.c32;
  const int greedy = dr.greedy;
  int32_t* xs = dr.xs;
  const double* u_draft = dr.u;
  float* zd = dr.draft_logits + ((size_t)b * gamma + j) * V;
  float m = neg_inf_f();
  uint64_t best = 0;
  for (int k = lane; k < V; k += kWave) {
    const float v = z[k];
    zd[k] = v;
    m = fmaxf(m, v);
    const uint64_t w = ((uint64_t)logit_key(v) << 32) | (uint32_t)~(uint32_t)k;
    best = w > best ? w : best;
  }
  if (greedy) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const uint32_t lo = __shfl_xor((uint32_t)best, o, kWave), hi = __shfl_xor((uint32_t)(best >> 32), o, kWave);
      const uint64_t w = ((uint64_t)hi << 32) | lo;
      best = w > best ? w : best;
    }
    if (lane == 0) xs[(size_t)b * gamma + j] = (int32_t)~(uint32_t)best;
    return;
  }
  m = wave_max(m);
  double s = 0.0;
  for (int k = lane; k < V; k += kWave) s += (double)exp2_fast((z[k] - m) * c32);
  const double target = u_draft[(size_t)b * gamma + j] * wave_sum(s);
  double carry = 0.0;
  int t = -1, last = -1;
  for (int c0 = 0; c0 < V && t < 0; c0 += kWave) {
    const int k = c0 + lane;
    const float w = k < V ? exp2_fast((z[k] - m) * c32) : 0.f;
    const double incl = carry + wave_inclusive_scan((double)w, lane);
    const uint64_t hit = __ballot(k < V && incl > target);
    const uint64_t pos = __ballot(k < V && w > 0.f);
    if (pos) last = c0 + 63 - __builtin_clzll(pos);
    if (hit) t = c0 + __ffsll((long long)hit) - 1;
    carry = __shfl(incl, kWave - 1, kWave);
  }
  if (t < 0) t = last < 0 ? 0 : last;
  if (lane == 0) xs[(size_t)b * gamma + j] = t;
}

// Waves of a 16-row block workgroup; each product's 16-column tiles are dealt
// round-robin over them (16: 0.16 -> 0.14 ms per forward of the 4-layer
// width-96 model against 8, and 4 were slower still).
constexpr int kRowWaves = 16;
static_assert(16 % kRowWaves == 0 || kRowWaves % 16 == 0, "rows per wave");

// The product that follows a block of 16 rows held in LDS, by kRowWaves waves:
// LayerNorm of the rows (n_gain, n_bias) into Hs, then
//   NEXT_QKV:    q | k_new | v_new = Hs w_in (the next layer's), written
//                head-major ([B][H][n][D]) for its attention;
//   NEXT_LOGITS: logits = Hs w_vocab ([M][V]);
//   NEXT_NONE:   nothing (the vocabulary projection runs as its own launch).
enum { NEXT_NONE = 0, NEXT_QKV = 1, NEXT_LOGITS = 2 };
struct NextArgs {
  int mode;
  const float *n_gain, *n_bias, *W;  // W: [C][N]
  float *q, *kn, *vn;            // NEXT_QKV
  float* logits;                 // NEXT_LOGITS
  int N;                         // 3C or V
  int draw;                      // NEXT_LOGITS: then draw from each sequence's last row (dr)
  DrawSpec dr;
};

// LayerNorm of 16 rows (Rs -> Hs, row stride CP), a row per wave at a time:
// the mean, then the variance about it.
__device__ __forceinline__ void rows_ln16(const float* Rs, float* Hs, int CP, int C, const float* __restrict__ n_gain,
                                          const float* __restrict__ n_bias, int wave, int lane) {
  for (int r = wave; r < 16; r += kRowWaves) {
    float s = 0.f;
    for (int k = lane; k < C; k += kWave) s += Rs[r * CP + k];
    const float mu = wave_sum(s) / (float)C;
    float v = 0.f;
    for (int k = lane; k < C; k += kWave) {
      const float d = Rs[r * CP + k] - mu;
      v += d * d;
    }
    const float rstd = 1.f / sqrtf(wave_sum(v) / (float)C + kLnEps);
    for (int k = lane; k < C; k += kWave) Hs[r * CP + k] = (Rs[r * CP + k] - mu) * rstd * n_gain[k] + n_bias[k];
  }
}

// Rows [m0, m0 + 16) of Rs through the LayerNorm and product of nx.  Every
// thread of the 8-wave workgroup calls it; it starts with a barrier.
__device__ __forceinline__ void next_product(const NextArgs& nx, const float* Rs, float* Hs, int CP, int C, int m0,
                                             int M, int n, int H, int D, int wave, int lane) {
  if (nx.mode == NEXT_NONE) return;  // uniform
  __syncthreads();
  rows_ln16(Rs, Hs, CP, C, nx.n_gain, nx.n_bias, wave, lane);
  __syncthreads();
  const int lr = lane & 15, lgp = lane >> 4;
  const __amdgpu_buffer_rsrc_t wr = w_rsrc(nx.W, C, nx.N);
  for (int ct = wave; ct < (nx.N + 15) / 16; ct += kRowWaves) {
    const int col = 16 * ct + lr;
    const bool ok = col < nx.N;
    const f32x4 acc = mfma_tile16(Hs, CP, C, wr, nx.N, col, ok, lr, lgp);
    if (!ok) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + 4 * lgp + i;
      if (m >= M) break;
      if (nx.mode == NEXT_LOGITS) {
        nx.logits[(size_t)m * nx.N + col] = acc[i];
      } else {
        const int part = col / C, c = col - part * C, h = c / D, d = c - h * D;
        const int b = m / n, i2 = m - b * n;
        float* dst = part == 0 ? nx.q : (part == 1 ? nx.kn : nx.vn);
        dst[(((size_t)b * H + h) * n + i2) * D + d] = acc[i];
      }
    }
  }
  if (nx.mode == NEXT_LOGITS && nx.draw) {  // uniform
    __syncthreads();  // the block's logit rows are written (same CU)
    for (int r = wave; r < 16; r += kRowWaves) {
      const int m = m0 + r;
      if (m < M && m % n == n - 1) draw_row(nx.dr, nx.logits + (size_t)m * nx.N, nx.N, m / n, lane);
    }
  }
}

// The draws when the vocabulary projection is a launch of its own: one wave
// per sequence, from its last row of n.
__global__ __launch_bounds__(64) void draw_rows_kernel(DrawSpec dr, const float* __restrict__ logits, int n, int V) {
  const int b = blockIdx.x;
  draw_row(dr, logits + ((size_t)b * n + n - 1) * V, V, b, threadIdx.x);
}

// Token and position embeddings of 16 rows per workgroup of kRowWaves waves (NaN
// rows for a token or position out of range), then the first layer's
// LayerNorm and q/k/v product (next_product).  The tokens and positions come
// from src (TokenSource).
struct EmbArgs {
  const float *tok_emb, *pos_emb;
  TokenSource src;
  float* x;  // [M][C]
  NextArgs nx;
  int M, n, H, D, C, V, T;
};

// Token and position of row (b, i) of a call of n rows per sequence; a
// draft step's i = 0 row also stores the step's cache length of b.
__device__ __forceinline__ void row_input(const TokenSource& s, int b, int i, int n, int& tok, long& pos) {
  if (s.mode == SRC_ARRAYS) {
    tok = s.tokens[(size_t)b * n + i];
    pos = (long)s.cache_len[b] + i;
    return;
  }
  const int L = s.seq_len[b];
  const int32_t* sb = s.seq + (size_t)b * s.max_len;
  if (s.mode == SRC_DRAFT_STEP) {
    const int base = s.j == 0 ? s.base_len[b] : s.base_len[b] + s.j + 1;
    if (s.j == 0)
      tok = (L >= 2 && L <= s.max_len) ? sb[L - 2 + i] : -1;
    else
      tok = s.xs[(size_t)b * s.gamma + s.j - 1];
    if (i == 0) s.pos_out[b] = base;
    pos = (long)base + i;
  } else {  // SRC_VERIFY
    tok = i == 0 ? ((L >= 1 && L <= s.max_len) ? sb[L - 1] : -1) : s.xs[(size_t)b * s.gamma + i - 1];
    pos = (long)s.cache_len[b] + i;
  }
}

__global__ __launch_bounds__(64 * kRowWaves) void embed_qkv_kernel(EmbArgs g) {
  extern __shared__ float sm[];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int C = g.C, CP = C + kPad;
  float* Rs = sm;            // [16][CP]
  float* Hs = Rs + 16 * CP;  // [16][CP]
  __shared__ int s_tok[16];
  __shared__ long s_pos[16];
  const int m0 = blockIdx.x * 16;
  if (threadIdx.x < 16 && m0 + (int)threadIdx.x < g.M) {
    const int m = m0 + threadIdx.x, b = m / g.n;
    row_input(g.src, b, m - b * g.n, g.n, s_tok[threadIdx.x], s_pos[threadIdx.x]);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 16 * C; e += blockDim.x) {
    const int r = e / C, k = e - r * C, m = m0 + r;
    float v = 0.f;
    if (m < g.M) {
      const int t = s_tok[r];
      const long pos = s_pos[r];
      const bool ok = t >= 0 && t < g.V && pos >= 0 && pos < g.T;
      v = ok ? g.tok_emb[(size_t)t * C + k] + g.pos_emb[(size_t)pos * C + k] : __builtin_nanf("");
      g.x[(size_t)m * C + k] = v;
    }
    Rs[r * CP + k] = v;
  }
  next_product(g.nx, Rs, Hs, CP, C, m0, g.M, g.n, g.H, g.D, wave, lane);
}

// The half of a layer after its attention, for 16 rows per workgroup of
// kRowWaves waves, with every intermediate in LDS:
//   y = O w_out (O read head-major as [M][C]); X = x + y
//   u = gelu(LN2(X) w_up + b_up)
//   x = X + u w_down + b_down
// then the next layer's LayerNorm and q/k/v product, or the final LayerNorm
// and the vocabulary projection (next_product).  Waves take 16-column tiles
// of each product in turn (mfma_tile16).
struct MlpArgs {
  const float* O;  // [B][H][n][D]
  float* x;        // [M][C], updated in place
  const float *w_out, *n_gain, *n_bias, *w_up, *b_up, *w_down, *b_down;
  NextArgs nx;
  int M, n, H, D, C, F;
};

__global__ __launch_bounds__(64 * kRowWaves) void block_mlp_kernel(MlpArgs g) {
  extern __shared__ float sm[];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int lr = lane & 15, lgp = lane >> 4;
  const int C = g.C, F = g.F, CP = C + kPad, FP = F + kPad;
  float* Os = sm;            // [16][CP]
  float* Xs = Os + 16 * CP;  // [16][CP]
  float* Hs = Xs + 16 * CP;  // [16][CP]
  float* Us = Hs + 16 * CP;  // [16][FP]
  const int m0 = blockIdx.x * 16;

  for (int e = threadIdx.x; e < 16 * C; e += blockDim.x) {
    const int r = e / C, k = e - r * C, m = m0 + r;
    float a = 0.f;
    if (m < g.M) {
      const int b = m / g.n, i = m - b * g.n, h = k / g.D, d = k - h * g.D;
      a = g.O[(((size_t)b * g.H + h) * g.n + i) * g.D + d];
    }
    Os[r * CP + k] = a;
  }
  __syncthreads();
  {  // X = x + O w_out
    const __amdgpu_buffer_rsrc_t wr = w_rsrc(g.w_out, C, C);
    for (int ct = wave; ct < C / 16; ct += kRowWaves) {
      const int col = 16 * ct + lr;
      const f32x4 acc = mfma_tile16(Os, CP, C, wr, C, col, true, lr, lgp);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * lgp + i, m = m0 + r;
        Xs[r * CP + col] = (m < g.M ? g.x[(size_t)m * C + col] : 0.f) + acc[i];
      }
    }
  }
  __syncthreads();
  rows_ln16(Xs, Hs, CP, C, g.n_gain, g.n_bias, wave, lane);  // LN2
  __syncthreads();
  {  // u = gelu(H w_up + b_up)
    const __amdgpu_buffer_rsrc_t wr = w_rsrc(g.w_up, C, F);
    for (int ct = wave; ct < F / 16; ct += kRowWaves) {
      const int col = 16 * ct + lr;
      const f32x4 acc = mfma_tile16(Hs, CP, C, wr, F, col, true, lr, lgp);
#pragma unroll
      for (int i = 0; i < 4; ++i) Us[(4 * lgp + i) * FP + col] = gelu_tanh(acc[i] + g.b_up[col]);
    }
  }
  __syncthreads();
  {  // x = X + u w_down + b_down, also kept in Os (free since the first product)
    const __amdgpu_buffer_rsrc_t wr = w_rsrc(g.w_down, F, C);
    for (int ct = wave; ct < C / 16; ct += kRowWaves) {
      const int col = 16 * ct + lr;
      const f32x4 acc = mfma_tile16(Us, FP, F, wr, C, col, true, lr, lgp);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * lgp + i, m = m0 + r;
        const float xv = Xs[r * CP + col] + acc[i] + g.b_down[col];
        Os[r * CP + col] = xv;
        if (m < g.M) g.x[(size_t)m * C + col] = xv;
      }
    }
  }
  next_product(g.nx, Os, Hs, CP, C, m0, g.M, g.n, g.H, g.D, wave, lane);
}

static size_t mlp_lds_bytes(const ModelLayout& l) {
  return sizeof(float) * 16 * (3 * (size_t)(l.C + kPad) + l.F + kPad);
}

struct FwdPlan {
  size_t off_x, off_q, off_k, off_v, off_o, off_attn, attn_bytes, total;
};

static inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

static bool fwd_plan(const ModelLayout& l, int B, int n, int hint, FwdPlan* p) {
  const size_t M = (size_t)B * n;
  const size_t ab = spec_verify_attention_workspace_size(B, l.H, l.H, n, l.D, hint, SPEC_F32);
  if (ab == 0) return false;
  FwdPlan f{};
  size_t off = 0;
  f.off_x = off;
  off = align256(off + sizeof(float) * M * l.C);
  f.off_q = off;
  off = align256(off + sizeof(float) * M * l.C);
  f.off_k = off;
  off = align256(off + sizeof(float) * M * l.C);
  f.off_v = off;
  off = align256(off + sizeof(float) * M * l.C);
  f.off_o = off;
  off = align256(off + sizeof(float) * M * l.C);
  f.off_attn = off;
  f.attn_bytes = ab;
  off = align256(off + ab);
  f.total = off;
  *p = f;
  return true;
}

}  // namespace specv

using namespace specv;

extern "C" size_t spec_model_param_count(const spec_model_t* model) {
  ModelLayout l;
  return model_layout(model, &l) ? l.total : 0;
}

extern "C" size_t spec_verify_forward_workspace_size(const spec_model_t* model, int B, int n, int max_len_hint) {
  ModelLayout l;
  FwdPlan p;
  if (!model_layout(model, &l) || B < 1 || n < 1 || max_len_hint < 0) return 0;
  if (!fwd_plan(l, B, n, max_len_hint, &p)) return 0;
  return p.total;
}

namespace specv {

spec_status_t verify_forward(const spec_model_t* model, const float* params, const TokenSource& src,
                             float* kv_cache, int max_T, float* logits, int B, int n, int max_len_hint,
                             void* workspace, size_t workspace_bytes, hipStream_t stream, const DrawSpec* draw) {
  ModelLayout l;
  if (!model_layout(model, &l)) return SPEC_ERR_ARG;
  if (!params || !kv_cache || !logits || !workspace) return SPEC_ERR_ARG;
  // the attention's cache lengths: the caller's, or the ones a draft step writes
  const int32_t* cache_len = src.mode == SRC_DRAFT_STEP ? src.pos_out : src.cache_len;
  if (!cache_len || (src.mode == SRC_ARRAYS && !src.tokens)) return SPEC_ERR_ARG;
  if (B < 1 || n < 1 || max_T < 1 || max_len_hint < 0) return SPEC_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return SPEC_ERR_ARG;
  if ((long)max_len_hint + n > (long)max_T || (long)max_len_hint + n > (long)l.T) return SPEC_ERR_OVERFLOW;
  // the staged rows of a product tile and of block_mlp must fit in 64 KB of
  // LDS, and each lane group's quarter of K must be a multiple of 4 (C a
  // multiple of 16); together these allow C up to 144
  if ((size_t)kBM * (l.C + kPad) * sizeof(float) > 64 * 1024 || mlp_lds_bytes(l) > 64 * 1024 || l.C % 16 != 0)
    return SPEC_ERR_UNSUPPORTED;
  FwdPlan p;
  if (!fwd_plan(l, B, n, max_len_hint, &p)) return SPEC_ERR_UNSUPPORTED;
  if (workspace_bytes < p.total) return SPEC_ERR_ARG;
  if ((long)B * n * std::max(std::max(l.C, l.F), l.V) >= 0x7fffffffL) return SPEC_ERR_UNSUPPORTED;

  char* ws = static_cast<char*>(workspace);
  float* x = reinterpret_cast<float*>(ws + p.off_x);
  float* q = reinterpret_cast<float*>(ws + p.off_q);
  float* kn = reinterpret_cast<float*>(ws + p.off_k);
  float* vn = reinterpret_cast<float*>(ws + p.off_v);
  float* o = reinterpret_cast<float*>(ws + p.off_o);
  void* aws = ws + p.off_attn;
  const int M = B * n;
  const size_t plane = (size_t)B * l.H * max_T * l.D;  // one layer's K (or V) cache

  // The vocabulary projection joins the last layer's launch up to this width;
  // a wider one is a launch of 32 x 32 tiles of its own.
  const bool fuse_logits = l.V <= kFusedVocabMax;
  auto qkv_of = [&](int layer) {
    const float* P = params + l.layer0 + (size_t)layer * l.layer_stride;
    NextArgs nx{};
    nx.mode = NEXT_QKV;
    nx.n_gain = P + l.n1_gain;
    nx.n_bias = P + l.n1_bias;
    nx.W = P + l.w_in;
    nx.q = q;
    nx.kn = kn;
    nx.vn = vn;
    nx.N = 3 * l.C;
    return nx;
  };
  const unsigned row_blocks = (unsigned)((M + 15) / 16);

  // x = tok_emb[token] + pos_emb[position]; q | k_new | v_new = LN1(x) w_in (layer 0)
  EmbArgs ea{};
  ea.tok_emb = params + l.tok_emb;
  ea.pos_emb = params + l.pos_emb;
  ea.src = src;
  ea.x = x;
  ea.nx = qkv_of(0);
  ea.M = M;
  ea.n = n;
  ea.H = l.H;
  ea.D = l.D;
  ea.C = l.C;
  ea.V = l.V;
  ea.T = l.T;
  hipLaunchKernelGGL(embed_qkv_kernel, dim3(row_blocks), dim3(64 * kRowWaves), sizeof(float) * 2 * 16 * (l.C + kPad),
                     stream, ea);
  if (hipGetLastError() != hipSuccess) return SPEC_ERR_LAUNCH;

  for (int layer = 0; layer < l.L; ++layer) {
    const float* P = params + l.layer0 + (size_t)layer * l.layer_stride;
    // append + causal attention over the layer's cache
    float* kc = kv_cache + (size_t)(2 * layer) * plane;
    float* vc = kv_cache + (size_t)(2 * layer + 1) * plane;
    const spec_status_t st = spec_verify_attention(q, kn, vn, kc, vc, cache_len, o, B, l.H, l.H, n, l.D, max_T,
                                                   max_len_hint, 1.f / sqrtf((float)l.D), SPEC_F32, aws,
                                                   p.attn_bytes, stream);
    if (st != SPEC_OK) return st;

    // x += O w_out; x += gelu(LN2(x) w_up + b_up) w_down + b_down; then the next layer's
    // q | k_new | v_new, or the logits, 16 rows per workgroup
    MlpArgs ma{};
    ma.O = o;
    ma.x = x;
    ma.w_out = P + l.w_out;
    ma.n_gain = P + l.n2_gain;
    ma.n_bias = P + l.n2_bias;
    ma.w_up = P + l.w_up;
    ma.b_up = P + l.b_up;
    ma.w_down = P + l.w_down;
    ma.b_down = P + l.b_down;
    if (layer + 1 < l.L) {
      ma.nx = qkv_of(layer + 1);
    } else if (fuse_logits) {
      ma.nx.mode = NEXT_LOGITS;
      ma.nx.n_gain = params + l.nf_gain;
      ma.nx.n_bias = params + l.nf_bias;
      ma.nx.W = params + l.w_vocab;
      ma.nx.logits = logits;
      ma.nx.N = l.V;
      if (draw) {
        ma.nx.draw = 1;
        ma.nx.dr = *draw;
      }
    } else {
      ma.nx.mode = NEXT_NONE;
    }
    ma.M = M;
    ma.n = n;
    ma.H = l.H;
    ma.D = l.D;
    ma.C = l.C;
    ma.F = l.F;
    hipLaunchKernelGGL(block_mlp_kernel, dim3(row_blocks), dim3(64 * kRowWaves), mlp_lds_bytes(l), stream, ma);
    if (hipGetLastError() != hipSuccess) return SPEC_ERR_LAUNCH;
  }

  if (!fuse_logits) {  // logits = LNf(x) w_vocab
    GemmArgs g{};
    g.M = M;
    g.A = x;
    g.K = l.C;
    g.N = l.V;
    g.W = params + l.w_vocab;
    g.n_gain = params + l.nf_gain;
    g.n_bias = params + l.nf_bias;
    g.out = logits;
    if (gemm(g, stream) != hipSuccess) return SPEC_ERR_LAUNCH;
    if (draw) {
      hipLaunchKernelGGL(draw_rows_kernel, dim3((unsigned)B), dim3(kWave), 0, stream, *draw, logits, n, l.V);
      if (hipGetLastError() != hipSuccess) return SPEC_ERR_LAUNCH;
    }
  }
  return SPEC_OK;
}

}  // namespace specv

extern "C" spec_status_t spec_verify_forward(const spec_model_t* model, const float* params, const int32_t* tokens,
                                             const int32_t* cache_len, float* kv_cache, int max_T, float* logits,
                                             int B, int n, int max_len_hint, void* workspace, size_t workspace_bytes,
                                             hipStream_t stream) {
  if (!tokens || !cache_len) return SPEC_ERR_ARG;
  TokenSource src{};
  src.mode = SRC_ARRAYS;
  src.tokens = tokens;
  src.cache_len = cache_len;
  return verify_forward(model, params, src, kv_cache, max_T, logits, B, n, max_len_hint, workspace, workspace_bytes,
                        stream);
}
