// Causal multi-query verify attention with KV append (gfx950, MFMA).
//
// [P2] "LLM推論の高速化｜KVキャッシュと投機的デコーディングを自作で実測":
//   section numpyで小さなTransformerを自作する (forward_cached: the n new
//   tokens' K/V go to cache rows [p0, p0+n), the i-th new row attends to rows
//   [0, p0+i], scores scaled by 1/sqrt(D) and soft-maxed);
//   section GQA・MQAでKVキャッシュを減らす (query heads share KV heads; decode
//   attention time is the time to read the cache).
//
// Work decomposition.  One wave (= one 64-thread workgroup) per work item
// (b, g, rg, sp): sequence b, KV head g, row group rg, key split sp.  The
// wave holds every query row of its group -- the G = Hq/Hkv heads that share
// KV head g, times the n_q verify positions, padded to 16-row MFMA tiles --
// so each K/V tile read from HBM serves all of them (the GQA reuse), and the
// wave walks its split's keys in blocks of 32 with an online softmax.  The
// partial (max, sum, unnormalised output) of each split goes to the workspace;
// attn_combine merges the splits of (b, g, rg) and writes the output.
//
// MFMA layouts (gfx950, wave64).  For v_mfma_f32_16x16x32_bf16 lane l holds
// A[l%16][8(l/16) .. 8(l/16)+7], B[8(l/16) .. +7][l%16] and returns
// C[4(l/16) + j][l%16], j = 0..3; v_mfma_f32_16x16x4_f32 holds one element,
// A[l%16][l/16], B[l/16][l%16], with the same C layout.
//   Scores are computed transposed, S^T = K Q^T (A = 16 keys x D, B = D x 16
//   rows), so each lane ends with 4 keys x 1 row: the row statistics need
//   only a reduction over the 4 lane groups, and the probabilities are
//   already where the B operand of O^T = V^T P^T wants them (keys along the
//   contraction).  The contraction over keys may take the keys in any order,
//   so the 8 keys a lane holds from two 16-key tiles, {4(l/16) + j, 16 +
//   4(l/16) + j}, form its 8 contiguous MFMA k-slots, and V^T is gathered in
//   that same key order.
//   V^T needs D along the rows and keys along the contraction, the transpose
//   of how the cache stores V; a wave stages its 32 x D V block in LDS
//   (coalesced 16-byte rows) and reads it back transposed.  For fp32 each
//   MFMA takes one key per lane, so V is read straight from memory.
//
// Keys [0, L_b) come from the cache, keys [L_b, L_b + n_q) from k_new/v_new
// directly (so the append in the same launch is never read back), and keys at
// or past L_b + n_q are zero and masked.  The cache rows past L_b are never
// read.  Row i of the verify block sees keys <= L_b + i.
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "spec_common.h"
#include "spec_verify.h"

namespace specv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int KB = 32;  // keys per block

struct ML {  // per split and row: running max (log2 units) and sum
  float m, l;
};

template <typename T>
struct Tr;

template <>
struct Tr<uint16_t> {  // bfloat16 storage
  static constexpr int KSTEP = 32;  // contraction per MFMA
  using frag = bf16x8;
  __device__ static frag zero() { return frag{}; }
  __device__ static frag load(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }
  __device__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Tr<float> {
  static constexpr int KSTEP = 4;
  using frag = float;
  __device__ static frag zero() { return 0.f; }
  __device__ static frag load(const float* p) { return *p; }
  __device__ static f32x4 mma(frag a, frag b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0); }
};

struct AttnArgs {
  const void* q;
  const void* kn;
  const void* vn;
  void* kc;
  void* vc;
  const int32_t* len;
  void* out;
  float* part_o;
  ML* part_ml;
  int B, Hq, Hkv, n_q, G, M, RG, NSP, C, max_T, hint;
  float qk_scale;  // scale * log2(e)
};

// Row pointer of key `key` of (b, g): cache row, new row, or null (masked).
template <typename T>
__device__ __forceinline__ const T* key_row(const T* cache, const T* fresh, int key, int L, int Ltot, int n_q,
                                            int max_T, int D, long bg) {
  if (key < L) return cache + ((size_t)bg * max_T + key) * D;
  if (key < Ltot) return fresh + ((size_t)bg * n_q + (key - L)) * D;
  return nullptr;
}

template <typename T, int D, int RT>
__global__ __launch_bounds__(64) void attn_split(AttnArgs a) {
  using TR = Tr<T>;
  using frag = typename TR::frag;
  constexpr bool BF = sizeof(T) == 2;
  constexpr int KSTEP = TR::KSTEP;
  constexpr int DS = D / KSTEP;          // MFMA steps over D for the scores
  constexpr int DT = (D + 15) / 16;      // 16-wide output tiles over D
  constexpr int VP = D + 8;              // LDS pitch of the staged V block (bf16)
  __shared__ uint16_t vs[BF ? KB * VP : 1];

  const int lane = threadIdx.x;
  const int lr = lane & 15;  // row (or key) within a 16-tile
  const int lg = lane >> 4;  // lane group 0..3
  long item = blockIdx.x;
  const int sp = (int)(item % a.NSP);
  item /= a.NSP;
  const int rg = (int)(item % a.RG);
  item /= a.RG;
  const int g = (int)(item % a.Hkv);
  const int b = (int)(item / a.Hkv);
  const long bg = (long)b * a.Hkv + g;

  const int L = a.len[b];
  if (L < 0 || L > a.hint) return;  // flagged by attn_combine
  const int Ltot = L + a.n_q;
  const int k0 = sp * a.C;
  if (k0 >= Ltot) return;
  const int k1 = min(k0 + a.C, Ltot);

  const T* q = static_cast<const T*>(a.q);
  const T* kn = static_cast<const T*>(a.kn);
  const T* vn = static_cast<const T*>(a.vn);
  const T* kc = static_cast<const T*>(a.kc);
  const T* vc = static_cast<const T*>(a.vc);

  // A1: append the n_q new rows (done once per (b, g); no wave reads them
  // from the cache in this launch).
  if (sp == 0 && rg == 0) {
    constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
    const int chunks = a.n_q * D / EPC;
    const uint4* skn = reinterpret_cast<const uint4*>(kn + (size_t)bg * a.n_q * D);
    const uint4* svn = reinterpret_cast<const uint4*>(vn + (size_t)bg * a.n_q * D);
    uint4* dkc = reinterpret_cast<uint4*>(static_cast<T*>(a.kc) + ((size_t)bg * a.max_T + L) * D);
    uint4* dvc = reinterpret_cast<uint4*>(static_cast<T*>(a.vc) + ((size_t)bg * a.max_T + L) * D);
    for (int c = lane; c < chunks; c += kWave) {
      dkc[c] = skn[c];
      dvc[c] = svn[c];
    }
  }

  // Query fragments (B operand of S^T = K Q^T) and each row's causal limit.
  frag qf[RT][DS];
  int lim[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int m = rg * 16 * RT + 16 * r + lr;
    const bool valid = m < a.M;
    const int h = g * a.G + (valid ? m / a.n_q : 0);
    const int i = valid ? m % a.n_q : a.n_q - 1;
    lim[r] = L + i;
    const T* qrow = q + (((size_t)b * a.Hq + h) * a.n_q + i) * D;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      const int d = BF ? s * KSTEP + 8 * lg : s * KSTEP + lg;
      qf[r][s] = valid ? TR::load(qrow + d) : TR::zero();
    }
  }

  float mrow[RT], lsum[RT];
  f32x4 oacc[RT][DT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    mrow[r] = neg_inf_f();
    lsum[r] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[r][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // K fragments of a block: kf[kt][s] = K[kb + 16 kt + lr][s*KSTEP + (8 lg | lg) ...]
  auto load_k = [&](int kb, frag (&kf)[2][DS]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const T* row = key_row<T>(kc, kn, kb + 16 * kt + lr, L, Ltot, a.n_q, a.max_T, D, bg);
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        const int d = BF ? s * KSTEP + 8 * lg : s * KSTEP + lg;
        kf[kt][s] = row ? TR::load(row + d) : TR::zero();
      }
    }
  };

  frag kcur[2][DS], knext[2][DS];
  load_k(k0, kcur);

  for (int kb = k0; kb < k1; kb += KB) {
    const bool has_next = kb + KB < k1;
    if (has_next) load_k(kb + KB, knext);

    // V of this block: bf16 rows into registers now, to LDS after the scores.
    constexpr int VCH = BF ? (KB * D / 8) / kWave : 1;  // 16-byte chunks per lane
    uint4 vreg[BF ? VCH : 1];
    if constexpr (BF) {
#pragma unroll
      for (int c = 0; c < VCH; ++c) {
        const int ch = lane + c * kWave;
        const int krow = ch / (D / 8), kcol = ch % (D / 8);
        const T* row = key_row<T>(vc, vn, kb + krow, L, Ltot, a.n_q, a.max_T, D, bg);
        vreg[c] = row ? *reinterpret_cast<const uint4*>(row + 8 * kcol) : make_uint4(0, 0, 0, 0);
      }
    }

    // Scores S^T for 2 key tiles x RT row tiles; lane holds keys
    // kb + 16 kt + 4 lg + j of row 16 r + lr.
    f32x4 sacc[2][RT];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < DS; ++s) c = TR::mma(kcur[kt][s], qf[r][s], c);
        sacc[kt][r] = c * a.qk_scale;
      }
    if (kb + KB > L) {  // block reaches the new rows or the end: causal mask
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int key = kb + 16 * kt + 4 * lg + j;
            if (key >= Ltot || key > lim[r]) sacc[kt][r][j] = neg_inf_f();
          }
    }

    // Online softmax (log2 domain).
    float pr[2][RT][4];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      float mx = neg_inf_f();
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) mx = fmaxf(mx, sacc[kt][r][j]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const float mnew = fmaxf(mrow[r], mx);
      const bool none = (mnew == neg_inf_f());
      const float alpha = none ? 1.f : exp2_fast(mrow[r] - mnew);
      float ps = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p = none ? 0.f : exp2_fast(sacc[kt][r][j] - mnew);
          pr[kt][r][j] = p;
          ps += p;
        }
      lsum[r] = lsum[r] * alpha + ps;
      mrow[r] = mnew;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[r][dt] *= alpha;
    }

    if constexpr (BF) {
      // Stage V (32 x D) in LDS, then gather V^T fragments in the key order
      // the P fragments use.
      __syncthreads();
#pragma unroll
      for (int c = 0; c < VCH; ++c) {
        const int ch = lane + c * kWave;
        const int krow = ch / (D / 8), kcol = ch % (D / 8);
        *reinterpret_cast<uint4*>(&vs[krow * VP + 8 * kcol]) = vreg[c];
      }
      __syncthreads();
      bf16x8 pf[RT];
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int j = 0; j < 8; ++j) pf[r][j] = (__bf16)pr[j >> 2][r][j & 3];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        s16x8 vv;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int krow = (j < 4) ? (4 * lg + j) : (16 + 4 * lg + (j - 4));
          vv[j] = (short)vs[krow * VP + 16 * dt + lr];
        }
        const bf16x8 vf = __builtin_bit_cast(bf16x8, vv);
#pragma unroll
        for (int r = 0; r < RT; ++r) oacc[r][dt] = TR::mma(vf, pf[r], oacc[r][dt]);
      }
    } else {
      // fp32: one key per lane per MFMA; lane group lg supplies key
      // kb + 16 kt + 4 lg + j at step (kt, j).
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const T* row = key_row<T>(vc, vn, kb + 16 * kt + 4 * lg + j, L, Ltot, a.n_q, a.max_T, D, bg);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const int d = 16 * dt + lr;
            const float vv = (row && d < D) ? reinterpret_cast<const float*>(row)[d] : 0.f;
#pragma unroll
            for (int r = 0; r < RT; ++r) oacc[r][dt] = TR::mma(vv, pr[kt][r][j], oacc[r][dt]);
          }
        }
    }

    if (has_next) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int s = 0; s < DS; ++s) kcur[kt][s] = knext[kt][s];
    }
  }

  // Write this split's partial: O^T tile (d = 16 dt + 4 lg + j, row 16 r + lr).
  const long item_id = blockIdx.x;
  float* po = a.part_o + (size_t)item_id * (16 * RT) * D;
  ML* pml = a.part_ml + (size_t)item_id * (16 * RT);
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    float lt = lsum[r];
    lt += __shfl_xor(lt, 16, kWave);
    lt += __shfl_xor(lt, 32, kWave);
    const int row = 16 * r + lr;
    if (lg == 0) pml[row] = ML{mrow[r], lt};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = 16 * dt + 4 * lg;
      if (d < D) *reinterpret_cast<f32x4*>(po + (size_t)row * D + d) = oacc[r][dt];
    }
  }
}

// Merge the splits of (b, g, rg) and write out[b][h][i][:].
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_combine(AttnArgs a, int RT) {
  constexpr int MAXSP = 64;  // splits handled per pass of the weight table
  __shared__ float coef[16 * 5][MAXSP];
  const int rows = 16 * RT;
  long item = blockIdx.x;
  const int rg = (int)(item % a.RG);
  item /= a.RG;
  const int g = (int)(item % a.Hkv);
  const int b = (int)(item / a.Hkv);
  const int L = a.len[b];
  T* out = static_cast<T*>(a.out);
  const int tid = threadIdx.x;
  const int row0 = rg * rows;
  const int nrows = min(rows, a.M - row0);
  auto out_ptr = [&](int row) {
    const int m = row0 + row;
    const int h = g * a.G + m / a.n_q, i = m % a.n_q;
    return out + (((size_t)b * a.Hq + h) * a.n_q + i) * D;
  };
  if (L < 0 || L > a.hint) {  // invalid length: NaN rows, nothing else touched
    for (int e = tid; e < nrows * D; e += blockDim.x) {
      T* o = out_ptr(e / D);
      if constexpr (sizeof(T) == 2)
        o[e % D] = (T)0x7fc0;
      else
        o[e % D] = __builtin_nanf("");
    }
    return;
  }
  const int nsp = (L + a.n_q + a.C - 1) / a.C;
  const long base_item = ((long)b * a.Hkv + g) * a.RG + rg;  // item = base_item * NSP + sp
  // Accumulate in register per (row, d) element, NSP in passes of MAXSP.
  constexpr int EPT = (16 * 5 * D + 255) / 256;  // elements per thread (upper bound)
  float acc[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) acc[k] = 0.f;
  // Global max and denominator per row (over all splits).
  __shared__ float rowmax[16 * 5], rowden[16 * 5];
  if (tid < nrows) {
    float mx = neg_inf_f();
    for (int sp = 0; sp < nsp; ++sp) mx = fmaxf(mx, a.part_ml[(base_item * a.NSP + sp) * rows + tid].m);
    float den = 0.f;
    for (int sp = 0; sp < nsp; ++sp) {
      const ML e = a.part_ml[(base_item * a.NSP + sp) * rows + tid];
      den += e.l * exp2_fast(e.m - mx);
    }
    rowmax[tid] = mx;
    rowden[tid] = den;
  }
  for (int sp0 = 0; sp0 < nsp; sp0 += MAXSP) {
    const int cnt = min(MAXSP, nsp - sp0);
    __syncthreads();
    for (int e = tid; e < nrows * cnt; e += blockDim.x) {
      const int row = e / cnt, k = e % cnt;
      const ML ml = a.part_ml[(base_item * a.NSP + sp0 + k) * rows + row];
      coef[row][k] = exp2_fast(ml.m - rowmax[row]) / rowden[row];
    }
    __syncthreads();
    for (int k = 0; k < cnt; ++k) {
      const float* po = a.part_o + (size_t)(base_item * a.NSP + sp0 + k) * rows * D;
#pragma unroll
      for (int t = 0; t < EPT; ++t) {
        const int e = tid + t * 256;
        if (e < nrows * D) acc[t] += coef[e / D][k] * po[e];
      }
    }
  }
#pragma unroll
  for (int t = 0; t < EPT; ++t) {
    const int e = tid + t * 256;
    if (e < nrows * D) {
      T* o = out_ptr(e / D);
      if constexpr (sizeof(T) == 2)
        o[e % D] = f32_to_bf16(acc[t]);
      else
        o[e % D] = acc[t];
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

static inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct AttnPlan {
  int RT, RG, C, NSP;
  size_t off_o, off_ml, total;
};

static int max_rt(spec_dtype_t dt, int D) {
  if (dt == SPEC_BF16) return 5;
  return D <= 32 ? 4 : (D <= 64 ? 2 : 1);
}

static bool supported(spec_dtype_t dt, int D) {
  if (dt == SPEC_BF16) return D == 64 || D == 128;
  if (dt == SPEC_F32) return D == 24 || D == 32 || D == 64 || D == 128;
  return false;
}

static AttnPlan attn_plan(int B, int Hq, int Hkv, int n_q, int D, int hint, spec_dtype_t dt) {
  AttnPlan p{};
  const int M = (Hq / Hkv) * n_q;
  const int tiles = (M + 15) / 16;
  p.RG = (tiles + max_rt(dt, D) - 1) / max_rt(dt, D);
  p.RT = (tiles + p.RG - 1) / p.RG;
  // Split length: aim at ~8192 waves; a power of two in [128, 4096] keys.
  const long keys = (long)B * Hkv * p.RG * (long)(hint + n_q);
  long want = (keys + 8191) / 8192;
  int C = 128;
  while (C < want && C < 4096) C <<= 1;
  p.C = C;
  p.NSP = (hint + n_q + C - 1) / C;
  const size_t items = (size_t)B * Hkv * p.RG * p.NSP;
  size_t off = 0;
  p.off_o = off;
  off = align256(off + sizeof(float) * items * 16 * p.RT * D);
  p.off_ml = off;
  off = align256(off + sizeof(ML) * items * 16 * p.RT);
  p.total = off;
  return p;
}

template <typename T, int D, int RT>
static hipError_t attn_launch_rt(const AttnArgs& a, hipStream_t s) {
  const size_t items = (size_t)a.B * a.Hkv * a.RG * a.NSP;
  hipLaunchKernelGGL((attn_split<T, D, RT>), dim3((unsigned)items), dim3(64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_combine<T, D>), dim3((unsigned)((size_t)a.B * a.Hkv * a.RG)), dim3(256), 0, s, a, RT);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t attn_launch_d(const AttnArgs& a, int RT, hipStream_t s) {
  switch (RT) {
    case 1: return attn_launch_rt<T, D, 1>(a, s);
    case 2: return attn_launch_rt<T, D, 2>(a, s);
    case 3: if constexpr (sizeof(T) == 2 || D <= 32) return attn_launch_rt<T, D, 3>(a, s); else break;
    case 4: if constexpr (sizeof(T) == 2 || D <= 32) return attn_launch_rt<T, D, 4>(a, s); else break;
    case 5: if constexpr (sizeof(T) == 2) return attn_launch_rt<T, D, 5>(a, s); else break;
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace specv

using namespace specv;

extern "C" size_t spec_verify_attention_workspace_size(int B, int Hq, int Hkv, int n_q, int D, int max_len_hint,
                                                       spec_dtype_t dtype) {
  if (B < 1 || Hq < 1 || Hkv < 1 || n_q < 1 || n_q > 16 || D < 1 || max_len_hint < 0) return 0;
  if (Hq % Hkv != 0 || (Hq / Hkv) * n_q > 256 || !supported(dtype, D)) return 0;
  // Bound on the split count over every hint h' <= max_len_hint: the split
  // length C(h') is a power of two in [128, 4096] no smaller than
  // K (h' + n_q) / 8192, so NSP(h') <= ceil(8192 / K) unless C is capped at
  // 4096, and NSP(h') <= ceil((h' + n_q) / 128) always.  Both are monotone.
  const AttnPlan p = attn_plan(B, Hq, Hkv, n_q, D, max_len_hint, dtype);
  const long K = (long)B * Hkv * p.RG;
  const long span = (long)max_len_hint + n_q;
  long nsp = std::max((8192 + K - 1) / K, (span + 4095) / 4096);
  nsp = std::min(nsp, (span + 127) / 128);
  nsp = std::max(nsp, (long)p.NSP);
  const size_t items = (size_t)K * nsp;
  return align256(sizeof(float) * items * 16 * p.RT * D) + align256(sizeof(ML) * items * 16 * p.RT);
}

extern "C" spec_status_t spec_verify_attention(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                               void* v_cache, const int32_t* cache_len, void* out, int B, int Hq,
                                               int Hkv, int n_q, int D, int max_T, int max_len_hint, float scale,
                                               spec_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                               hipStream_t stream) {
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !cache_len || !out || !workspace) return SPEC_ERR_ARG;
  if (B < 1 || Hq < 1 || Hkv < 1 || n_q < 1 || D < 1 || max_T < 1 || max_len_hint < 0) return SPEC_ERR_ARG;
  if (Hq % Hkv != 0) return SPEC_ERR_ARG;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return SPEC_ERR_ARG;
  const uintptr_t al = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_new) |
                       reinterpret_cast<uintptr_t>(v_new) | reinterpret_cast<uintptr_t>(k_cache) |
                       reinterpret_cast<uintptr_t>(v_cache) | reinterpret_cast<uintptr_t>(out);
  if (al % 16 != 0 || reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return SPEC_ERR_ARG;
  if ((long)max_len_hint + n_q > (long)max_T) return SPEC_ERR_OVERFLOW;
  if (n_q > 16 || (Hq / Hkv) * n_q > 256 || !supported(dtype, D)) return SPEC_ERR_UNSUPPORTED;
  const AttnPlan p = attn_plan(B, Hq, Hkv, n_q, D, max_len_hint, dtype);
  if (workspace_bytes < p.total) return SPEC_ERR_ARG;
  if ((size_t)B * Hkv * p.RG * p.NSP > 0x7fffffffu) return SPEC_ERR_UNSUPPORTED;

  AttnArgs a;
  a.q = q;
  a.kn = k_new;
  a.vn = v_new;
  a.kc = k_cache;
  a.vc = v_cache;
  a.len = cache_len;
  a.out = out;
  a.part_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.off_o);
  a.part_ml = reinterpret_cast<ML*>(static_cast<char*>(workspace) + p.off_ml);
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.n_q = n_q;
  a.G = Hq / Hkv;
  a.M = a.G * n_q;
  a.RG = p.RG;
  a.NSP = p.NSP;
  a.C = p.C;
  a.max_T = max_T;
  a.hint = max_len_hint;
  a.qk_scale = scale * 1.4426950408889634f;

  hipError_t e = hipErrorInvalidValue;
  if (dtype == SPEC_BF16) {
    if (D == 128) e = attn_launch_d<uint16_t, 128>(a, p.RT, stream);
    else if (D == 64) e = attn_launch_d<uint16_t, 64>(a, p.RT, stream);
  } else {
    if (D == 24) e = attn_launch_d<float, 24>(a, p.RT, stream);
    else if (D == 32) e = attn_launch_d<float, 32>(a, p.RT, stream);
    else if (D == 64) e = attn_launch_d<float, 64>(a, p.RT, stream);
    else if (D == 128) e = attn_launch_d<float, 128>(a, p.RT, stream);
  }
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_LAUNCH;
}
