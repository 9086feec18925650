// Causal multi-query verify attention with KV append (gfx950, MFMA).
//
// [P2] "LLM推論の高速化｜KVキャッシュと投機的デコーディングを自作で実測":
//   section numpyで小さなTransformerを自作する (forward_cached: the n new
//   tokens' K/V go to cache rows [p0, p0+n), the i-th new row attends to rows
//   [0, p0+i], scores scaled by 1/sqrt(D) and soft-maxed);
//   section GQA・MQAでKVキャッシュを減らす (query heads share KV heads; decode
//   attention time is the time to read the cache).
//
// Work decomposition.  A slab is (b, g, rg): sequence b, KV head g, row group
// rg.  The rows of (b, g) are the G = Hq/Hkv query heads sharing KV head g
// times the n_q verify positions, padded to 16-row MFMA tiles; all of them
// read the same K/V tiles (the GQA reuse).  A piece of a slab walks a range
// of its keys in blocks of 32 with an online softmax and leaves its (max,
// sum, unnormalised output) in the workspace, or writes the output directly
// when it is the whole slab; the pieces are merged afterwards.
//   bf16 (B <= 1024): the stream scheme.  One workgroup per resident slot;
//   the slabs' key blocks are laid end to end and cut into equal shares, one
//   per workgroup, so every workgroup has the same work whatever the lengths.
//   Long shares merge each slab's pieces inside the launch (the last of its
//   workgroups to finish); short ones in a combine launch.
//   fp32: fixed splits of C keys, one wave each; up to 8 splits of a slab
//   are the waves of one workgroup and merge in LDS, more go through a
//   combine launch.  bf16 with B > 1024: fixed splits and a combine launch.
//
// MFMA layouts (gfx950, wave64, checked on the hardware).  For
// v_mfma_f32_16x16x32_bf16 lane l holds A[l%16][8(l/16) .. +7],
// B[8(l/16) .. +7][l%16] and returns C[4(l/16) + j][l%16], j = 0..3;
// v_mfma_f32_16x16x4_f32 holds A[l%16][l/16], B[l/16][l%16], same C layout.
//   Scores are computed transposed, S^T = K Q^T (A = 16 keys x D, B = D x 16
//   rows), so each lane ends with 4 keys x 1 row: row statistics need only a
//   reduction over the 4 lane groups, and the probabilities are already where
//   the B operand of O^T = V^T P^T wants them (keys along the contraction).
//   The contraction may take keys in any order, so the 8 keys a lane holds
//   from two 16-key tiles, {4(l/16) + j, 16 + 4(l/16) + j}, are its 8 MFMA
//   k-slots and V^T is gathered in the same order.
//
// bf16 kernels.  One wave per 16-row tile.  K and
// V blocks (32 keys x D) are copied from HBM straight into LDS with
// global_load_lds (no registers, asynchronous, non-temporal) through two LDS
// stages, the next block in flight while one is computed, and read by
// every wave of the workgroup: K as 16-byte A fragments (ds_read_b128), V
// transposed with ds_read_b64_tr_b16 (within each 16-lane group, lane i
// receives element i mod 4 of the 8-byte pieces of lanes 4k + i/4, k = 0..3;
// pointing lane 4k+q at V[key_k][d0 + 4q] hands lane i V[key_0..3][d0 + i]).
// Each 16-byte column slot of a staged row is XOR-swizzled by the row so both
// read patterns are free of LDS bank conflicts; the swizzle is applied on the
// global side of the copy, which keeps every 16 lanes of a copy on one
// contiguous row.
//
// fp32 kernel.  One wave per split holding every row tile; one key per lane
// per MFMA, so V is read straight from memory.
//
// int8 kernel ([P2] section PagedAttentionとKVキャッシュの量子化).  The stream
// scheme with one-wave workgroups holding every row tile of a slab: each raw
// int8 block is widened once (K exactly to f16 for f16 products, V
// dequantised to bf16 for the bf16 PV product) and used by every tile; the
// probabilities are taken against a fixed per-row reference, with an exact
// fp32 path for the rare slab whose scores outgrow it (see its section).
//
// Keys [0, L_b) come from the cache, keys [L_b, L_b + n_q) from k_new/v_new
// directly (so the append in the same launch is never read back), and keys at
// or past L_b + n_q are masked (they read a finite dummy row).  Cache rows at
// or past L_b are never read.  Row i of the verify block sees keys <= L_b + i.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "spec_common.h"
#include "spec_verify.h"

namespace specv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int KB = 32;  // keys per block

// The 16-bit element of the bf16 kernels' layout: bf16, or IEEE half (F16).
// Both are 2 bytes, staged and transposed alike; only the MFMA, the
// conversions and the NaN pattern differ.
template <bool F16>
struct Half16;
template <>
struct Half16<false> {
  typedef bf16x8 v8;
  typedef __bf16 elem;
  static constexpr uint16_t kNaN = 0x7fc0;
  __device__ static f32x4 mfma(v8 a, v8 b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0); }
  __device__ static uint16_t bits(float f) { return f32_to_bf16(f); }
};
template <>
struct Half16<true> {
  typedef f16x8 v8;
  typedef _Float16 elem;
  static constexpr uint16_t kNaN = 0x7e00;
  __device__ static f32x4 mfma(v8 a, v8 b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }
  __device__ static uint16_t bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }  // round to nearest even
};

struct ML {  // per split and row: running max (log2 units) and sum
  float m, l;
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
  uint32_t* ovf;  // int8 stream scheme: per slab, 1 if a piece left it to the exact path
  int* pre;  // stream scheme: [B + 1] blocks per slab before sequence b
  uint32_t* scnt;  // stream scheme merged in the kernel: pieces finished per slab
  int B, Hq, Hkv, n_q, G, M, RG, RT, NSP, C, max_T, hint;
  int P, MINB, JP;  // stream scheme: workgroups, minimum share, partial slots per slab
  // Paged cache: kc / vc are [Hkv][num_pages][page][D]; table[b * max_blocks + i]
  // is the page of logical block i of sequence b.
  const int32_t* table;  // null: contiguous cache [B][Hkv][max_T][D]
  int page, max_blocks, num_pages;
  // int8 cache: kc / vc are int8 [B][Hkv][max_T][D], ksc / vsc their fp16
  // scales [B][Hkv][max_T]; nkq / nvq and nks / nvs hold the new rows
  // quantised by quant_new_rows ([B][Hkv][n_q][D] int8, [B][Hkv][n_q] fp16).
  const uint16_t* ksc;
  const uint16_t* vsc;
  int8_t* nkq;
  int8_t* nvq;
  uint16_t* nks;
  uint16_t* nvs;
  float qk_scale;  // scale * log2(e)
};

// Decode blockIdx into (b, g, rg, sp); sp varies fastest, so consecutive
// workgroups stream neighbouring parts of one (b, g) slab.  Partials are
// stored at this index, id = ((b Hkv + g) RG + rg) NSP + sp.
struct Item {
  int b, g, rg, sp;
  long bg;
  size_t id;
};

__device__ __forceinline__ Item decode_item(const AttnArgs& a) {
  long item = blockIdx.x;
  Item it;
  it.id = (size_t)item;
  it.sp = (int)(item % a.NSP);
  item /= a.NSP;
  it.rg = (int)(item % a.RG);
  item /= a.RG;
  it.g = (int)(item % a.Hkv);
  it.b = (int)(item / a.Hkv);
  it.bg = (long)it.b * a.Hkv + it.g;
  return it;
}

// Row of key `key` of (b, g): the cache row, the new row, or null (masked).
template <typename T>
__device__ __forceinline__ const T* key_row(const T* cache, const T* fresh, int key, int L, int Ltot, int n_q,
                                            int max_T, int D, long bg) {
  if (key < L) return cache + ((size_t)bg * max_T + key) * D;
  if (key < Ltot) return fresh + ((size_t)bg * n_q + (key - L)) * D;
  return nullptr;
}

// A1: copy the n_q new rows of (b, g) into the cache at rows [L, L + n_q).
template <typename T, int D>
__device__ __forceinline__ void append_rows(const AttnArgs& a, long bg, int L, int tid, int nthreads) {
  constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
  const int chunks = a.n_q * D / EPC;
  const uint4* skn = reinterpret_cast<const uint4*>(static_cast<const T*>(a.kn) + (size_t)bg * a.n_q * D);
  const uint4* svn = reinterpret_cast<const uint4*>(static_cast<const T*>(a.vn) + (size_t)bg * a.n_q * D);
  uint4* dkc = reinterpret_cast<uint4*>(static_cast<T*>(a.kc) + ((size_t)bg * a.max_T + L) * D);
  uint4* dvc = reinterpret_cast<uint4*>(static_cast<T*>(a.vc) + ((size_t)bg * a.max_T + L) * D);
  for (int c = tid; c < chunks; c += nthreads) {
    dkc[c] = skn[c];
    dvc[c] = svn[c];
  }
}

// A1 into a paged cache: row L + r of (b, g) goes to slot (L + r) % PG of the
// page the table lists for block (L + r) / PG (entries checked by the caller).
template <int D, int PG>
__device__ __forceinline__ void append_rows_paged(const AttnArgs& a, int b, int g, int L, int tid, int nthreads) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  const int chunks = a.n_q * CPR;
  const long bg = (long)b * a.Hkv + g;
  const uint4* skn = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.kn) + (size_t)bg * a.n_q * D);
  const uint4* svn = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.vn) + (size_t)bg * a.n_q * D);
  for (int c = tid; c < chunks; c += nthreads) {
    const int pos = L + c / CPR;
    const size_t page = (size_t)a.table[(size_t)b * a.max_blocks + pos / PG];
    const size_t row = (((size_t)g * a.num_pages + page) * PG + pos % PG) * CPR + c % CPR;
    reinterpret_cast<uint4*>(a.kc)[row] = skn[c];
    reinterpret_cast<uint4*>(a.vc)[row] = svn[c];
  }
}

// Online-softmax update of one row from 8 scaled scores (log2 domain);
// returns the rescale factor of the previous state and writes the new
// probabilities into s in place.
__device__ __forceinline__ float softmax_update(float (&s)[8], float& mrow, float& lsum) {
  float mx = s[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) mx = fmaxf(mx, s[j]);
  mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
  mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
  const float mnew = fmaxf(mrow, mx);
  const bool none = (mnew == neg_inf_f());
  const float alpha = none ? 1.f : exp2_fast(mrow - mnew);
  float ps = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float p = none ? 0.f : exp2_fast(s[j] - mnew);
    s[j] = p;
    ps += p;
  }
  lsum = lsum * alpha + ps;
  mrow = mnew;
  return alpha;
}

// ---------------------------------------------------------------------------
// bf16 split kernel: NW waves, one 16-row tile each, K/V staged in LDS
// ---------------------------------------------------------------------------

template <int D>
struct BfLayout {
  static constexpr int CH = D / 8;               // 16-byte slots per row
  static constexpr int RP = 256 / (2 * D);       // rows per 256-byte bank line (>= 1)
  static constexpr int TILE = KB * D;            // elements per staged tile
  static constexpr int NI = TILE * 2 / 1024;     // 1 KB global_load_lds copies per tile
  // K rows are read 16 at a time at one slot: spread them over 16 slots.
  __host__ __device__ static constexpr int kslot(int row, int c) { return c ^ ((row / RP) % CH); }
  // V rows are read 8 at a time at a 32-byte slot pair: spread them over 8 pairs.
  __host__ __device__ static constexpr int vslot(int row, int c) { return c ^ (2 * ((row / RP) % (CH / 2))); }
  static constexpr bool same_swizzle_16_rows_apart() {
    for (int r = 0; r < 16; ++r)
      for (int c = 0; c < CH; ++c)
        if (kslot(r + 16, c) != kslot(r, c) || vslot(r + 16, c) != vslot(r, c)) return false;
    return true;
  }
};

// Wait until at most N of this wave's vector-memory operations are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without a global memory fence.  __syncthreads() also
// fences, which makes the compiler wait for every outstanding global_load_lds
// copy, including those of later blocks still meant to be in flight.  Here
// each wave has already waited for its own copies of the current block; it
// drains its own LDS reads (so none of them can still be reading a stage
// another wave is about to refill) and the asm statements keep the compiler
// from moving LDS accesses across the barrier.
__device__ __forceinline__ void block_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

template <int V>
using IC = std::integral_constant<int, V>;

// Max / sum across the four 16-lane groups of a wave (lanes l, l^16, l^32,
// l^48) with the gfx950 lane-swap instructions: swapping a register with
// itself across 16-lane (32-lane) halves hands every lane its partner's value.
__device__ __forceinline__ float group_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Waves per SIMD the compiler budgets registers for: 4 keeps a kernel within
// 128 VGPRs, so two 5-wave workgroups share a CU.
constexpr int kAttnWavesPerEU = 4;
constexpr int kStreamWavesPerEU = 4;
// Cache policy of the cache-block loads, which stream every key once per
// call: non-temporal (nt = 2).
constexpr int kKvCachePolicy = 2;

// One LDS object per stage and tensor: reads of one stage then provably do
// not alias the asynchronous copies into another, so the compiler does not
// make them wait for those copies.
#define SPECV_BF16_STAGE_LDS \
  __shared__ __attribute__((aligned(1024))) uint16_t k0s[LY::TILE], v0s[LY::TILE]; \
  __shared__ __attribute__((aligned(1024))) uint16_t k1s[LY::TILE], v1s[LY::TILE]; \
  __shared__ __attribute__((aligned(1024))) uint16_t k2s[NST > 2 ? LY::TILE : 8], v2s[NST > 2 ? LY::TILE : 8]; \
  auto kbuf = [&](auto S) -> uint16_t* { \
    if constexpr (decltype(S)::value == 0) return k0s; \
    else if constexpr (decltype(S)::value == 1) return k1s; \
    else return k2s; \
  }; \
  auto vbuf = [&](auto S) -> uint16_t* { \
    if constexpr (decltype(S)::value == 0) return v0s; \
    else if constexpr (decltype(S)::value == 1) return v1s; \
    else return v2s; \
  };

// Device-scope (write-through) stores and loads of piece partials that
// another workgroup merges within the same launch.
__device__ __forceinline__ void co_store2(float* p, float x, float y) {
  const unsigned long long v = (unsigned long long)__float_as_uint(x) | ((unsigned long long)__float_as_uint(y) << 32);
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 co_load2(const float* p) {
  const unsigned long long v =
      __hip_atomic_load(reinterpret_cast<const unsigned long long*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}

// One piece of one (b, g, rg): keys [k0, k1) of sequence b (length L, valid),
// rows of row group rg of KV head g.  Writes the normalised output when the
// piece is the whole of (b, g, rg) (whole), else its (max, sum, unnormalised
// output) at partial slot `slot`.  append: also copy the n_q new rows of
// (b, g) into the cache (A1).  kbuf / vbuf map a stage index to its LDS
// objects.  Every wave of the workgroup calls it with the same arguments.
// CO: partials through device-scope stores (merged within the launch).
template <int D, int NW, int NST, int PG, bool CO = false, bool F16 = false, typename KBuf, typename VBuf>
__device__ __forceinline__ void bf16_piece(const AttnArgs& a, KBuf kbuf, VBuf vbuf, int b, int g, int rg, int L,
                                           int k0, int k1, bool whole, size_t slot, bool append,
                                           const int32_t* __restrict__ table = nullptr) {
  using LY = BfLayout<D>;
  using H = Half16<F16>;
  constexpr int DS = D / 32;  // MFMA steps over D for the scores
  constexpr int DT = D / 16;  // 16-wide output tiles over D
  constexpr int NCP = 2 * LY::NI;                             // 1 KB copies per block (K then V)
  constexpr int WI = NW >= 4 ? 4 : (NW >= 2 ? 2 : 1);         // waves that issue copies
  constexpr int CPW = NCP / WI;                               // copies per issuing wave per block
  static_assert(NCP % WI == 0, "copies must split evenly over the issuing waves");
  static_assert(NST >= 2 && NST <= 3 && (NST - 2) * CPW <= 63, "stages");
  // The thread index passes through an empty asm, so lane-derived values are
  // recomputed per piece rather than hoisted out of a caller's piece loop
  // and kept live across it.
  int tid = threadIdx.x;
  __asm__ volatile("" : "+v"(tid));
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform per wave
  const int lane = tid & (kWave - 1);
  const int lr = lane & 15;
  const int lg = lane >> 4;
  const long bg = (long)b * a.Hkv + g;
  const int Ltot = L + a.n_q;
  const int nblk = (k1 - k0 + KB - 1) / KB;
  static_assert(PG == 0 || PG == 16 || PG == 32, "page size");
  // The table comes in as a read-only, non-aliased kernel argument, so the
  // uniform per-block lookups below are scalar loads: a vector load would
  // need a wait on the vector-memory counter, draining the copies in flight.
  const int32_t* __restrict__ tab = PG ? table + (size_t)b * a.max_blocks : nullptr;
  if constexpr (PG > 0) {
    // Every table entry this piece will use (the committed keys it reads and,
    // if it appends, the pages of the new rows) must name a page; otherwise
    // the piece reads nothing and leaves NaN (every wave finds the same).
    bool badp = false;
    const int e1 = (min(k1, L) + PG - 1) / PG;
    for (int e = k0 / PG + lane; e < e1; e += 8 * kWave) {
      int pg[8];  // eight loads in flight per lane before any test
#pragma unroll
      for (int t = 0; t < 8; ++t) pg[t] = e + t * kWave < e1 ? tab[e + t * kWave] : 0;
#pragma unroll
      for (int t = 0; t < 8; ++t) badp |= pg[t] < 0 || pg[t] >= a.num_pages;
    }
    if (append) {
      for (int e = L / PG + lane; e <= (Ltot - 1) / PG; e += kWave) {
        const int pg = tab[e];
        badp |= pg < 0 || pg >= a.num_pages;
      }
    }
    if (__ballot(badp)) {
      const float qnan = __builtin_nanf("");
      const int m = rg * 16 * NW + 16 * wave + lr;
      if (whole) {
        if (m < a.M && lg == 0) {
          uint16_t* o = static_cast<uint16_t*>(a.out) +
                        (((size_t)b * a.Hq + g * a.G + m / a.n_q) * a.n_q + m % a.n_q) * D;
          for (int d = 0; d < D; ++d) o[d] = H::kNaN;
        }
      } else {
        const int row = 16 * wave + lr;
        float* po = a.part_o + slot * (16 * NW) * D + (size_t)row * D;
        if constexpr (CO) {
          if (lg == 0) co_store2(reinterpret_cast<float*>(a.part_ml + slot * (16 * NW) + row), qnan, qnan);
          for (int d = 2 * lg; d < D; d += 8) co_store2(po + d, qnan, qnan);
        } else {
          if (lg == 0) a.part_ml[slot * (16 * NW) + row] = ML{qnan, qnan};
          for (int d = lg; d < D; d += 4) po[d] = qnan;
        }
      }
      return;
    }
  }

  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  // Contiguous cache: the (b, g) slab.  Paged: the page array (per-block bases below).
  const uint16_t* kc = static_cast<const uint16_t*>(a.kc) + (PG ? 0 : (size_t)bg * a.max_T * D);
  const uint16_t* vc = static_cast<const uint16_t*>(a.vc) + (PG ? 0 : (size_t)bg * a.max_T * D);
  const uint16_t* knb = static_cast<const uint16_t*>(a.kn) + (size_t)bg * a.n_q * D;
  const uint16_t* vnb = static_cast<const uint16_t*>(a.vn) + (size_t)bg * a.n_q * D;

  // Copies of one block: copy c (first NI for K, then NI for V) is issued by
  // wave c % WI, as its i-th copy with c = wave + i WI (so copies i < NI/WI
  // are K).  Lane l fills LDS slot (64 c' + l) of its tile (c' = c mod NI):
  // row (64 c' + l) / CH at swizzled slot (64 c' + l) % CH, which holds the
  // row's 16-byte chunk given by the same XOR.  Every issuing wave issues CPW
  // copies per block, so a fixed vmcnt tells it when an older block landed.
  // coff[i]: element offset, within a staged block, of the 16-byte chunk this
  // lane copies in copy i (row crow = coff / D, chunk 8 cchunk = coff % D).
  // A copy's rows are 512 / D consecutive rows of one 16-row half, so a
  // copy never spans two 16-position pages.
  uint32_t coff[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const bool is_v = i >= LY::NI / WI;
    const int cc = (wave + i * WI) - (is_v ? LY::NI : 0);
    const int p = cc * kWave + lane;
    const int crow = p / LY::CH;
    const int sl = p % LY::CH;
    const int cchunk = is_v ? LY::vslot(crow, sl) : LY::kslot(crow, sl);  // XOR is its own inverse
    coff[i] = (uint32_t)(crow * D + 8 * cchunk);
  }
  static_assert(16 % (512 / D) == 0, "a copy stays inside one 16-row half");
  // Paged: the page(s) of a block holding committed keys (kb is a multiple of
  // 32, so a block is one 32-page or two 16-pages), read one block ahead of
  // its copies so the scalar load's latency is not on the copy issue path.
  auto pages_of = [&](int kb, int& p0, int& p1) {
    if constexpr (PG > 0) {
      if (kb < L) p0 = tab[kb / PG];
      if constexpr (PG == 16) {
        if (kb + 16 < L) p1 = tab[kb / PG + 1];
      }
    }
  };
  auto issue_block = [&](int kb, auto S, int p0, int p1) {
    if (wave >= WI) return;
    const bool full = kb + KB <= L;  // every key of the block is committed cache
    // Element offset of the block's row 0 in the cache (contiguous), or of
    // its page's row 0 (paged; pbase1 + 16 D is the 16-page holding rows
    // 16..31).
    size_t pbase0 = (size_t)kb * D, pbase1 = 0;
    if constexpr (PG > 0) {
      if (kb < L) pbase0 = ((size_t)g * a.num_pages + p0) * PG * D;
      if constexpr (PG == 16) {
        if (kb + 16 < L) pbase1 = ((size_t)g * a.num_pages + p1) * PG * D - (size_t)16 * D;
      }
    }
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const bool is_v = i >= LY::NI / WI;
      const int cc = (wave + i * WI) - (is_v ? LY::NI : 0);
      const uint16_t* cache = is_v ? vc : kc;
      const uint16_t* fresh = is_v ? vnb : knb;
      // The copy's base is uniform across the wave: its rows sit in one page.
      const bool hi_half = PG == 16 && (cc * kWave) / LY::CH >= 16;
      const uint16_t* cbase = cache + (hi_half ? pbase1 + (size_t)16 * D : pbase0);
      const uint32_t loff = coff[i] - (hi_half ? 16 * D : 0);  // element offset from cbase
      uint16_t* dst = (is_v ? vbuf(S) : kbuf(S)) + cc * 512;
      if (full) {
        // Buffer load: the base in a scalar descriptor whose range is the
        // block's (or page's) rows, the lane's byte offset in one VGPR.
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc((void*)cbase, (short)0, (PG == 16 ? 16 : KB) * D * 2, 0x00020000);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (void __attribute__((address_space(3)))*)dst, 16,
                                                 (int)(loff * 2), 0, 0, kKvCachePolicy);
      } else {  // new rows from k_new/v_new; keys past the end read a finite dummy row
        const int crow = (int)(coff[i] / D);
        const int key = kb + crow;
        const uint16_t* src =
            (key < L ? cbase + loff : fresh + (size_t)(key < Ltot ? key - L : 0) * D + coff[i] % D);
        __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                         (void __attribute__((address_space(3)))*)dst, 16, 0, 0);
      }
    }
  };

  // Query fragment of this wave's tile (B operand of S^T = K Q^T).
  const int m = rg * 16 * NW + 16 * wave + lr;
  const bool valid = m < a.M;
  const int h = g * a.G + (valid ? m / a.n_q : 0);
  const int qi = valid ? m % a.n_q : a.n_q - 1;
  const int lim = L + qi;  // last visible key of this row
  typename H::v8 qf[DS];
  {
    const uint16_t* qrow = q + (((size_t)b * a.Hq + h) * a.n_q + qi) * D;
#pragma unroll
    for (int s = 0; s < DS; ++s)
      qf[s] = valid ? *reinterpret_cast<const typename H::v8*>(qrow + 32 * s + 8 * lg) : typename H::v8{};
  }

  int pf0 = 0, pf1 = 0;  // pages of the next block to issue
  pages_of(k0, pf0, pf1);
  issue_block(k0, IC<0>{}, pf0, pf1);
  if constexpr (NST > 2) {
    if (nblk > 1) {
      pages_of(k0 + KB, pf0, pf1);
      issue_block(k0 + KB, IC<1>{}, pf0, pf1);
    }
  }
  if (NST - 1 < nblk) pages_of(k0 + (NST - 1) * KB, pf0, pf1);

  // Loop-invariant LDS element offsets of this lane's reads within a stage:
  // K fragment (kt = 0) for each D step, and V^T pieces (hh = 0) for each D
  // tile; kt = 1 / hh = 1 add 16 rows.
  int kofs[DS], vofs[DT];
#pragma unroll
  for (int s = 0; s < DS; ++s) kofs[s] = lr * D + 8 * LY::kslot(lr, 4 * s + lg);
  {
    const int vrow = 4 * lg + (lr >> 2), q4 = lr & 3;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vofs[dt] = vrow * D + 8 * LY::vslot(vrow, 2 * dt + (q4 >> 1)) + 4 * (q4 & 1);
  }
  // kt = 1 and hh = 1 reuse these offsets 16 rows further: rows 16 apart
  // have the same swizzle.
  static_assert(LY::same_swizzle_16_rows_apart(), "kt / hh offsets");

  const float c = a.qk_scale;
  float mrow = neg_inf_f(), lsum = 0.f;  // running max (scaled, log2 units) and partial sum
  f32x4 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Block j lives in stage S = j mod NST.
  auto step = [&](auto S, int j) {
    const int kb = k0 + j * KB;
    // This wave's copies of block j have landed (only blocks issued after it
    // may still be in flight); after the barrier every wave's have, and every
    // wave has finished reading the stage the next copy refills.
    if (NST > 2 && j + 1 < nblk)
      wait_vmcnt<(NST > 2 ? CPW : 0)>();
    else
      wait_vmcnt<0>();
    block_barrier();
    if (j + NST - 1 < nblk) {
      issue_block(kb + (NST - 1) * KB, IC<(decltype(S)::value + NST - 1) % NST>{}, pf0, pf1);
      if (j + NST < nblk) pages_of(kb + NST * KB, pf0, pf1);
    }

    const uint16_t* ks = kbuf(S);
    const uint16_t* vs = vbuf(S);
    // Raw scores: lane holds keys kb + 16 kt + 4 lg + jj of row lr of the tile.
    float sc[8];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        const typename H::v8 kf = *reinterpret_cast<const typename H::v8*>(ks + kofs[s] + 16 * kt * D);
        acc = H::mfma(kf, qf[s], acc);
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) sc[4 * kt + jj] = acc[jj];
    }
    // Online softmax in the log2 domain: p = 2^(s c - m) with m the running
    // max of s c.
    float mx = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
    float alpha;
    if (kb + KB <= L) {
      // Every key is visible to every row: scores are finite.
      const float mnew = fmaxf(mrow, group_max(mx) * c);
      alpha = exp2_fast(mrow - mnew);
      float ps = 0.f;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        sc[jj] = exp2_fast(fmaf(sc[jj], c, -mnew));
        ps += sc[jj];
      }
      lsum = fmaf(lsum, alpha, ps);
      mrow = mnew;
    } else {
      // The block reaches the new rows or the end: causal mask, and a row may
      // have seen no visible key yet.
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int key = kb + 16 * kt + 4 * lg + jj;
          if (key >= Ltot || key > lim) sc[4 * kt + jj] = neg_inf_f();
        }
      mx = sc[0];
#pragma unroll
      for (int jj = 1; jj < 8; ++jj) mx = fmaxf(mx, sc[jj]);
      const float mnew = fmaxf(mrow, group_max(mx) * c);
      const bool none = (mnew == neg_inf_f());
      alpha = none ? 1.f : exp2_fast(mrow - mnew);
      float ps = 0.f;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        sc[jj] = none ? 0.f : exp2_fast(fmaf(sc[jj], c, -mnew));
        ps += sc[jj];
      }
      lsum = fmaf(lsum, alpha, ps);
      mrow = mnew;
    }
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
    }
    typename H::v8 pf;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) pf[jj] = (typename H::elem)sc[jj];

    // V^T fragments: half hh covers keys 16 hh + 4 lg + (0..3); lane lr of
    // the group points at V[16 hh + 4 lg + lr/4][16 dt + 4 (lr%4)].
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      s16x4 v2[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        v2[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vs + vofs[dt] + 16 * hh * D));
      const typename H::v8 vf =
          __builtin_bit_cast(typename H::v8, __builtin_shufflevector(v2[0], v2[1], 0, 1, 2, 3, 4, 5, 6, 7));
      oacc[dt] = H::mfma(vf, pf, oacc[dt]);
    }
  };

  for (int j = 0; j < nblk; j += NST) {
    step(IC<0>{}, j);
    if (j + 1 < nblk) step(IC<1>{}, j + 1);
    if constexpr (NST > 2) {
      if (j + 2 < nblk) step(IC<2>{}, j + 2);
    }
  }

  // A1 (once per (b, g)); nothing in this launch reads these rows.
  if (append) {
    if constexpr (PG == 0) {
      append_rows<uint16_t, D>(a, bg, L, tid, 64 * NW);
    } else {
      append_rows_paged<D, PG>(a, b, g, L, tid, 64 * NW);
    }
  }

  const float lt = group_sum(lsum);  // row sum over the 4 lane groups
  const int row = 16 * wave + lr;    // row within the item
  if (whole) {
    // The whole of (b, g, rg) is here: normalise and write the output.
    if (valid) {
      uint16_t* o = static_cast<uint16_t*>(a.out) + (((size_t)b * a.Hq + h) * a.n_q + qi) * D;
      const float inv = 1.f / lt;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = 16 * dt + 4 * lg;
        uint2 pk;
        pk.x = uint32_t(H::bits(oacc[dt][0] * inv)) | (uint32_t(H::bits(oacc[dt][1] * inv)) << 16);
        pk.y = uint32_t(H::bits(oacc[dt][2] * inv)) | (uint32_t(H::bits(oacc[dt][3] * inv)) << 16);
        *reinterpret_cast<uint2*>(o + d) = pk;
      }
    }
    return;
  }
  float* po = a.part_o + slot * (16 * NW) * D;
  if constexpr (CO) {
    if (lg == 0) co_store2(reinterpret_cast<float*>(a.part_ml + slot * (16 * NW) + row), mrow, lt);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      float* pd = po + (size_t)row * D + 16 * dt + 4 * lg;
      co_store2(pd, oacc[dt][0], oacc[dt][1]);
      co_store2(pd + 2, oacc[dt][2], oacc[dt][3]);
    }
  } else {
    if (lg == 0) a.part_ml[slot * (16 * NW) + row] = ML{mrow, lt};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(po + (size_t)row * D + 16 * dt + 4 * lg) = oacc[dt];
  }
}

template <int D, int NW, int NST>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(kAttnWavesPerEU)))
void attn_split_bf16(AttnArgs a) {
  using LY = BfLayout<D>;
  SPECV_BF16_STAGE_LDS
  const Item it = decode_item(a);
  const int L = a.len[it.b];
  if (L < 0 || L > a.hint) return;  // flagged by attn_combine
  const int Ltot = L + a.n_q;
  const int k0 = it.sp * a.C;
  if (k0 >= Ltot) return;
  bf16_piece<D, NW, NST, 0>(a, kbuf, vbuf, it.b, it.g, it.rg, L, k0, min(k0 + a.C, Ltot), Ltot <= a.C, it.id,
                         it.sp == 0 && it.rg == 0);
}

// Inclusive prefix sum of ints over the 64 lanes in lane order.
__device__ __forceinline__ int wave_inclusive_scan_int(int v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}

// A wave-uniform 64-bit value moved to scalar registers.
__device__ __forceinline__ long long uniform64(long long v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (long long)(((uint64_t)hi << 32) | lo);
}

// Blocks of KB keys in one (b, g, rg) slab of sequence b; 0 for a length the
// call rejects (the combine writes NaN rows for it).
__device__ __forceinline__ int slab_blocks(const AttnArgs& a, int b) {
  const int L = a.len[b];
  return (L < 0 || L > a.hint) ? 0 : (L + a.n_q + KB - 1) / KB;
}

// Blocks per workgroup: the total W spread over the P workgroups, but never
// below MINB, so a slab is cut into at most JP pieces.
__device__ __forceinline__ long long stream_share(const AttnArgs& a, long long W) {
  return max((W + a.P - 1) / a.P, (long long)a.MINB);
}

// bf16 stream kernel: P persistent workgroups share the key blocks of every
// slab evenly.  The slabs (b, g, rg) are laid end to end in that order (b
// slowest), slab (b, .) holding slab_blocks(b) blocks, W blocks in all;
// workgroup w takes blocks [w share, (w + 1) share) of that sequence, which
// may end inside one slab and run on through the next ones.  Each piece it
// covers is run like a split: a slab it covers whole gets its output
// directly, otherwise the piece's state goes to partial slot j of the slab,
// j = w - (first workgroup touching the slab), and attn_combine_stream merges
// the pieces.  Equal shares keep every CU busy to the end whatever the
// lengths, and one workgroup per slot means no workgroup waits to be
// dispatched.  Workgroup 0 also stores the per-slab block prefix pre[b] for
// the combine.
// The stream scheme's walk, shared by the stream kernels: find this
// workgroup's share of the slabs' key blocks and call
// piece(b, g, rg, L, k0, k1, whole, slot, append, np) for every slab piece in it
// (np: the number of pieces the slab is cut into),
// in order (every wave of the workgroup makes the same calls; a workgroup
// barrier separates consecutive pieces).
template <typename Piece>
__device__ __forceinline__ void stream_walk(const AttnArgs& a, Piece&& piece) {
  __shared__ long long sh_x[3];
  __shared__ int sh_b[2];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int HR = a.Hkv * a.RG;

  // Locate this workgroup's first block (wave 0; two passes over the lengths).
  if (tid < kWave) {
    int run = 0;
    for (int c0 = 0; c0 < a.B; c0 += kWave) {
      const int bb = c0 + lane;
      const int nb = bb < a.B ? slab_blocks(a, bb) : 0;
      const int incl = run + wave_inclusive_scan_int(nb, lane);
      if (blockIdx.x == 0 && bb < a.B) a.pre[bb + 1] = incl;
      run = __shfl(incl, kWave - 1, kWave);
    }
    if (blockIdx.x == 0 && lane == 0) a.pre[0] = 0;
    const long long W = (long long)HR * run;
    const long long share = stream_share(a, W);
    const long long x0 = (long long)blockIdx.x * share;
    int b0 = a.B, pre0 = 0;
    if (x0 < W) {
      run = 0;
      for (int c0 = 0; c0 < a.B; c0 += kWave) {
        const int bb = c0 + lane;
        const int nb = bb < a.B ? slab_blocks(a, bb) : 0;
        const int incl = run + wave_inclusive_scan_int(nb, lane);
        const uint64_t hit = __ballot(bb < a.B && (long long)HR * incl > x0);
        if (hit) {
          const int l = __ffsll((long long)hit) - 1;
          b0 = c0 + l;
          pre0 = __shfl(incl - nb, l, kWave);
          break;
        }
        run = __shfl(incl, kWave - 1, kWave);
      }
    }
    if (lane == 0) {
      sh_x[0] = x0;
      sh_x[1] = min(x0 + share, W);
      sh_x[2] = share;
      sh_b[0] = b0;
      sh_b[1] = pre0;
    }
  }
  __syncthreads();
  // The piece walk is the same for every wave: keep its state in scalar
  // registers.
  const long long x1 = uniform64(sh_x[1]);
  long long x = uniform64(sh_x[0]);
  if (x >= x1) return;  // uniform: nothing left for this workgroup
  const long long share = uniform64(sh_x[2]);
  int b = __builtin_amdgcn_readfirstlane(sh_b[0]);
  long long preb = __builtin_amdgcn_readfirstlane(sh_b[1]);  // blocks per slab before sequence b
  auto ufl = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
  int nbb = ufl(slab_blocks(a, b));
  const long long q0 = x - (long long)HR * preb;
  int sidx = ufl((int)(q0 / nbb));
  int off = ufl((int)(q0 % nbb));
  bool first = true;
  while (x < x1 && b < a.B) {
    if (nbb == 0) {  // a rejected length holds no blocks
      ++b;
      nbb = b < a.B ? ufl(slab_blocks(a, b)) : 0;
      sidx = 0;
      off = 0;
      continue;
    }
    const int take = ufl((int)min((long long)(nbb - off), x1 - x));
    const int end = off + take;
    const int g = ufl(sidx / a.RG), rg = ufl(sidx % a.RG);
    const long long S0 = (long long)HR * preb + (long long)sidx * nbb;  // first block of the slab
    const int j = ufl((int)((long long)blockIdx.x - S0 / share));
    const bool whole = (off == 0 && end == nbb);
    if (whole || (j >= 0 && j < a.JP)) {
      if (!first) block_barrier();  // every wave is done with the previous piece's stages
      first = false;
      const int L = ufl(a.len[b]);
      const size_t slot = (((size_t)b * a.Hkv + g) * a.RG + rg) * a.JP + (size_t)j;
      const int np = ufl((int)min((S0 + nbb - 1) / share - S0 / share + 1, (long long)a.JP));  // pieces of the slab
      piece(b, g, rg, L, off * KB, min(end * KB, L + a.n_q), whole, slot, off == 0 && rg == 0, np);
    }
    x = uniform64(x + take);
    off = 0;
    if (++sidx == HR) {
      sidx = 0;
      preb = uniform64(preb + nbb);
      ++b;
      nbb = b < a.B ? ufl(slab_blocks(a, b)) : 0;
    }
  }
}

// The piece-merge hand-off inside the stream launch: after a workgroup's
// partial for one piece of a slab (device-scope stores, waited for), it
// counts itself in scnt[slab] (zeroed by attn_stream_prep); the workgroup
// whose add completes the count merges the slab's np partials (device-scope
// loads) and writes the output, as attn_combine_stream would.  Every wave
// calls it.
template <int D, int ROWS, int NT, bool F16>
__device__ __forceinline__ void stream_merge(const AttnArgs& a, int b, int g, int rg, size_t slot, int np) {
  using H = Half16<F16>;
  __shared__ int sh_last;
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  const size_t slab = slot / (size_t)a.JP;
  if (threadIdx.x == 0)
    sh_last = __hip_atomic_fetch_add(a.scnt + slab, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(np - 1);
  __syncthreads();
  if (!sh_last) return;  // uniform over the workgroup
  constexpr int D4 = D / 4;
  const int row0 = rg * ROWS;
  const int nrows = min(ROWS, a.M - row0);
  const size_t base = slab * (size_t)a.JP;
  uint16_t* out = static_cast<uint16_t*>(a.out);
  for (int e = threadIdx.x; e < nrows * D4; e += NT) {
    const int row = e / D4, d = 4 * (e % D4);
    float mx = neg_inf_f(), den = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    bool flagged = false;  // a piece that met a bad page entry left m = NaN
    for (int j0 = 0; j0 < np; j0 += 4) {
      float2 ml[4];
      f32x4 po[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bool in = j0 + t < np;
        const size_t pj = (base + j0 + t) * ROWS + row;
        ml[t] = in ? co_load2(reinterpret_cast<const float*>(a.part_ml + pj)) : make_float2(neg_inf_f(), 0.f);
        const float2 lo = in ? co_load2(a.part_o + pj * D + d) : make_float2(0.f, 0.f);
        const float2 hi = in ? co_load2(a.part_o + pj * D + d + 2) : make_float2(0.f, 0.f);
        po[t] = f32x4{lo.x, lo.y, hi.x, hi.y};
        flagged |= ml[t].x != ml[t].x;
      }
      // fmaxf drops NaN: the flag above, not the maxima, carries it
      const float mc = fmaxf(fmaxf(ml[0].x, ml[1].x), fmaxf(ml[2].x, ml[3].x));
      const float mn = fmaxf(mx, mc);
      if (mn == neg_inf_f()) continue;  // no visible key in these pieces yet
      const float r = exp2_fast(mx - mn);
      den *= r;
      acc *= r;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float w = exp2_fast(ml[t].x - mn);
        den += w * ml[t].y;
        acc += w * po[t];
      }
      mx = mn;
    }
    acc *= flagged ? __builtin_nanf("") : 1.f / den;
    const int m = row0 + row;
    uint2 pk;
    pk.x = uint32_t(H::bits(acc[0])) | (uint32_t(H::bits(acc[1])) << 16);
    pk.y = uint32_t(H::bits(acc[2])) | (uint32_t(H::bits(acc[3])) << 16);
    *reinterpret_cast<uint2*>(out + (((size_t)b * a.Hq + g * a.G + m / a.n_q) * a.n_q + m % a.n_q) * D + d) = pk;
  }
}

// MERGE: the pieces of a slab are merged by the last of its workgroups
// (stream_merge) instead of by attn_combine_stream.
template <int D, int NW, int NST, int PG, bool MERGE, bool F16 = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(kStreamWavesPerEU)))
void attn_stream_bf16(AttnArgs a, const int32_t* __restrict__ table) {
  using LY = BfLayout<D>;
  SPECV_BF16_STAGE_LDS
  stream_walk(a, [&](int b, int g, int rg, int L, int k0, int k1, bool whole, size_t slot, bool append, int np) {
    bf16_piece<D, NW, NST, PG, MERGE, F16>(a, kbuf, vbuf, b, g, rg, L, k0, k1, whole, slot, append, table);
    if constexpr (MERGE) {
      if (!whole) stream_merge<D, 16 * NW, 64 * NW, F16>(a, b, g, rg, slot, np);
    }
  });
}

// Before a merging stream launch: zero the per-slab counters, and write NaN
// rows for the slabs of a rejected length (the stream walk skips them).
template <int D, bool F16 = false>
__global__ __launch_bounds__(256) void attn_stream_prep(AttnArgs a) {
  const long slabs = (long)a.B * a.Hkv * a.RG;
  for (long sl = (long)blockIdx.x * blockDim.x + threadIdx.x; sl < slabs; sl += (long)gridDim.x * blockDim.x) {
    a.scnt[sl] = 0u;
    const int rg = (int)(sl % a.RG);
    const int g = (int)((sl / a.RG) % a.Hkv);
    const int b = (int)(sl / ((long)a.RG * a.Hkv));
    if (slab_blocks(a, b) != 0) continue;
    const int rows = 16 * a.RT, row0 = rg * rows, nrows = min(rows, a.M - row0);
    uint16_t* out = static_cast<uint16_t*>(a.out);
    for (int row = 0; row < nrows; ++row) {
      const int m = row0 + row;
      uint16_t* o = out + (((size_t)b * a.Hq + g * a.G + m / a.n_q) * a.n_q + m % a.n_q) * D;
      for (int d = 0; d < D; ++d) o[d] = Half16<F16>::kNaN;
    }
  }
}


// ---------------------------------------------------------------------------
// int8 cache ([P2] PagedAttentionとKVキャッシュの量子化: rows rounded to int8
// with a per-(head, position) absmax scale kept in fp16)
// ---------------------------------------------------------------------------

// Quantise the n_q new K and V rows of each (b, g) into the workspace: s =
// max|x| / 127, q = round-half-even(x / s) clipped to +-127 (fp32, correctly
// rounded division), scale stored as fp16(s); a zero row gives s = 0, q = 0.
// Grid B * Hkv; 16 lanes per row.
template <int D>
__global__ __launch_bounds__(256) void quant_new_rows(AttnArgs a) {
  constexpr int EPL = D / 16;  // elements per lane
  const long bg = blockIdx.x;
  if ((int)threadIdx.x < a.RG) a.ovf[bg * a.RG + threadIdx.x] = 0u;  // this call's slabs start unmarked
  const int grp = threadIdx.x >> 4, gl = threadIdx.x & 15;
  for (int r = grp; r < 2 * a.n_q; r += 16) {
    const bool is_v = r >= a.n_q;
    const int rr = is_v ? r - a.n_q : r;
    const uint16_t* src = static_cast<const uint16_t*>(is_v ? a.vn : a.kn) + ((size_t)bg * a.n_q + rr) * D + gl * EPL;
    float x[EPL];
    float m = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      x[e] = bf16_to_f32(src[e]);
      m = fmaxf(m, fabsf(x[e]));
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 16));
    const float sc = m / 127.f;
    int8_t* dq = (is_v ? a.nvq : a.nkq) + ((size_t)bg * a.n_q + rr) * D + gl * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float qv = sc > 0.f ? fminf(fmaxf(__builtin_rintf(x[e] / sc), -127.f), 127.f) : 0.f;
      dq[e] = (int8_t)(int)qv;
    }
    if (gl == 0) {
      const _Float16 h = (_Float16)sc;
      (is_v ? a.nvs : a.nks)[(size_t)bg * a.n_q + rr] = __builtin_bit_cast(uint16_t, h);
    }
  }
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// ---------------------------------------------------------------------------
// int8 cache: one wave per workgroup
// ---------------------------------------------------------------------------
//
// A wave holds all RT row tiles of its row group, so each key block is
// widened once and used by every tile (a design that shared each widened
// block between the waves of a workgroup moved it through LDS about 14 times
// its HBM bytes, which bounded it; here a block costs LDS 4 times its
// bytes).  Raw blocks are copied by the wave into I8W_STAGES private LDS
// stages (global_load_lds: no registers held while in flight).  K goes from its stage
// straight into the MFMA operand: the order of d inside the contraction is
// permuted so that lane (lr, lg) takes bytes [lg D/4, (lg + 1) D/4) of key row
// lr -- step s of the product its bytes [8 s, 8 s + 8) -- and the query
// fragments follow the same permutation, which leaves every score unchanged.
// K is widened exactly to f16 (two byte permutes and a packed subtract per
// four values) and the products run in f16 against the query converted to
// f16; the key's scale multiplies the score.  V is widened dequantised,
// bf16(q s) (one rounding, as the probabilities get), into a wave-private
// bf16 tile in the bf16 kernel's swizzled layout, then read transposed
// (ds_read_b64_tr_b16) as there.
//
// The output accumulators (RT x D / 4 floats a lane) stay in the MFMA
// accumulator registers: no vector instruction rewrites them (a rescale of
// them would need all of them in vector registers, more than a wave has), so
// the usual online-softmax rescale (O *= exp2(m_old - m_new) when a row's
// maximum grows) is replaced by a fixed reference per row.  A row's reference
// is the largest score of the first block in which it sees a key, and every
// probability is exp2(score - reference) -- exact softmax terms up to a
// common factor that the final division removes.  Later scores may exceed the
// reference; while the row sum stays within 2^64 so does every (positive)
// term, and then no sum can have overflowed (2^64 x 2^15 keys x |v| < 2^23
// stays below 2^128).  A piece with a larger, infinite or NaN row sum (scores
// growing by some 64 / (scale log2 e) along a row after its first block;
// never for scores of ordinary size) marks its slab, and the combine launch
// computes that slab again on an exact path with the usual rescaling
// (attn_combine_i8).  The row sums themselves come from the MFMA.
//
// Each step overlaps the MFMA work of one block with the vector work of the
// next: the previous block's PV runs while this block's V is dequantised and
// its K widened, and the score products of tile r + 1 run under the
// probabilities of tile r.

// Raw int8 stages: 16-byte chunk c of row r sits at chunk c ^ swz(r) of its
// row, so that the 16 rows an operand read touches (one chunk each) fall on
// 16 different 16-byte bank groups of a 256-byte bank line.
template <int D>
struct I8Layout {
  static constexpr int CH = D / 16;         // 16-byte chunks per row
  static constexpr int RP = 256 / D;        // rows per 256-byte bank line
  static constexpr int NI = KB * D / 1024;  // 1 KB copies per tile
  static constexpr int CPB = 2 * NI + 1;    // copies per block: K, V, scales
  __host__ __device__ static constexpr int swz(int r) { return (r / RP) % CH; }
  // Byte offset of chunk c of row r.
  __host__ __device__ static constexpr int at(int r, int c) { return r * D + 16 * (c ^ swz(r)); }
};
constexpr int I8W_STAGES = 3;

// One copy of 16 bytes per lane from global memory into LDS: lane l's bytes
// land at LDS byte lds + 16 l.  Written out (the instruction has no register
// results) so that the compiler does not track it: it cannot tell the stages
// apart and would make every LDS access wait for every copy in flight.  The
// waits for the copies are explicit (wait_vmcnt), and the memory clobber keeps
// LDS accesses on their side of each copy.  M0 takes the LDS address; one
// wait state separates the write of M0 from the copy that reads it.  M0 is a
// reserved register, so the compiler ignores it in the clobber list (it warns)
// and assumes M0 unchanged across the statement: nothing here may rely on a
// value it keeps in M0.  The int8 kernels that use this copy have no other M0
// user (their generated code writes M0 only right before these copies); a
// kernel that added one (an LDS-direct builtin, indexed register access) would
// have to keep it away from these statements.
__device__ __forceinline__ void lds_copy16(const void* src, uint32_t lds) {
  __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "s"(lds)
                   : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ float ubyte_f32(uint32_t flipped, int i) {
  return (float)((flipped >> (8 * i)) & 0xffu);
}

// Eight int8 values (two words, little-endian) as f16, exactly: with every
// byte's top bit flipped, byte b = q + 128 becomes the low byte of the f16
// 0x64bb = 1024 + b (high byte 0x64: exponent 10, so the low byte counts
// units), and subtracting 1152 leaves q.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f16x8 widen8_f16(uint32_t w0, uint32_t w1) {
  const f16x2 off = {(_Float16)1152.f, (_Float16)1152.f};
  uint32_t o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t x = (k < 2 ? w0 : w1) ^ 0x80808080u;
    const uint32_t h = __builtin_amdgcn_perm(0x64646464u, x, (k & 1) ? 0x04030402u : 0x04010400u);
    o[k] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, h) - off);
  }
  return __builtin_bit_cast(f16x8, make_uint4(o[0], o[1], o[2], o[3]));
}

// Eight int8 values as bf16(q s): (q + 128) s - 128 s in one fma, rounded.
__device__ __forceinline__ bf16x8 widen8_scaled(uint32_t w0, uint32_t w1, float s, float m128s) {
  bf16x8 o;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t word = (i < 4 ? w0 : w1) ^ 0x80808080u;
    o[i] = (__bf16)fmaf(ubyte_f32(word, i & 3), s, m128s);
  }
  return o;
}

// Returns false when the piece left its slab to the exact path (its partial
// is then not written).  MERGE: partials through device-scope stores, for the
// in-launch merge.
template <int D, int RT, bool MERGE, typename KS, typename VS, typename SS>
__device__ __forceinline__ bool i8w_piece(const AttnArgs& a, KS kst, VS vst, SS sst, uint16_t* __restrict__ vt, int b,
                                          int g, int rg, int L, int k0, int k1, bool whole, size_t slot, bool append) {
  using LY = BfLayout<D>;
  using IL = I8Layout<D>;
  constexpr int NST = I8W_STAGES;
  constexpr int DS = D / 32;  // product steps over D
  constexpr int DT = D / 16;  // 16-wide output tiles over D
  constexpr int ROWS = 16 * RT;
  const int lane = threadIdx.x & (kWave - 1);
  const int lr = lane & 15, lg = lane >> 4;
  const long bg = (long)b * a.Hkv + g;
  const int Ltot = L + a.n_q;
  const int nblk = (k1 - k0 + KB - 1) / KB;
  const int kb_last = k0 + (nblk - 1) * KB;

  const int8_t* kc = static_cast<const int8_t*>(a.kc) + (size_t)bg * a.max_T * D;
  const int8_t* vc = static_cast<const int8_t*>(a.vc) + (size_t)bg * a.max_T * D;
  const int8_t* knb = a.nkq + (size_t)bg * a.n_q * D;
  const int8_t* vnb = a.nvq + (size_t)bg * a.n_q * D;
  const uint16_t* ksr = a.ksc + (size_t)bg * a.max_T;
  const uint16_t* vsr = a.vsc + (size_t)bg * a.max_T;
  const uint16_t* ksn = a.nks + (size_t)bg * a.n_q;
  const uint16_t* vsn = a.nvs + (size_t)bg * a.n_q;

  // A1: the quantised new rows and their scales into the cache (only rows
  // [L, L + n_q), which no piece reads from the cache).
  if (append) {
    constexpr int CPR = D / 16;  // 16-byte chunks per int8 row
    for (int cidx = lane; cidx < 2 * a.n_q * CPR; cidx += kWave) {
      const bool is_v = cidx >= a.n_q * CPR;
      const int cc = is_v ? cidx - a.n_q * CPR : cidx;
      const uint4* src = reinterpret_cast<const uint4*>(is_v ? vnb : knb) + cc;
      uint4* dst = reinterpret_cast<uint4*>(static_cast<int8_t*>(is_v ? a.vc : a.kc) + ((size_t)bg * a.max_T + L) * D) + cc;
      *dst = *src;
    }
    if (lane < 2 * a.n_q) {
      const bool is_v = lane >= a.n_q;
      const int r = is_v ? lane - a.n_q : lane;
      uint16_t* dst = const_cast<uint16_t*>(is_v ? a.vsc : a.ksc) + (size_t)bg * a.max_T + L + r;
      *dst = (is_v ? vsn : ksn)[r];
    }
  }

  // Copy i of a tile: lane l moves chunk (t % CH) ^ swz(r) of row r = t / CH,
  // t = 64 i + l, to byte 16 t of the stage.  Rows past the new rows copy
  // row 0 (masked).  Every block issues CPB copies, so waits stay static.
  auto issue = [&](int kb, auto S) {
    if (kb + KB <= L) {  // the whole block is in the cache
      const int8_t* kbase = kc + (size_t)kb * D;
      const int8_t* vbase = vc + (size_t)kb * D;
#pragma unroll
      for (int i = 0; i < IL::NI; ++i) {
        const int t = 64 * i + lane, r = t / IL::CH;
        const int off = r * D + 16 * ((t % IL::CH) ^ IL::swz(r));
        lds_copy16(kbase + off, lds_addr(kst(S) + 1024 * i));
        lds_copy16(vbase + off, lds_addr(vst(S) + 1024 * i));
      }
    } else {
#pragma unroll
      for (int i = 0; i < IL::NI; ++i) {
        const int t = 64 * i + lane, r = t / IL::CH;
        const int cb = 16 * ((t % IL::CH) ^ IL::swz(r));
        const int key = kb + r;
        const bool cached = key < L, fresh = !cached && key < Ltot;
        const size_t ro = cached ? (size_t)key * D : (fresh ? (size_t)(key - L) * D : 0);
        lds_copy16((fresh ? knb : kc) + ro + cb, lds_addr(kst(S) + 1024 * i));
        lds_copy16((fresh ? vnb : vc) + ro + cb, lds_addr(vst(S) + 1024 * i));
      }
    }
    if (lane < 8) {
      // 8 K scales (lanes 0-3) or V scales (4-7) from a multiple of 8; a
      // clamped copy only serves keys past the new rows.
      const int key = min(kb + 8 * (lane & 3), a.max_T - 8);
      lds_copy16((lane < 4 ? ksr : vsr) + key, lds_addr(sst(S)));
    }
  };
  // Query fragments of the RT tiles, d permuted: step s, lane group lg hold
  // d = lg D/4 + 8 s + (0..7).  The products run in f16, which holds every
  // bf16 value of magnitude up to 65504 exactly (bf16's 8 significant bits
  // fit f16's 11; below 2^-14 fewer bits remain, a change far below the
  // scores' rounding); a larger or non-finite query leaves the slab to the
  // exact path.
  f16x8 qf[RT][DS];
  bool qbad = false;
  int lim[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int m = rg * ROWS + 16 * r + lr;
    const bool valid = m < a.M;
    const int h = g * a.G + (valid ? m / a.n_q : 0);
    const int qi = valid ? m % a.n_q : a.n_q - 1;
    lim[r] = L + qi;
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + (((size_t)b * a.Hq + h) * a.n_q + qi) * D;
#pragma unroll
    for (int st = 0; st < DS; ++st) {
      const bf16x8 qv = valid ? *reinterpret_cast<const bf16x8*>(qrow + lg * (D / 4) + 8 * st) : bf16x8{};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = (float)qv[i];
        qbad |= !(fabsf(x) <= 65504.f);
        qf[r][st][i] = (_Float16)x;
      }
    }
  }
  // (taken as a wave-uniform flag here: left per lane until the end, the
  // check kept more registers alive)
  const bool qbad_any = __builtin_amdgcn_readfirstlane(__ballot(qbad) != 0);
  // LDS element offsets of this lane's V^T reads (hh = 0; hh = 1 adds 16 rows)
  int vofs[DT];
  {
    const int vrow = 4 * lg + (lr >> 2), q4 = lr & 3;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vofs[dt] = vrow * D + 8 * LY::vslot(vrow, 2 * dt + (q4 >> 1)) + 4 * (q4 & 1);
  }
  static_assert(LY::same_swizzle_16_rows_apart(), "hh offsets");

  const float c = a.qk_scale;
  // reference (scaled, log2 units; -inf until the row sees a key); the row
  // sums come from the MFMA: an all-ones A fragment against the bf16
  // probabilities adds each row's block sum to every element of lacc[r]
  // (the sum of exactly the values the PV product uses).
  float mref[RT];
  f32x4 lacc[RT];
  f32x4 oacc[RT][DT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    mref[r] = neg_inf_f();
    lacc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[r][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  issue(k0, IC<0>{});
  issue(min(k0 + KB, kb_last), IC<1>{});
  if constexpr (NST > 2) issue(min(k0 + 2 * KB, kb_last), IC<2>{});

  // PV of the previous block (its probabilities pprev, its dequantised V in
  // the tile) is issued while this block's V is dequantised into the same
  // tile: for each 16-wide d tile dt, the tile's reads for dt precede, in
  // program order, this block's writes of those d (a wave's LDS accesses
  // take effect in order, and the compiler keeps possibly aliasing accesses
  // in order).  The MFMA work of one block then overlaps the vector work of
  // the next.  Lane l dequantises row l % 32, bf16 chunks 2 dt + l / 32.
  const int vrow_w = lane & 31, vhalf = lane >> 5;
  bf16x8 pprev[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) pprev[r] = bf16x8{};
  // PV of the previous block: 5 MFMAs per 16-wide d tile dt (dt 0 also
  // adds the row sums).
  const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));
  auto pv_tile = [&](int dt) {
    s16x4 v2[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      v2[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(vt + vofs[dt] + 16 * hh * D));
    const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v2[0], v2[1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
    for (int r = 0; r < RT; ++r) oacc[r][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pprev[r], oacc[r][dt], 0, 0, 0);
    if (dt == 0) {
#pragma unroll
      for (int r = 0; r < RT; ++r) lacc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pprev[r], lacc[r], 0, 0, 0);
    }
  };

  // Everything a block needs from its stage, read into registers one step
  // ahead (after the block's copies have landed).
  struct Raw {
    uint4 k[2][D / 64];
    uint2 v[DT];
    uint2 sk[2];
    uint16_t sv;
  };
  auto read_stage = [&](Raw& R, auto S) {
    wait_vmcnt<(NST - 1) * IL::CPB>();  // this block's copies have landed
    const int8_t* ks = kst(S);
    const int8_t* vs = vst(S);
    const uint16_t* ss = sst(S);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int hh = 0; hh < D / 64; ++hh)
        R.k[kt][hh] = *reinterpret_cast<const uint4*>(ks + IL::at(16 * kt + lr, lg * (D / 64) + hh));
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) R.v[dt] = *reinterpret_cast<const uint2*>(vs + IL::at(vrow_w, dt) + 8 * vhalf);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) R.sk[kt] = *reinterpret_cast<const uint2*>(ss + 16 * kt + 4 * lg);
    R.sv = ss[32 + vrow_w];
  };
  Raw R;

  auto step = [&](int j, auto S) {
    const int kb = k0 + j * KB;
    // the block reaches the new rows (or past them): the only blocks with
    // per-key cases, handled in branches of their own
    const bool tail = __builtin_amdgcn_readfirstlane(kb + KB > L);
    // The block's stage was read into R at the end of the previous step: once
    // those reads are done, refill the stage with the block NST ahead (the
    // last block again past the end).
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    issue(min(kb + NST * KB, kb_last), S);
    const auto& kr = R.k;
    const auto& vr = R.v;
    const auto& skr = R.sk;
    float sv = f16_to_f32(R.sv);
    if (tail) {
      const int key = kb + vrow_w;
      if (key >= L) sv = key < Ltot ? f16_to_f32(vsn[key - L]) : 0.f;
    }
    // The previous block's PV, with this block's V dequantised into the tile
    // behind it and its K fragments widened (exact f16, each then used by
    // every tile) alongside.
    const float m128 = -128.f * sv;
    f16x8 kf[2][DS];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      pv_tile(dt);
      const int chunk = 2 * dt + vhalf;
      *reinterpret_cast<bf16x8*>(vt + vrow_w * D + 8 * LY::vslot(vrow_w, chunk)) =
          widen8_scaled(vr[dt].x, vr[dt].y, sv, m128);
      if (dt < 2 * DS) {
        const int kt = dt / DS, st = dt % DS;
        const uint4 u = kr[kt][st / 2];
        kf[kt][st] = (st & 1) ? widen8_f16(u.z, u.w) : widen8_f16(u.x, u.y);
      }
    }
    // K scales of this lane's 8 keys kb + 16 kt + 4 lg + jj, times c.
    float skc[8];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      skc[4 * kt + 0] = f16_to_f32((uint16_t)(skr[kt].x & 0xffffu)) * c;
      skc[4 * kt + 1] = f16_to_f32((uint16_t)(skr[kt].x >> 16)) * c;
      skc[4 * kt + 2] = f16_to_f32((uint16_t)(skr[kt].y & 0xffffu)) * c;
      skc[4 * kt + 3] = f16_to_f32((uint16_t)(skr[kt].y >> 16)) * c;
    }
    if (tail) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int key = kb + 16 * (jj >> 2) + 4 * lg + (jj & 3);
        if (key >= L) skc[jj] = key < Ltot ? f16_to_f32(ksn[key - L]) * c : 0.f;
      }
    }
    // The next block's stage into R, under this block's scores.
    if (j + 1 < nblk) {
      if constexpr (decltype(S)::value == NST - 1)
        read_stage(R, IC<0>{});
      else
        read_stage(R, IC<decltype(S)::value + 1>{});
    }

    // Scores of tile r (the products of tile r + 1 can run under the vector
    // work of tile r), then its probabilities.
    auto qk = [&](int r, f32x4 (&acc)[2]) {
      acc[0] = acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < DS; ++st)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) acc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[kt][st], qf[r][st], acc[kt], 0, 0, 0);
    };
    auto probs = [&](int r, const float (&e)[8]) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) pprev[r][jj] = (__bf16)exp2_fast(e[jj]);
    };
    if (j == 0 || tail) {
      // rows without a reference yet take this block's largest visible
      // score; keys a row does not see get no weight
      auto masked = [&](int r, int jj) {
        const int key = kb + 16 * (jj >> 2) + 4 * lg + (jj & 3);
        return key >= Ltot || key > lim[r];
      };
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        f32x4 acc[2];
        qk(r, acc);
        float t[8], mx = neg_inf_f();
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          t[jj] = masked(r, jj) ? neg_inf_f() : acc[jj >> 2][jj & 3] * skc[jj];
          mx = fmaxf(mx, t[jj]);
        }
        mx = group_max(mx);
        if (mref[r] == neg_inf_f()) mref[r] = mx;
        const float mr = mref[r] == neg_inf_f() ? 0.f : mref[r];  // such a row sees no key here
        float e[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) e[jj] = t[jj] - mr;
        probs(r, e);
      }
    } else {
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        f32x4 acc[2];
        qk(r, acc);
        float e[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) e[jj] = fmaf(acc[jj >> 2][jj & 3], skc[jj], -mref[r]);
        probs(r, e);
      }
    }
  };

  read_stage(R, IC<0>{});
  for (int j = 0; j < nblk; j += NST) {
    step(j, IC<0>{});
    if (j + 1 < nblk) step(j + 1, IC<1>{});
    if constexpr (NST > 2) {
      if (j + 2 < nblk) step(j + 2, IC<2>{});
    }
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) pv_tile(dt);  // the last block's PV
  // The copies still in flight (the last block again) land before the stages
  // serve another piece.
  wait_vmcnt<0>();
  float lt[RT];
  bool over = qbad_any;
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    lt[r] = lacc[r][0];
    over |= !(lt[r] <= 18446744073709551616.f);  // 2^64
  }
  if (__ballot(over)) {
    if (lane == 0) a.ovf[bg * a.RG + rg] = 1u;
    return false;
  }

#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int m = rg * ROWS + 16 * r + lr;
    if (whole) {
      if (m < a.M) {
        uint16_t* o = static_cast<uint16_t*>(a.out) + (((size_t)b * a.Hq + g * a.G + m / a.n_q) * a.n_q + m % a.n_q) * D;
        const float inv = 1.f / lt[r];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int d = 16 * dt + 4 * lg;
          uint2 pk;
          pk.x = uint32_t(f32_to_bf16(oacc[r][dt][0] * inv)) | (uint32_t(f32_to_bf16(oacc[r][dt][1] * inv)) << 16);
          pk.y = uint32_t(f32_to_bf16(oacc[r][dt][2] * inv)) | (uint32_t(f32_to_bf16(oacc[r][dt][3] * inv)) << 16);
          *reinterpret_cast<uint2*>(o + d) = pk;
        }
      }
    } else {
      const int row = 16 * r + lr;
      float* po = a.part_o + slot * ROWS * D;
      if constexpr (MERGE) {
        if (lg == 0) co_store2(reinterpret_cast<float*>(a.part_ml + slot * ROWS + row), mref[r], lt[r]);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          float* pd = po + (size_t)row * D + 16 * dt + 4 * lg;
          co_store2(pd, oacc[r][dt][0], oacc[r][dt][1]);
          co_store2(pd + 2, oacc[r][dt][2], oacc[r][dt][3]);
        }
      } else {
        if (lg == 0) a.part_ml[slot * ROWS + row] = ML{mref[r], lt[r]};
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(po + (size_t)row * D + 16 * dt + 4 * lg) = oacc[r][dt];
      }
    }
  }
  return true;
}

// MERGE: the pieces of a slab are merged by the last of its workgroups
// (stream_merge, as in the bf16 kernel); a piece that leaves its slab to the
// exact path does not count itself, so that slab is never merged here.
template <int D, int RT, bool MERGE>
__global__ __launch_bounds__(64) void attn_stream_i8w(AttnArgs a) {
  constexpr int T = KB * D;
  __shared__ __attribute__((aligned(1024))) int8_t stg[I8W_STAGES][2 * T];  // K tile, V tile
  __shared__ __attribute__((aligned(16))) uint16_t ssc[I8W_STAGES][64];      // 32 K, 32 V scales
  __shared__ __attribute__((aligned(1024))) uint16_t vt[KB * D];
  // The bf16 tile starts as zeros: the first block of every piece issues a PV
  // of zero probabilities against it.
  for (int i = threadIdx.x; i < KB * D / 8; i += kWave) reinterpret_cast<uint4*>(vt)[i] = make_uint4(0, 0, 0, 0);
  auto kst = [&](auto S) -> int8_t* { return stg[decltype(S)::value]; };
  auto vst = [&](auto S) -> int8_t* { return stg[decltype(S)::value] + T; };
  auto sst = [&](auto S) -> uint16_t* { return ssc[decltype(S)::value]; };
  stream_walk(a, [&](int b, int g, int rg, int L, int k0, int k1, bool whole, size_t slot, bool append, int np) {
    const bool counted = i8w_piece<D, RT, MERGE>(a, kst, vst, sst, vt, b, g, rg, L, k0, k1, whole, slot, append);
    if constexpr (MERGE) {
      if (!whole && counted) stream_merge<D, 16 * RT, kWave, false>(a, b, g, rg, slot, np);
    }
  });
}

// Merge the pieces of each (b, g, rg) slab the stream kernel cut; one
// workgroup per slab.  Slabs covered whole were written by the stream kernel.
template <int D, bool F16 = false>
__device__ __forceinline__ void combine_stream_slab(const AttnArgs& a, long slab, int chunk, int nchunk) {
  using H = Half16<F16>;
  const int rg = (int)(slab % a.RG);
  const int g = (int)((slab / a.RG) % a.Hkv);
  const int b = (int)(slab / ((long)a.RG * a.Hkv));
  const int rows = 16 * a.RT;
  const int row0 = rg * rows;
  const int nrows = min(rows, a.M - row0);
  uint16_t* out = static_cast<uint16_t*>(a.out);
  auto out_ptr = [&](int row) {
    const int m = row0 + row;
    return out + (((size_t)b * a.Hq + g * a.G + m / a.n_q) * a.n_q + m % a.n_q) * D;
  };
  const int nbb = slab_blocks(a, b);
  if (nbb == 0) {  // rejected length: NaN rows, nothing else touched
    for (int e = chunk * blockDim.x + threadIdx.x; e < nrows * D; e += nchunk * blockDim.x) out_ptr(e / D)[e % D] = H::kNaN;
    return;
  }
  const int HR = a.Hkv * a.RG;
  const long long share = stream_share(a, (long long)HR * a.pre[a.B]);
  const long long S0 = (long long)HR * a.pre[b] + (long long)(g * a.RG + rg) * nbb;
  const long long w0 = S0 / share, w1 = (S0 + nbb - 1) / share;
  if (w0 == w1) return;
  const int np = (int)min(w1 - w0 + 1, (long long)a.JP);
  const size_t base = (size_t)slab * a.JP;
  constexpr int D4 = D / 4;
  for (int e = chunk * blockDim.x + threadIdx.x; e < nrows * D4; e += nchunk * blockDim.x) {
    const int row = e / D4, d = 4 * (e % D4);
    // Online merge, four pieces at a time with all their loads in flight
    // (the piece count is only known at run time).
    float mx = neg_inf_f(), den = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    bool flagged = false;  // a piece that met a bad page entry left m = NaN
    for (int j0 = 0; j0 < np; j0 += 4) {
      ML ml[4];
      f32x4 po[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bool in = j0 + t < np;
        const size_t pj = (base + j0 + t) * rows + row;
        ml[t] = in ? a.part_ml[pj] : ML{neg_inf_f(), 0.f};
        po[t] = in ? *reinterpret_cast<const f32x4*>(a.part_o + pj * D + d) : f32x4{0.f, 0.f, 0.f, 0.f};
        flagged |= ml[t].m != ml[t].m;
      }
      // fmaxf drops NaN: the flag above, not the maxima, carries it
      const float mc = fmaxf(fmaxf(ml[0].m, ml[1].m), fmaxf(ml[2].m, ml[3].m));
      const float mn = fmaxf(mx, mc);
      if (mn == neg_inf_f()) continue;  // no visible key in these pieces yet
      const float r = exp2_fast(mx - mn);
      den *= r;
      acc *= r;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float w = exp2_fast(ml[t].m - mn);
        den += w * ml[t].l;
        acc += w * po[t];
      }
      mx = mn;
    }
    acc *= flagged ? __builtin_nanf("") : 1.f / den;
    uint2 pk;
    pk.x = uint32_t(H::bits(acc[0])) | (uint32_t(H::bits(acc[1])) << 16);
    pk.y = uint32_t(H::bits(acc[2])) | (uint32_t(H::bits(acc[3])) << 16);
    *reinterpret_cast<uint2*>(out_ptr(row) + d) = pk;
  }
}

// Workgroups of the combine launches per slab: one output item (4 values of
// a row) per thread, so each thread's loads are in flight at once.
template <int D>
__host__ __device__ constexpr int combine_chunks(int RT) {
  return (16 * RT * (D / 4) + 255) / 256;
}

template <int D, bool F16 = false>
__global__ __launch_bounds__(256) void attn_combine_stream(AttnArgs a) {
  const int nchunk = combine_chunks<D>(a.RT);
  combine_stream_slab<D, F16>(a, blockIdx.x / nchunk, (int)(blockIdx.x % nchunk), nchunk);
}

// The exact path of the int8 call for a slab its stream pieces gave up on (a
// probability term beyond the wave kernel's headroom): the plain online
// softmax -- running maximum, sums rescaled whenever it grows -- over the
// dequantised keys, fp32 throughout, two threads per row (each one half of
// the output's D values; both compute every score).  Slow, and only run for
// scores that grow by more than 64 / (scale log2 e) along a row.
template <int D>
__device__ void i8_slab_exact(const AttnArgs& a, long slab) {
  const int rg = (int)(slab % a.RG);
  const int g = (int)((slab / a.RG) % a.Hkv);
  const int b = (int)(slab / ((long)a.RG * a.Hkv));
  const int rows = 16 * a.RT, row0 = rg * rows, nrows = min(rows, a.M - row0);
  const int row = threadIdx.x >> 1, half = threadIdx.x & 1;
  if (row >= nrows) return;
  constexpr int DH = D / 2;
  const int m = row0 + row, h = g * a.G + m / a.n_q, qi = m % a.n_q;
  const long bg = (long)b * a.Hkv + g;
  const int L = a.len[b];
  const uint16_t* q = static_cast<const uint16_t*>(a.q) + (((size_t)b * a.Hq + h) * a.n_q + qi) * D;
  const int8_t* kc = static_cast<const int8_t*>(a.kc) + (size_t)bg * a.max_T * D;
  const int8_t* vc = static_cast<const int8_t*>(a.vc) + (size_t)bg * a.max_T * D;
  const int8_t* knb = a.nkq + (size_t)bg * a.n_q * D;
  const int8_t* vnb = a.nvq + (size_t)bg * a.n_q * D;
  float acc[DH];
#pragma unroll
  for (int d = 0; d < DH; ++d) acc[d] = 0.f;
  float mx = neg_inf_f(), l = 0.f;
  for (int j = 0; j <= L + qi; ++j) {  // the keys this row sees
    const bool cached = j < L;
    const int8_t* kr = cached ? kc + (size_t)j * D : knb + (size_t)(j - L) * D;
    const int8_t* vr = (cached ? vc + (size_t)j * D : vnb + (size_t)(j - L) * D) + half * DH;
    const float sk = f16_to_f32(cached ? a.ksc[bg * a.max_T + j] : a.nks[bg * a.n_q + (j - L)]);
    const float sv = f16_to_f32(cached ? a.vsc[bg * a.max_T + j] : a.nvs[bg * a.n_q + (j - L)]);
    float dot = 0.f;
    for (int d = 0; d < D; ++d) dot = fmaf(bf16_to_f32(q[d]), (float)kr[d], dot);
    const float sc = dot * sk * a.qk_scale;  // log2 units
    const float mn = fmaxf(mx, sc);
    const float r = exp2_fast(mx - mn);  // 0 for the first key
    const float p = exp2_fast(sc - mn);
    l = fmaf(l, r, p);
#pragma unroll
    for (int d = 0; d < DH; ++d) acc[d] = fmaf(acc[d], r, p * sv * (float)vr[d]);
    mx = mn;
  }
  uint16_t* o = static_cast<uint16_t*>(a.out) + (((size_t)b * a.Hq + h) * a.n_q + qi) * D + half * DH;
  const float inv = 1.f / l;
#pragma unroll
  for (int d = 0; d < DH; ++d) o[d] = f32_to_bf16(acc[d] * inv);
}

// Combine launch of the int8 call: slabs marked by the wave kernel take the
// exact path, the others are merged as in the bf16 call.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_i8(AttnArgs a) {
  const int nchunk = combine_chunks<D>(a.RT);
  const long slab = blockIdx.x / nchunk;
  const int chunk = (int)(blockIdx.x % nchunk);
  if (a.ovf[slab] != 0u && slab_blocks(a, (int)(slab / ((long)a.RG * a.Hkv))) > 0) {
    if (chunk == 0) i8_slab_exact<D>(a, slab);  // the whole slab, by one workgroup
    return;
  }
  combine_stream_slab<D, false>(a, slab, chunk, nchunk);
}

// After a merging int8 stream launch: only the slabs marked for the exact
// path have work.
template <int D>
__global__ __launch_bounds__(256) void attn_exact_i8(AttnArgs a) {
  const long slab = blockIdx.x;
  if (a.ovf[slab] != 0u && slab_blocks(a, (int)(slab / ((long)a.RG * a.Hkv))) > 0) i8_slab_exact<D>(a, slab);
}

// ---------------------------------------------------------------------------
// fp32 kernel: one wave per split of C keys holding RT row tiles.
//   NWK = 0: one wave per workgroup and item; its state goes to the partial
//            slots and attn_combine merges the splits.
//   NWK > 0: one workgroup per (b, g, rg) whose wave w takes split w (at most
//            NWK splits); the waves' states are merged through LDS and the
//            workgroup writes the output itself.
// ---------------------------------------------------------------------------

// Blocks of K/V held per wave (one computed, the rest in flight): three at
// the small head dimensions, where a block takes 28 registers, else two.
constexpr int kF32RingSmallD = 3;  // blocks per wave at D <= 32
template <int D>
constexpr int kF32Ring = D <= 32 ? kF32RingSmallD : 2;

// LDS of the in-workgroup merge: every wave's O rows and (max, sum).
template <int D, int RT, int NWK>
constexpr size_t f32_merge_lds() {
  return (size_t)NWK * 16 * RT * (D * sizeof(float) + sizeof(ML));
}

template <int D, int RT, int NWK>
__global__ __launch_bounds__(64 * (NWK > 0 ? NWK : 1)) void attn_split_f32(AttnArgs a) {
  constexpr bool kWG = NWK > 0;
  constexpr int DS = D / 4;
  constexpr int DT = (D + 15) / 16;
  const int lane = threadIdx.x & (kWave - 1);
  const int lr = lane & 15;
  const int lg = lane >> 4;
  Item it;
  if constexpr (kWG) {
    long item = blockIdx.x;
    it.rg = (int)(item % a.RG);
    item /= a.RG;
    it.g = (int)(item % a.Hkv);
    it.b = (int)(item / a.Hkv);
    it.bg = (long)it.b * a.Hkv + it.g;
    it.sp = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    it.id = 0;
  } else {
    it = decode_item(a);
  }
  const int L = a.len[it.b];
  const bool bad = L < 0 || L > a.hint;
  if (!kWG && bad) return;
  const int Ltot = L + a.n_q;
  const int k0 = it.sp * a.C;
  if (!kWG && k0 >= Ltot) return;
  // an idle wave of a workgroup (bad length, or no keys in its split) runs
  // no blocks and merges as an empty state
  const int k1 = (bad || k0 >= Ltot) ? k0 : min(k0 + a.C, Ltot);
  const float* q = static_cast<const float*>(a.q);
  const float* kn = static_cast<const float*>(a.kn);
  const float* vn = static_cast<const float*>(a.vn);
  const float* kc = static_cast<const float*>(a.kc);
  const float* vc = static_cast<const float*>(a.vc);

  if (!bad && it.sp == 0 && it.rg == 0) append_rows<float, D>(a, it.bg, L, lane, kWave);

  float qf[RT][DS];
  int lim[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int m = it.rg * 16 * RT + 16 * r + lr;
    const bool valid = m < a.M;
    const int h = it.g * a.G + (valid ? m / a.n_q : 0);
    const int i = valid ? m % a.n_q : a.n_q - 1;
    lim[r] = L + i;
    const float* qrow = q + (((size_t)it.b * a.Hq + h) * a.n_q + i) * D;
#pragma unroll
    for (int s = 0; s < DS; ++s) qf[r][s] = valid ? qrow[4 * s + lg] : 0.f;
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

  // The K and V values of the block this lane feeds to the products: K as
  // [kt][s] (key kb + 16 kt + lr, dims 4 s + lg), V as [4 kt + jj][dt] (key
  // kb + 16 kt + 4 lg + jj, dim 16 dt + lr).  The next block's are loaded
  // before the current block's products, so one block's loads are in flight
  // during the other's arithmetic.
  auto load_kv = [&](int kb, float (&kf)[2][DS], float (&vf)[8][DT]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const float* row = key_row<float>(kc, kn, kb + 16 * kt + lr, L, Ltot, a.n_q, a.max_T, D, it.bg);
#pragma unroll
      for (int s = 0; s < DS; ++s) kf[kt][s] = row ? row[4 * s + lg] : 0.f;
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float* row = key_row<float>(vc, vn, kb + 16 * kt + 4 * lg + jj, L, Ltot, a.n_q, a.max_T, D, it.bg);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int d = 16 * dt + lr;
          vf[4 * kt + jj][dt] = (row && d < D) ? row[d] : 0.f;
        }
      }
  };
  // Block j's products, from ring slot kf/vf.
  auto block = [&](int kb, const float (&kf)[2][DS], const float (&vf)[8][DT]) {
    float sc[RT][8];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < DS; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[kt][s], qf[r][s], c, 0, 0, 0);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sc[r][4 * kt + jj] = c[jj] * a.qk_scale;
      }
    if (kb + KB > L) {
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int key = kb + 16 * kt + 4 * lg + jj;
            if (key >= Ltot || key > lim[r]) sc[r][4 * kt + jj] = neg_inf_f();
          }
    }
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const float alpha = softmax_update(sc[r], mrow[r], lsum[r]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[r][dt] *= alpha;
    }
    // One key per lane per MFMA: lane group lg supplies key kb + 16 kt + 4 lg + jj.
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < RT; ++r)
            oacc[r][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf[4 * kt + jj][dt], sc[r][4 * kt + jj], oacc[r][dt],
                                                               0, 0, 0);
  };
  // A ring of NR blocks: block j + NR - 1 is loaded into the slot block j - 1
  // used before block j is computed, so NR - 1 blocks are in flight during
  // the products (the ring index is a compile-time constant).
  constexpr int NR = kF32Ring<D>;
  float kf[NR][2][DS], vf[NR][8][DT];
  const int nblk = (k1 - k0 + KB - 1) / KB;
#pragma unroll
  for (int q = 0; q < NR - 1; ++q)
    if (q < nblk) load_kv(k0 + q * KB, kf[q], vf[q]);
  for (int j0 = 0; j0 < nblk; j0 += NR) {
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      const int j = j0 + q;
      if (j < nblk) {  // uniform
        const int nxt = (q + NR - 1) % NR;  // constant once the q loop is unrolled
        if (j + NR - 1 < nblk) load_kv(k0 + (j + NR - 1) * KB, kf[nxt], vf[nxt]);
        block(k0 + j * KB, kf[q], vf[q]);
      }
    }
  }

  constexpr int ROWS = 16 * RT;
  float* po;
  ML* pml;
  if constexpr (kWG) {
    __shared__ __attribute__((aligned(16))) char merge_lds[f32_merge_lds<D, RT, NWK>()];
    po = reinterpret_cast<float*>(merge_lds) + (size_t)it.sp * ROWS * D;
    pml = reinterpret_cast<ML*>(merge_lds + (size_t)NWK * ROWS * D * sizeof(float)) + it.sp * ROWS;
  } else {
    po = a.part_o + it.id * ROWS * D;
    pml = a.part_ml + it.id * ROWS;
  }
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
  if constexpr (kWG) {
    __syncthreads();
    // merge the NWK states of each row (weights 2^(m_w - max)) and write out
    const float* so = po - (size_t)it.sp * ROWS * D;
    const ML* sml = pml - it.sp * ROWS;
    const int row0 = it.rg * ROWS;
    const int nrows = min(ROWS, a.M - row0);
    float* out = static_cast<float*>(a.out);
    auto out_ptr = [&](int row) {
      const int m = row0 + row;
      return out + (((size_t)it.b * a.Hq + it.g * a.G + m / a.n_q) * a.n_q + m % a.n_q) * D;
    };
    if (bad) {  // NaN rows, nothing else touched
      for (int e = threadIdx.x; e < nrows * D; e += blockDim.x) out_ptr(e / D)[e % D] = __builtin_nanf("");
      return;
    }
    constexpr int D4 = D / 4;
    for (int e = threadIdx.x; e < nrows * D4; e += blockDim.x) {
      const int row = e / D4, d = 4 * (e % D4);
      float mx = neg_inf_f();
#pragma unroll
      for (int w = 0; w < NWK; ++w) mx = fmaxf(mx, sml[w * ROWS + row].m);
      float den = 0.f;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < NWK; ++w) {
        const ML ml = sml[w * ROWS + row];
        const float wt = exp2_fast(ml.m - mx);
        den += wt * ml.l;
        acc += wt * *reinterpret_cast<const f32x4*>(so + ((size_t)w * ROWS + row) * D + d);
      }
      acc *= 1.f / den;
      *reinterpret_cast<f32x4*>(out_ptr(row) + d) = acc;
    }
  }
}

// ---------------------------------------------------------------------------
// combine: merge the splits of (b, g, rg) and write out[b][h][i][:]
// ---------------------------------------------------------------------------

template <typename T, int D>
__global__ __launch_bounds__(256) void attn_combine(AttnArgs a, int skip_single) {
  const Item it = [&] {
    long item = blockIdx.x;
    Item x;
    x.rg = (int)(item % a.RG);
    item /= a.RG;
    x.g = (int)(item % a.Hkv);
    x.b = (int)(item / a.Hkv);
    x.bg = (long)x.b * a.Hkv + x.g;
    x.sp = 0;
    return x;
  }();
  const int rows = 16 * a.RT;
  const int row0 = it.rg * rows;
  const int nrows = min(rows, a.M - row0);
  const int L = a.len[it.b];
  T* out = static_cast<T*>(a.out);
  auto out_ptr = [&](int row) {
    const int m = row0 + row;
    return out + (((size_t)it.b * a.Hq + it.g * a.G + m / a.n_q) * a.n_q + m % a.n_q) * D;
  };
  constexpr int D4 = D / 4;
  if (L < 0 || L > a.hint) {  // invalid length: NaN rows, nothing else touched
    for (int e = threadIdx.x; e < nrows * D; e += blockDim.x) {
      if constexpr (sizeof(T) == 2)
        out_ptr(e / D)[e % D] = (T)0x7fc0;
      else
        out_ptr(e / D)[e % D] = __builtin_nanf("");
    }
    return;
  }
  const int nsp = (L + a.n_q + a.C - 1) / a.C;
  if (skip_single && nsp == 1) return;  // written by the split kernel
  const size_t base = (((size_t)it.b * a.Hkv + it.g) * a.RG + it.rg) * a.NSP;  // item of split 0
  for (int e = threadIdx.x; e < nrows * D4; e += blockDim.x) {
    const int row = e / D4, d = 4 * (e % D4);
    float mx = neg_inf_f();
    for (int sp = 0; sp < nsp; ++sp) mx = fmaxf(mx, a.part_ml[(base + sp) * rows + row].m);
    float den = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < nsp; ++sp) {
      const ML ml = a.part_ml[(base + sp) * rows + row];
      const float w = exp2_fast(ml.m - mx);
      den += w * ml.l;
      acc += w * *reinterpret_cast<const f32x4*>(a.part_o + ((base + sp) * rows + row) * D + d);
    }
    acc *= 1.f / den;
    T* o = out_ptr(row) + d;
    if constexpr (sizeof(T) == 2) {
      uint2 pk;
      pk.x = uint32_t(f32_to_bf16(acc[0])) | (uint32_t(f32_to_bf16(acc[1])) << 16);
      pk.y = uint32_t(f32_to_bf16(acc[2])) | (uint32_t(f32_to_bf16(acc[3])) << 16);
      *reinterpret_cast<uint2*>(o) = pk;
    } else {
      *reinterpret_cast<f32x4*>(o) = acc;
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

static inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct SplitPolicy {
  int cmin, cmax;  // split length: a power of two in [cmin, cmax]
  long target;     // aim for about this many work items
};

constexpr int kSplitItems16 = 2048;   // bf16 fixed splits: aim for this many items
constexpr int kSplitCmax16 = 8192;    // bf16: longest split
constexpr int kSplitItemsF32 = 8192;  // fp32: aim for this many items
constexpr int kSplitCminF32 = 128;    // fp32: shortest split

static SplitPolicy policy(spec_dtype_t dt) {
  // bf16: workgroups of one wave per row tile, a few resident per CU; fp32:
  // single-wave items.
  return dt != SPEC_F32 ? SplitPolicy{256, kSplitCmax16, kSplitItems16}
                         : SplitPolicy{kSplitCminF32, 4096, kSplitItemsF32};
}

static int max_rt(spec_dtype_t dt, int D) {
  if (dt != SPEC_F32) return 8;  // waves per workgroup
  return D <= 32 ? 4 : (D <= 64 ? 2 : 1);
}

static bool supported(spec_dtype_t dt, int D) {
  if (dt == SPEC_BF16 || dt == SPEC_F16) return D == 64 || D == 128;
  if (dt == SPEC_F32) return D == 24 || D == 32 || D == 64 || D == 128;
  return false;
}

struct AttnPlan {
  int RT, RG, C, NSP;
  size_t off_o, off_ml, total;
};

static AttnPlan attn_plan(int B, int Hq, int Hkv, int n_q, int D, int hint, spec_dtype_t dt) {
  AttnPlan p{};
  const int M = (Hq / Hkv) * n_q;
  const int tiles = (M + 15) / 16;
  p.RG = (tiles + max_rt(dt, D) - 1) / max_rt(dt, D);
  p.RT = (tiles + p.RG - 1) / p.RG;
  const SplitPolicy sp = policy(dt);
  const long keys = (long)B * Hkv * p.RG * (long)(hint + n_q);
  const long want = (keys + sp.target - 1) / sp.target;
  int C = sp.cmin;
  while (C < want && C < sp.cmax) C <<= 1;
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

// Two stages measured faster than three with non-temporal loads (4.6%,
// 32K-key caches), and halve the LDS.
constexpr int kStages = 2;  // LDS stages; blocks in flight per workgroup: kStages - 1

// ---- stream scheme ---------------------------------------------------------

// Upper bound on the workgroups of a stream launch: 256 CUs, at most 3
// resident workgroups each (LDS).  The partial slots per slab follow from it,
// so the workspace size does not depend on the device.
// Workgroups per CU of the bf16 stream kernel.  Its 2-wave build fits 3 per
// CU but ran faster at 2 (fewer, longer shares: 78 -> 75 us at B = 32 with
// 1-4K-key caches; 1 and 1.5 per CU were slower everywhere).  The int8
// kernel keeps 3 (87 us against 109 us at 2).
constexpr int kStreamMaxWG = 768;
// The int8 kernel runs one-wave workgroups, one or two per SIMD.
constexpr int kStreamMaxWG8 = 2048;
constexpr int kMergeMinShare = 256;  // blocks per workgroup from which the launch merges pieces
constexpr int kBf16PerCU = 2;        // resident 16-bit stream workgroups per CU

// Sizes the stream scheme handles: every workgroup scans the B lengths, and
// block counts stay in int.
static bool stream_ok(spec_dtype_t dt, int B, int Hkv, int RG, int n_q, int hint) {
  const long nbmax = ((long)hint + n_q + KB - 1) / KB;
  return (dt == SPEC_BF16 || dt == SPEC_F16) && B <= 1024 && (long)Hkv * RG * B * nbmax < (1L << 30);
}

struct StreamPlan {
  int JP, MINB;
  size_t off_o, off_ml, off_pre, off_cnt, total;
};

static StreamPlan stream_plan(int B, int Hkv, int RG, int RT, int n_q, int D, int hint, int maxwg = kStreamMaxWG) {
  StreamPlan p{};
  const long slabs = (long)B * Hkv * RG;
  // With shares of at least MINB = ceil(nbmax / jcap) blocks a slab is cut
  // into at most jcap + 1 pieces.  jcap is large enough that MINB stays below
  // the even share W / P (P <= maxwg) unless most lengths are far below the hint.
  const long jcap = std::max(2L, 2 * ((maxwg + slabs - 1) / slabs) + 2);
  const long nbmax = ((long)hint + n_q + KB - 1) / KB;
  p.JP = (int)(jcap + 1);
  p.MINB = (int)std::max(1L, (nbmax + jcap - 1) / jcap);
  const size_t slots = (size_t)slabs * p.JP;
  size_t off = 0;
  p.off_o = off;
  off = align256(off + sizeof(float) * slots * 16 * RT * D);
  p.off_ml = off;
  off = align256(off + sizeof(ML) * slots * 16 * RT);
  p.off_pre = off;
  off = align256(off + sizeof(int) * ((size_t)B + 1));
  p.off_cnt = off;
  off = align256(off + sizeof(uint32_t) * (size_t)slabs);
  p.total = off;
  return p;
}

// Workgroups of a stream launch on the current device: CUs x resident
// workgroups per CU.  Residency is the occupancy query's answer, further
// limited because the waves of a workgroup are spread round-robin over the 4
// SIMDs of a CU: a workgroup of NW waves puts ceil(NW / 4) on one SIMD, which
// holds 512 / VGPRs waves.  Cached per kernel (the template argument) and
// device.
template <auto kernel>
static int stream_workgroups(int NW, int max_per_cu, int maxwg = kStreamMaxWG) {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  std::atomic<int>* slot = dev < 64 ? &cache[dev] : nullptr;
  if (slot && slot->load(std::memory_order_relaxed) > 0) return slot->load(std::memory_order_relaxed);
  int cus = 0, occ = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(kernel), 64 * NW, 0) !=
          hipSuccess ||
      occ < 1)
    occ = 1;
  hipFuncAttributes fa{};
  int per_simd = 4;
  if (hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(kernel)) == hipSuccess && fa.numRegs > 0)
    per_simd = 512 / ((fa.numRegs + 7) / 8 * 8);
  // Up to 4 waves a workgroup takes one slot on each of NW SIMDs; a larger
  // one takes ceil(NW / 4) slots on every SIMD, and never more than 2 fit
  // (measured: 5-, 6- and 8-wave workgroups fit 2 per CU whatever their
  // registers and LDS; a build that used fewer registers and launched 3 per
  // CU left a third of them waiting for a slot).
  const int by_slots = NW <= 4 ? 4 * per_simd / NW : std::min(2, per_simd / ((NW + 3) / 4));
  int k = std::max(1, std::min(std::min(occ, by_slots), max_per_cu));
  const int P = std::min(maxwg, cus * k);
  if (slot) slot->store(P, std::memory_order_relaxed);
  return P;
}

template <int D, int NW, int PG, bool kMerge, bool F16>
static hipError_t launch_stream_as(const AttnArgs& a0, hipStream_t s) {
  AttnArgs a = a0;
  const size_t slabs = (size_t)a.B * a.Hkv * a.RG;
  if constexpr (kMerge) {
    hipLaunchKernelGGL((attn_stream_prep<D, F16>), dim3((unsigned)std::min<size_t>((slabs + 255) / 256, 1024)),
                       dim3(256), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  a.P = stream_workgroups<attn_stream_bf16<D, NW, kStages, PG, kMerge, F16>>(NW, kBf16PerCU);
  hipLaunchKernelGGL((attn_stream_bf16<D, NW, kStages, PG, kMerge, F16>), dim3((unsigned)a.P), dim3(64 * NW), 0, s,
                     a, a.table);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || kMerge) return e;
  hipLaunchKernelGGL((attn_combine_stream<D, F16>), dim3((unsigned)(slabs * combine_chunks<D>(a.RT))), dim3(256), 0, s, a);
  return hipGetLastError();
}

// The in-launch merge costs every workgroup a few microseconds per piece
// (the write-through partials, the count, the last one's merge) and the
// counters a launch of their own; the combine launch costs a fixed time that
// grows with the slab count.  Merge when a workgroup's share can reach
// kMergeMinShare blocks (measured: 32K-key caches, B = 256: 3.36 ->
// 3.32 ms; 1-4K-key caches, B = 32: 74 -> 87 us, so those combine).
template <int D, int NW, int PG, bool F16 = false>
static hipError_t launch_stream(const AttnArgs& a, hipStream_t s) {
  const long nbmax = ((long)a.hint + a.n_q + KB - 1) / KB;
  const long wmax = (long)a.B * a.Hkv * a.RG * nbmax;
  const int P = stream_workgroups<attn_stream_bf16<D, NW, kStages, PG, true, F16>>(NW, kBf16PerCU);
  if (wmax >= (long)kMergeMinShare * P) return launch_stream_as<D, NW, PG, true, F16>(a, s);
  return launch_stream_as<D, NW, PG, false, F16>(a, s);
}

// As for bf16, shares of kMergeMinShare blocks or more merge their pieces in
// the stream launch (a small prep launch zeroes the counters and writes the
// NaN rows of rejected lengths; the exact-path launch after it has work only
// for marked slabs); shorter ones keep the combine launch.
template <int D, int RT>
static hipError_t launch_i8(const AttnArgs& a0, hipStream_t s) {
  AttnArgs a = a0;
  const size_t slabs = (size_t)a.B * a.Hkv * a.RG;
  hipLaunchKernelGGL((quant_new_rows<D>), dim3((unsigned)((size_t)a.B * a.Hkv)), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long nbmax = ((long)a.hint + a.n_q + KB - 1) / KB;
  const int Pm = stream_workgroups<attn_stream_i8w<D, RT, true>>(1, 8, kStreamMaxWG8);
  if ((long)slabs * nbmax >= (long)kMergeMinShare * Pm) {
    a.P = Pm;
    hipLaunchKernelGGL((attn_stream_prep<D, false>), dim3((unsigned)std::min<size_t>((slabs + 255) / 256, 1024)),
                       dim3(256), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_stream_i8w<D, RT, true>), dim3((unsigned)a.P), dim3(64), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_exact_i8<D>), dim3((unsigned)slabs), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  a.P = stream_workgroups<attn_stream_i8w<D, RT, false>>(1, 8, kStreamMaxWG8);
  hipLaunchKernelGGL((attn_stream_i8w<D, RT, false>), dim3((unsigned)a.P), dim3(64), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_combine_i8<D>), dim3((unsigned)((size_t)a.B * a.Hkv * a.RG * combine_chunks<D>(a.RT))),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_i8_d(const AttnArgs& a, hipStream_t s) {
  switch (a.RT) {
    case 1: return launch_i8<D, 1>(a, s);
    case 2: return launch_i8<D, 2>(a, s);
    case 3: return launch_i8<D, 3>(a, s);
    case 4: return launch_i8<D, 4>(a, s);
    case 5: return launch_i8<D, 5>(a, s);
    case 6: return launch_i8<D, 6>(a, s);
    case 7: return launch_i8<D, 7>(a, s);
    case 8: return launch_i8<D, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// F16: IEEE-half elements, stream scheme only.
template <int D, int NW, bool F16 = false>
static hipError_t launch_bf16(const AttnArgs& a0, hipStream_t s) {
  if constexpr (F16) {
    if (!a0.pre) return hipErrorInvalidValue;  // rejected on the host before
    if (a0.table) return a0.page == 16 ? launch_stream<D, NW, 16, true>(a0, s) : launch_stream<D, NW, 32, true>(a0, s);
    return launch_stream<D, NW, 0, true>(a0, s);
  }
  if (a0.pre) {  // stream scheme
    if (a0.table) return a0.page == 16 ? launch_stream<D, NW, 16>(a0, s) : launch_stream<D, NW, 32>(a0, s);
    return launch_stream<D, NW, 0>(a0, s);
  }
  const AttnArgs& a = a0;
  const size_t items = (size_t)a.B * a.Hkv * a.RG * a.NSP;
  hipLaunchKernelGGL((attn_split_bf16<D, NW, kStages>), dim3((unsigned)items), dim3(64 * NW), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_combine<uint16_t, D>), dim3((unsigned)((size_t)a.B * a.Hkv * a.RG)), dim3(256), 0, s, a, 1);
  return hipGetLastError();
}

template <int D, bool F16 = false>
static hipError_t launch_bf16_d(const AttnArgs& a, hipStream_t s) {
  switch (a.RT) {
    case 1: return launch_bf16<D, 1, F16>(a, s);
    case 2: return launch_bf16<D, 2, F16>(a, s);
    case 3: return launch_bf16<D, 3, F16>(a, s);
    case 4: return launch_bf16<D, 4, F16>(a, s);
    case 5: return launch_bf16<D, 5, F16>(a, s);
    case 6: return launch_bf16<D, 6, F16>(a, s);
    case 7: return launch_bf16<D, 7, F16>(a, s);
    case 8: return launch_bf16<D, 8, F16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D, int RT, int NWK>
static hipError_t launch_f32_wg(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((attn_split_f32<D, RT, NWK>), dim3((unsigned)((size_t)a.B * a.Hkv * a.RG)), dim3(64 * NWK), 0, s,
                     a);
  return hipGetLastError();
}

// Up to 8 splits per (b, g, rg) run as the waves of one workgroup, merged in
// LDS (no partials in HBM, no second launch); more go through attn_combine.
template <int D, int RT>
static hipError_t launch_f32(const AttnArgs& a, hipStream_t s) {
  constexpr size_t kMaxLds = 48 * 1024;
  if (a.NSP <= 1) return launch_f32_wg<D, RT, 1>(a, s);
  if (a.NSP <= 2) return launch_f32_wg<D, RT, 2>(a, s);
  if (a.NSP <= 4) {
    if constexpr (f32_merge_lds<D, RT, 4>() <= kMaxLds) return launch_f32_wg<D, RT, 4>(a, s);
  } else if (a.NSP <= 8) {
    if constexpr (f32_merge_lds<D, RT, 8>() <= kMaxLds) return launch_f32_wg<D, RT, 8>(a, s);
  }
  const size_t items = (size_t)a.B * a.Hkv * a.RG * a.NSP;
  hipLaunchKernelGGL((attn_split_f32<D, RT, 0>), dim3((unsigned)items), dim3(64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_combine<float, D>), dim3((unsigned)((size_t)a.B * a.Hkv * a.RG)), dim3(256), 0, s, a, 0);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_f32_d(const AttnArgs& a, hipStream_t s) {
  switch (a.RT) {
    case 1: return launch_f32<D, 1>(a, s);
    case 2: return launch_f32<D, 2>(a, s);
    case 3: if constexpr (D <= 32) return launch_f32<D, 3>(a, s); else break;
    case 4: if constexpr (D <= 32) return launch_f32<D, 4>(a, s); else break;
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
  // length C(h') is a power of two in [cmin, cmax] no smaller than
  // K (h' + n_q) / target, so NSP(h') <= ceil(target / K) unless C is capped
  // at cmax, and NSP(h') <= ceil((h' + n_q) / cmin) always.  Both bounds grow
  // with the hint.
  const AttnPlan p = attn_plan(B, Hq, Hkv, n_q, D, max_len_hint, dtype);
  const SplitPolicy sp = policy(dtype);
  const long K = (long)B * Hkv * p.RG;
  const long span = (long)max_len_hint + n_q;
  long nsp = std::max((sp.target + K - 1) / K, (span + sp.cmax - 1) / sp.cmax);
  nsp = std::min(nsp, (span + sp.cmin - 1) / sp.cmin);
  nsp = std::max(nsp, (long)p.NSP);
  const size_t items = (size_t)K * nsp;
  const size_t split_bytes = align256(sizeof(float) * items * 16 * p.RT * D) + align256(sizeof(ML) * items * 16 * p.RT);
  // bf16 uses the stream scheme while stream_ok holds, which for a larger
  // hint can stop holding: cover both then.
  if (dtype == SPEC_F32 || B > 1024) return split_bytes;
  const size_t stream_bytes = stream_plan(B, Hkv, p.RG, p.RT, n_q, D, max_len_hint).total;
  if (stream_ok(dtype, B, Hkv, p.RG, n_q, max_len_hint)) return stream_bytes;
  return std::max(split_bytes, stream_bytes);
}

// Shared by the contiguous and the paged entry points.  Paged: table != null,
// k_cache / v_cache are the page arrays, max_T is unused.
static spec_status_t verify_attention(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                      void* v_cache, const int32_t* cache_len, void* out, int B, int Hq, int Hkv,
                                      int n_q, int D, int max_T, int max_len_hint, float scale, spec_dtype_t dtype,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream,
                                      const int32_t* table, int page, int num_pages, int max_blocks) {
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !cache_len || !out || !workspace) return SPEC_ERR_ARG;
  if (B < 1 || Hq < 1 || Hkv < 1 || n_q < 1 || D < 1 || max_T < 1 || max_len_hint < 0) return SPEC_ERR_ARG;
  if (Hq % Hkv != 0) return SPEC_ERR_ARG;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16 && dtype != SPEC_F16) return SPEC_ERR_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return SPEC_ERR_ARG;
  const uintptr_t al = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_new) |
                       reinterpret_cast<uintptr_t>(v_new) | reinterpret_cast<uintptr_t>(k_cache) |
                       reinterpret_cast<uintptr_t>(v_cache) | reinterpret_cast<uintptr_t>(out);
  if (al % 16 != 0 || reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return SPEC_ERR_ARG;
  if ((long)max_len_hint + n_q > (long)max_T) return SPEC_ERR_OVERFLOW;
  if (n_q > 16 || (Hq / Hkv) * n_q > 256 || !supported(dtype, D)) return SPEC_ERR_UNSUPPORTED;
  const AttnPlan p = attn_plan(B, Hq, Hkv, n_q, D, max_len_hint, dtype);
  const bool use_stream = stream_ok(dtype, B, Hkv, p.RG, n_q, max_len_hint);
  if (table && !use_stream) return SPEC_ERR_UNSUPPORTED;  // paged: bf16, B <= 1024
  if (dtype == SPEC_F16 && !use_stream) return SPEC_ERR_UNSUPPORTED;  // fp16: B <= 1024
  const StreamPlan sp = use_stream ? stream_plan(B, Hkv, p.RG, p.RT, n_q, D, max_len_hint) : StreamPlan{};
  if (workspace_bytes < (use_stream ? sp.total : p.total)) return SPEC_ERR_ARG;
  if ((size_t)B * Hkv * p.RG * p.NSP > 0x7fffffffu) return SPEC_ERR_UNSUPPORTED;

  AttnArgs a;
  a.q = q;
  a.kn = k_new;
  a.vn = v_new;
  a.kc = k_cache;
  a.vc = v_cache;
  a.len = cache_len;
  a.out = out;
  char* ws = static_cast<char*>(workspace);
  a.part_o = reinterpret_cast<float*>(ws + (use_stream ? sp.off_o : p.off_o));
  a.part_ml = reinterpret_cast<ML*>(ws + (use_stream ? sp.off_ml : p.off_ml));
  a.pre = use_stream ? reinterpret_cast<int*>(ws + sp.off_pre) : nullptr;
  a.scnt = use_stream ? reinterpret_cast<uint32_t*>(ws + sp.off_cnt) : nullptr;
  a.P = 0;
  a.MINB = sp.MINB;
  a.JP = sp.JP;
  a.table = table;
  a.page = page;
  a.max_blocks = max_blocks;
  a.num_pages = num_pages;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.n_q = n_q;
  a.G = Hq / Hkv;
  a.M = a.G * n_q;
  a.RG = p.RG;
  a.RT = p.RT;
  a.NSP = p.NSP;
  a.C = p.C;
  a.max_T = max_T;
  a.hint = max_len_hint;
  a.qk_scale = scale * 1.4426950408889634f;

  hipError_t e = hipErrorInvalidValue;
  if (dtype == SPEC_BF16) {
    if (D == 128) e = launch_bf16_d<128>(a, stream);
    else if (D == 64) e = launch_bf16_d<64>(a, stream);
  } else if (dtype == SPEC_F16) {
    if (D == 128) e = launch_bf16_d<128, true>(a, stream);
    else if (D == 64) e = launch_bf16_d<64, true>(a, stream);
  } else {
    if (D == 24) e = launch_f32_d<24>(a, stream);
    else if (D == 32) e = launch_f32_d<32>(a, stream);
    else if (D == 64) e = launch_f32_d<64>(a, stream);
    else if (D == 128) e = launch_f32_d<128>(a, stream);
  }
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_LAUNCH;
}

extern "C" spec_status_t spec_verify_attention(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                               void* v_cache, const int32_t* cache_len, void* out, int B, int Hq,
                                               int Hkv, int n_q, int D, int max_T, int max_len_hint, float scale,
                                               spec_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                               hipStream_t stream) {
  return verify_attention(q, k_new, v_new, k_cache, v_cache, cache_len, out, B, Hq, Hkv, n_q, D, max_T, max_len_hint,
                          scale, dtype, workspace, workspace_bytes, stream, nullptr, 0, 0, 0);
}

extern "C" spec_status_t spec_verify_attention_paged(const void* q, const void* k_new, const void* v_new,
                                                     void* k_pages, void* v_pages, const int32_t* block_table,
                                                     const int32_t* cache_len, void* out, int B, int Hq, int Hkv,
                                                     int n_q, int D, int page_size, int num_pages, int max_blocks,
                                                     int max_len_hint, float scale, spec_dtype_t dtype,
                                                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!block_table) return SPEC_ERR_ARG;
  if (page_size != 16 && page_size != 32) return SPEC_ERR_UNSUPPORTED;
  if (num_pages < 1 || max_blocks < 1) return SPEC_ERR_ARG;
  if (dtype != SPEC_BF16 && dtype != SPEC_F16) return SPEC_ERR_UNSUPPORTED;
  // The logical capacity of a sequence is max_blocks pages.
  const long cap = (long)max_blocks * page_size;
  if (cap > 0x7fffffffL) return SPEC_ERR_ARG;
  return verify_attention(q, k_new, v_new, k_pages, v_pages, cache_len, out, B, Hq, Hkv, n_q, D, (int)cap,
                          max_len_hint, scale, dtype, workspace, workspace_bytes, stream, block_table, page_size,
                          num_pages, max_blocks);
}

// ---- int8 cache entry points ------------------------------------------------

// Stream-scheme workspace followed by the quantised new rows (int8 K, int8 V,
// fp16 K scales, fp16 V scales) and the per-slab exact-path marks.
struct I8Plan {
  StreamPlan sp;
  size_t off_nkq, off_nvq, off_nks, off_nvs, off_ovf, total;
};

static I8Plan i8_plan(int B, int Hq, int Hkv, int n_q, int D, int hint) {
  I8Plan p{};
  const AttnPlan ap = attn_plan(B, Hq, Hkv, n_q, D, hint, SPEC_BF16);
  p.sp = stream_plan(B, Hkv, ap.RG, ap.RT, n_q, D, hint, kStreamMaxWG8);
  const size_t rows = (size_t)B * Hkv * n_q;
  size_t off = p.sp.total;
  p.off_nkq = off;
  off = align256(off + rows * D);
  p.off_nvq = off;
  off = align256(off + rows * D);
  p.off_nks = off;
  off = align256(off + rows * 2);
  p.off_nvs = off;
  off = align256(off + rows * 2);
  p.off_ovf = off;
  off = align256(off + sizeof(uint32_t) * (size_t)B * Hkv * ap.RG);
  p.total = off;
  return p;
}

extern "C" size_t spec_verify_attention_int8_workspace_size(int B, int Hq, int Hkv, int n_q, int D, int max_len_hint) {
  if (B < 1 || B > 1024 || Hq < 1 || Hkv < 1 || n_q < 1 || n_q > 16 || max_len_hint < 0) return 0;
  if (Hq % Hkv != 0 || (Hq / Hkv) * n_q > 256 || (D != 64 && D != 128)) return 0;
  const AttnPlan ap = attn_plan(B, Hq, Hkv, n_q, D, max_len_hint, SPEC_BF16);
  if (!stream_ok(SPEC_BF16, B, Hkv, ap.RG, n_q, max_len_hint)) return 0;
  return i8_plan(B, Hq, Hkv, n_q, D, max_len_hint).total;
}

extern "C" spec_status_t spec_verify_attention_int8(const void* q, const void* k_new, const void* v_new,
                                                    void* k_cache, void* k_scale, void* v_cache, void* v_scale,
                                                    const int32_t* cache_len, void* out, int B, int Hq, int Hkv,
                                                    int n_q, int D, int max_T, int max_len_hint, float scale,
                                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!q || !k_new || !v_new || !k_cache || !k_scale || !v_cache || !v_scale || !cache_len || !out || !workspace)
    return SPEC_ERR_ARG;
  if (B < 1 || Hq < 1 || Hkv < 1 || n_q < 1 || D < 1 || max_T < 1 || max_len_hint < 0) return SPEC_ERR_ARG;
  if (Hq % Hkv != 0) return SPEC_ERR_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return SPEC_ERR_ARG;
  const uintptr_t al = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_new) |
                       reinterpret_cast<uintptr_t>(v_new) | reinterpret_cast<uintptr_t>(k_cache) |
                       reinterpret_cast<uintptr_t>(v_cache) | reinterpret_cast<uintptr_t>(k_scale) |
                       reinterpret_cast<uintptr_t>(v_scale) | reinterpret_cast<uintptr_t>(out);
  if (al % 16 != 0 || reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return SPEC_ERR_ARG;
  if (max_T % 8 != 0) return SPEC_ERR_ARG;  // scale rows are copied 8 at a time
  if ((long)max_len_hint + n_q > (long)max_T) return SPEC_ERR_OVERFLOW;
  if (n_q > 16 || (Hq / Hkv) * n_q > 256 || (D != 64 && D != 128)) return SPEC_ERR_UNSUPPORTED;
  const AttnPlan p = attn_plan(B, Hq, Hkv, n_q, D, max_len_hint, SPEC_BF16);
  if (!stream_ok(SPEC_BF16, B, Hkv, p.RG, n_q, max_len_hint)) return SPEC_ERR_UNSUPPORTED;
  const I8Plan ip = i8_plan(B, Hq, Hkv, n_q, D, max_len_hint);
  if (workspace_bytes < ip.total) return SPEC_ERR_ARG;

  AttnArgs a{};
  a.q = q;
  a.kn = k_new;
  a.vn = v_new;
  a.kc = k_cache;
  a.vc = v_cache;
  a.len = cache_len;
  a.out = out;
  char* ws = static_cast<char*>(workspace);
  a.part_o = reinterpret_cast<float*>(ws + ip.sp.off_o);
  a.part_ml = reinterpret_cast<ML*>(ws + ip.sp.off_ml);
  a.pre = reinterpret_cast<int*>(ws + ip.sp.off_pre);
  a.MINB = ip.sp.MINB;
  a.JP = ip.sp.JP;
  a.ksc = static_cast<const uint16_t*>(k_scale);
  a.vsc = static_cast<const uint16_t*>(v_scale);
  a.nkq = reinterpret_cast<int8_t*>(ws + ip.off_nkq);
  a.nvq = reinterpret_cast<int8_t*>(ws + ip.off_nvq);
  a.nks = reinterpret_cast<uint16_t*>(ws + ip.off_nks);
  a.nvs = reinterpret_cast<uint16_t*>(ws + ip.off_nvs);
  a.ovf = reinterpret_cast<uint32_t*>(ws + ip.off_ovf);
  a.scnt = reinterpret_cast<uint32_t*>(ws + ip.sp.off_cnt);
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.n_q = n_q;
  a.G = Hq / Hkv;
  a.M = a.G * n_q;
  a.RG = p.RG;
  a.RT = p.RT;
  a.NSP = p.NSP;
  a.C = p.C;
  a.max_T = max_T;
  a.hint = max_len_hint;
  a.qk_scale = scale * 1.4426950408889634f;
  const hipError_t e = D == 128 ? launch_i8_d<128>(a, stream) : launch_i8_d<64>(a, stream);
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_LAUNCH;
}
