// Modified rejection sampler for one verification round (gfx950).
//
// [P1] "投機的デコーディングとドラフトモデル" section 受理判定の数理：修正版棄却サンプリング;
// [P2] "LLM推論の高速化｜KVキャッシュと投機的デコーディングを自作で実測" section
//      投機的デコーディングとは (the verify listing);
// [P3] "Speculative Decoding（投機的デコーディング）とは？…" section
//      受理・棄却の規則と出力分布が変わらない理由 (the five steps, bonus token).
//
// The pages' loop is sequential (test position i, stop at the first
// rejection, then draw).  Here every position is judged in parallel and the
// first rejection is found afterwards: the test at i reads only row i, so
// judging positions past the first rejection changes nothing but wasted work,
// and the data-parallel pass reads every logit exactly once.
//
// Two kernels:
//   rs_stats   per segment of every target and draft row: max and sum of
//              exp((z - max)/T) (every logit read once).
//   rs_resid   per (sequence, group of segments of its decided row): merges
//              each row's segments, evaluates p_i(x_i), q_i(x_i) and the
//              accept tests, finds n (every workgroup of the sequence alike;
//              the first also writes n, p and q), then sums the residual
//              weights max(0, p_n - q_n) (or p_gamma for the bonus) over its
//              segments; the last of the sequence's workgroups to finish
//              locates the segment where the fp64 prefix sum first exceeds
//              u * total, re-scans it and writes the tokens.
// The hand-off between the kernels is the kernel boundary.  Inside rs_resid
// the segment sums pass between a sequence's workgroups through device-scope
// (write-through) stores, completed before a device-scope counter add, and
// device-scope loads by the workgroup whose add completes the count: a few
// workgroups per counter, so the adds do not queue, and nobody waits.  (A
// fence-based hand-off would cost more than the pass itself on this chip: an
// agent-scope release or acquire writes back or invalidates a whole per-XCD
// L2.)  Every merge is in fp64 and in a fixed order.  The counters are zeroed
// by rs_stats; no other workspace word is read before this call has written
// it, so a workspace needs no initialisation and may be shared by calls of
// any sizes.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>


#include "spec_common.h"
#include "spec_verify.h"

namespace specv {

constexpr int kLaneBytes = 64;     // bytes of a row per lane per segment
// The sampler's statistics pass over a small batch (at most kStatsSmallSegs
// row segments in all) runs one segment per wave in 4-wave workgroups, so the
// launch ends in finer pieces; a larger batch runs two segments per wave (all
// loads issued before the arithmetic) in 16-wave workgroups (measured against
// two per wave in 4-wave workgroups for both: about 3% off the call at B = 32
// over 151,936 tokens, about 2% at B = 256 over 128,256).
constexpr long kStatsSmallSegs = 65536;
constexpr int kStatsSmallWaves = 4;
constexpr int kStatsLargeWaves = 16;
constexpr int kStatsLargeSegsPerWave = 2;
// The greedy pass: one segment per wave in 8-wave workgroups (measured: 91
// against 94 us with two segments per wave in 4-wave workgroups at B = 256,
// gamma = 8 over 128,256 tokens; no change at B = 32 over 151,936).
constexpr int kGreedySegsPerWave = 1;
constexpr int kGreedyWaves = 8;
constexpr int kResidPerCU = 2;     // residual workgroups per CU to aim for

struct RowPart {  // one wave's segment of one row
  float M;
  float pad;
  double S;
};

template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t v) { return bf16_to_f32(v); }

// Load VEC consecutive elements (aligned to VEC * sizeof(T)) as fp32.
template <typename T, int VEC>
__device__ __forceinline__ void load_vec(const T* __restrict__ p, float (&o)[VEC]) {
  constexpr int BYTES = VEC * (int)sizeof(T);
  if constexpr (BYTES == 16) {
    uint4 r = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        o[2 * k] = __uint_as_float(w[k] << 16);
        o[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = __uint_as_float(w[k]);
    }
  } else if constexpr (BYTES == 8) {
    uint2 r = *reinterpret_cast<const uint2*>(p);
    const uint32_t w[2] = {r.x, r.y};
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        o[2 * k] = __uint_as_float(w[k] << 16);
        o[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
      }
    } else {
      o[0] = __uint_as_float(w[0]);
      o[1] = __uint_as_float(w[1]);
    }
  } else if constexpr (BYTES == 4) {
    uint32_t w = *reinterpret_cast<const uint32_t*>(p);
    if constexpr (sizeof(T) == 2) {
      o[0] = __uint_as_float(w << 16);
      o[1] = __uint_as_float(w & 0xffff0000u);
    } else {
      o[0] = __uint_as_float(w);
    }
  } else {
    o[0] = to_f32<T>(*p);
  }
}

// Pairwise sum of a fixed-size array (depth log2 N, fixed association).
template <int N>
__device__ __forceinline__ float tree_sum(const float* a) {
  if constexpr (N == 1) {
    return a[0];
  } else {
    constexpr int H = N / 2;
    return tree_sum<H>(a) + tree_sum<N - H>(a + H);
  }
}

// ---------------------------------------------------------------------------
// pass 1: row statistics; accept tests and the first rejection per sequence
// ---------------------------------------------------------------------------

// Max and sum of 2^((v - m) c) over one segment held in registers.  v - m is
// exact for bf16 inputs, so the only rounding in the exponent is the product
// with c (relative 2^-24 of a small number); lanes merge in fp64.
template <int NIT, int VEC>
__device__ __forceinline__ RowPart segment_stats(const float (&v)[NIT][VEC], float c32) {
  float m = neg_inf_f();
#pragma unroll
  for (int it = 0; it < NIT; ++it)
#pragma unroll
    for (int k = 0; k < VEC; ++k) m = fmaxf(m, v[it][k]);
  float terms[NIT * VEC];
#pragma unroll
  for (int it = 0; it < NIT; ++it)
#pragma unroll
    for (int k = 0; k < VEC; ++k) terms[it * VEC + k] = exp2_fast((v[it][k] - m) * c32);
  const float s = (m == neg_inf_f()) ? 0.f : tree_sum<NIT * VEC>(terms);
  const float M = wave_max(m);
  const double sc = (m == neg_inf_f()) ? 0.0 : (double)s * (double)exp2_fast((m - M) * c32);
  RowPart rp;
  rp.M = M;
  rp.pad = 0.f;
  rp.S = wave_sum(sc);
  return rp;
}

// Raw storage of one VEC-element vector (the loaded bits, converted later).
template <int BYTES>
struct RawVec;
template <>
struct RawVec<16> { using type = uint4; };
template <>
struct RawVec<8> { using type = uint2; };
template <>
struct RawVec<4> { using type = uint32_t; };
template <>
struct RawVec<2> { using type = uint16_t; };

// One raw vector through a buffer resource: a scalar base and a 32-bit byte
// offset, so no 64-bit address is built in (and waits on) vector registers;
// offsets past the resource's size read 0 and never fault.
constexpr int kResidCachePolicy = 0;  // cache policy bits of the residual pass's buffer loads
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
template <typename Raw>
__device__ __forceinline__ Raw buf_raw(__amdgpu_buffer_rsrc_t r, uint32_t off);
template <>
__device__ __forceinline__ uint4 buf_raw<uint4>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kResidCachePolicy);
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <>
__device__ __forceinline__ uint2 buf_raw<uint2>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kResidCachePolicy);
  return make_uint2(v.x, v.y);
}
template <>
__device__ __forceinline__ uint32_t buf_raw<uint32_t>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kResidCachePolicy);
}
template <>
__device__ __forceinline__ uint16_t buf_raw<uint16_t>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, kResidCachePolicy);
}

template <typename T, int VEC>
__device__ __forceinline__ void raw_to_f32(const typename RawVec<VEC * sizeof(T)>::type& r, float (&o)[VEC]) {
  constexpr int BYTES = VEC * (int)sizeof(T);
  uint32_t w[(BYTES + 3) / 4];
  if constexpr (BYTES == 16) {
    w[0] = r.x; w[1] = r.y; w[2] = r.z; w[3] = r.w;
  } else if constexpr (BYTES == 8) {
    w[0] = r.x; w[1] = r.y;
  } else {
    w[0] = r;
  }
  if constexpr (sizeof(T) == 2) {
    if constexpr (BYTES == 2) {
      o[0] = __uint_as_float(w[0] << 16);
    } else {
#pragma unroll
      for (int k = 0; k < BYTES / 4; ++k) {
        o[2 * k] = __uint_as_float(w[k] << 16);
        o[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < VEC; ++k) o[k] = __uint_as_float(w[k]);
  }
}

// Grid: x = chunk of rows (one workgroup per cpr-th of a row), rows in
// position order gamma, gamma-1, ..., 0 and within a position by sequence,
// the target row before the draft row; each wave owns SPW consecutive
// segments and issues every load of all of them before the arithmetic (as
// many bytes in flight per wave as possible); a segment's elements past V
// read as -inf.  Position 0 comes last because the decided row is most often
// an early position (each position is reached only if all before it were
// accepted): read last, its rows are the likeliest still to be in the
// memory-side cache when rs_resid reads the decided row again.
// The statistics pass reads every logit once: non-temporal loads.
// A logit vector of the single streaming pass.
template <typename R>
__device__ __forceinline__ R stream_load(const R* p) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  typedef unsigned int v2u __attribute__((ext_vector_type(2)));
  if constexpr (sizeof(R) == 16) return __builtin_bit_cast(R, __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p)));
  else if constexpr (sizeof(R) == 8) return __builtin_bit_cast(R, __builtin_nontemporal_load(reinterpret_cast<const v2u*>(p)));
  else if constexpr (sizeof(R) == 4) return __builtin_bit_cast(R, __builtin_nontemporal_load(reinterpret_cast<const unsigned int*>(p)));
  else return __builtin_bit_cast(R, __builtin_nontemporal_load(reinterpret_cast<const unsigned short*>(p)));
}

template <typename T, int VEC, int NIT, int SPW>
__global__ __launch_bounds__(1024) void rs_stats(const T* __restrict__ tgt, const T* __restrict__ drf, int B, int G,
                                                 int V, int nseg, int cpr, float c32, RowPart* __restrict__ part,
                                                 uint32_t* __restrict__ cnt) {
  constexpr int SEG = kWave * VEC * NIT;
  using Raw = typename RawVec<VEC * sizeof(T)>::type;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if (blockIdx.x == 0)  // rs_resid's arrival counters start at zero
    for (int i = threadIdx.x; i < B; i += blockDim.x) cnt[i] = 0u;
  const int q = blockIdx.x / cpr, c = blockIdx.x - q * cpr;
  const int seg0 = (c * (blockDim.x / kWave) + wave) * SPW;
  if (seg0 >= nseg) return;  // uniform per wave
  int b, r;
  if (q < B) {  // position gamma: the bonus row, target only
    b = q;
    r = G;
  } else {
    const int q2 = q - B, pos = G - 1 - q2 / (2 * B), rem = q2 % (2 * B);
    b = rem >> 1;
    r = (rem & 1) ? G + 1 + pos : pos;
  }
  const int R = 2 * G + 1;
  const int rowid = b * R + r;
  const T* row = (r <= G) ? tgt + ((size_t)b * (G + 1) + r) * V : drf + ((size_t)b * G + (r - G - 1)) * V;
  RowPart* out = part + (size_t)rowid * nseg;
  // Strided, fully coalesced loads: iteration it of a segment covers 64*VEC
  // consecutive elements.  Order does not matter for a max and a sum.  FULL:
  // every element of the wave's segments lies in the row (all but a row's
  // last segment), so no element needs a bounds test or -inf padding; the
  // arithmetic is the same either way.
  auto body = [&](auto FULL) {
    constexpr bool kFull = decltype(FULL)::value;
    Raw raw[SPW][NIT];
    bool ok[SPW][NIT];
#pragma unroll
    for (int k = 0; k < SPW; ++k)
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int idx = (seg0 + k) * SEG + (it * kWave + lane) * VEC;
        ok[k][it] = kFull || idx < V;
        if (ok[k][it]) raw[k][it] = stream_load(reinterpret_cast<const Raw*>(row + idx));
      }
#pragma unroll
    for (int k = 0; k < SPW; ++k) {
      const int seg = seg0 + k;
      if (!kFull && seg >= nseg) break;
      float v[NIT][VEC];
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        if (ok[k][it]) {
          raw_to_f32<T, VEC>(raw[k][it], v[it]);
        } else {
#pragma unroll
          for (int e = 0; e < VEC; ++e) v[it][e] = neg_inf_f();
        }
      }
      const RowPart rp = segment_stats<NIT, VEC>(v, c32);
      if (lane == 0) out[seg] = rp;
    }
  };
  if ((long)(seg0 + SPW) * SEG <= V)  // uniform per wave
    body(std::true_type{});
  else
    body(std::false_type{});
}

// ---------------------------------------------------------------------------
// pass 2: one workgroup per sequence -- accept tests, first rejection,
// residual / bonus inverse-CDF draw
// ---------------------------------------------------------------------------

constexpr int kMaxSeg = 1024;  // segments of one row held in LDS

// p_n of one element, and its residual weight max(0, p - q), each with the
// roundings written out (one product for p, one fma for p - q) so that the
// residual pass's segment sums and the draw's re-scan round alike whatever
// the compiler would contract.
__device__ __forceinline__ float residual_p(float zt, float Mt, float c32, float inv_st) {
#pragma clang fp contract(off)
  return exp2_fast((zt - Mt) * c32) * inv_st;
}
__device__ __forceinline__ float residual_w(float p, float zd, float Md, float c32, float inv_sd) {
  return fmaxf(fmaf(-exp2_fast((zd - Md) * c32), inv_sd, p), 0.f);
}

// Weights of the E = VEC*NIT contiguous elements starting at idx0 (used by
// the final re-scan, in index order).  resid: max(0, p - q); else p.
template <typename T, int VEC, int NIT>
__device__ __forceinline__ void lane_weights(const T* __restrict__ rt, const T* __restrict__ rd, int idx0, int V,
                                             float c32, float Mt, float inv_st, float Md, float inv_sd, bool resid,
                                             float (&w)[NIT * VEC]) {
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int idx = idx0 + it * VEC;
    float zt[VEC], zd[VEC];
    if (idx < V) {
      load_vec<T, VEC>(rt + idx, zt);
      if (resid) load_vec<T, VEC>(rd + idx, zd);
#pragma unroll
      for (int k = 0; k < VEC; ++k) {
        const float p = residual_p(zt[k], Mt, c32, inv_st);
        w[it * VEC + k] = resid ? residual_w(p, zd[k], Md, c32, inv_sd) : p;
      }
    } else {
#pragma unroll
      for (int k = 0; k < VEC; ++k) w[it * VEC + k] = 0.f;
    }
  }
}

// Wait until every vector memory access this wave has issued is complete
// (for device-scope stores: visible to every XCD).
__device__ __forceinline__ void wait_vm_all() { __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// One segment sum pair (residual, p) through device-scope stores and loads:
// written by every workgroup of a sequence, read by the one that draws.
__device__ __forceinline__ void store_segsum(double2* p, double w, double pp) {
  unsigned long long* q = reinterpret_cast<unsigned long long*>(p);
  __hip_atomic_store(q, (unsigned long long)__double_as_longlong(w), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 1, (unsigned long long)__double_as_longlong(pp), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double load_segsum(const double2* p, int half) {
  const unsigned long long* q = reinterpret_cast<const unsigned long long*>(p) + half;
  return __longlong_as_double((long long)__hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// The draw of sequence b, by every thread of a workgroup (waves beyond the
// fourth only take the barriers).  Wave 0 takes the fp64 total of the segment
// sums in a fixed order and the first segment whose prefix exceeds u * total;
// then four waves re-scan that segment in index order (lane l of wave w holds
// the E/4 contiguous elements starting at (64 w + l) E/4; the prefix is the
// segment's base, the totals of the waves before, then the lane scan) and
// write the emitted tokens.  The segment sums and the re-scan agree to
// rounding, which only matters for a draw within rounding of a segment
// boundary -- inside the 1e-6 band.
template <typename T, int VEC, int NIT>
__device__ __forceinline__ void draw_tokens(const T* __restrict__ rt, const T* __restrict__ rd,
                                            const int32_t* __restrict__ xtok, const double* __restrict__ uni,
                                            int b, int G, int V, int nseg, float c32, int n, bool resid, float Mt,
                                            float inv_st, float Md, float inv_sd, const double2* __restrict__ sb,
                                            int32_t* __restrict__ tok_out) {
  constexpr int E = VEC * NIT;
  constexpr int SEG = kWave * E;
  constexpr int E4 = E / 4;
  static_assert(NIT % 4 == 0, "the re-scan splits a segment over four waves");
  __shared__ double sh_base, sh_target, sh_wtot[4];
  __shared__ int sh_kseg, sh_from_last, sh_use_p, sh_hit[4], sh_lastj[4];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

  if (wave == 0) {
    double W = 0.0;
    for (int c0 = 0; c0 < nseg; c0 += kWave) {
      const double v = (c0 + lane < nseg) ? load_segsum(sb + c0 + lane, 0) : 0.0;
      W += __shfl(wave_inclusive_scan(v, lane), kWave - 1, kWave);
    }
    const bool use_p = resid && !(W > 0.0);  // zero residual mass: draw from p_n
    if (use_p) {
      W = 0.0;
      for (int c0 = 0; c0 < nseg; c0 += kWave) {
        const double v = (c0 + lane < nseg) ? load_segsum(sb + c0 + lane, 1) : 0.0;
        W += __shfl(wave_inclusive_scan(v, lane), kWave - 1, kWave);
      }
    }
    const double target = uni[(size_t)b * (G + 1) + G] * W;
    int kseg = -1, last_pos = -1;
    double base = 0.0, carry = 0.0;
    for (int c0 = 0; c0 < nseg && kseg < 0; c0 += kWave) {
      const bool in = c0 + lane < nseg;
      const double v = in ? load_segsum(sb + c0 + lane, use_p ? 1 : 0) : 0.0;
      const double incl = carry + wave_inclusive_scan(v, lane);
      const double prev = __shfl_up(incl, 1, kWave);
      const double excl = (lane == 0) ? carry : prev;
      const uint64_t hit = __ballot(in && incl > target);
      const uint64_t pos = __ballot(in && v > 0.0);
      if (pos) last_pos = c0 + 63 - __builtin_clzll(pos);
      if (hit) {
        const int l = __ffsll((long long)hit) - 1;
        kseg = c0 + l;
        base = __shfl(excl, l, kWave);
      }
      carry = __shfl(incl, kWave - 1, kWave);
    }
    const bool from_last = kseg < 0;  // the target reached the total by rounding
    if (from_last) kseg = last_pos < 0 ? 0 : last_pos;
    if (lane == 0) {
      sh_kseg = kseg;
      sh_from_last = from_last;
      sh_use_p = use_p;
      sh_base = base;
      sh_target = target;
    }
  }
  __syncthreads();

  const int kseg = __builtin_amdgcn_readfirstlane(sh_kseg);
  const bool from_last = sh_from_last;
  const double target = sh_target;
  float w[E4];
  double incl2 = 0.0;
  const int j0 = kseg * SEG + (wave * kWave + lane) * E4;
  if (wave < 4) {
    lane_weights<T, VEC, NIT / 4>(rt, rd, j0, V, c32, Mt, inv_st, Md, inv_sd, resid && !sh_use_p, w);
    double l2 = 0.0;
#pragma unroll
    for (int k = 0; k < E4; ++k) l2 += (double)w[k];
    incl2 = wave_inclusive_scan(l2, lane);
    if (lane == kWave - 1) sh_wtot[wave] = incl2;
  }
  __syncthreads();
  if (wave < 4) {
    double run = sh_base;
    for (int q = 0; q < wave; ++q) run += sh_wtot[q];
    const double prev2 = __shfl_up(incl2, 1, kWave);
    run += (lane == 0 ? 0.0 : prev2);  // this lane's exclusive prefix
    int hit_j = 0x7fffffff, last_j = -1;
#pragma unroll
    for (int k = 0; k < E4; ++k) {
      run += (double)w[k];
      if (w[k] > 0.f) {
        last_j = j0 + k;
        if (!from_last && hit_j == 0x7fffffff && run > target) hit_j = j0 + k;
      }
    }
    hit_j = wave_min(hit_j);
    last_j = wave_max(last_j);
    if (lane == 0) {
      sh_hit[wave] = hit_j;
      sh_lastj[wave] = last_j;
    }
  }
  __syncthreads();
  if (wave != 0) return;
  int t = min(min(sh_hit[0], sh_hit[1]), min(sh_hit[2], sh_hit[3]));
  if (t == 0x7fffffff) t = max(max(sh_lastj[0], sh_lastj[1]), max(sh_lastj[2], sh_lastj[3]));
  int32_t* ob = tok_out + (size_t)b * (G + 1);
  if (lane < n) ob[lane] = xtok[(size_t)b * G + lane];
  if (lane == n) ob[lane] = t;
  if (lane > n && lane <= G) ob[lane] = -1;
}


// Merges the segments of every row of sequence b into rowM / rowS (fp64,
// fixed order).  Waves over rows, two rows at a time; each part is loaded
// once, 128 parts of a row per step (one step for up to 128 segments), and
// the steps merge online.
__device__ __forceinline__ void merge_rows(const RowPart* __restrict__ pb, int R, int nseg, float c32, int wave,
                                           int nwave, int lane, float* rowM, double* rowS) {
  for (int rr0 = wave; rr0 < R; rr0 += 2 * nwave) {
    float m[2] = {neg_inf_f(), neg_inf_f()};
    double sum[2] = {0.0, 0.0};
    for (int c0 = 0; c0 < nseg; c0 += 2 * kWave) {
      RowPart e[2][2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int rr = rr0 + j * nwave, k = c0 + h * kWave + lane;
          if (rr < R && k < nseg) {
            e[j][h] = pb[(size_t)rr * nseg + k];
          } else {
            e[j][h].M = neg_inf_f();
            e[j][h].S = 0.0;
          }
        }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float mc = wave_max(fmaxf(e[j][0].M, e[j][1].M));
        if (mc == neg_inf_f()) continue;  // uniform: nothing in this step
        double sc = 0.0;
#pragma unroll
        for (int h = 0; h < 2; ++h)
          if (e[j][h].M != neg_inf_f()) sc += e[j][h].S * (double)exp2_fast((e[j][h].M - mc) * c32);
        sc = wave_sum(sc);
        if (mc > m[j]) {
          sum[j] = (m[j] == neg_inf_f() ? 0.0 : sum[j] * (double)exp2_fast((m[j] - mc) * c32)) + sc;
          m[j] = mc;
        } else {
          sum[j] += sc * (double)exp2_fast((mc - m[j]) * c32);
        }
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int rr = rr0 + j * nwave;
        if (rr < R) {
          rowM[rr] = m[j];
          rowS[rr] = sum[j];
        }
      }
    }
  }
}

// Grid: x = sequence b, y = group of kResidWaves * spw segments of the
// decided row; kResidWaves waves, spw segments each.  Every workgroup of b merges b's rows and takes the
// decision (the same arithmetic in each, so all agree); workgroup y = 0 also
// writes n_accepted, p_draft and q_draft.  Then the workgroup sums the
// residual weights max(0, p_n - q_n) (or p_gamma for the bonus) and p_n (for
// the zero-residual fallback) over its segments, every load of them issued
// before the arithmetic; lane sums in fp64.  The last of b's workgroups to
// count itself in cnt[b] (zeroed by rs_stats) then draws (draw_tokens).
constexpr int kResidWaves = 8;

template <typename T, int VEC, int NIT>
__global__ __launch_bounds__(kResidWaves * kWave) void rs_resid(
    const T* __restrict__ tgt, const T* __restrict__ drf, const int32_t* __restrict__ xtok,
    const double* __restrict__ uni, int G, int V, int nseg, int spw, float c32, double c64,
    const RowPart* __restrict__ part, double2* __restrict__ segsum, uint32_t* __restrict__ cnt,
    int32_t* __restrict__ n_out, int32_t* __restrict__ tok_out, float* __restrict__ p_out,
    float* __restrict__ q_out) {
  constexpr int E = VEC * NIT;
  constexpr int SEG = kWave * E;
  using Raw = typename RawVec<VEC * sizeof(T)>::type;
  __shared__ float rowM[64];
  __shared__ double rowS[64];
  __shared__ int sh_n, sh_valid, sh_last;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int R = 2 * G + 1;
  const int b = blockIdx.x;
  const bool lead = blockIdx.y == 0;

  merge_rows(part + (size_t)b * R * nseg, R, nseg, c32, wave, kResidWaves, lane, rowM, rowS);
  __syncthreads();

  // wave 0: lane i < G judges position i against target row i and draft row
  // G+1+i; n is the first rejection.
  if (wave == 0) {
    bool bad = false, reject = false;
    if (lane < G) {
      const int x = xtok[(size_t)b * G + lane];
      double p = __builtin_nan(""), q = __builtin_nan("");
      if (x < 0 || x >= V) {
        bad = true;
      } else {
        const double zt = (double)to_f32<T>(tgt[((size_t)b * (G + 1) + lane) * V + x]);
        const double zd = (double)to_f32<T>(drf[((size_t)b * G + lane) * V + x]);
        p = exp2((zt - (double)rowM[lane]) * c64) / rowS[lane];
        q = exp2((zd - (double)rowM[G + 1 + lane]) * c64) / rowS[G + 1 + lane];
        const double u = uni[(size_t)b * (G + 1) + lane];
        // u < min(1, p/q): q = 0 < p gives +inf (accept), p = q = 0 gives
        // NaN (reject), as the IEEE comparison with a NaN-propagating min.
        const double ratio = p / q;
        reject = !((u < 1.0) && (u < ratio));
      }
      if (lead && p_out) p_out[(size_t)b * G + lane] = (float)p;
      if (lead && q_out) q_out[(size_t)b * G + lane] = (float)q;
    }
    const uint64_t rej_mask = __ballot(reject);
    const uint64_t bad_mask = __ballot(bad);
    const int n = rej_mask ? (__ffsll((long long)rej_mask) - 1) : G;
    if (lane == 0) {
      sh_n = n;
      sh_valid = bad_mask ? 0 : 1;
    }
    if (lead) {
      if (lane == 0) n_out[b] = bad_mask ? -1 : n;
      if (bad_mask && lane <= G) tok_out[(size_t)b * (G + 1) + lane] = -1;
    }
  }
  __syncthreads();
  if (!sh_valid) return;  // uniform over the workgroup
  // Uniform values in scalar registers: the row bases stay scalar.
  const int n = __builtin_amdgcn_readfirstlane(sh_n);
  const bool resid = n < G;
  const T* rt = tgt + ((size_t)b * (G + 1) + n) * V;
  const T* rd = drf + ((size_t)b * G + min(n, G - 1)) * V;  // never read unless resid
  const float Mt = rowM[n], Md = resid ? rowM[G + 1 + n] : 0.f;
  const float inv_st = (float)(1.0 / rowS[n]), inv_sd = resid ? (float)(1.0 / rowS[G + 1 + n]) : 1.f;
  const __amdgpu_buffer_rsrc_t rsrc_t =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(rt), 0, (int)((long)V * sizeof(T)), 0x00020000);
  const __amdgpu_buffer_rsrc_t rsrc_d =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(rd), 0, (int)((long)V * sizeof(T)), 0x00020000);

  // wave w takes segments [s0, s1) of this workgroup's spw * kResidWaves,
  // two at a time; the decided row's case (a residual, or the bonus row
  // alone) is fixed outside the element loops
  const int s0 = (blockIdx.y * kResidWaves + wave) * spw;
  const int s1 = min(s0 + spw, nseg);
  auto sums = [&](auto RESID) {
    constexpr bool kResid = decltype(RESID)::value;
    for (int seg0 = s0; seg0 < s1; seg0 += 2) {  // uniform per wave
      Raw at[2][NIT], ad[2][NIT];
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
          // elements past V read 0 from the buffer and are masked out below
          const uint32_t off = (uint32_t)((seg0 + k) * SEG + (it * kWave + lane) * VEC) * (uint32_t)sizeof(T);
          at[k][it] = buf_raw<Raw>(rsrc_t, off);
          if constexpr (kResid) ad[k][it] = buf_raw<Raw>(rsrc_d, off);
        }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int seg = seg0 + k;
        if (seg >= s1) break;
        double lw = 0.0, lp = 0.0;
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
          const int idx = seg * SEG + (it * kWave + lane) * VEC;
          if (idx < V) {
            float zt[VEC], zd[VEC];
            raw_to_f32<T, VEC>(at[k][it], zt);
            if constexpr (kResid) raw_to_f32<T, VEC>(ad[k][it], zd);
            float sw = 0.f, sp = 0.f;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
              const float p = residual_p(zt[e], Mt, c32, inv_st);
              if constexpr (kResid)
                sw += residual_w(p, zd[e], Md, c32, inv_sd);
              else
                sw += p;
              sp += p;
            }
            lw += (double)sw;
            lp += (double)sp;
          }
        }
        lw = wave_sum(lw);
        lp = wave_sum(lp);
        if (lane == 0) store_segsum(segsum + (size_t)b * nseg + seg, lw, lp);
      }
    }
  };
  if (resid)
    sums(std::true_type{});
  else
    sums(std::false_type{});
  // The last of b's workgroups to finish draws: its count follows every
  // other workgroup's completed segment stores (device-scope, write-through).
  wait_vm_all();
  __syncthreads();
  if (threadIdx.x == 0)
    sh_last = __hip_atomic_fetch_add(cnt + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.y - 1;
  __syncthreads();
  if (!sh_last) return;  // uniform over the workgroup
  draw_tokens<T, VEC, NIT>(rt, rd, xtok, uni, b, G, V, nseg, c32, n, resid, Mt, inv_st, Md, inv_sd,
                           segsum + (size_t)b * nseg, tok_out);
}

// ---------------------------------------------------------------------------
// temperature 0: greedy verification
// ---------------------------------------------------------------------------
//
// [P2] "LLM推論の高速化｜KVキャッシュと投機的デコーディングを自作で実測",
// section 投機的デコーディングとは: the listing there leaves out its
// temperature-0 branch; the results after it say that the accept test then
// asks whether the draft token is the target's most likely token, and that the
// output is the target's own greedy decoding.  So: a_i = (argmax z_t[i] == x_i),
// n = leading accepts, t = argmax z_t[n].  argmax is the first index of the
// largest value, a NaN counting as largest.  Only the gamma+1 target rows are
// read.
//
//   gs_stats  wave per segment of a target row: the segment's argmax as one
//             64-bit key (ordered value key, then inverted index).
//   gs_tail   workgroup per sequence: merges each row's keys, then one wave
//             makes the decisions and writes the outputs.

// Ordered key of a logit: a larger value gives a larger key; -0 and +0 are
// equal; every NaN is above +inf.  Key 0 is below every value (padding).
__device__ __forceinline__ uint32_t order_key(float v) {
  if (v != v) return 0xffffffffu;
  const uint32_t u = (v == 0.f) ? 0u : __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// (key, index) -> one comparable word: larger key first, then smaller index.
__device__ __forceinline__ uint64_t arg_word(uint32_t key, int idx) {
  return ((uint64_t)key << 32) | (uint32_t)~(uint32_t)idx;
}
__device__ __forceinline__ int arg_index(uint64_t w) { return (int)~(uint32_t)w; }

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, o, kWave), hi = __shfl_xor((uint32_t)(v >> 32), o, kWave);
    const uint64_t w = ((uint64_t)hi << 32) | lo;
    v = w > v ? w : v;
  }
  return v;
}

// Word j (of 32 bits) of a raw vector.
template <typename R>
__device__ __forceinline__ uint32_t raw_word(const R& r, int j) {
  if constexpr (sizeof(R) == 16) return j == 0 ? r.x : j == 1 ? r.y : j == 2 ? r.z : r.w;
  else if constexpr (sizeof(R) == 8) return j == 0 ? r.x : r.y;
  else return (uint32_t)r;
}

// The two bf16 values packed in w as two 16-bit keys (packed integer
// arithmetic, both halves at once) whose unsigned order is the values' order
// for every bit pattern but NaN, with -0 one below +0: a positive value's bits
// with the sign bit set, a negative value's bits inverted.  +inf maps to
// 0xff80 and -inf to 0x007f; a positive NaN lands above +inf (0xff81 and up),
// a negative one below -inf (0x007e and down).
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u16x2 bf16_pair_keys(uint32_t w) {
  const s16x2 x = __builtin_bit_cast(s16x2, w);
  const uint32_t neg = __builtin_bit_cast(uint32_t, x >> (s16x2){15, 15});  // 0xffff for a negative half
  return __builtin_bit_cast(u16x2, w ^ (neg | 0x80008000u));
}
constexpr int kKeyPosInf = 0xff80, kKeyNegInf = 0x007f, kKeyNegZero = 0x7fff, kKeyPosZero = 0x8000;

// Grid: x = target row b * (gamma + 1) + r, y = group of waves along the row.
//
// bf16 rows take a packed pass: per pair of elements, three integer
// operations make the two keys, and the lane keeps their largest and smallest
// (per group of VEC elements for the largest).  The wave's largest key then
// names the largest value, and only the lanes that hold it look for its first
// index.  A segment with a NaN (a key above +inf's or below -inf's) or whose
// largest value is a zero (where -0 and +0 must tie) takes the elementwise
// pass instead, which implements the rule directly.  Both give the same word.
template <typename T, int VEC, int NIT, int SPW>
__global__ __launch_bounds__(1024) void gs_stats(const T* __restrict__ tgt, int V, int nseg, uint64_t* __restrict__ part) {
  constexpr int SEG = kWave * VEC * NIT;
  using Raw = typename RawVec<VEC * sizeof(T)>::type;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int seg0 = (blockIdx.y * (blockDim.x / kWave) + wave) * SPW;
  if (seg0 >= nseg) return;  // uniform per wave
  const T* row = tgt + (size_t)blockIdx.x * V;
  uint64_t* out = part + (size_t)blockIdx.x * nseg;
  // FULL: every element of the wave's segments lies in the row (all but a
  // row's last segment), so no element needs a bounds test.
  auto body = [&](auto FULL) {
    constexpr bool kFull = decltype(FULL)::value;
    Raw raw[SPW][NIT];
    bool ok[SPW][NIT];
#pragma unroll
    for (int k = 0; k < SPW; ++k)
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int idx = (seg0 + k) * SEG + (it * kWave + lane) * VEC;
        ok[k][it] = kFull || idx < V;
        if (ok[k][it]) raw[k][it] = stream_load(reinterpret_cast<const Raw*>(row + idx));
      }
#pragma unroll
    for (int k = 0; k < SPW; ++k) {
      const int seg = seg0 + k;
      if (!kFull && seg >= nseg) break;
      if constexpr (sizeof(T) == 2 && VEC % 2 == 0) {
        constexpr int WPG = VEC / 2;  // words per group
        u16x2 gmax[NIT];
        u16x2 kmax = {0, 0}, kmin = {0xffff, 0xffff};
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
          gmax[it] = (u16x2){0, 0};
          if (!ok[k][it]) continue;
#pragma unroll
          for (int j = 0; j < WPG; ++j) {
            const u16x2 key = bf16_pair_keys(raw_word(raw[k][it], j));
            gmax[it] = __builtin_elementwise_max(gmax[it], key);
            kmin = __builtin_elementwise_min(kmin, key);
          }
          kmax = __builtin_elementwise_max(kmax, gmax[it]);
        }
        // A lane without elements keeps 0 as its largest key, below every
        // element's (NaN aside, and a NaN sends the segment elementwise).
        const int lmax = max((int)kmax.x, (int)kmax.y);
        const int lmin = min((int)kmin.x, (int)kmin.y);
        const int wmax = wave_max(lmax);
        const bool elementwise = __ballot(lmax > kKeyPosInf || lmin < kKeyNegInf) != 0ull || wmax == kKeyNegZero ||
                                 wmax == kKeyPosZero;
        if (!elementwise) {  // uniform over the wave
          int first = 0x7fffffff;
          if (lmax == wmax) {
            bool found = false;
#pragma unroll
            for (int it = 0; it < NIT; ++it) {
              if (found || !ok[k][it] || (gmax[it].x != wmax && gmax[it].y != wmax)) continue;
              const int idx0 = seg * SEG + (it * kWave + lane) * VEC;
#pragma unroll
              for (int j = 0; j < WPG; ++j) {
                const u16x2 key = bf16_pair_keys(raw_word(raw[k][it], j));
                if (!found && key.x == wmax) {
                  first = idx0 + 2 * j;
                  found = true;
                }
                if (!found && key.y == wmax) {
                  first = idx0 + 2 * j + 1;
                  found = true;
                }
              }
            }
          }
          first = wave_min(first);
          // The value with key wmax: a positive one's bits are the key without
          // its top bit, a negative one's the key inverted.
          const uint32_t bits = wmax >= kKeyPosZero ? (uint32_t)(wmax ^ 0x8000) : (uint32_t)(~wmax & 0xffff);
          if (lane == 0) out[seg] = arg_word(order_key(bf16_to_f32((uint16_t)bits)), first);
          continue;
        }
      }
      // A lane sees its elements in increasing index order, so a strict '>'
      // keeps the first of equal keys.  Every value's key exceeds 0.
      uint32_t best = 0u;
      int bidx = 0;
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        if (!ok[k][it]) continue;
        float v[VEC];
        raw_to_f32<T, VEC>(raw[k][it], v);
        const int idx0 = seg * SEG + (it * kWave + lane) * VEC;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const uint32_t key = order_key(v[e]);
          if (key > best) {
            best = key;
            bidx = idx0 + e;
          }
        }
      }
      const uint64_t w = wave_max_u64(best == 0u ? 0ull : arg_word(best, bidx));
      if (lane == 0) out[seg] = w;
    }
  };
  if ((long)(seg0 + SPW) * SEG <= V)  // uniform per wave
    body(std::true_type{});
  else
    body(std::false_type{});
}

__global__ __launch_bounds__(1024) void gs_tail(const int32_t* __restrict__ xtok, int G, int V, int nseg,
                                                const uint64_t* __restrict__ part, int32_t* __restrict__ n_out,
                                                int32_t* __restrict__ tok_out, float* __restrict__ p_out,
                                                float* __restrict__ q_out) {
  __shared__ int arg[32];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int nwave = blockDim.x / kWave;
  const int b = blockIdx.x;
  const uint64_t* pb = part + (size_t)b * (G + 1) * nseg;
  for (int r = wave; r <= G; r += nwave) {
    uint64_t m = 0;
    for (int k = lane; k < nseg; k += kWave) {
      const uint64_t w = pb[(size_t)r * nseg + k];
      m = w > m ? w : m;
    }
    m = wave_max_u64(m);
    if (lane == 0) arg[r] = arg_index(m);
  }
  __syncthreads();
  if (wave != 0) return;
  bool bad = false, reject = false;
  if (lane < G) {
    const int x = xtok[(size_t)b * G + lane];
    bad = x < 0 || x >= V;
    reject = bad || arg[lane] != x;
    if (p_out) p_out[(size_t)b * G + lane] = bad ? __builtin_nanf("") : (arg[lane] == x ? 1.f : 0.f);
    if (q_out) q_out[(size_t)b * G + lane] = __builtin_nanf("");  // the draft side is not read
  }
  const uint64_t bad_mask = __ballot(bad);
  const uint64_t rej_mask = __ballot(reject);
  const int n = rej_mask ? (__ffsll((long long)rej_mask) - 1) : G;
  int32_t* ob = tok_out + (size_t)b * (G + 1);
  if (bad_mask) {
    if (lane == 0) n_out[b] = -1;
    if (lane <= G) ob[lane] = -1;
    return;
  }
  if (lane == 0) n_out[b] = n;
  if (lane < n) ob[lane] = xtok[(size_t)b * G + lane];
  if (lane == n) ob[lane] = arg[n];
  if (lane > n && lane <= G) ob[lane] = -1;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

static inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Compute units of the current device (cached per device).
static int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  std::atomic<int>* slot = dev < 64 ? &cache[dev] : nullptr;
  if (slot && slot->load(std::memory_order_relaxed) > 0) return slot->load(std::memory_order_relaxed);
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
  if (slot) slot->store(cus, std::memory_order_relaxed);
  return cus;
}

struct RsPlan {
  int vec, nit, seg, nseg;
  size_t off_part1, off_seg, off_cnt, total;
};

static int pick_vec(int V, int esize, uintptr_t a, uintptr_t b) {
  for (int vec = 16 / esize; vec > 1; vec >>= 1) {
    const int bytes = vec * esize;
    if (V % vec == 0 && a % bytes == 0 && b % bytes == 0) return vec;
  }
  return 1;
}

static RsPlan rs_plan(int B, int G, int V, int esize, int vec) {
  RsPlan p{};
  p.vec = vec;
  // kLaneBytes bytes of each row per lane per segment
  p.nit = std::max(1, kLaneBytes / (vec * esize));
  p.seg = kWave * vec * p.nit;
  p.nseg = (V + p.seg - 1) / p.seg;
  const int R = 2 * G + 1;
  p.off_part1 = 0;
  p.off_seg = align256(sizeof(RowPart) * (size_t)B * R * p.nseg);
  p.off_cnt = p.off_seg + align256(sizeof(double2) * (size_t)B * p.nseg);
  p.total = p.off_cnt + align256(sizeof(uint32_t) * (size_t)B);
  return p;
}

// The statistics pass: SPW segments per wave, up to max_wpb waves per
// workgroup, the workgroups of a row consecutive.
template <typename T, int VEC, int NIT, int SPW>
static hipError_t rs_stats_launch(const RsPlan& pl, const void* tgt, const void* drf, int B, int G, int V, float c32,
                                  RowPart* part1, uint32_t* cnt, int max_wpb, hipStream_t stream) {
  const int R = 2 * G + 1;
  const int waves_row = (pl.nseg + SPW - 1) / SPW;
  const int wpb = std::min(max_wpb, waves_row);  // waves per block
  const int cpr = (waves_row + wpb - 1) / wpb;   // workgroups per row
  hipLaunchKernelGGL((rs_stats<T, VEC, NIT, SPW>), dim3((unsigned)((long)B * R * cpr)), dim3(kWave * wpb), 0, stream,
                     (const T*)tgt, (const T*)drf, B, G, V, pl.nseg, cpr, c32, part1, cnt);
  return hipGetLastError();
}

template <typename T, int VEC, int NIT>
static hipError_t rs_launch(const RsPlan& pl, const void* tgt, const void* drf, const int32_t* x, const double* u,
                            int B, int G, int V, float c32, double c64, char* ws, int32_t* n_out, int32_t* tok_out,
                            float* p_out, float* q_out, hipStream_t stream) {
  const int R = 2 * G + 1;
  RowPart* part1 = reinterpret_cast<RowPart*>(ws + pl.off_part1);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(ws + pl.off_cnt);
  hipError_t e = (long)B * R * pl.nseg <= kStatsSmallSegs
                     ? rs_stats_launch<T, VEC, NIT, 1>(pl, tgt, drf, B, G, V, c32, part1, cnt, kStatsSmallWaves, stream)
                     : rs_stats_launch<T, VEC, NIT, kStatsLargeSegsPerWave>(pl, tgt, drf, B, G, V, c32, part1, cnt,
                                                                           kStatsLargeWaves, stream);
  if (e != hipSuccess) return e;
  double2* segsum = reinterpret_cast<double2*>(ws + pl.off_seg);
  // About two residual workgroups per CU, at least two segments per wave.
  const int ngrp = std::max(1, std::min((kResidPerCU * device_cus() + B - 1) / B,
                                        (pl.nseg + 2 * kResidWaves - 1) / (2 * kResidWaves)));
  int spw = (pl.nseg + ngrp * kResidWaves - 1) / (ngrp * kResidWaves);
  spw += spw & 1;
  const int ny = (pl.nseg + spw * kResidWaves - 1) / (spw * kResidWaves);
  hipLaunchKernelGGL((rs_resid<T, VEC, NIT>), dim3((unsigned)B, (unsigned)ny), dim3(kWave * kResidWaves), 0, stream,
                     (const T*)tgt, (const T*)drf, x, u, G, V, pl.nseg, spw, c32, c64, part1, segsum, cnt, n_out,
                     tok_out, p_out, q_out);
  return hipGetLastError();
}

template <typename T>
static hipError_t rs_dispatch(const RsPlan& pl, const void* tgt, const void* drf, const int32_t* x, const double* u,
                              int B, int G, int V, float c32, double c64, char* ws, int32_t* n_out, int32_t* tok_out,
                              float* p_out, float* q_out, hipStream_t s) {
#define RS_CASE(VEC_, NIT_)                                                                                     \
  if (pl.vec == VEC_ && pl.nit == NIT_)                                                                         \
    return rs_launch<T, VEC_, NIT_>(pl, tgt, drf, x, u, B, G, V, c32, c64, ws, n_out, tok_out, p_out, q_out, s);
  constexpr int LB = kLaneBytes;
  if constexpr (sizeof(T) == 2) {
    RS_CASE(8, LB / 16)
    RS_CASE(4, LB / 8)
    RS_CASE(2, LB / 4)
    RS_CASE(1, LB / 2)
  } else {
    RS_CASE(4, LB / 16)
    RS_CASE(2, LB / 8)
    RS_CASE(1, LB / 4)
  }
#undef RS_CASE
  return hipErrorInvalidValue;
}

template <typename T, int VEC, int NIT>
static hipError_t gs_launch(const RsPlan& pl, const void* tgt, const int32_t* x, int B, int G, int V, char* ws,
                            int32_t* n_out, int32_t* tok_out, float* p_out, float* q_out, hipStream_t stream) {
  uint64_t* part = reinterpret_cast<uint64_t*>(ws + pl.off_part1);
  constexpr int SPW = kGreedySegsPerWave;
  const int waves_row = (pl.nseg + SPW - 1) / SPW;
  const int wpb = std::min(kGreedyWaves, waves_row);
  hipLaunchKernelGGL((gs_stats<T, VEC, NIT, SPW>), dim3((unsigned)((long)B * (G + 1)), (unsigned)((waves_row + wpb - 1) / wpb)),
                     dim3(kWave * wpb), 0, stream, (const T*)tgt, V, pl.nseg, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nw = std::min(16, G + 1);
  hipLaunchKernelGGL(gs_tail, dim3((unsigned)B), dim3(kWave * nw), 0, stream, x, G, V, pl.nseg, part, n_out, tok_out,
                     p_out, q_out);
  return hipGetLastError();
}

template <typename T>
static hipError_t gs_dispatch(const RsPlan& pl, const void* tgt, const int32_t* x, int B, int G, int V, char* ws,
                              int32_t* n_out, int32_t* tok_out, float* p_out, float* q_out, hipStream_t s) {
#define GS_CASE(VEC_, NIT_) \
  if (pl.vec == VEC_ && pl.nit == NIT_) return gs_launch<T, VEC_, NIT_>(pl, tgt, x, B, G, V, ws, n_out, tok_out, p_out, q_out, s);
  constexpr int LB = kLaneBytes;
  if constexpr (sizeof(T) == 2) {
    GS_CASE(8, LB / 16)
    GS_CASE(4, LB / 8)
    GS_CASE(2, LB / 4)
    GS_CASE(1, LB / 2)
  } else {
    GS_CASE(4, LB / 16)
    GS_CASE(2, LB / 8)
    GS_CASE(1, LB / 4)
  }
#undef GS_CASE
  return hipErrorInvalidValue;
}

}  // namespace specv

using namespace specv;

extern "C" size_t spec_reject_sample_workspace_size(int B, int gamma, int V, spec_dtype_t dtype) {
  if (B < 1 || gamma < 1 || gamma > 31 || V < 1) return 0;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return 0;
  const int esize = dtype == SPEC_BF16 ? 2 : 4;
  // The smallest vector width gives the most segments: size for it.
  return rs_plan(B, gamma, V, esize, 1).total;
}

extern "C" spec_status_t spec_reject_sample(const void* target_logits, const void* draft_logits,
                                            const int32_t* draft_tokens, const double* uniforms, int B, int gamma,
                                            int V, float temperature, spec_dtype_t dtype, int32_t* n_accepted,
                                            int32_t* out_tokens, float* p_draft, float* q_draft, void* workspace,
                                            size_t workspace_bytes, hipStream_t stream) {
  const bool greedy = temperature == 0.f;
  if (!target_logits || !draft_tokens || !n_accepted || !out_tokens || !workspace) return SPEC_ERR_ARG;
  if (!greedy && (!draft_logits || !uniforms)) return SPEC_ERR_ARG;  // greedy reads neither
  if (B < 1 || gamma < 1 || gamma > 31 || V < 1) return SPEC_ERR_ARG;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_ARG;
  if (!greedy && (!(temperature > 0.f) || !isfinite(temperature))) return SPEC_ERR_ARG;
  if (workspace_bytes < spec_reject_sample_workspace_size(B, gamma, V, dtype)) return SPEC_ERR_ARG;
  {
    const int nseg1 = rs_plan(B, gamma, V, dtype == SPEC_BF16 ? 2 : 4, 1).nseg;
    if (nseg1 > kMaxSeg) return SPEC_ERR_UNSUPPORTED;
    // the statistics grid (one workgroup per chunk of every row) must fit in
    // int: a grid of over kStatsSmallSegs segments has chunks of this size
    const long long chunk = (long long)kStatsLargeWaves * kStatsLargeSegsPerWave;
    if ((long long)B * (2 * gamma + 1) * ((nseg1 + chunk - 1) / chunk) > 0x7fffffffLL) return SPEC_ERR_UNSUPPORTED;
  }
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return SPEC_ERR_ARG;
  const int esize = dtype == SPEC_BF16 ? 2 : 4;
  const int vec = pick_vec(V, esize, reinterpret_cast<uintptr_t>(target_logits),
                           reinterpret_cast<uintptr_t>(greedy ? target_logits : draft_logits));
  const RsPlan pl = rs_plan(B, gamma, V, esize, vec);
  if (greedy) {
    char* ws = static_cast<char*>(workspace);
    const hipError_t e = dtype == SPEC_BF16
                             ? gs_dispatch<uint16_t>(pl, target_logits, draft_tokens, B, gamma, V, ws, n_accepted,
                                                     out_tokens, p_draft, q_draft, stream)
                             : gs_dispatch<float>(pl, target_logits, draft_tokens, B, gamma, V, ws, n_accepted,
                                                  out_tokens, p_draft, q_draft, stream);
    return e == hipSuccess ? SPEC_OK : SPEC_ERR_LAUNCH;
  }
  // 2^((z - M) * c) = exp((z - M) / T)
  const double c64 = 1.4426950408889634073599246810019 / (double)temperature;
  const float c32 = (float)c64;
  char* ws = static_cast<char*>(workspace);
  hipError_t e;
  if (dtype == SPEC_BF16)
    e = rs_dispatch<uint16_t>(pl, target_logits, draft_logits, draft_tokens, uniforms, B, gamma, V, c32, c64, ws,
                              n_accepted, out_tokens, p_draft, q_draft, stream);
  else
    e = rs_dispatch<float>(pl, target_logits, draft_logits, draft_tokens, uniforms, B, gamma, V, c32, c64, ws,
                           n_accepted, out_tokens, p_draft, q_draft, stream);
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_LAUNCH;
}

// ---------------------------------------------------------------------------
// the same call without a caller workspace
// ---------------------------------------------------------------------------
//
// spec_reject_sample_noalloc uses this array as its workspace.  Every GPU the
// library runs on holds its own copy (zero-initialised when the code object is
// loaded) until the process ends.  Host code never passes the array's name to
// a kernel: the name stands for a host-side shadow, so its device address is
// looked up once per device with hipGetSymbolAddress and kept.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// The device address of this device's `scratch`, looked up on the first call
// made with the device current; nullptr if the lookup fails.
static void* scratch_address() {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

extern "C" spec_status_t spec_reject_sample_noalloc(const void* target_logits, const void* draft_logits,
                                                    const int32_t* draft_tokens, const double* uniforms, int B,
                                                    int gamma, int V, float temperature, spec_dtype_t dtype,
                                                    int32_t* n_accepted, int32_t* out_tokens, float* p_draft,
                                                    float* q_draft, hipStream_t stream) {
  const size_t need = spec_reject_sample_workspace_size(B, gamma, V, dtype);
  if (need == 0) return SPEC_ERR_ARG;
  if (need > kNoAllocScratchBytes) return SPEC_ERR_SCRATCH;
  void* ws = scratch_address();
  if (!ws) return SPEC_ERR_LAUNCH;
  // Every scratch word the kernels read is written earlier in the same call
  // (the arrival counters are zeroed by its first kernel), so nothing is
  // cleared here and no memory is allocated.
  return spec_reject_sample(target_logits, draft_logits, draft_tokens, uniforms, B, gamma, V, temperature, dtype,
                            n_accepted, out_tokens, p_draft, q_draft, ws, kNoAllocScratchBytes, stream);
}
