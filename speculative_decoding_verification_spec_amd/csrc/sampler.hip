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
// Four kernels; the hand-offs between them are kernel boundaries (a
// cross-workgroup hand-off inside a kernel would need device-scope release /
// acquire, which on this chip writes back and invalidates the per-XCD L2):
//   rs_stats    wave (b, row, segment): max and sum of exp((z - max)/T) over a
//               segment of one target or draft row.
//   rs_finalize workgroup b: merges the segments of all 2*gamma+1 rows,
//               evaluates p_i(x_i), q_i(x_i), the accept tests and n.
//   rs_resolve  wave (b, segment) of the decided row n: residual weights
//               max(0, p_n - q_n) (or p_gamma for the bonus) summed per
//               segment.
//   rs_draw     wave b: locates the segment where the fp64 prefix sum first
//               exceeds u * total, re-scans it and writes the emitted tokens.
// Every merge is in fp64 and in a fixed order.  No workspace word is read
// before this call has written it, so a workspace needs no initialisation and
// may be shared by calls of different sizes.
#include <math.h>
#include <stdint.h>

#include <algorithm>

#ifndef SPECV_RS_LANE_BYTES
#define SPECV_RS_LANE_BYTES 64
#endif

#include "spec_common.h"
#include "spec_verify.h"

namespace specv {

struct RowPart {  // one wave's segment of one row
  float M;
  float pad;
  double S;
};

struct SeqState {  // 32 bytes
  int n;           // leading accepted positions, 0..gamma
  int valid;       // 0 if a draft token was outside [0, V)
  float Mt, Md;    // row maxima of target row n and draft row n
  double St, Sd;   // sum of 2^((z - M) c) over those rows
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

template <typename T, int VEC, int NIT>
__global__ __launch_bounds__(256) void rs_stats(const T* __restrict__ tgt, const T* __restrict__ drf,
                                                int B, int G, int V, int nseg, float c32,
                                                RowPart* __restrict__ part) {
  constexpr int SEG = kWave * VEC * NIT;
  const int lane = threadIdx.x & (kWave - 1);
  const int R = 2 * G + 1;
  const long gw = (long)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (gw >= (long)B * R * nseg) return;  // uniform per wave
  const int seg = (int)(gw % nseg);
  const int r = (int)((gw / nseg) % R);
  const int b = (int)(gw / ((long)nseg * R));
  const T* row = (r <= G) ? tgt + ((size_t)b * (G + 1) + r) * V : drf + ((size_t)b * G + (r - G - 1)) * V;

  // Strided, fully coalesced loads: iteration it covers 64 * VEC consecutive
  // elements.  Order does not matter for a max and a sum.
  float v[NIT][VEC];
  const int s0 = seg * SEG;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int idx = s0 + (it * kWave + lane) * VEC;
    if (idx < V) {
      load_vec<T, VEC>(row + idx, v[it]);
    } else {
#pragma unroll
      for (int k = 0; k < VEC; ++k) v[it][k] = neg_inf_f();
    }
  }
  float m = neg_inf_f();
#pragma unroll
  for (int it = 0; it < NIT; ++it)
#pragma unroll
    for (int k = 0; k < VEC; ++k) m = fmaxf(m, v[it][k]);
  // Terms 2^((v - m) c): v - m is exact for bf16 inputs, so the only rounding
  // in the exponent is the product with c (relative 2^-24 of a small number).
  float terms[NIT * VEC];
#pragma unroll
  for (int it = 0; it < NIT; ++it)
#pragma unroll
    for (int k = 0; k < VEC; ++k) terms[it * VEC + k] = exp2_fast((v[it][k] - m) * c32);
  const float s = (m == neg_inf_f()) ? 0.f : tree_sum<NIT * VEC>(terms);
  const float M = wave_max(m);
  const double sc = (m == neg_inf_f()) ? 0.0 : (double)s * (double)exp2_fast((m - M) * c32);
  const double S = wave_sum(sc);
  if (lane == 0) {
    RowPart rp;
    rp.M = M;
    rp.pad = 0.f;
    rp.S = S;
    part[gw] = rp;
  }
}

// One workgroup per sequence: its waves merge the segments of the 2*gamma+1
// rows (fp64, fixed order) into LDS; then one wave evaluates p_i(x_i),
// q_i(x_i) and the accept tests, finds n and records the decided row's
// statistics for the resolve pass.
template <typename T>
__global__ __launch_bounds__(256) void rs_finalize(const T* __restrict__ tgt, const T* __restrict__ drf,
                                                   const int32_t* __restrict__ xtok, const double* __restrict__ uni,
                                                   int B, int G, int V, int nseg, float c32, double c64,
                                                   const RowPart* __restrict__ part, SeqState* __restrict__ st,
                                                   int32_t* __restrict__ n_out, int32_t* __restrict__ tok_out,
                                                   float* __restrict__ p_out, float* __restrict__ q_out) {
  __shared__ float rowM[64];
  __shared__ double rowS[64];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nwave = blockDim.x / kWave;
  const int R = 2 * G + 1;
  const int b = blockIdx.x;
  const RowPart* pb = part + (size_t)b * R * nseg;
  for (int rr = wave; rr < R; rr += nwave) {
    float mm = neg_inf_f();
    for (int k = lane; k < nseg; k += kWave) mm = fmaxf(mm, pb[rr * nseg + k].M);
    mm = wave_max(mm);
    double ss = 0.0;
    if (mm != neg_inf_f()) {
      for (int k = lane; k < nseg; k += kWave) {
        const RowPart e = pb[rr * nseg + k];
        if (e.M != neg_inf_f()) ss += e.S * (double)exp2_fast((e.M - mm) * c32);
      }
    }
    ss = wave_sum(ss);
    if (lane == 0) {
      rowM[rr] = mm;
      rowS[rr] = ss;
    }
  }
  __syncthreads();
  if (wave != 0) return;
  // Lane i < G judges position i against target row i and draft row G+1+i.
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
      // u < min(1, p/q): q = 0 < p gives +inf (accept), p = q = 0 gives NaN
      // (reject), exactly as the IEEE comparison with a NaN-propagating min.
      const double ratio = p / q;
      reject = !((u < 1.0) && (u < ratio));
    }
    if (p_out) p_out[(size_t)b * G + lane] = (float)p;
    if (q_out) q_out[(size_t)b * G + lane] = (float)q;
  }
  const uint64_t rej_mask = __ballot(reject);
  const uint64_t bad_mask = __ballot(bad);
  const int n = rej_mask ? (__ffsll((long long)rej_mask) - 1) : G;
  if (lane == 0) {
    SeqState s_;
    s_.n = n;
    s_.valid = bad_mask ? 0 : 1;
    s_.Mt = rowM[n];
    s_.St = rowS[n];
    s_.Md = n < G ? rowM[G + 1 + n] : 0.f;
    s_.Sd = n < G ? rowS[G + 1 + n] : 1.0;
    st[b] = s_;
    n_out[b] = bad_mask ? -1 : n;
  }
  if (bad_mask && lane <= G) tok_out[(size_t)b * (G + 1) + lane] = -1;
}

// ---------------------------------------------------------------------------
// pass 2: residual / bonus inverse-CDF draw on the decided row
// ---------------------------------------------------------------------------

// Weights of the E = VEC*NIT contiguous elements starting at idx0, computed
// identically in the segment pass and in the re-scan.  mode 0: residual
// max(0, p - q); mode 1: p alone (bonus row, or the zero-residual fallback).
// pw receives p (used for the fallback mass) when want_p is set.
template <typename T, int VEC, int NIT, bool want_p>
__device__ __forceinline__ void lane_weights(const T* __restrict__ rt, const T* __restrict__ rd, int idx0, int V,
                                             float c32, float Mt, float inv_st, float Md, float inv_sd, bool resid,
                                             float (&w)[NIT * VEC], float (&pw)[NIT * VEC]) {
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int idx = idx0 + it * VEC;
    float zt[VEC], zd[VEC];
    if (idx < V) {
      load_vec<T, VEC>(rt + idx, zt);
      if (resid) load_vec<T, VEC>(rd + idx, zd);
#pragma unroll
      for (int k = 0; k < VEC; ++k) {
        const float p = exp2_fast((zt[k] - Mt) * c32) * inv_st;
        float wk = p;
        if (resid) wk = fmaxf(p - exp2_fast((zd[k] - Md) * c32) * inv_sd, 0.f);
        w[it * VEC + k] = wk;
        if constexpr (want_p) pw[it * VEC + k] = p;
      }
    } else {
#pragma unroll
      for (int k = 0; k < VEC; ++k) {
        w[it * VEC + k] = 0.f;
        if constexpr (want_p) pw[it * VEC + k] = 0.f;
      }
    }
  }
}

template <typename T, int VEC, int NIT>
__global__ __launch_bounds__(256) void rs_resolve(const T* __restrict__ tgt, const T* __restrict__ drf, int B, int G,
                                                  int V, int nseg, float c32, const SeqState* __restrict__ st,
                                                  double2* __restrict__ part) {
  constexpr int SEG = kWave * VEC * NIT;
  const int lane = threadIdx.x & (kWave - 1);
  const long gw = (long)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (gw >= (long)B * nseg) return;
  const int seg = (int)(gw % nseg);
  const int b = (int)(gw / nseg);
  const SeqState s = st[b];
  if (!s.valid || s.n < 0 || s.n > G) return;  // rs_draw skips this sequence
  const int n = s.n;
  const bool resid = n < G;
  const T* rt = tgt + ((size_t)b * (G + 1) + n) * V;
  const T* rd = resid ? drf + ((size_t)b * G + n) * V : rt;
  const float inv_st = (float)(1.0 / s.St), inv_sd = (float)(1.0 / s.Sd);
  // Segment sums with coalesced loads (iteration it covers 64*VEC consecutive
  // elements).  rs_draw re-scans the chosen segment in index order; the two
  // summation orders agree to rounding, which only matters for a draw that
  // sits within rounding of a segment boundary (inside the 1e-6 band).
  const float mt_c = s.Mt, md_c = s.Md;
  double lw = 0.0, lp = 0.0;
  const int s0 = seg * SEG;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int idx = s0 + (it * kWave + lane) * VEC;
    if (idx < V) {
      float zt[VEC], zd[VEC];
      load_vec<T, VEC>(rt + idx, zt);
      if (resid) load_vec<T, VEC>(rd + idx, zd);
      float sw = 0.f, sp = 0.f;
#pragma unroll
      for (int k = 0; k < VEC; ++k) {
        const float p = exp2_fast((zt[k] - mt_c) * c32) * inv_st;
        const float w = resid ? fmaxf(p - exp2_fast((zd[k] - md_c) * c32) * inv_sd, 0.f) : p;
        sw += w;
        sp += p;
      }
      lw += (double)sw;
      lp += (double)sp;
    }
  }
  const double segw = __shfl(wave_inclusive_scan(lw, lane), kWave - 1, kWave);
  const double segp = __shfl(wave_inclusive_scan(lp, lane), kWave - 1, kWave);
  if (lane == 0) part[gw] = make_double2(segw, segp);
}

// One wave per sequence: fp64 total of the segment sums, the first segment
// whose prefix exceeds u * total, then the first token inside it.
template <typename T, int VEC, int NIT>
__global__ __launch_bounds__(256) void rs_draw(const T* __restrict__ tgt, const T* __restrict__ drf,
                                               const int32_t* __restrict__ xtok, const double* __restrict__ uni,
                                               int B, int G, int V, int nseg, float c32,
                                               const SeqState* __restrict__ st, const double2* __restrict__ part,
                                               int32_t* __restrict__ tok_out) {
  constexpr int E = VEC * NIT;
  constexpr int SEG = kWave * E;
  const int lane = threadIdx.x & (kWave - 1);
  const long b = (long)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (b >= B) return;
  const SeqState s = st[b];
  if (!s.valid || s.n < 0 || s.n > G) return;  // tokens already set to -1
  const int n = s.n;
  const bool resid = n < G;
  const T* rt = tgt + ((size_t)b * (G + 1) + n) * V;
  const T* rd = resid ? drf + ((size_t)b * G + n) * V : rt;
  const float inv_st = (float)(1.0 / s.St), inv_sd = (float)(1.0 / s.Sd);

  const double2* pb = part + (size_t)b * nseg;
  double W = 0.0;  // fixed-order fp64 total of the weights
  for (int c0 = 0; c0 < nseg; c0 += kWave) {
    const double v = (c0 + lane < nseg) ? pb[c0 + lane].x : 0.0;
    W += __shfl(wave_inclusive_scan(v, lane), kWave - 1, kWave);
  }
  const bool use_p = resid && !(W > 0.0);  // zero residual mass: draw from p_n
  if (use_p) {
    W = 0.0;
    for (int c0 = 0; c0 < nseg; c0 += kWave) {
      const double v = (c0 + lane < nseg) ? pb[c0 + lane].y : 0.0;
      W += __shfl(wave_inclusive_scan(v, lane), kWave - 1, kWave);
    }
  }
  const double target = uni[(size_t)b * (G + 1) + G] * W;
  // First segment whose inclusive prefix exceeds the target; base = the
  // prefix before it.  The carry chain matches the total W above.
  int kseg = -1, last_pos = -1;
  double base = 0.0, carry = 0.0;
  for (int c0 = 0; c0 < nseg && kseg < 0; c0 += kWave) {
    const bool in = c0 + lane < nseg;
    const double v = in ? (use_p ? pb[c0 + lane].y : pb[c0 + lane].x) : 0.0;
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

  // Re-scan the chosen segment with the same per-lane weights (with the
  // fallback, the weights are p itself: residual switched off).
  float w[E], pw[E];
  const int j0 = kseg * SEG + lane * E;
  lane_weights<T, VEC, NIT, false>(rt, rd, j0, V, c32, s.Mt, inv_st, s.Md, inv_sd, resid && !use_p, w, pw);
  double l2 = 0.0;
#pragma unroll
  for (int k = 0; k < E; ++k) l2 += (double)w[k];
  const double incl2 = wave_inclusive_scan(l2, lane);
  const double prev2 = __shfl_up(incl2, 1, kWave);
  double run = base + (lane == 0 ? 0.0 : prev2);  // this lane's exclusive prefix
  int hit_j = 0x7fffffff, last_j = -1;
#pragma unroll
  for (int k = 0; k < E; ++k) {
    run += (double)w[k];
    if (w[k] > 0.f) {
      last_j = j0 + k;
      if (!from_last && hit_j == 0x7fffffff && run > target) hit_j = j0 + k;
    }
  }
  int t = wave_min(hit_j);
  if (t == 0x7fffffff) t = wave_max(last_j);
  int32_t* ob = tok_out + (size_t)b * (G + 1);
  if (lane < n) ob[lane] = xtok[(size_t)b * G + lane];
  if (lane == n) ob[lane] = t;
  if (lane > n && lane <= G) ob[lane] = -1;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

static inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct RsPlan {
  int vec, nit, seg, nseg;
  size_t off_part1, off_state, off_part2, total;
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
  // about 64 bytes of each row per lane per segment
  // SPECV_RS_LANE_BYTES bytes of each row per lane per segment
  p.nit = std::max(1, SPECV_RS_LANE_BYTES / (vec * esize));
  p.seg = kWave * vec * p.nit;
  p.nseg = (V + p.seg - 1) / p.seg;
  const int R = 2 * G + 1;
  size_t off = 0;
  p.off_part1 = off;
  off = align256(off + sizeof(RowPart) * (size_t)B * R * p.nseg);
  p.off_state = off;
  off = align256(off + sizeof(SeqState) * (size_t)B);
  p.off_part2 = off;
  off = align256(off + sizeof(double2) * (size_t)B * p.nseg);
  p.total = off;
  return p;
}

template <typename T, int VEC, int NIT>
static hipError_t rs_launch(const RsPlan& pl, const void* tgt, const void* drf, const int32_t* x, const double* u,
                            int B, int G, int V, float c32, double c64, char* ws, int32_t* n_out, int32_t* tok_out,
                            float* p_out, float* q_out, hipStream_t stream) {
  const int R = 2 * G + 1;
  const long waves1 = (long)B * R * pl.nseg;
  const long waves2 = (long)B * pl.nseg;
  constexpr int WPB = 4;  // waves per 256-thread block
  RowPart* part1 = reinterpret_cast<RowPart*>(ws + pl.off_part1);
  SeqState* state = reinterpret_cast<SeqState*>(ws + pl.off_state);
  double2* part2 = reinterpret_cast<double2*>(ws + pl.off_part2);
  hipLaunchKernelGGL((rs_stats<T, VEC, NIT>), dim3((unsigned)((waves1 + WPB - 1) / WPB)), dim3(256), 0, stream,
                     (const T*)tgt, (const T*)drf, B, G, V, pl.nseg, c32, part1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((rs_finalize<T>), dim3((unsigned)B), dim3(256), 0, stream, (const T*)tgt, (const T*)drf, x, u, B,
                     G, V, pl.nseg, c32, c64, part1, state, n_out, tok_out, p_out, q_out);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((rs_resolve<T, VEC, NIT>), dim3((unsigned)((waves2 + WPB - 1) / WPB)), dim3(256), 0, stream,
                     (const T*)tgt, (const T*)drf, B, G, V, pl.nseg, c32, state, part2);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((rs_draw<T, VEC, NIT>), dim3((unsigned)((B + WPB - 1) / WPB)), dim3(256), 0, stream,
                     (const T*)tgt, (const T*)drf, x, u, B, G, V, pl.nseg, c32, state, part2, tok_out);
  return hipGetLastError();
}

template <typename T>
static hipError_t rs_dispatch(const RsPlan& pl, const void* tgt, const void* drf, const int32_t* x, const double* u,
                              int B, int G, int V, float c32, double c64, char* ws, int32_t* n_out, int32_t* tok_out,
                              float* p_out, float* q_out, hipStream_t s) {
#define RS_CASE(VEC_, NIT_)                                                                                     \
  if (pl.vec == VEC_ && pl.nit == NIT_)                                                                         \
    return rs_launch<T, VEC_, NIT_>(pl, tgt, drf, x, u, B, G, V, c32, c64, ws, n_out, tok_out, p_out, q_out, s);
  constexpr int LB = SPECV_RS_LANE_BYTES;
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
  if (!target_logits || !draft_logits || !draft_tokens || !uniforms || !n_accepted || !out_tokens || !workspace)
    return SPEC_ERR_ARG;
  if (B < 1 || gamma < 1 || gamma > 31 || V < 1) return SPEC_ERR_ARG;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_ARG;
  if (temperature == 0.f) return SPEC_ERR_UNSUPPORTED;
  if (!(temperature > 0.f) || !isfinite(temperature)) return SPEC_ERR_ARG;
  if (workspace_bytes < spec_reject_sample_workspace_size(B, gamma, V, dtype)) return SPEC_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return SPEC_ERR_ARG;
  const int esize = dtype == SPEC_BF16 ? 2 : 4;
  const int vec = pick_vec(V, esize, reinterpret_cast<uintptr_t>(target_logits),
                           reinterpret_cast<uintptr_t>(draft_logits));
  const RsPlan pl = rs_plan(B, gamma, V, esize, vec);
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
