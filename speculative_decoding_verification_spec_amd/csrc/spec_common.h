// Device helpers shared by the verification kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specv {

constexpr int kWave = 64;

__device__ __forceinline__ float neg_inf_f() { return -__builtin_huge_valf(); }
__device__ __forceinline__ double neg_inf_d() { return -__builtin_huge_val(); }

// 2^x on the hardware transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// bfloat16 bit pattern <-> fp32.  Widening is exact; narrowing rounds to
// nearest, ties to even (NaN kept quiet).
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// ---- wave-wide reductions and scans (64 lanes, all active) ----------------
//
// Reductions stay in the VALU: rotations of each 16-lane row by 8, 4, 2, 1
// (DPP row_ror) leave every lane of a row with the row's result, then the
// gfx950 lane swaps across 16- and 32-lane halves (v_permlane16/32_swap)
// combine the four rows.  The association order is fixed, so equal inputs
// give equal results in every lane.

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xf, 0xf, false);
}
constexpr int kRowRor8 = 0x128, kRowRor4 = 0x124, kRowRor2 = 0x122, kRowRor1 = 0x121;

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) { return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v))); }

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = __double_as_longlong(v);
  const uint64_t lo = dpp_u32<CTRL>((uint32_t)u), hi = dpp_u32<CTRL>((uint32_t)(u >> 32));
  return __longlong_as_double((long long)((hi << 32) | lo));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<kRowRor8>(v));
  v = fmaxf(v, dpp_f32<kRowRor4>(v));
  v = fmaxf(v, dpp_f32<kRowRor2>(v));
  v = fmaxf(v, dpp_f32<kRowRor1>(v));
  {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<kRowRor8>(v);
  v += dpp_f32<kRowRor4>(v);
  v += dpp_f32<kRowRor2>(v);
  v += dpp_f32<kRowRor1>(v);
  {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return v;
}

// The two results of a lane swap, in a fixed order (lower half's value first),
// so a sum of them is the same in both lanes of a pair.
__device__ __forceinline__ double pair_sum_16(double v) {
  const uint64_t u = __double_as_longlong(v);
  const auto rl = __builtin_amdgcn_permlane16_swap((uint32_t)u, (uint32_t)u, false, false);
  const auto rh = __builtin_amdgcn_permlane16_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
  const double a = __longlong_as_double((long long)(((uint64_t)rh[0] << 32) | rl[0]));
  const double b = __longlong_as_double((long long)(((uint64_t)rh[1] << 32) | rl[1]));
  return a + b;
}
__device__ __forceinline__ double pair_sum_32(double v) {
  const uint64_t u = __double_as_longlong(v);
  const auto rl = __builtin_amdgcn_permlane32_swap((uint32_t)u, (uint32_t)u, false, false);
  const auto rh = __builtin_amdgcn_permlane32_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
  const double a = __longlong_as_double((long long)(((uint64_t)rh[0] << 32) | rl[0]));
  const double b = __longlong_as_double((long long)(((uint64_t)rh[1] << 32) | rl[1]));
  return a + b;
}

__device__ __forceinline__ double wave_sum(double v) {
  v += dpp_f64<kRowRor8>(v);
  v += dpp_f64<kRowRor4>(v);
  v += dpp_f64<kRowRor2>(v);
  v += dpp_f64<kRowRor1>(v);
  v = pair_sum_16(v);
  return pair_sum_32(v);
}

__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
  return v;
}

// Inclusive prefix sum over the 64 lanes in lane order (Hillis-Steele).  The
// association is fixed by the lane index, so equal inputs give equal outputs.
__device__ __forceinline__ double wave_inclusive_scan(double v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    double t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}

}  // namespace specv
