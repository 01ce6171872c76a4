// sv_device.hpp -- gfx950 device helpers: 16-byte row units and wave64
// reductions shared by the verify kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <float.h>
#include <math.h>
#include <stdint.h>

#include "sv_plan.hpp"

namespace sv {

constexpr double kLog2E = 1.4426950408889634074;

__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A 16-byte unit of a logits row, widened to fp32. bf16 is the upper half of an
// IEEE binary32, so widening is a shift (exact).
template <int DT>
struct Unit;

template <>
struct Unit<0> {  // fp32
  static constexpr int kEsz = 4;
  static constexpr int kEpu = 4;
  float x[4];
  __device__ __forceinline__ void unpack(const uint4& w) {
    x[0] = __uint_as_float(w.x);
    x[1] = __uint_as_float(w.y);
    x[2] = __uint_as_float(w.z);
    x[3] = __uint_as_float(w.w);
  }
};

template <>
struct Unit<1> {  // bf16
  static constexpr int kEsz = 2;
  static constexpr int kEpu = 8;
  float x[8];
  __device__ __forceinline__ void unpack(const uint4& w) {
    x[0] = __uint_as_float(w.x << 16);
    x[1] = __uint_as_float(w.x & 0xffff0000u);
    x[2] = __uint_as_float(w.y << 16);
    x[3] = __uint_as_float(w.y & 0xffff0000u);
    x[4] = __uint_as_float(w.z << 16);
    x[5] = __uint_as_float(w.z & 0xffff0000u);
    x[6] = __uint_as_float(w.w << 16);
    x[7] = __uint_as_float(w.w & 0xffff0000u);
  }
};

// Replace the slots of unit u that lie at or beyond V by -inf (neutral for
// max, sum-exp and argmax). Only the last unit of a row can hold such slots.
template <int DT>
__device__ __forceinline__ void mask_tail(Unit<DT>& un, int64_t u, int V) {
  constexpr int E = Unit<DT>::kEpu;
  int64_t e0 = u * E;
#pragma unroll
  for (int k = 0; k < E; ++k)
    if (e0 + k >= V) un.x[k] = -INFINITY;
}

template <int DT>
__device__ __forceinline__ float unit_max(const Unit<DT>& un) {
  float m = un.x[0];
#pragma unroll
  for (int k = 1; k < Unit<DT>::kEpu; ++k) m = fmaxf(m, un.x[k]);
  return m;
}

// Streaming 16-byte load with the non-temporal hint: logits are read once, so
// they should not displace other lines in the caches (measured on MI355X: a
// pure read of 4 GiB runs at ~7.0 TB/s this way against ~6.3 TB/s without).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16(const char* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------------------
// wave64 reductions (xor butterfly: fixed order, so results are deterministic)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int wave_or(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v |= __shfl_xor(v, o, kWave);
  return v;
}

// (value desc, index asc) argmax; NaN values never enter (callers flag them).
__device__ __forceinline__ void arg_combine(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float v2 = __shfl_xor(v, o, kWave);
    int i2 = __shfl_xor(i, o, kWave);
    arg_combine(v, i, v2, i2);
  }
}

// inclusive prefix sum over the wave, lane order
__device__ __forceinline__ double wave_incl_scan(double v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    double t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}

// Temperature usable iff finite, positive and a normal binary32.
__device__ __forceinline__ bool temp_ok(float T) { return T >= FLT_MIN && T <= FLT_MAX; }

// log2(e) / T rounded once to fp32.
__device__ __forceinline__ float log2e_over(float T) { return (float)(kLog2E / (double)T); }

}  // namespace sv
