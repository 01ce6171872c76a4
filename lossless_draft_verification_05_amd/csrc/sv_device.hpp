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
// wave64 reductions in registers (DPP). Within each 16-lane row a butterfly
// over quad_perm / row_ror leaves the row's result in every lane; the four row
// results are then read from lanes 0, 16, 32, 48 and combined in a fixed
// order, so the result is the same in every lane and deterministic. All 64
// lanes must be active.
// ---------------------------------------------------------------------------
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(dpp_i32<CTRL>(__float_as_int(v)));
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const int lo = dpp_i32<CTRL>(__double2loint(v));
  const int hi = dpp_i32<CTRL>(__double2hiint(v));
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ float readlane_f32(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ double readlane_f64(double v, int l) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(v), l);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(v), l);
  return __hiloint2double(hi, lo);
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f32<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_f32<kDppRowRor4>(v));
  v = fmaxf(v, dpp_f32<kDppRowRor8>(v));
  return fmaxf(fmaxf(readlane_f32(v, 0), readlane_f32(v, 16)), fmaxf(readlane_f32(v, 32), readlane_f32(v, 48)));
}

__device__ __forceinline__ double wave_max_f64(double v) {
  v = fmax(v, dpp_f64<kDppQuadXor1>(v));
  v = fmax(v, dpp_f64<kDppQuadXor2>(v));
  v = fmax(v, dpp_f64<kDppRowRor4>(v));
  v = fmax(v, dpp_f64<kDppRowRor8>(v));
  return fmax(fmax(readlane_f64(v, 0), readlane_f64(v, 16)), fmax(readlane_f64(v, 32), readlane_f64(v, 48)));
}

__device__ __forceinline__ double wave_sum(double v) {
  v += dpp_f64<kDppQuadXor1>(v);
  v += dpp_f64<kDppQuadXor2>(v);
  v += dpp_f64<kDppRowRor4>(v);
  v += dpp_f64<kDppRowRor8>(v);
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}
// The same fixed-order reduction in fp32 (every lane gets the sum).
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += dpp_f32<kDppQuadXor1>(v);
  v += dpp_f32<kDppQuadXor2>(v);
  v += dpp_f32<kDppRowRor4>(v);
  v += dpp_f32<kDppRowRor8>(v);
  return (readlane_f32(v, 0) + readlane_f32(v, 16)) + (readlane_f32(v, 32) + readlane_f32(v, 48));
}

// (value desc, index asc) argmax; NaN values never enter (callers flag them).
__device__ __forceinline__ void arg_combine(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

template <int CTRL>
__device__ __forceinline__ void arg_step(float& v, int& i) {
  const float v2 = dpp_f32<CTRL>(v);
  const int i2 = dpp_i32<CTRL>(i);
  arg_combine(v, i, v2, i2);
}

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  arg_step<kDppQuadXor1>(v, i);
  arg_step<kDppQuadXor2>(v, i);
  arg_step<kDppRowRor4>(v, i);
  arg_step<kDppRowRor8>(v, i);
  float rv = readlane_f32(v, 0);
  int ri = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
  for (int r = 16; r < 64; r += 16) arg_combine(rv, ri, readlane_f32(v, r), __builtin_amdgcn_readlane(i, r));
  v = rv;
  i = ri;
}

// inclusive prefix sum over the wave in lane order: Hillis-Steele within rows
// (row_shr 1, 2, 4, 8 with zero fill), then row 15 / 31 broadcasts
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_f64_masked(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, ROWS, 0xf, true);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, ROWS, 0xf, true);
  return __hiloint2double(hi, lo);
}

__device__ __forceinline__ double wave_incl_scan(double v, int /*lane*/) {
  v += dpp_f64_masked<kDppRowShr1, 0xf>(v);
  v += dpp_f64_masked<kDppRowShr2, 0xf>(v);
  v += dpp_f64_masked<kDppRowShr4, 0xf>(v);
  v += dpp_f64_masked<kDppRowShr8, 0xf>(v);
  v += dpp_f64_masked<kDppRowBcast15, 0xa>(v);
  v += dpp_f64_masked<kDppRowBcast31, 0xc>(v);
  return v;
}

// Temperature usable iff finite, positive and a normal binary32.
__device__ __forceinline__ bool temp_ok(float T) { return T >= FLT_MIN && T <= FLT_MAX; }

// log2(e) / T rounded once to fp32.
__device__ __forceinline__ float log2e_over(float T) { return (float)(kLog2E / (double)T); }

}  // namespace sv
