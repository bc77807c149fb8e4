// Device helpers shared by the chunked prefill and backward kernels (gfx950): the
// hardware exponential, fp64 lane scans over DPP, 4-element loads and stores, and
// the LDS transpose read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace gdr {

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Lane j of 16-lane group g receives M[r0 + 4g + e][c0 + j], e = 0..3, of a row-major
// 16-bit matrix M in LDS (leading dimension ld elements): the gfx950 LDS transpose
// load, each lane s of the group naming the 8 bytes at row r0 + 4g + s/4, column
// c0 + 4 (s % 4).
template <typename T>
__device__ __forceinline__ s16x4 read_tr(const T *base, int ld, int r0, int c0, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const T *p = base + (r0 + 4 * g + (s >> 2)) * ld + c0 + 4 * (s & 3);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4 *)(p));
}

// B fragment of a row-major fp16 matrix M (rows = contraction index k0 .. k0+31,
// columns n0 .. n0+15), equivalently the A fragment of M^T: two transposed reads.
__device__ __forceinline__ Mma<false>::frag frag_tr(const _Float16 *base, int ld, int k0, int n0,
                                                   int lane) {
  const s16x4 lo = read_tr(base, ld, k0, n0, lane);
  const s16x4 hi = read_tr(base, ld, k0 + 16, n0, lane);
  Mma<false>::frag f;
  f.v = __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  return f;
}

// exp(x) on the hardware base-2 exponential
__device__ __forceinline__ float fexp(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// One DPP lane move of a double (both halves with the same control); lanes
// whose source is outside the pattern, or whose row is masked off, read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double x) {
  const long long b = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(b), CTRL, ROW_MASK, 0xf, false);
  const int hi =
      __builtin_amdgcn_update_dpp(0, static_cast<int>(b >> 32), CTRL, ROW_MASK, 0xf, false);
  return __longlong_as_double((static_cast<long long>(hi) << 32) |
                              static_cast<unsigned int>(lo));
}

// Inclusive prefix sum over lanes 0..31 of a wave (the whole wave must be
// active): shifts by 1, 2, 4, 8 inside each 16-lane row, then lane 15's total
// is broadcast into the next row.
__device__ __forceinline__ double prefix_sum32(double x) {
  x += dpp_f64<0x111, 0xf>(x);   // row_shr:1
  x += dpp_f64<0x112, 0xf>(x);   // row_shr:2
  x += dpp_f64<0x114, 0xf>(x);   // row_shr:4
  x += dpp_f64<0x118, 0xf>(x);   // row_shr:8
  x += dpp_f64<0x142, 0xa>(x);   // row_bcast:15 into rows 1 and 3
  return x;
}

__device__ __forceinline__ double readlane_f64(double x, int l) {
  const long long b = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_readlane(static_cast<int>(b), l);
  const int hi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), l);
  return __longlong_as_double((static_cast<long long>(hi) << 32) |
                              static_cast<unsigned int>(lo));
}

// four consecutive input elements (8- or 16-byte aligned) as float
__device__ __forceinline__ void load4(const uint16_t *p, float (&x)[4]) {
  const uint2 u = *reinterpret_cast<const uint2 *>(p);
  x[0] = __uint_as_float(u.x << 16);
  x[1] = __uint_as_float(u.x & 0xffff0000u);
  x[2] = __uint_as_float(u.y << 16);
  x[3] = __uint_as_float(u.y & 0xffff0000u);
}
__device__ __forceinline__ void load4(const float *p, float (&x)[4]) {
  const float4 a = *reinterpret_cast<const float4 *>(p);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
}

// four consecutive output elements
__device__ __forceinline__ void store4(__bf16 *p, const float (&o)[4]) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 h;
#pragma unroll
  for (int i = 0; i < 4; ++i) h[i] = static_cast<__bf16>(o[i]);
  *reinterpret_cast<bf16x4 *>(p) = h;
}
__device__ __forceinline__ void store4(float *p, const float (&o)[4]) {
  *reinterpret_cast<float4 *>(p) = make_float4(o[0], o[1], o[2], o[3]);
}

// four consecutive operand elements in LDS (8 bytes for fp16, 16 for fp32)
__device__ __forceinline__ void store4e(_Float16 *p, const float (&x)[4]) {
  f16x4 h;
#pragma unroll
  for (int i = 0; i < 4; ++i) h[i] = static_cast<_Float16>(x[i]);
  *reinterpret_cast<f16x4 *>(p) = h;
}
__device__ __forceinline__ void store4e(float *p, const float (&x)[4]) {
  *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
}

// 64-lane inclusive prefix sum of a double (the whole wave must be active): the
// 32-lane scan, then lane 31's total broadcast into rows 2 and 3.
__device__ __forceinline__ double prefix_sum64(double x) {
  x = prefix_sum32(x);
  x += dpp_f64<0x143, 0xc>(x);   // row_bcast:31 into rows 2 and 3
  return x;
}

}  // namespace gdr
