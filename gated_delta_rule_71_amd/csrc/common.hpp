// Device helpers for the gfx950 (CDNA4) kernels: element conversions and the
// 16x16 matrix-core tile conventions used by the chunked prefill.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

constexpr int kWave = 64;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---- element conversions ------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T> __device__ __forceinline__ float load_f32(const T *p);
template <> __device__ __forceinline__ float load_f32<float>(const float *p) { return *p; }
template <> __device__ __forceinline__ float load_f32<uint16_t>(const uint16_t *p) {
  return bf16_to_f32(*p);
}

template <typename T> __device__ __forceinline__ void store_f32(T *p, float x);
template <> __device__ __forceinline__ void store_f32<float>(float *p, float x) { *p = x; }
template <> __device__ __forceinline__ void store_f32<uint16_t>(uint16_t *p, float x) {
  *p = f32_to_bf16(x);
}

// Eight consecutive input elements as float (16-byte or 32-byte aligned).
__device__ __forceinline__ void load8(const uint16_t *p, float (&x)[8]) {
  const uint4 u = *reinterpret_cast<const uint4 *>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float *p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4 *>(p);
  const float4 b = *reinterpret_cast<const float4 *>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// Eight consecutive input elements held raw in registers between a global load
// and their use (lets a workgroup issue a whole chunk of loads at once).
template <typename T> struct Seg8;
template <> struct Seg8<uint16_t> {
  uint4 u;
  __device__ __forceinline__ void load(const uint16_t *p) {
    u = *reinterpret_cast<const uint4 *>(p);
  }
  __device__ __forceinline__ void zero() { u = make_uint4(0u, 0u, 0u, 0u); }
  __device__ __forceinline__ void store(uint16_t *p) const { *reinterpret_cast<uint4 *>(p) = u; }
  __device__ __forceinline__ void get(float (&x)[8]) const {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <> struct Seg8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float *p) {
    a = *reinterpret_cast<const float4 *>(p);
    b = *reinterpret_cast<const float4 *>(p + 4);
  }
  __device__ __forceinline__ void zero() {
    a = make_float4(0.f, 0.f, 0.f, 0.f);
    b = a;
  }
  __device__ __forceinline__ void store(float *p) const {
    *reinterpret_cast<float4 *>(p) = a;
    *reinterpret_cast<float4 *>(p + 4) = b;
  }
  __device__ __forceinline__ void get(float (&x)[8]) const {
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
};

// ---- 16x16 matrix-core tiles --------------------------------------------------
//
// Accumulator ("C layout") of a 16x16 float tile D: lane l holds
//   D[4*(l/16) + i][l%16], i = 0..3.
// Operand fragments cover a 32-deep slice of the contraction index.  For an A
// operand (16 rows x 32) lane l supplies row l%16, for a B operand (32 x 16
// columns) column l%16, and in both cases the eight values at contraction
// indices
//   kidx(g, e) = 4g + e          (e = 0..3)
//              = 16 + 4g + e - 4 (e = 4..7),     g = l/16.
// The same map is used for A and B, so each product pairs equal indices.  It is
// chosen so that two stacked accumulator tiles (rows 0..15 and 16..31 of the
// slice) ARE a B fragment without moving data between lanes: the state matrix
// and the per-chunk deltas stay in registers between products.
//
// Mma<false>: fp16 operands, one v_mfma_f32_16x16x32_f16 per slice.
// Mma<true> : fp32 operands, eight v_mfma_f32_16x16x4_f32 per slice (step e
//             contracts index kidx(g, e) of each lane group g).

template <bool F32> struct Mma;

template <> struct Mma<false> {
  using elem = _Float16;
  struct frag { f16x8 v; };
  static __device__ __forceinline__ f32x4 mma(const frag &a, const frag &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v, b.v, c, 0, 0, 0);
  }
  // rows/cols from a row-major LDS matrix: base[(row) * ld + kcol]
  static __device__ __forceinline__ frag load(const elem *base, int ld, int row, int k0,
                                              int lane) {
    const int g = lane >> 4;
    const elem *p = base + row * ld + k0 + 4 * g;
    // Two separate 8-byte reads.  The compiler would otherwise pair them into one
    // ds_read2_b64, whose two addresses 32 bytes apart collide in the LDS banks
    // (about four times the cycles of two single reads at these row strides); the
    // empty asm with a memory clobber keeps them apart.
    const f16x4 lo = *reinterpret_cast<const f16x4 *>(p);
    asm volatile("" ::: "memory");
    const f16x4 hi = *reinterpret_cast<const f16x4 *>(p + 16);
    asm volatile("" ::: "memory");
    frag f;
    f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return f;
  }
  static __device__ __forceinline__ frag from_acc(const f32x4 &t0, const f32x4 &t1) {
    frag f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f.v[i] = static_cast<_Float16>(t0[i]);
      f.v[4 + i] = static_cast<_Float16>(t1[i]);
    }
    return f;
  }
  static __device__ __forceinline__ frag zero() {
    frag f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f.v[i] = static_cast<_Float16>(0.0f);
    return f;
  }
  static __device__ __forceinline__ elem cvt(float x) { return static_cast<_Float16>(x); }
};

template <> struct Mma<true> {
  using elem = float;
  struct frag { float v[8]; };
  static __device__ __forceinline__ f32x4 mma(const frag &a, const frag &b, f32x4 c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], c, 0, 0, 0);
    return c;
  }
  static __device__ __forceinline__ frag load(const elem *base, int ld, int row, int k0,
                                              int lane) {
    const int g = lane >> 4;
    const float *p = base + row * ld + k0 + 4 * g;
    const float4 lo = *reinterpret_cast<const float4 *>(p);
    const float4 hi = *reinterpret_cast<const float4 *>(p + 16);
    frag f;
    f.v[0] = lo.x; f.v[1] = lo.y; f.v[2] = lo.z; f.v[3] = lo.w;
    f.v[4] = hi.x; f.v[5] = hi.y; f.v[6] = hi.z; f.v[7] = hi.w;
    return f;
  }
  static __device__ __forceinline__ frag from_acc(const f32x4 &t0, const f32x4 &t1) {
    frag f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f.v[i] = t0[i];
      f.v[4 + i] = t1[i];
    }
    return f;
  }
  static __device__ __forceinline__ frag zero() {
    frag f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f.v[i] = 0.0f;
    return f;
  }
  static __device__ __forceinline__ elem cvt(float x) { return x; }
};

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.0f, 0.0f, 0.0f, 0.0f}; }

// ---- gates from raw projections ----------------------------------------------
// GatedDeltaNet._compute_gates (page "core.ssm.gated_delta_net.gdn") turns the
// per-token projections alpha and b into the gates with the per-head parameters
// A_log and dt_bias; read as the softplus time-step parametrisation those names
// denote:  g = -exp(A_log) softplus(alpha + dt_bias),  beta = sigmoid(b).
// Evaluated in float32 with the library's correctly rounded-to-1-ulp expf and
// log1pf (softplus split at 0, so that exp never overflows); a float32 g carries
// the same information as a float32 g given as input.
__device__ __forceinline__ float softplus_f32(float x) {
  return x > 0.0f ? x + log1pf(expf(-x)) : log1pf(expf(x));
}
// g from the raw decay projection; A = exp(A_log[h]) is passed precomputed
__device__ __forceinline__ float gate_decay(float alpha, float A, float dt_bias) {
  return -A * softplus_f32(alpha + dt_bias);
}
__device__ __forceinline__ float gate_beta(float b) { return 1.0f / (1.0f + expf(-b)); }

// element e of a fragment, from a float
__device__ __forceinline__ void set_frag(Mma<false>::frag &f, int e, float x) {
  f.v[e] = static_cast<_Float16>(x);
}
__device__ __forceinline__ void set_frag(Mma<true>::frag &f, int e, float x) { f.v[e] = x; }

// eight floats -> eight consecutive operand elements in LDS (one 16-byte store
// for fp16, two for fp32)
__device__ __forceinline__ void store8(_Float16 *dst, const float (&x)[8]) {
  f16x8 h;
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = static_cast<_Float16>(x[e]);
  *reinterpret_cast<f16x8 *>(dst) = h;
}
__device__ __forceinline__ void store8(float *dst, const float (&x)[8]) {
  *reinterpret_cast<float4 *>(dst) = make_float4(x[0], x[1], x[2], x[3]);
  *reinterpret_cast<float4 *>(dst + 4) = make_float4(x[4], x[5], x[6], x[7]);
}

// two floats -> two consecutive operand elements in LDS (one 32-bit store for fp16)
__device__ __forceinline__ void store2(_Float16 *dst, float a, float b) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  f16x2 h;
  h[0] = static_cast<_Float16>(a);
  h[1] = static_cast<_Float16>(b);
  *reinterpret_cast<f16x2 *>(dst) = h;
}
__device__ __forceinline__ void store2(float *dst, float a, float b) {
  *reinterpret_cast<float2 *>(dst) = make_float2(a, b);
}
// eight consecutive operand elements in LDS -> floats
__device__ __forceinline__ void load8(const _Float16 *p, float (&x)[8]) {
  const f16x8 h = *reinterpret_cast<const f16x8 *>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = static_cast<float>(h[e]);
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t b) { return bf16_to_f32(b); }

// Accumulator -> LDS float matrix (row-major, leading dimension ld).
__device__ __forceinline__ void store_acc(float *base, int ld, int row0, int col0,
                                          const f32x4 &t, int lane) {
  const int c = lane & 15, r = 4 * (lane >> 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) base[(row0 + r + i) * ld + col0 + c] = t[i];
}

// XCD-aware work mapping.  Work items come in groups of `gsize` consecutive
// items that read the same inputs (the value-column tiles and grouped value
// heads of one query/key head).  Workgroups are dispatched round-robin over the
// eight XCDs, so group j is placed on XCD j % 8 and its members on consecutive
// dispatch slots there: members share that XCD's L2.  Returns -1 for the
// padding blocks of the rounded-up grid.
__device__ __forceinline__ int xcd_work_item(int block, int gsize, int ngroups) {
  const int xcd = block & 7;
  const int pos = block >> 3;
  const int group = (pos / gsize) * 8 + xcd;
  if (group >= ngroups) return -1;
  return group * gsize + pos % gsize;
}

}  // namespace gdr
