// The steps on either side of the recurrence in a Gated DeltaNet / Gated Delta
// Product layer (Megatron Core API pages "core.ssm.gated_delta_net.gdn" and
// "core.ssm.gated_delta_product"):
//   * the short depthwise causal convolution over the packed V/K/Q projection
//     (GatedDeltaProductMixer d_conv = 4, _prepare_qkv with conv_initial_states
//     for chunked prefill, _decode_conv for the cached decode step), with a
//     slot-indexed conv state holding each request's last W-1 inputs;
//   * the gated RMS normalisation of the recurrence output (ExtendedRMSNorm, an
//     RMSNormGated; norm_before_gate chooses where the gate applies).
// All three kernels are bandwidth-bound streams: consecutive threads take
// consecutive channel groups (16-byte accesses where the width allows), the conv
// window lives in registers, and the norm reduces each (token, head) group across
// G/8 lanes, several rows per lane group in flight.

#include "common.hpp"
#include "gdr_internal.hpp"

namespace gdr {

namespace {

// SiLU(x) = x / (1 + e^-x) on the hardware base-2 exponential and reciprocal
// (about one ulp each); e^-x = inf for very negative x gives x * 0 = -0.
__device__ __forceinline__ float silu(float x) {
  const float e = __builtin_amdgcn_exp2f(-x * 1.4426950408889634f);
  return x * __builtin_amdgcn_rcpf(1.0f + e);
}

__device__ __forceinline__ void load4in(const uint16_t *p, float (&x)[4]) {
  const uint2 u = *reinterpret_cast<const uint2 *>(p);
  x[0] = __uint_as_float(u.x << 16);
  x[1] = __uint_as_float(u.x & 0xffff0000u);
  x[2] = __uint_as_float(u.y << 16);
  x[3] = __uint_as_float(u.y & 0xffff0000u);
}
__device__ __forceinline__ void load4in(const float *p, float (&x)[4]) {
  const float4 a = *reinterpret_cast<const float4 *>(p);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
}
__device__ __forceinline__ void store4out(uint16_t *p, const float (&y)[4]) {
  const uint2 u = {static_cast<uint32_t>(f32_to_bf16(y[0])) |
                       (static_cast<uint32_t>(f32_to_bf16(y[1])) << 16),
                   static_cast<uint32_t>(f32_to_bf16(y[2])) |
                       (static_cast<uint32_t>(f32_to_bf16(y[3])) << 16)};
  *reinterpret_cast<uint2 *>(p) = u;
}
__device__ __forceinline__ void store4out(float *p, const float (&y)[4]) {
  *reinterpret_cast<float4 *>(p) = make_float4(y[0], y[1], y[2], y[3]);
}

// N consecutive channels (N = 4 or 8; 8-, 16- or 32-byte accesses)
template <int N>
__device__ __forceinline__ void loadN(const uint16_t *p, float (&x)[N]) {
  if constexpr (N == 8) {
    load8(p, x);
  } else {
    load4in(p, x);
  }
}
template <int N>
__device__ __forceinline__ void loadN(const float *p, float (&x)[N]) {
  if constexpr (N == 8) {
    load8(p, x);
  } else {
    load4in(p, x);
  }
}
template <int N>
__device__ __forceinline__ void storeN(uint16_t *p, const float (&y)[N]) {
  if constexpr (N == 8) {
    uint4 u;
    uint32_t *w = reinterpret_cast<uint32_t *>(&u);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(f32_to_bf16(y[2 * i])) |
             (static_cast<uint32_t>(f32_to_bf16(y[2 * i + 1])) << 16);
    *reinterpret_cast<uint4 *>(p) = u;
  } else {
    store4out(p, y);
  }
}
template <int N>
__device__ __forceinline__ void storeN(float *p, const float (&y)[N]) {
#pragma unroll
  for (int i = 0; i < N; i += 4)
    *reinterpret_cast<float4 *>(p + i) = make_float4(y[i], y[i + 1], y[i + 2], y[i + 3]);
}

// sequence holding token t: the last n with cu[n] <= t (cu non-decreasing)
__device__ __forceinline__ int find_seq(const int32_t *cu, int num_seqs, int t) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

constexpr int kConvTokens = 64;   // tokens per thread in the prefill conv

// One output token: y = act(b + sum_j w_j x[t - (W-1) + j]); win holds the W-1
// previous inputs (oldest first), N channels.
template <int W, int N>
__device__ __forceinline__ void conv_step(const float (&w)[N][W], const float (&b)[N],
                                          float (&win)[W - 1][N], const float (&x)[N],
                                          int act, float (&y)[N]) {
#pragma unroll
  for (int c = 0; c < N; ++c) {
    float acc = b[c] + w[c][W - 1] * x[c];
#pragma unroll
    for (int j = 0; j < W - 1; ++j) acc += w[c][j] * win[j][c];
    y[c] = act ? silu(acc) : acc;
  }
#pragma unroll
  for (int j = 0; j + 1 < W - 1; ++j)
#pragma unroll
    for (int c = 0; c < N; ++c) win[j][c] = win[j + 1][c];
#pragma unroll
  for (int c = 0; c < N; ++c) win[W - 2][c] = x[c];
}

template <int W, int N>
__device__ __forceinline__ void load_weights(const ConvParams &p, int c0, float (&w)[N][W],
                                             float (&b)[N]) {
#pragma unroll
  for (int c = 0; c < N; ++c) {
#pragma unroll
    for (int j = 0; j < W; ++j) w[c][j] = p.weight[static_cast<size_t>(c0 + c) * W + j];
    b[c] = p.bias ? p.bias[c0 + c] : 0.0f;
  }
}

// window of the W-1 inputs before sequence n's first token: its conv state row
template <int W, int N>
__device__ __forceinline__ void load_window(const ConvParams &p, int n, int c0,
                                            float (&win)[W - 1][N]) {
  const float *st = nullptr;
  if (p.conv_state) {
    const int idx = p.state_indices ? p.state_indices[n] : n;
    st = p.conv_state + (static_cast<size_t>(idx < 0 ? 0 : idx) * p.C + c0) * (W - 1);
  }
#pragma unroll
  for (int c = 0; c < N; ++c)
#pragma unroll
    for (int j = 0; j < W - 1; ++j) win[j][c] = st ? st[c * (W - 1) + j] : 0.0f;
}

// ---- prefill: outputs ---------------------------------------------------------------
// Each thread runs N consecutive channels through kConvTokens tokens, kAhead tokens'
// inputs in flight at a time, with the window in registers.
template <typename T, int W, int N>
__global__ void __launch_bounds__(256) conv_prefill_kernel(const ConvParams p) {
  const int cg = blockIdx.y * 256 + threadIdx.x;   // N-channel group
  if (cg * N >= p.C) return;
  const int c0 = N * cg;
  const int tb = blockIdx.x * kConvTokens;
  const int te = min(tb + kConvTokens, p.tokens);
  if (tb >= te) return;
  float w[N][W], b[N];
  load_weights<W, N>(p, c0, w, b);
  const T *x = static_cast<const T *>(p.x);
  T *y = static_cast<T *>(p.out);

  int n = find_seq(p.cu_seqlens, p.num_seqs, tb);
  float win[W - 1][N];
  // window before token tb: inputs of this sequence where they exist, else its state
  {
    const int t0 = p.cu_seqlens[n];
    float sw[W - 1][N];
    load_window<W, N>(p, n, c0, sw);
#pragma unroll
    for (int j = 0; j < W - 1; ++j) {
      const int tau = tb - (W - 1) + j;
      if (tau >= t0) {
        float v[N];
        loadN<N>(x + static_cast<size_t>(tau) * p.C + c0, v);
#pragma unroll
        for (int c = 0; c < N; ++c) win[j][c] = v[c];
      } else {
        // tau - t0 in [-(W-1), -1] -> state entry (W-1) + (tau - t0)
        const int e = (W - 1) + (tau - t0);
#pragma unroll
        for (int c = 0; c < N; ++c) {
          float sv = 0.0f;
#pragma unroll
          for (int k = 0; k < W - 1; ++k) sv = (k == e) ? sw[k][c] : sv;
          win[j][c] = sv;
        }
      }
    }
  }
  int next = p.cu_seqlens[n + 1];
  constexpr int kAhead = 4;
  for (int tg = tb; tg < te; tg += kAhead) {
    float v[kAhead][N];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      const int t = min(tg + u, te - 1);   // clamped; only t < te is used
      loadN<N>(x + static_cast<size_t>(t) * p.C + c0, v[u]);
    }
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      const int t = tg + u;
      if (t >= te) break;
      if (t >= next) {   // a new sequence starts at t: its window is its state
        while (n + 1 < p.num_seqs && p.cu_seqlens[n + 1] <= t) ++n;
        next = p.cu_seqlens[n + 1];
        load_window<W, N>(p, n, c0, win);
      }
      float o[N];
      conv_step<W, N>(w, b, win, v[u], p.activation, o);
      storeN<N>(y + static_cast<size_t>(t) * p.C + c0, o);
    }
  }
}

// ---- prefill: conv states (after the outputs, so that no state is overwritten
// before the first tokens of its sequence have read it) ---------------------------------
template <typename T, int W>
__global__ void __launch_bounds__(256) conv_state_kernel(const ConvParams p) {
  const int cg = blockIdx.x * 256 + threadIdx.x;
  const int n = blockIdx.y;
  if (cg * 4 >= p.C) return;
  const int idx = p.state_indices ? p.state_indices[n] : n;
  if (idx < 0) return;   // padding writes nothing
  const int c0 = 4 * cg;
  const int t0 = p.cu_seqlens[n], t1 = p.cu_seqlens[n + 1];
  float *st = p.conv_state + (static_cast<size_t>(idx) * p.C + c0) * (W - 1);
  float old[W - 1][4], nw[W - 1][4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int j = 0; j < W - 1; ++j) old[j][c] = st[c * (W - 1) + j];
  const T *x = static_cast<const T *>(p.x);
#pragma unroll
  for (int j = 0; j < W - 1; ++j) {
    const int tau = t1 - (W - 1) + j;   // the last W-1 inputs, oldest first
    if (tau >= t0) {
      float v[4];
      load4in(x + static_cast<size_t>(tau) * p.C + c0, v);
#pragma unroll
      for (int c = 0; c < 4; ++c) nw[j][c] = v[c];
    } else {
      const int e = (W - 1) + (tau - t0);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float s = 0.0f;
#pragma unroll
        for (int k = 0; k < W - 1; ++k) s = (k == e) ? old[k][c] : s;
        nw[j][c] = s;
      }
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int j = 0; j < W - 1; ++j) st[c * (W - 1) + j] = nw[j][c];
}

// ---- decode: T tokens per request over the cached window --------------------------------
template <typename T, int W>
__global__ void __launch_bounds__(256) conv_decode_kernel(const ConvParams p) {
  const int cg = blockIdx.x * 256 + threadIdx.x;
  const int i = blockIdx.y;   // request
  if (cg * 4 >= p.C) return;
  const int c0 = 4 * cg;
  const int r = p.state_indices ? p.state_indices[i] : i;
  float *st = p.conv_state + (static_cast<size_t>(r < 0 ? 0 : r) * p.C + c0) * (W - 1);
  float w[4][W], b[4], win[W - 1][4];
  load_weights<W, 4>(p, c0, w, b);
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int j = 0; j < W - 1; ++j) win[j][c] = st[c * (W - 1) + j];
  const T *x = static_cast<const T *>(p.x);
  T *y = static_cast<T *>(p.out);
  for (int t = 0; t < p.num_tokens; ++t) {
    const size_t row = static_cast<size_t>(i) * p.num_tokens + t;
    float v[4], o[4];
    load4in(x + row * p.C + c0, v);
    conv_step<W, 4>(w, b, win, v, p.activation, o);
    store4out(y + row * p.C + c0, o);
    if (p.intermediate_state && r >= 0) {
      float *is = p.intermediate_state + (row * p.C + c0) * (W - 1);
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int j = 0; j < W - 1; ++j) is[c * (W - 1) + j] = win[j][c];
    }
  }
  if (r < 0) return;   // padding writes nothing
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int j = 0; j < W - 1; ++j) st[c * (W - 1) + j] = win[j][c];
}

// ---- gated RMS norm: G/8 lanes per (token, head) group, 8 elements per lane ------------
__device__ __forceinline__ void load8e(const uint16_t *p, float (&x)[8]) { load8(p, x); }
__device__ __forceinline__ void load8e(const float *p, float (&x)[8]) { load8(p, x); }
__device__ __forceinline__ void store8e(uint16_t *p, const float (&y)[8]) {
  const float a[4] = {y[0], y[1], y[2], y[3]}, b[4] = {y[4], y[5], y[6], y[7]};
  store4out(p, a);
  store4out(p + 4, b);
}
__device__ __forceinline__ void store8e(float *p, const float (&y)[8]) {
  *reinterpret_cast<float4 *>(p) = make_float4(y[0], y[1], y[2], y[3]);
  *reinterpret_cast<float4 *>(p + 4) = make_float4(y[4], y[5], y[6], y[7]);
}

// Each group of G/8 lanes normalises kNormRows rows (the rows of a block, RPB apart):
// all their x and z loads are issued before the first reduction, so that 2 kNormRows
// 16-byte loads per lane are in flight.
constexpr int kNormRows = 4;

template <typename T, int G>
__global__ void __launch_bounds__(256) gated_rmsnorm_kernel(const NormParams p) {
  constexpr int LPR = G / 8;            // lanes per row
  constexpr int RPB = 256 / LPR;        // rows per block and step
  constexpr int R = kNormRows;
  const int sub = threadIdx.x % LPR;
  const long row0 = static_cast<long>(blockIdx.x) * RPB * R + threadIdx.x / LPR;
  float xv[R][8], zv[R][8];
  size_t base[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const long row = row0 + static_cast<long>(k) * RPB;
    const long r = row < p.rows ? row : p.rows - 1;   // clamped: every lane of a group reduces
    base[k] = static_cast<size_t>(r) * G + 8 * sub;
    load8e(static_cast<const T *>(p.x) + base[k], xv[k]);
    load8e(static_cast<const T *>(p.z) + base[k], zv[k]);
  }
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const long row = row0 + static_cast<long>(k) * RPB;
    const long r = row < p.rows ? row : p.rows - 1;
    const int head = static_cast<int>(r % p.heads);
    float u[8], ss = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      u[e] = p.norm_before_gate ? xv[k][e] : xv[k][e] * silu(zv[k][e]);
      ss += u[e] * u[e];
    }
#pragma unroll
    for (int o = LPR / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    const float rs = 1.0f / sqrtf(ss / G + p.eps);
    const float *wt = p.weight + static_cast<size_t>(head) * G + 8 * sub;
    const float4 w0 = *reinterpret_cast<const float4 *>(wt);
    const float4 w1 = *reinterpret_cast<const float4 *>(wt + 4);
    const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    float yv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      yv[e] = u[e] * rs * wv[e];
      if (p.norm_before_gate) yv[e] *= silu(zv[k][e]);
    }
    if (row < p.rows) store8e(static_cast<T *>(p.out) + base[k], yv);
  }
}

template <typename T>
hipError_t conv_dispatch(const ConvParams &p, int mode, hipStream_t s) {
  const int groups = p.C / 4;
  const dim3 block(256);
  auto go = [&](auto width) -> hipError_t {
    constexpr int W = decltype(width)::value;
    if (mode == 0) {
      if (p.tokens > 0) {
        const int tb = (p.tokens + kConvTokens - 1) / kConvTokens;
        // 4 channels (8-byte bf16 accesses) and 4 tokens in flight per thread: measured
        // on the packed workload's shape, within 5% of 8 channels or 8 tokens and
        // without their register cost
        hipLaunchKernelGGL((conv_prefill_kernel<T, W, 4>), dim3(tb, (groups + 255) / 256), block,
                           0, s, p);
      }
      if (p.conv_state && p.num_seqs > 0)
        hipLaunchKernelGGL((conv_state_kernel<T, W>), dim3((groups + 255) / 256, p.num_seqs),
                           block, 0, s, p);
    } else {
      hipLaunchKernelGGL((conv_decode_kernel<T, W>), dim3((groups + 255) / 256, p.batch), block,
                         0, s, p);
    }
    return hipGetLastError();
  };
  if (p.W == 2) return go(std::integral_constant<int, 2>());
  if (p.W == 3) return go(std::integral_constant<int, 3>());
  if (p.W == 4) return go(std::integral_constant<int, 4>());
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t norm_dispatch(const NormParams &p, hipStream_t s) {
  const dim3 block(256);
  auto grid = [&](int g) {
    const long per_block = static_cast<long>(256 / (g / 8)) * kNormRows;
    return dim3(static_cast<unsigned>((p.rows + per_block - 1) / per_block));
  };
  if (p.group == 64)
    hipLaunchKernelGGL((gated_rmsnorm_kernel<T, 64>), grid(64), block, 0, s, p);
  else if (p.group == 128)
    hipLaunchKernelGGL((gated_rmsnorm_kernel<T, 128>), grid(128), block, 0, s, p);
  else if (p.group == 256)
    hipLaunchKernelGGL((gated_rmsnorm_kernel<T, 256>), grid(256), block, 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_conv(const ConvParams &p, int f32, int mode, hipStream_t stream) {
  return f32 ? conv_dispatch<float>(p, mode, stream) : conv_dispatch<uint16_t>(p, mode, stream);
}

hipError_t launch_gated_rmsnorm(const NormParams &p, int f32, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  return f32 ? norm_dispatch<float>(p, stream) : norm_dispatch<uint16_t>(p, stream);
}

}  // namespace gdr
