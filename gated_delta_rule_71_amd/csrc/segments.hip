// Long batched sequences split into segments that run in parallel.
//
// The recurrence is linear in the state: a segment entering with state H_in (the
// [K, V] matrix S^T) leaves with
//     H_out = A H_in + F,
// where F is what the segment leaves from a zero state and A (K x K) is the
// segment's transition: the same recurrence run with zero values from the identity
// (each step maps H to exp(g) (I - beta k k^T) H, applied to the left of the stored
// [K, V] state).  So a sequence of S segments needs
//   1. every segment from a zero state (F, no outputs),
//   2. every segment with zero values from the identity (A, no outputs),
//   3. the entering states H_in, one segment after another (this file: a K x K by
//      K x V product per segment), and
//   4. every segment from its true entering state, writing the outputs,
// where 1, 2 and 4 are ordinary chunked prefills over the segments as packed
// sequences.  The chain of dependent chunk steps per workgroup shortens by the
// factor S at the cost of three passes instead of one; the host takes this path
// only when the sequences alone leave most compute units idle.

#include "common.hpp"
#include "gdr_internal.hpp"

namespace gdr {

// cu_seqlens of the segments, and identity states [segments, Hv, DK, DK].  Packed
// sequences are planned by one thread: sequence n gets max(1, ceil(L_n / seg_len))
// consecutive slots (the host sizes seg_len so that they never exceed S; the count is
// still clamped so that no write leaves the slot arrays), and the remaining slots are
// empty segments at the end of the tokens.
__global__ void segment_setup_kernel(const SegmentParams p, long n_ident) {
  const long i = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (p.src_cu) {
    if (i == 0) {
      int s = 0;
      for (int n = 0; n < p.batch; ++n) {
        const int a = p.src_cu[n], e = p.src_cu[n + 1];
        int c = e > a ? (e - a + p.seg_len - 1) / p.seg_len : 1;
        if (c > p.S - s) c = p.S - s;
        p.first[n] = s;
        for (int j = 0; j < c; ++j) p.cu[s + j] = a + j * p.seg_len;
        s += c;
      }
      p.first[p.batch] = s;
      for (; s <= p.S; ++s) p.cu[s] = p.src_cu[p.batch];
    }
  } else {
    const int nseq = p.batch * p.S;
    if (i <= nseq) {
      const int b = static_cast<int>(i / p.S), s = static_cast<int>(i % p.S);
      p.cu[i] = i == nseq ? p.batch * p.seqlen : b * p.seqlen + min(s * p.seg_len, p.seqlen);
    }
  }
  if (i < n_ident) {
    const int e = static_cast<int>(i % (static_cast<long>(p.DK) * p.DK));
    p.ident[i] = (e / p.DK == e % p.DK) ? 1.0f : 0.0f;
  }
}

// One workgroup per (batch row, value head, 16 state columns): H starts from the
// initial state (or zero); for each segment s, H_in[s] = H, then H <- A_s H + F_s;
// the last H is the final state.  The whole K x K transition of a segment sits in
// LDS; the next segment's is fetched into registers (16-byte loads) while the
// current product runs, so each segment exposes at most one load latency.  The
// product A_s H runs on the fp32 matrix cores (v_mfma_f32_16x16x4f32): each of the
// four waves owns DK / 64 tiles of 16 rows x 16 columns of H in accumulator
// layout (lane l: column l % 16, rows 4 (l / 16) + v).
constexpr int kCombineCols = 16;

template <int DK>
__global__ void __launch_bounds__(256) segment_combine_kernel(const SegmentParams p) {
  constexpr int TC = kCombineCols;
  // LDS strides against the 64 four-byte banks: A is read with 16 lanes on 16
  // rows and 4 along a row (stride 4 mod 64 words), H with 16 lanes along a row
  // and 4 rows (stride 16)
  constexpr int LDA = DK + 4, LDH = TC;
  constexpr int NT = DK / 64;                   // 16-row tiles per wave
  constexpr int A4 = DK * DK / 4 / 256;         // 16-byte pieces of A per thread
  constexpr int KB = 4;                         // k-steps per batch of operand reads
  static_assert(TC == 16 && NT >= 1, "combine tiling");
  __shared__ float sA[DK * LDA];
  __shared__ float sH[DK * LDH];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int ntile = p.DV / TC;
  const int vt = blockIdx.x % ntile;
  const int h = (blockIdx.x / ntile) % p.Hv;
  const int b = blockIdx.x / ntile / p.Hv;
  const size_t sv = static_cast<size_t>(DK) * p.DV, sa = static_cast<size_t>(DK) * DK;
  // this row's segments, and where its state comes from and goes (slot -1: read
  // slot 0, write nothing)
  const int s_begin = p.src_cu ? p.first[b] : b * p.S;
  const int s_end = p.src_cu ? p.first[b + 1] : s_begin + p.S;
  int src = b, dst = b;
  if (p.state_indices) {
    const int idx = p.state_indices[b];
    src = idx < 0 ? 0 : idx;
    dst = idx;
  }
  // row of this lane's element v of tile t
  auto row = [&](int t, int v) { return 16 * (wave * NT + t) + 4 * g + v; };
  const size_t col = static_cast<size_t>(TC) * vt + i;
  f32x4 H[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v)
      H[t][v] = p.initial_state
                    ? p.initial_state[(static_cast<size_t>(src) * p.Hv + h) * sv +
                                      static_cast<size_t>(row(t, v)) * p.DV + col]
                    : 0.0f;
  float4 ra[A4];
  auto fetchA = [&](const float *A) {
#pragma unroll
    for (int j = 0; j < A4; ++j) ra[j] = reinterpret_cast<const float4 *>(A)[tid + 256 * j];
  };
  if (s_begin < s_end) fetchA(p.A + (static_cast<size_t>(s_begin) * p.Hv + h) * sa);
  for (int s = s_begin; s < s_end; ++s) {
    const size_t seq = static_cast<size_t>(s);
    float *hin = p.H_in + (seq * p.Hv + h) * sv + col;
    const float *F = p.F + (seq * p.Hv + h) * sv + col;
    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[t][v] = F[static_cast<size_t>(row(t, v)) * p.DV];
    __syncthreads();   // the previous segment's product has read sA and sH
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        hin[static_cast<size_t>(row(t, v)) * p.DV] = H[t][v];
        sH[row(t, v) * LDH + i] = H[t][v];
      }
#pragma unroll
    for (int j = 0; j < A4; ++j) {
      const int e = 4 * (tid + 256 * j), r = e / DK, q = e % DK;
      float *d = sA + r * LDA + q;
      d[0] = ra[j].x;
      d[1] = ra[j].y;
      d[2] = ra[j].z;
      d[3] = ra[j].w;
    }
    __syncthreads();
    if (s + 1 < s_end) fetchA(p.A + ((seq + 1) * p.Hv + h) * sa);
    // acc += A_s H over k, the operands of KB k-steps read before their products
    const float *a0 = sA + (16 * wave * NT + i) * LDA + g;
    const float *b0 = sH + g * LDH + i;
#pragma unroll
    for (int k = 0; k < DK; k += 4 * KB) {
      float xa[KB][NT], xb[KB];
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        xb[u] = b0[(k + 4 * u) * LDH];
#pragma unroll
        for (int t = 0; t < NT; ++t) xa[u][t] = a0[16 * t * LDA + k + 4 * u];
      }
#pragma unroll
      for (int u = 0; u < KB; ++u)
#pragma unroll
        for (int t = 0; t < NT; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[u][t], xb[u], acc[t], 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) H[t] = acc[t];
  }
  if (p.final_state && dst >= 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        p.final_state[(static_cast<size_t>(dst) * p.Hv + h) * sv +
                      static_cast<size_t>(row(t, v)) * p.DV + col] = H[t][v];
  }
}

hipError_t launch_segment_setup(const SegmentParams &p, hipStream_t stream) {
  const long nseg = p.src_cu ? p.S : static_cast<long>(p.batch) * p.S;
  const long n_ident = nseg * p.Hv * p.DK * p.DK;
  const long n = n_ident > nseg + 1 ? n_ident : nseg + 1;
  hipLaunchKernelGGL(segment_setup_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, p,
                     n_ident);
  return hipGetLastError();
}

hipError_t launch_segment_combine(const SegmentParams &p, hipStream_t stream) {
  const dim3 grid(p.batch * p.Hv * (p.DV / kCombineCols));
  if (p.DK == 64)
    hipLaunchKernelGGL(segment_combine_kernel<64>, grid, dim3(256), 0, stream, p);
  else if (p.DK == 128)
    hipLaunchKernelGGL(segment_combine_kernel<128>, grid, dim3(256), 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace gdr
