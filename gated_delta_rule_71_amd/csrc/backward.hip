// Chunked backward of the gated delta rule on gfx950 (training through
// torch_chunk_gated_delta_rule, Megatron Core API page
// "core.ssm.gated_delta_net.gdn"; the chunked training kernels of the Gated
// DeltaNet and Gated Delta Product pages).
//
// Given the gradients dO of the outputs and dH_T of the final state, produce the
// gradients of q, k, v, g, beta and the initial state.  With the state kept as
// H = S^T (K x V) and one chunk of n = 64 tokens entering with state H0
// (G the cumulative decay inside the chunk, Gamma[r, i] = exp(G_r - G_i)):
//   forward   A = strict_lower(diag(beta) (K K^T) * Gamma),  T = (I + A)^-1,
//             R = diag(beta) V - diag(beta e^G) K H0,  D = T R,
//             O = diag(scale e^G) Q H0 + P D,  P = scale (Q K^T) * Gamma * [i <= r],
//             H_n = e^{G_n} H0 + K~^T D,  K~ = diag(e^{G_n - G}) K;
//   backward  dD = P^T dO + K~ dH_n,  dR = T^T dD,  dV = diag(beta) dR,
//             dH0 = e^{G_n} dH_n + Q^T diag(scale e^G) dO - K^T diag(beta e^G) dR,
//             dA = -strict_lower(dR D^T),  dP = lower(dO D^T),
//             dQ = diag(scale e^G) dO H0^T + dPs K,
//             dK = dAs K + dAs^T K + dPs^T Q - diag(beta e^G) dR H0^T
//                  + diag(e^{G_n - G}) D dH_n^T,
//   with dAs = dA * diag(beta) Gamma, dPs = scale dP * Gamma, and dbeta, dg from
//   the same quantities (row sums, see bwd_grads_kernel).
// With n_h Householder sub-steps per token (the gated delta product) the same
// algebra runs on rows t * n_h + j: k, v, beta per row, g on each token's first row,
// q and dO on its last row (zero on the others).
// Only the dH0 recursion is sequential over a sequence's chunks; everything else
// is local to a chunk once the chunk's entering state H0 and leaving gradient
// dH_n are known.  Hence four launches after a table of chunk offsets:
//   1. the forward prefill with a boundary state every 64 tokens (the H0 of every
//      chunk after the first) into the workspace;
//   2. bwd_local_kernel, one workgroup per (chunk, value head): Gamma, A, P,
//      T = (I + A)^-1 (by 16 x 16 blocks) and D = T R;
//   3. bwd_sweep_kernel, one workgroup per (sequence, value head, 32 or 16 value
//      columns), last chunk to first: dH_n of every chunk, dR, dV and dH0;
//   4. bwd_grads_kernel, one workgroup per (chunk, value head): dQ, dK, dbeta, dg;
//   5. with grouped heads (Hv > Hk), a sum of dQ, dK over each group.
// The contractions run on the fp32 matrix cores (v_mfma_f32_16x16x4f32) with
// operands in LDS; the cumulative decay is summed in fp64 so that differences of
// large sums stay exact.

#include "chunk_helpers.hpp"
#include "common.hpp"
#include "gdr_internal.hpp"

namespace gdr {
namespace {

constexpr int BC = 64;        // tokens per backward chunk
constexpr int BT = 512;       // threads per workgroup (two waves per SIMD)
constexpr int kCUs = 256;     // compute units
constexpr int NW = BT / 64;   // waves per workgroup
constexpr int LDC = BC + 1;   // 64 x 64 tiles read one row or one column per thread

// LDS row strides (floats) for matrix-core operands, against the 64 four-byte LDS
// banks.  An operand read in mmf has 16 lanes along one index of the matrix and 4
// along the other.  With the 16 lanes on 16 rows (4 along a row) the read is
// conflict-free at a stride of 4 x odd (mod 64); with the 16 lanes along a row (4
// rows) at 16 x odd (mod 64); a matrix read both ways takes 17 (mod 64), where only
// 3 lane pairs share a bank.  (A stride of n + 1 makes such reads up to 4-way.)
constexpr int ld_up(int n, int m, int r) { return n + ((r - n) % m + m) % m; }
constexpr int ld_row_read(int n) { return ld_up(n, 8, 4); }
constexpr int ld_col_read(int n) { return ld_up(n, 32, 16); }
constexpr int ld_any_read(int n) { return ld_up(n, 64, 17); }
static_assert(ld_row_read(32) == 36 && ld_row_read(128) == 132 && ld_col_read(16) == 16 &&
                  ld_col_read(32) == 48 && ld_col_read(64) == 80 && ld_any_read(128) == 145,
              "LDS strides");

// Wave-tiled fp32 matrix-core products.  An M x N output is cut into 16 x 16
// tiles, numbered row by row; wave w owns the TPW consecutive tiles w*TPW ..
// w*TPW + TPW - 1, which lie in one tile row (TPW divides N / 16).  Lane l holds,
// of each of its tiles, column l % 16 and rows 4 (l / 16) + v, v = 0..3: the
// accumulator layout of v_mfma_f32_16x16x4f32, whose operands are A[l % 16][l / 16]
// (16 rows x 4) and B[l / 16][l % 16] (4 x 16 columns).
template <int N, int TPW>
struct WTile {
  static_assert((N / 16) % TPW == 0, "a wave's tiles share one tile row");
  int r0, c0;
  __device__ __forceinline__ explicit WTile(int wave) {
    const int idx = wave * TPW;
    r0 = (idx / (N / 16)) * 16;
    c0 = (idx % (N / 16)) * 16;
  }
  __device__ __forceinline__ int row(int v, int lane) const { return r0 + 4 * (lane >> 4) + v; }
  __device__ __forceinline__ int col(int t, int lane) const { return c0 + 16 * t + (lane & 15); }
};

// The products acc_j[t] += A_j(rows of the tile row, p) B(p, columns of tile t)
// over p in [0, P), j < NA, sharing the B fragments (each read from LDS once), with
// A_j(r, p) = A_j[r * ars_j + p * acs_j] and B(p, c) = B[p * brs + c * bcs] in LDS,
// P % 16 == 0 (every caller passes 16, 32, 64 or 128).  The operands are read in
// batches of four k-steps, each batch issued before the matrix-core instructions of
// the previous one, so that the reads are in flight while the previous batch
// multiplies (reading and multiplying one k-step at a time would make every
// instruction wait out its own LDS round trip).  mul(j, t, a, b) applies one
// instruction to product j, tile t.
constexpr int KB = 4;   // k-steps per batch
template <int NA, int TPW>
struct OperandBatch {
  float a[KB][NA], b[KB][TPW];
};
template <int NA, int N, int TPW, typename Mul>
__device__ __forceinline__ void mmf_batched(const WTile<N, TPW> &w, const float *const (&A)[NA],
                                            const int (&ars)[NA], const int (&acs)[NA],
                                            const float *B, int brs, int bcs, int P, int lane,
                                            Mul mul) {
  const int i = lane & 15, g = lane >> 4;
  const float *a[NA];
#pragma unroll
  for (int j = 0; j < NA; ++j) a[j] = A[j] + (w.r0 + i) * ars[j] + g * acs[j];
  const float *b = B + g * brs + (w.c0 + i) * bcs;
  auto load = [&](OperandBatch<NA, TPW> &x, int p) {
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int q = p + 4 * u;
#pragma unroll
      for (int j = 0; j < NA; ++j) x.a[u][j] = a[j][q * acs[j]];
#pragma unroll
      for (int t = 0; t < TPW; ++t) x.b[u][t] = b[q * brs + 16 * t * bcs];
    }
  };
  auto multiply = [&](const OperandBatch<NA, TPW> &x) {
#pragma unroll
    for (int u = 0; u < KB; ++u)
#pragma unroll
      for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int j = 0; j < NA; ++j) mul(j, t, x.a[u][j], x.b[u][t]);
  };
  OperandBatch<NA, TPW> x0, x1;
  load(x0, 0);
#pragma unroll
  for (int p = 0; p < P; p += 8 * KB) {
    if (p + 4 * KB < P) load(x1, p + 4 * KB);
    multiply(x0);
    if (p + 4 * KB < P) {
      if (p + 8 * KB < P) load(x0, p + 8 * KB);
      multiply(x1);
    }
  }
}

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// acc += A B (one product)
template <int N, int TPW>
__device__ __forceinline__ void mmf(f32x4 (&acc)[TPW], const WTile<N, TPW> &w, const float *A,
                                    int ars, int acs, const float *B, int brs, int bcs, int P,
                                    int lane) {
  const float *const As[1] = {A};
  const int r[1] = {ars}, c[1] = {acs};
  mmf_batched<1>(w, As, r, c, B, brs, bcs, P, lane,
                 [&](int, int t, float x, float y) { acc[t] = mfma4(x, y, acc[t]); });
}

// acc1 += A1 B, acc2 += A2 B (, acc3 += A3 B); the accumulators may be one array
template <int N, int TPW>
__device__ __forceinline__ void mmf2(f32x4 (&acc1)[TPW], f32x4 (&acc2)[TPW],
                                     const WTile<N, TPW> &w, const float *A1, int ars1, int acs1,
                                     const float *A2, int ars2, int acs2, const float *B, int brs,
                                     int bcs, int P, int lane) {
  const float *const As[2] = {A1, A2};
  const int r[2] = {ars1, ars2}, c[2] = {acs1, acs2};
  mmf_batched<2>(w, As, r, c, B, brs, bcs, P, lane, [&](int j, int t, float x, float y) {
    if (j == 0)
      acc1[t] = mfma4(x, y, acc1[t]);
    else
      acc2[t] = mfma4(x, y, acc2[t]);
  });
}
template <int N, int TPW>
__device__ __forceinline__ void mmf3(f32x4 (&acc1)[TPW], f32x4 (&acc2)[TPW], f32x4 (&acc3)[TPW],
                                     const WTile<N, TPW> &w, const float *A1, int ars1, int acs1,
                                     const float *A2, int ars2, int acs2, const float *A3, int ars3,
                                     int acs3, const float *B, int brs, int bcs, int P, int lane) {
  const float *const As[3] = {A1, A2, A3};
  const int r[3] = {ars1, ars2, ars3}, c[3] = {acs1, acs2, acs3};
  mmf_batched<3>(w, As, r, c, B, brs, bcs, P, lane, [&](int j, int t, float x, float y) {
    if (j == 0)
      acc1[t] = mfma4(x, y, acc1[t]);
    else if (j == 1)
      acc2[t] = mfma4(x, y, acc2[t]);
    else
      acc3[t] = mfma4(x, y, acc3[t]);
  });
}

// fp16 matrix-core products of the form acc_j[t] += X_j Y^T over k in [0, K), both
// row-major fp16 in LDS with k contiguous (leading dimensions ldx, ldy halves, rows
// 16-byte aligned): tile t of wave tile w covers rows r0 .. r0 + 15 of X_j and rows
// c0 + 16 t .. + 15 of Y.  v_mfma_f32_16x16x32_f16: lane l supplies row l % 16 of X_j
// and of Y with contraction indices 8 (l / 16) .. + 7, one 16-byte read each, and its
// accumulator layout is that of the fp32 products above.
template <int NA, int N, int TPW>
__device__ __forceinline__ void mmh_xyt(f32x4 *const (&acc)[NA], const WTile<N, TPW> &w,
                                        const _Float16 *const (&X)[NA], int ldx,
                                        const _Float16 *Y, int ldy, int K, int lane) {
  const int i = lane & 15, g = lane >> 4;
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 32) {
    f16x8 a[NA], b[TPW];
#pragma unroll
    for (int j = 0; j < NA; ++j)
      a[j] = *reinterpret_cast<const f16x8 *>(X[j] + (w.r0 + i) * ldx + k0 + 8 * g);
#pragma unroll
    for (int t = 0; t < TPW; ++t)
      b[t] = *reinterpret_cast<const f16x8 *>(Y + (w.c0 + 16 * t + i) * ldy + k0 + 8 * g);
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int j = 0; j < NA; ++j)
        acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[j], b[t], acc[j][t], 0, 0, 0);
  }
}

template <int TPW>
__device__ __forceinline__ void zero(f32x4 (&acc)[TPW]) {
#pragma unroll
  for (int t = 0; t < TPW; ++t) acc[t] = zero4();
}

// the sequence holding global chunk c: the last n with cb[n] <= c
__device__ __forceinline__ int chunk_seq(const int32_t *cb, int N, int c) {
  int lo = 0, hi = N;   // cb[lo] <= c < cb[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cb[mid] <= c) lo = mid; else hi = mid;
  }
  return lo;
}

// the rows [t0, t1) of sequence n: with n_h Householder sub-steps per token, row
// t * n_h + j is sub-step j of token t (k, v, beta and their gradients are per row;
// q, dO and dq sit on each token's last row, g and dg on its first)
__device__ __forceinline__ void seq_span(const BackwardParams &p, int n, int &t0, int &t1) {
  if (p.cu_seqlens) {
    t0 = p.cu_seqlens[n];
    t1 = p.cu_seqlens[n + 1];
  } else {
    t0 = n * p.seqlen;
    t1 = t0 + p.seqlen;
  }
  t0 *= p.nh;
  t1 *= p.nh;
}

// Per-chunk row factors in LDS: the fp64 cumulative decay G (restarting at the
// chunk), beta, e^G and e^{G_n - G} (rows past the sequence end carry g = beta = 0,
// so that G_63 is the decay of the whole chunk).  Wave 0 runs the scan.
struct RowFactors {
  double G[BC];
  float beta[BC], eG[BC], eGl[BC];
};
// g and beta of one chunk's rows in registers (thread r < 64 holds row r), so that
// a sweep can fetch them one chunk ahead
struct RowInputs {
  float g, beta;
  __device__ __forceinline__ void fetch(const BackwardParams &p, int h, int ts, int rows,
                                        int tid) {
    g = 0.0f;
    beta = 0.0f;
    if (tid < rows) {
      const int row = ts + tid;
      beta = p.beta[static_cast<size_t>(row) * p.Hv + h];
      if (row % p.nh == 0) g = p.g[static_cast<size_t>(row / p.nh) * p.Hv + h];
    }
  }
};
// the row factors of one chunk, on all 64 lanes of wave 0: the fp64 prefix sum of g
// runs on DPP lane moves (the prefill's scan)
__device__ __forceinline__ void row_factors(RowFactors &rf, const RowInputs &ri, int tid) {
  if (tid < BC) {
    const double x = prefix_sum64(static_cast<double>(ri.g));
    const double last = readlane_f64(x, BC - 1);
    rf.G[tid] = x;
    rf.beta[tid] = ri.beta;
    rf.eG[tid] = expf(static_cast<float>(x));
    rf.eGl[tid] = expf(static_cast<float>(last - x));
  }
}
__device__ __forceinline__ void row_factors(RowFactors &rf, const BackwardParams &p, int h, int ts,
                                            int rows, int tid) {
  RowInputs ri;
  ri.fetch(p, h, ts, rows, tid);
  row_factors(rf, ri, tid);
}

// Rows [0, 64) x NC columns (from col0) of a [tokens, heads, D] input (head `hd`),
// fetched into registers with 8-element loads (addresses clamped to the sequence),
// then stored as fp32 LDS rows of leading dimension ld with rows past `rows` zero.
// Fetch and store are separate so that a fetch can be in flight during other work.
template <typename TIn, int D, int NC>
struct RowsRegs {
  static constexpr int SEGS = NC / 8, UNITS = BC * SEGS, PER = (UNITS + BT - 1) / BT;
  Seg8<TIn> buf[PER];
  // nh > 1: a per-token input (q, dO) read on rows, token (ts + r) / nh, present
  // only on each token's last row
  __device__ __forceinline__ void fetch(const TIn *src, int heads, int hd, int ts, int rows,
                                        int col0, int tid, int nh = 1) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int u = tid + j * BT;
      const int r = min(u / SEGS, rows - 1), sg = u % SEGS;
      if (UNITS % BT == 0 || u < UNITS)
        buf[j].load(src + (static_cast<size_t>((ts + r) / nh) * heads + hd) * D + col0 + 8 * sg);
    }
  }
  __device__ __forceinline__ void store(float *dst, int ld, int rows, int tid, int ts = 0,
                                        int nh = 1) const {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int u = tid + j * BT;
      const int r = u / SEGS, sg = u % SEGS;
      if (UNITS % BT == 0 || u < UNITS) {
        const bool ok = r < rows && (nh == 1 || (ts + r) % nh == nh - 1);
        float x[8];
        buf[j].get(x);
#pragma unroll
        for (int e = 0; e < 8; ++e) dst[r * ld + 8 * sg + e] = ok ? x[e] : 0.0f;
      }
    }
  }
  // the same rows as fp16 (one 16-byte store per segment)
  __device__ __forceinline__ void store_h(_Float16 *dst, int ld, int rows, int tid, int ts = 0,
                                          int nh = 1) const {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int u = tid + j * BT;
      const int r = u / SEGS, sg = u % SEGS;
      if (UNITS % BT == 0 || u < UNITS) {
        const bool ok = r < rows && (nh == 1 || (ts + r) % nh == nh - 1);
        float x[8];
        buf[j].get(x);
        f16x8 h;
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = static_cast<_Float16>(ok ? x[e] : 0.0f);
        *reinterpret_cast<f16x8 *>(dst + r * ld + 8 * sg) = h;
      }
    }
  }
};

template <typename TIn, int D, int NC>
__device__ __forceinline__ void load_rows(float *dst, int ld, const TIn *src, int heads, int hd,
                                          int ts, int rows, int col0, int tid, int nh = 1) {
  RowsRegs<TIn, D, NC> r;
  r.fetch(src, heads, hd, ts, rows, col0, tid, nh);
  r.store(dst, ld, rows, tid, ts, nh);
}

// An NR x NC float32 matrix (global row stride gs; NULL reads as zeros) through
// registers (16-byte loads) into LDS (leading dimension ld).
template <int NR, int NC>
struct MatRegs {
  static constexpr int Q4 = NC / 4, UNITS = NR * Q4, PER = (UNITS + BT - 1) / BT;
  float4 buf[PER];
  __device__ __forceinline__ void fetch(const float *src, size_t gs, int tid) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int u = tid + j * BT;
      buf[j] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (src && (UNITS % BT == 0 || u < UNITS))
        buf[j] = *reinterpret_cast<const float4 *>(src + (u / Q4) * gs + 4 * (u % Q4));
    }
  }
  __device__ __forceinline__ void store(float *dst, int ld, int tid) const {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int u = tid + j * BT;
      if (UNITS % BT == 0 || u < UNITS) {
        float *d = dst + (u / Q4) * ld + 4 * (u % Q4);
        d[0] = buf[j].x;
        d[1] = buf[j].y;
        d[2] = buf[j].z;
        d[3] = buf[j].w;
      }
    }
  }
  // the same matrix as fp16 (one 8-byte store per four values)
  __device__ __forceinline__ void store_h(_Float16 *dst, int ld, int tid) const {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int u = tid + j * BT;
      if (UNITS % BT == 0 || u < UNITS) {
        f16x4 h = {static_cast<_Float16>(buf[j].x), static_cast<_Float16>(buf[j].y),
                   static_cast<_Float16>(buf[j].z), static_cast<_Float16>(buf[j].w)};
        *reinterpret_cast<f16x4 *>(dst + (u / Q4) * ld + 4 * (u % Q4)) = h;
      }
    }
  }
  // as an fp16 pair hi + lo (lo = the rounding error of hi, in fp16): two products
  // with the pair carry ~22 bits of the fp32 value instead of 11
  __device__ __forceinline__ void store_hl(_Float16 *hi, _Float16 *lo, int ld, int tid) const {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int u = tid + j * BT;
      if (UNITS % BT == 0 || u < UNITS) {
        const float x[4] = {buf[j].x, buf[j].y, buf[j].z, buf[j].w};
        f16x4 a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = static_cast<_Float16>(x[e]);
          b[e] = static_cast<_Float16>(x[e] - static_cast<float>(a[e]));
        }
        const int off = (u / Q4) * ld + 4 * (u % Q4);
        *reinterpret_cast<f16x4 *>(hi + off) = a;
        *reinterpret_cast<f16x4 *>(lo + off) = b;
      }
    }
  }
  // sum over this thread's values of the elementwise product with another matrix held
  // the same way
  __device__ __forceinline__ float dot(const MatRegs &o) const {
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      s = fmaf(buf[j].x, o.buf[j].x, s);
      s = fmaf(buf[j].y, o.buf[j].y, s);
      s = fmaf(buf[j].z, o.buf[j].z, s);
      s = fmaf(buf[j].w, o.buf[j].w, s);
    }
    return s;
  }
};

template <int NR, int NC>
__device__ __forceinline__ void load_mat(float *dst, int ld, const float *src, size_t gs, int tid) {
  MatRegs<NR, NC> m;
  m.fetch(src, gs, tid);
  m.store(dst, ld, tid);
}

// the state a chunk enters with: the initial state for a sequence's first chunk,
// else the forward's boundary state after the previous chunk (NULL = zeros)
__device__ __forceinline__ const float *entry_state(const BackwardParams &p, int n, int j, int h,
                                                    int D) {
  const size_t ss = static_cast<size_t>(D) * D;
  if (j == 0)
    return p.initial_state ? p.initial_state + (static_cast<size_t>(n) * p.Hv + h) * ss : nullptr;
  return p.states + (static_cast<size_t>(p.bb[n] + j - 1) * p.Hv + h) * ss;
}

}  // namespace

// chunk table: cb[n] = first global chunk of sequence n (cb[N] = chunk count),
// bb[n] = first boundary state of sequence n (sum of floor(L_m / 64), m < n)
__global__ void bwd_table_kernel(const BackwardParams p) {
  if (threadIdx.x != 0) return;
  int cb = 0, bb = 0;
  for (int n = 0; n < p.num_seqs; ++n) {
    p.cb[n] = cb;
    p.bb[n] = bb;
    int t0, t1;
    seq_span(p, n, t0, t1);
    const int L = t1 - t0;
    cb += (L + BC - 1) / BC;
    bb += L / BC;
  }
  p.cb[p.num_seqs] = cb;
  p.bb[p.num_seqs] = bb;
}

// Per (chunk, value head): Araw = strict_lower((K K^T) * Gamma), P, T = (I + A)^-1
// with A = diag(beta) Araw, and D = T R, R = diag(beta) (V - diag(e^G) K H0).
// The local pass of bf16 inputs (q, k exact in fp16): K K^T and Q K^T exactly on the
// fp16 matrix cores, and the inverse T = (I + A)^-1 on the fp32 path (substitution and
// 16 x 16 block steps).  It writes Araw, P and T only (see the gradient kernel for D).
template <typename TIn, typename TQK, int D>
__device__ __forceinline__ void bwd_local_h16(const BackwardParams &p) {
  using M = Mma<false>;
  using frag = M::frag;
  constexpr int LDA = ld_row_read(BC);   // A: by rows
  constexpr int LDT = ld_row_read(BC);   // T: by rows (by columns only in the block steps)
  constexpr int LDKH = D + 8;            // K, Q rows (fp16)
  constexpr int TPC = (BC / 16) * (BC / 16) / NW;
  // no D = T R here: the gradient kernel forms it slice by slice from H0, which it
  // reads anyway, so this pass reads no state and its LDS fits two workgroups per CU
  __shared__ __align__(16) _Float16 hK[BC * LDKH];
  __shared__ __align__(16) _Float16 hQ[BC * LDKH];
  __shared__ float sA[BC * LDA];
  __shared__ float sT[BC * LDT];
  __shared__ float sM[(BC / 16) * 16 * 17];   // the block steps' 16 x 16 blocks
  __shared__ RowFactors rf;

  const int c = blockIdx.x, h = blockIdx.y;
  if (c >= p.cb[p.num_seqs]) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15;
  const int n = chunk_seq(p.cb, p.num_seqs, c);
  const int j = c - p.cb[n];
  int t0, t1;
  seq_span(p, n, t0, t1);
  const int ts = t0 + BC * j, rows = min(BC, t1 - ts);
  const int hk = h / (p.Hv / p.Hk);

  RowsRegs<TQK, D, D> fk, fq;
  RowInputs fr;
  fr.fetch(p, h, ts, rows, tid);
  fk.fetch(static_cast<const TQK *>(p.k), p.Hk, hk, ts, rows, 0, tid);
  fq.fetch(static_cast<const TQK *>(p.q), p.Hk, hk, ts, rows, 0, tid, p.nh);
  fk.store_h(hK, LDKH, rows, tid);
  fq.store_h(hQ, LDKH, rows, tid, ts, p.nh);
  row_factors(rf, fr, tid);
  __syncthreads();

  const size_t cc = static_cast<size_t>(c) * p.Hv + h;
  {
    // K K^T and Q K^T: operands exact in fp16, one product per 32-deep slice
    const WTile<BC, TPC> w(wave);
    f32x4 kk[TPC], qk[TPC];
    zero(kk);
    zero(qk);
#pragma unroll
    for (int k0 = 0; k0 < D; k0 += 32) {
      const frag ka = M::load(hK, LDKH, w.r0 + l16, k0, lane);
      const frag qa = M::load(hQ, LDKH, w.r0 + l16, k0, lane);
#pragma unroll
      for (int t = 0; t < TPC; ++t) {
        const frag kb = M::load(hK, LDKH, w.c0 + 16 * t + l16, k0, lane);
        kk[t] = M::mma(ka, kb, kk[t]);
        qk[t] = M::mma(qa, kb, qk[t]);
      }
    }
    float *araw = p.araw + cc * BC * BC;
    float *pm = p.pmat + cc * BC * BC;
#pragma unroll
    for (int t = 0; t < TPC; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = w.row(v, lane), q = w.col(t, lane);
        // mask before the exponential
        const float gam = q <= r ? expf(static_cast<float>(rf.G[r] - rf.G[q])) : 0.0f;
        const float a = q < r ? kk[t][v] * gam : 0.0f;
        araw[r * BC + q] = a;
        pm[r * BC + q] = q <= r ? p.scale * qk[t][v] * gam : 0.0f;
        sA[r * LDA + q] = rf.beta[r] * a;
      }
  }
  __syncthreads();

  // T = (I + A)^-1 by 16 x 16 blocks, as in the fp32 local pass
  {
    for (int idx = tid; idx < BC * BC; idx += BT) sT[(idx / BC) * LDT + idx % BC] = 0.0f;
    __syncthreads();
    if (wave < BC / 16 && lane < 16) {
      const int b = 16 * wave, jc = lane;
      float t[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = r == jc ? 1.0f : 0.0f;
#pragma unroll
        for (int i = 0; i < r; ++i) x = fmaf(-sA[(b + r) * LDA + b + i], t[i], x);
        t[r] = x;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sT[(b + r) * LDT + b + jc] = t[r];
    }
    __syncthreads();
    constexpr int LDM = 17;
    const WTile<16, 1> w0(0);
    for (int i = 1; i < BC / 16; ++i) {
      if (wave < i) {
        const int jb = wave;
        f32x4 m[1];
        zero(m);
        for (int k = jb; k < i; ++k)
          mmf(m, w0, sA + (16 * i) * LDA + 16 * k, LDA, 1, sT + (16 * k) * LDT + 16 * jb, LDT, 1,
              16, lane);
#pragma unroll
        for (int v = 0; v < 4; ++v) sM[jb * 16 * LDM + w0.row(v, lane) * LDM + w0.col(0, lane)] = m[0][v];
      }
      __syncthreads();
      if (wave < i) {
        const int jb = wave;
        f32x4 m[1];
        zero(m);
        mmf(m, w0, sT + (16 * i) * LDT + 16 * i, LDT, 1, sM + jb * 16 * LDM, LDM, 1, 16, lane);
#pragma unroll
        for (int v = 0; v < 4; ++v)
          sT[(16 * i + w0.row(v, lane)) * LDT + 16 * jb + w0.col(0, lane)] = -m[0][v];
      }
      __syncthreads();
    }
    float *tm = p.tmat + cc * BC * BC;
    for (int idx = tid; idx < BC * BC; idx += BT) tm[idx] = sT[(idx / BC) * LDT + idx % BC];
  }
}

template <typename TIn, typename TQK, int D>
__global__ void __launch_bounds__(BT) bwd_local_kernel(const BackwardParams p) {
  if constexpr (sizeof(TIn) == 2 && sizeof(TQK) == 2) {
    bwd_local_h16<TIn, TQK, D>(p);
  } else {
  constexpr int LDK = ld_row_read(D);    // K: by rows
  constexpr int LDQ = ld_any_read(D);    // Q by rows, R by columns
  constexpr int LDA = ld_row_read(BC);   // A: by rows
  constexpr int LDT = ld_row_read(BC);   // T: by rows (by columns only in the block steps)
  constexpr int LDH = ld_col_read(D);    // H0: by columns
  constexpr int TPC = (BC / 16) * (BC / 16) / NW;   // 64 x 64 tiles per wave
  constexpr int TPD = (BC / 16) * (D / 16) / NW;    // 64 x D tiles per wave
  __shared__ float sK[BC * LDK];
  __shared__ float sQ[BC * LDQ];    // later V, then R
  __shared__ float sA[BC * LDA];
  __shared__ float sT[BC * LDT];
  __shared__ float sH[32 * LDH];    // 32 rows of H0 at a time; also the solve's 16 x 16 blocks
  __shared__ RowFactors rf;

  const int c = blockIdx.x, h = blockIdx.y;
  if (c >= p.cb[p.num_seqs]) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = chunk_seq(p.cb, p.num_seqs, c);
  const int j = c - p.cb[n];
  int t0, t1;
  seq_span(p, n, t0, t1);
  const int ts = t0 + BC * j, rows = min(BC, t1 - ts);
  const int hk = h / (p.Hv / p.Hk);

  // every global input is fetched into registers up front: K, Q, g, beta first
  // (needed at once), then H0 and V, whose loads run under the K K^T products and
  // the inverse
  RowsRegs<TQK, D, D> fk, fq;
  RowInputs fr;
  fr.fetch(p, h, ts, rows, tid);
  fk.fetch(static_cast<const TQK *>(p.k), p.Hk, hk, ts, rows, 0, tid);
  fq.fetch(static_cast<const TQK *>(p.q), p.Hk, hk, ts, rows, 0, tid, p.nh);
  const float *h0 = entry_state(p, n, j, h, D);
  MatRegs<32, D> fh[D / 32];
#pragma unroll
  for (int b = 0; b < D / 32; ++b) fh[b].fetch(h0 ? h0 + static_cast<size_t>(32 * b) * D : nullptr, D, tid);
  RowsRegs<TIn, D, D> fv;
  fv.fetch(static_cast<const TIn *>(p.v), p.Hv, h, ts, rows, 0, tid);
  fk.store(sK, LDK, rows, tid);
  fq.store(sQ, LDQ, rows, tid, ts, p.nh);
  row_factors(rf, fr, tid);
  __syncthreads();

  const size_t cc = static_cast<size_t>(c) * p.Hv + h;
  {
    const WTile<BC, TPC> w(wave);
    f32x4 kk[TPC], qk[TPC];
    zero(kk);
    zero(qk);
    mmf2(kk, qk, w, sK, LDK, 1, sQ, LDQ, 1, sK, 1, LDK, D, lane);
    float *araw = p.araw + cc * BC * BC;
    float *pm = p.pmat + cc * BC * BC;
#pragma unroll
    for (int t = 0; t < TPC; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = w.row(v, lane), q = w.col(t, lane);
        // mask before the exponential
        const float gam = q <= r ? expf(static_cast<float>(rf.G[r] - rf.G[q])) : 0.0f;
        const float a = q < r ? kk[t][v] * gam : 0.0f;
        araw[r * BC + q] = a;
        pm[r * BC + q] = q <= r ? p.scale * qk[t][v] * gam : 0.0f;
        sA[r * LDA + q] = rf.beta[r] * a;
      }
  }
  __syncthreads();

  // T = (I + A)^-1 by 16 x 16 blocks (A strictly lower, so T is unit lower):
  //   diagonal blocks T_bb = (I + A_bb)^-1: wave b, lane jc < 16 solves column jc by
  //   forward substitution, t_r = [r == jc] - sum_{i<r} A_bb[r][i] t_i;
  //   off-diagonal blocks, block row by block row: T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj
  //   (16 x 16 matrix-core products, wave j takes block column j).
  {
    for (int idx = tid; idx < BC * BC; idx += BT) sT[(idx / BC) * LDT + idx % BC] = 0.0f;
    __syncthreads();
    if (wave < BC / 16 && lane < 16) {
      const int b = 16 * wave, jc = lane;
      float t[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = r == jc ? 1.0f : 0.0f;
#pragma unroll
        for (int i = 0; i < r; ++i) x = fmaf(-sA[(b + r) * LDA + b + i], t[i], x);
        t[r] = x;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sT[(b + r) * LDT + b + jc] = t[r];
    }
    __syncthreads();
    constexpr int LDM = 17;
    float *sM = sH;   // one 16 x 16 block per block column
    const WTile<16, 1> w0(0);
    for (int i = 1; i < BC / 16; ++i) {
      if (wave < i) {
        const int jb = wave;
        f32x4 m[1];
        zero(m);
        for (int k = jb; k < i; ++k)
          mmf(m, w0, sA + (16 * i) * LDA + 16 * k, LDA, 1, sT + (16 * k) * LDT + 16 * jb, LDT, 1,
              16, lane);
#pragma unroll
        for (int v = 0; v < 4; ++v) sM[jb * 16 * LDM + w0.row(v, lane) * LDM + w0.col(0, lane)] = m[0][v];
      }
      __syncthreads();
      if (wave < i) {
        const int jb = wave;
        f32x4 m[1];
        zero(m);
        mmf(m, w0, sT + (16 * i) * LDT + 16 * i, LDT, 1, sM + jb * 16 * LDM, LDM, 1, 16, lane);
#pragma unroll
        for (int v = 0; v < 4; ++v)
          sT[(16 * i + w0.row(v, lane)) * LDT + 16 * jb + w0.col(0, lane)] = -m[0][v];
      }
      __syncthreads();
    }
    float *tm = p.tmat + cc * BC * BC;
    for (int idx = tid; idx < BC * BC; idx += BT) tm[idx] = sT[(idx / BC) * LDT + idx % BC];
  }

  // X = K H0, H0 streamed 32 rows at a time
  const WTile<D, TPD> wd(wave);
  f32x4 x[TPD];
  zero(x);
  if (h0) {
#pragma unroll
    for (int b = 0; b < D / 32; ++b) {
      __syncthreads();
      fh[b].store(sH, LDH, tid);
      __syncthreads();
      mmf(x, wd, sK + 32 * b, LDK, 1, sH, LDH, 1, 32, lane);
    }
  }
  // R = diag(beta) (V - diag(e^G) X) -> sQ (V is staged there first)
  __syncthreads();
  fv.store(sQ, LDQ, rows, tid);
  __syncthreads();
#pragma unroll
  for (int t = 0; t < TPD; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = wd.row(v, lane);
      float &y = sQ[r * LDQ + wd.col(t, lane)];
      y = rf.beta[r] * (y - rf.eG[r] * x[t][v]);
    }
  __syncthreads();
  // D = T R
  f32x4 d[TPD];
  zero(d);
  mmf(d, wd, sT, LDT, 1, sQ, LDQ, 1, BC, lane);
  float *dm = p.dmat + cc * BC * D;
#pragma unroll
  for (int t = 0; t < TPD; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) dm[wd.row(v, lane) * D + wd.col(t, lane)] = d[t][v];
  }
}

// Per (sequence, value head, CW value columns), last chunk to first, carrying
// dH (D x CW columns): store dH_n, then dD = P^T dO + diag(e^{G_n - G}) K dH,
// dR = T^T dD (kept for bwd_grads_kernel), dV = diag(beta) dR, and
// dH <- e^{G_n} dH + Q^T diag(scale e^G) dO - K^T diag(beta e^G) dR.
// (CW = 32, or 16 when 32-column workgroups would leave compute units idle: the
// chain per workgroup stays the same, its products halve)
// The sweep of bf16 inputs (q, k, dO exact in fp16) on the fp16 matrix cores: the
// same steps as the fp32 sweep below, with every operand that is not an fp16 input (P,
// T, dD, dH, the scaled dO and dR) held as an fp16 pair hi + lo (~22 bits) and each
// product with such an operand taken as hi and lo terms (both pairs: hi hi + hi lo +
// lo hi).  Operands are read k-contiguous (8-byte reads in the contraction order of
// the fp16 tile helpers) or by LDS transpose reads.
template <typename TIn, typename TQK, int D, int CW>
__device__ __forceinline__ void bwd_sweep_h16(const BackwardParams &p) {
  using M = Mma<false>;
  using frag = M::frag;
  constexpr int LDKH = D + 8;      // K, Q rows (fp16)
  constexpr int LDS64 = BC + 8;    // P, T rows
  constexpr int LDO = CW + 16;     // 64 x CW operands: transposed reads conflict-free
  constexpr int LDHT = D + 8;      // dH^T rows (CW x D)
  constexpr int TPH = (D / 16) * (CW / 16) / NW;
  constexpr int NACT = (BC / 16) * (CW / 16) < NW ? (BC / 16) * (CW / 16) : NW;
  constexpr int TPS = (BC / 16) * (CW / 16) / NACT;
  static_assert(TPH >= 1 && TPS >= 1, "column tile");
  const bool sact = (threadIdx.x >> 6) < NACT;
  // K and the row factors are double-buffered: the last products of a step read them
  // while the next chunk is staged
  __shared__ __align__(16) _Float16 hK[2][BC * LDKH];
  __shared__ __align__(16) _Float16 hQ[BC * LDKH];
  __shared__ __align__(16) _Float16 hPh[BC * LDS64], hPl[BC * LDS64];
  __shared__ __align__(16) _Float16 hTh[BC * LDS64], hTl[BC * LDS64];
  __shared__ __align__(16) _Float16 hO[BC * LDO];                   // dO
  __shared__ __align__(16) _Float16 hDh[BC * LDO], hDl[BC * LDO];   // dD
  __shared__ __align__(16) _Float16 hSh[BC * LDO], hSl[BC * LDO];   // diag(scale e^G) dO
  __shared__ __align__(16) _Float16 hRh[BC * LDO], hRl[BC * LDO];   // -diag(beta e^G) dR
  __shared__ __align__(16) _Float16 hHh[CW * LDHT], hHl[CW * LDHT]; // dH^T
  __shared__ RowFactors rfs[2];
  auto put_hl = [](_Float16 *hi, _Float16 *lo, int i, float x) {
    const _Float16 a = static_cast<_Float16>(x);
    hi[i] = a;
    lo[i] = static_cast<_Float16>(x - static_cast<float>(a));
  };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15;
  constexpr int NVT = D / CW;
  const int item = xcd_work_item(blockIdx.x, NVT, p.num_seqs * p.Hv);
  if (item < 0) return;
  const int vt = item % NVT;
  const int h = (item / NVT) % p.Hv;
  const int n = item / NVT / p.Hv;
  const int col0 = CW * vt;
  const int hk = h / (p.Hv / p.Hk);
  int t0, t1;
  seq_span(p, n, t0, t1);
  const int nch = (t1 - t0 + BC - 1) / BC;
  // read once: a reload inside the loop would wait for every load and store in flight
  const int cb0 = p.cb[n];
  const size_t ss = static_cast<size_t>(D) * D;

  const WTile<CW, TPH> wh(wave);
  const WTile<CW, TPS> ws(wave);
  f32x4 dh[TPH];
  zero(dh);
  if (p.d_final_state) {
    const float *s = p.d_final_state + (static_cast<size_t>(n) * p.Hv + h) * ss;
#pragma unroll
    for (int t = 0; t < TPH; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) dh[t][v] = s[wh.row(v, lane) * D + col0 + wh.col(t, lane)];
  }
  const TIn *dO = static_cast<const TIn *>(p.d_out);
  RowsRegs<TQK, D, D> fk, fq;
  RowsRegs<TIn, D, CW> fo;
  MatRegs<BC, BC> fp, ft;
  RowInputs fr;
  auto fetch = [&](int jc) {
    const int ts = t0 + BC * jc, rows = min(BC, t1 - ts);
    const size_t cc = static_cast<size_t>(cb0 + jc) * p.Hv + h;
    fr.fetch(p, h, ts, rows, tid);
    fk.fetch(static_cast<const TQK *>(p.k), p.Hk, hk, ts, rows, 0, tid);
    fq.fetch(static_cast<const TQK *>(p.q), p.Hk, hk, ts, rows, 0, tid, p.nh);
    fo.fetch(dO, p.Hv, h, ts, rows, col0, tid, p.nh);
    fp.fetch(p.pmat + cc * BC * BC, BC, tid);
    ft.fetch(p.tmat + cc * BC * BC, BC, tid);
  };
  // chunk jc from the registers into LDS (K into buffer jc & 1)
  auto stage = [&](int jc) __attribute__((always_inline)) {
    const int ts = t0 + BC * jc, rows = min(BC, t1 - ts);
    fk.store_h(hK[jc & 1], LDKH, rows, tid);
    fq.store_h(hQ, LDKH, rows, tid, ts, p.nh);
    fo.store_h(hO, LDO, rows, tid, ts, p.nh);
    fp.store_hl(hPh, hPl, LDS64, tid);
    ft.store_hl(hTh, hTl, LDS64, tid);
    row_factors(rfs[jc & 1], fr, tid);
  };
  // dH leaving chunk jc (this wave's tiles): stored as dH_n, and as the fp16 pair of
  // the dD products
  auto put_dh = [&](int jc) __attribute__((always_inline)) {
    float *dhn = p.dhn + (static_cast<size_t>(cb0 + jc) * p.Hv + h) * ss;
#pragma unroll
    for (int t = 0; t < TPH; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = wh.row(v, lane), q = wh.col(t, lane);
        dhn[r * D + col0 + q] = dh[t][v];
        put_hl(hHh, hHl, q * LDHT + r, dh[t][v]);
      }
  };
  if (nch > 0) {
    put_dh(nch - 1);
    fetch(nch - 1);
    stage(nch - 1);
    if (nch > 1) fetch(nch - 2);
    // Three barriers per chunk: (1) dH and the chunk staged, (2) dD and
    // S = diag(scale e^G) dO, (3) dR and the Q^T S part of the update; then the K^T part,
    // after which this wave puts the next chunk's dH (its operand was last read before
    // barrier 2), stages the next chunk (every buffer written was last read before
    // barrier 3, K into the other buffer) and requests the one after.
    for (int jc = nch - 1; jc >= 0; --jc) {
      const int c = cb0 + jc;
      const int ts = t0 + BC * jc, rows = min(BC, t1 - ts);
      const size_t cc = static_cast<size_t>(c) * p.Hv + h;
      const _Float16 *hKc = hK[jc & 1];
      const RowFactors &rf = rfs[jc & 1];
      __syncthreads();

      // dD = P^T dO + diag(e^{G_n - G}) (K dH)
      if (sact) {
        f32x4 a1[TPS], a2[TPS];
        zero(a1);
        zero(a2);
#pragma unroll
        for (int k0 = 0; k0 < BC; k0 += 32) {
          const frag ph = frag_tr(hPh, LDS64, k0, ws.r0, lane);
          const frag pl = frag_tr(hPl, LDS64, k0, ws.r0, lane);
#pragma unroll
          for (int t = 0; t < TPS; ++t) {
            const frag ob = frag_tr(hO, LDO, k0, ws.c0 + 16 * t, lane);
            a1[t] = M::mma(pl, ob, M::mma(ph, ob, a1[t]));
          }
        }
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += 32) {
          const frag ka = M::load(hKc, LDKH, ws.r0 + l16, k0, lane);
#pragma unroll
          for (int t = 0; t < TPS; ++t) {
            const frag bh = M::load(hHh, LDHT, ws.c0 + 16 * t + l16, k0, lane);
            const frag bl = M::load(hHl, LDHT, ws.c0 + 16 * t + l16, k0, lane);
            a2[t] = M::mma(ka, bl, M::mma(ka, bh, a2[t]));
          }
        }
#pragma unroll
        for (int t = 0; t < TPS; ++t)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int r = ws.row(v, lane);
            put_hl(hDh, hDl, r * LDO + ws.col(t, lane), a1[t][v] + rf.eGl[r] * a2[t][v]);
          }
      }
      for (int idx = tid; idx < BC * CW; idx += BT) {
        const int r = idx / CW, q = idx % CW;
        put_hl(hSh, hSl, r * LDO + q, static_cast<float>(hO[r * LDO + q]) * (p.scale * rf.eG[r]));
      }
      __syncthreads();
      // dR = T^T dD; dR stored, dV = diag(beta) dR and -diag(beta e^G) dR for the update
      if (sact) {
        f32x4 dr[TPS];
        zero(dr);
#pragma unroll
        for (int k0 = 0; k0 < BC; k0 += 32) {
          const frag th = frag_tr(hTh, LDS64, k0, ws.r0, lane);
          const frag tl = frag_tr(hTl, LDS64, k0, ws.r0, lane);
#pragma unroll
          for (int t = 0; t < TPS; ++t) {
            const frag dhi = frag_tr(hDh, LDO, k0, ws.c0 + 16 * t, lane);
            const frag dlo = frag_tr(hDl, LDO, k0, ws.c0 + 16 * t, lane);
            dr[t] = M::mma(tl, dhi, M::mma(th, dlo, M::mma(th, dhi, dr[t])));
          }
        }
        float *drm = p.drmat + cc * BC * D;
#pragma unroll
        for (int t = 0; t < TPS; ++t)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int r = ws.row(v, lane), q = ws.col(t, lane);
            drm[r * D + col0 + q] = dr[t][v];
            if (r < rows)
              p.dv[(static_cast<size_t>(ts + r) * p.Hv + h) * D + col0 + q] =
                  rf.beta[r] * dr[t][v];
            put_hl(hRh, hRl, r * LDO + q, -rf.beta[r] * rf.eG[r] * dr[t][v]);
          }
      }
      // dH <- e^{G_n} dH + Q^T (diag(scale e^G) dO) ...
      {
        const float en = rf.eG[BC - 1];
#pragma unroll
        for (int t = 0; t < TPH; ++t) dh[t] *= en;
#pragma unroll
        for (int k0 = 0; k0 < BC; k0 += 32) {
          const frag qa = frag_tr(hQ, LDKH, k0, wh.r0, lane);
#pragma unroll
          for (int t = 0; t < TPH; ++t) {
            const int cn = wh.c0 + 16 * t;
            const frag sh = frag_tr(hSh, LDO, k0, cn, lane);
            const frag sl = frag_tr(hSl, LDO, k0, cn, lane);
            dh[t] = M::mma(qa, sl, M::mma(qa, sh, dh[t]));
          }
        }
      }
      __syncthreads();
      // ... + K^T (-diag(beta e^G) dR)
#pragma unroll
      for (int k0 = 0; k0 < BC; k0 += 32) {
        const frag ka = frag_tr(hKc, LDKH, k0, wh.r0, lane);
#pragma unroll
        for (int t = 0; t < TPH; ++t) {
          const int cn = wh.c0 + 16 * t;
          const frag rh = frag_tr(hRh, LDO, k0, cn, lane);
          const frag rl = frag_tr(hRl, LDO, k0, cn, lane);
          dh[t] = M::mma(ka, rl, M::mma(ka, rh, dh[t]));
        }
      }
      if (jc > 0) {
        put_dh(jc - 1);
        stage(jc - 1);
        if (jc > 1) fetch(jc - 2);
      }
    }
  }
  if (p.d_initial_state) {
    float *s = p.d_initial_state + (static_cast<size_t>(n) * p.Hv + h) * ss;
#pragma unroll
    for (int t = 0; t < TPH; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) s[wh.row(v, lane) * D + col0 + wh.col(t, lane)] = dh[t][v];
  }
}

template <typename TIn, typename TQK, int D, int CW>
__global__ void __launch_bounds__(BT) bwd_sweep_kernel(const BackwardParams p) {
  if constexpr (sizeof(TIn) == 2 && sizeof(TQK) == 2) {
    bwd_sweep_h16<TIn, TQK, D, CW>(p);
  } else {
  constexpr int LDK = ld_any_read(D);    // K: by rows (K dH) and by columns (K^T)
  constexpr int LDQ = ld_col_read(D);    // Q: by columns
  constexpr int LDP = ld_col_read(BC);   // P, T: by columns
  constexpr int LDV = ld_col_read(CW);   // dO, dD: by columns
  constexpr int LDH = ld_row_read(D);    // dH, stored transposed (CW x D): by rows
  static_assert(LDV <= LDP, "-diag(beta e^G) dR reuses the LDS of P");
  constexpr int TPH = (D / 16) * (CW / 16) / NW;   // D x CW tiles per wave
  // 64 x CW tiles: one per wave, on the first NACT waves
  constexpr int NACT = (BC / 16) * (CW / 16) < NW ? (BC / 16) * (CW / 16) : NW;
  constexpr int TPS = (BC / 16) * (CW / 16) / NACT;
  static_assert(TPH >= 1 && TPS >= 1, "column tile");
  const bool sact = (threadIdx.x >> 6) < NACT;   // wave-uniform
  __shared__ float sK[BC * LDK];
  __shared__ float sQ[BC * LDQ];
  __shared__ float sP[BC * LDP];
  __shared__ float sT[BC * LDP];
  __shared__ float sO[BC * LDV];    // dO columns, later diag(scale e^G) dO
  __shared__ float sD[BC * LDV];    // dD, later -diag(beta e^G) dR
  __shared__ float sdH[CW * LDH];   // dH^T
  __shared__ RowFactors rf;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int NVT = D / CW;
  // the NVT column tiles of one (sequence, head) read the same K, Q, P and T: they
  // go to one XCD, whose L2 then serves the re-reads
  const int item = xcd_work_item(blockIdx.x, NVT, p.num_seqs * p.Hv);
  if (item < 0) return;
  const int vt = item % NVT;
  const int h = (item / NVT) % p.Hv;
  const int n = item / NVT / p.Hv;
  const int col0 = CW * vt;
  const int hk = h / (p.Hv / p.Hk);
  int t0, t1;
  seq_span(p, n, t0, t1);
  const int nch = (t1 - t0 + BC - 1) / BC;
  const size_t ss = static_cast<size_t>(D) * D;

  const WTile<CW, TPH> wh(wave);
  const WTile<CW, TPS> ws(wave);
  f32x4 dh[TPH];
  zero(dh);
  if (p.d_final_state) {
    const float *s = p.d_final_state + (static_cast<size_t>(n) * p.Hv + h) * ss;
#pragma unroll
    for (int t = 0; t < TPH; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) dh[t][v] = s[wh.row(v, lane) * D + col0 + wh.col(t, lane)];
  }
  const TIn *dO = static_cast<const TIn *>(p.d_out);
  // the inputs of the chunk after next in the sweep are fetched into registers
  // while the current chunk's products run
  RowsRegs<TQK, D, D> fk, fq;
  RowsRegs<TIn, D, CW> fo;
  MatRegs<BC, BC> fp, ft;
  RowInputs fr;
  auto fetch = [&](int jc) {
    const int ts = t0 + BC * jc, rows = min(BC, t1 - ts);
    const size_t cc = static_cast<size_t>(p.cb[n] + jc) * p.Hv + h;
    fr.fetch(p, h, ts, rows, tid);
    fk.fetch(static_cast<const TQK *>(p.k), p.Hk, hk, ts, rows, 0, tid);
    fq.fetch(static_cast<const TQK *>(p.q), p.Hk, hk, ts, rows, 0, tid, p.nh);
    fo.fetch(dO, p.Hv, h, ts, rows, col0, tid, p.nh);
    fp.fetch(p.pmat + cc * BC * BC, BC, tid);
    ft.fetch(p.tmat + cc * BC * BC, BC, tid);
  };
  if (nch > 0) fetch(nch - 1);
  for (int jc = nch - 1; jc >= 0; --jc) {
    const int c = p.cb[n] + jc;
    const int ts = t0 + BC * jc, rows = min(BC, t1 - ts);
    const size_t cc = static_cast<size_t>(c) * p.Hv + h;
    float *dhn = p.dhn + cc * ss;
#pragma unroll
    for (int t = 0; t < TPH; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = wh.row(v, lane), q = wh.col(t, lane);
        dhn[r * D + col0 + q] = dh[t][v];
        sdH[q * LDH + r] = dh[t][v];
      }
    fk.store(sK, LDK, rows, tid);
    fq.store(sQ, LDQ, rows, tid, ts, p.nh);
    fo.store(sO, LDV, rows, tid, ts, p.nh);
    fp.store(sP, LDP, tid);
    ft.store(sT, LDP, tid);
    row_factors(rf, fr, tid);
    if (jc > 0) fetch(jc - 1);
    __syncthreads();

    // dD = P^T dO + diag(e^{G_n - G}) (K dH)
    if (sact) {
      f32x4 a1[TPS], a2[TPS];
      zero(a1);
      zero(a2);
      mmf(a1, ws, sP, 1, LDP, sO, LDV, 1, BC, lane);
      mmf(a2, ws, sK, LDK, 1, sdH, 1, LDH, D, lane);
#pragma unroll
      for (int t = 0; t < TPS; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = ws.row(v, lane);
          sD[r * LDV + ws.col(t, lane)] = a1[t][v] + rf.eGl[r] * a2[t][v];
        }
    }
    __syncthreads();
    // dR = T^T dD; then, in the same interval, dR is stored, dV = diag(beta) dR,
    // -diag(beta e^G) dR goes to the LDS of P (read only by dD, which is done) and
    // dO is scaled by diag(scale e^G) (dO is read next by the dH products)
    float *sR = sP;
    if (sact) {
      f32x4 dr[TPS];
      zero(dr);
      mmf(dr, ws, sT, 1, LDP, sD, LDV, 1, BC, lane);
      float *drm = p.drmat + cc * BC * D;
#pragma unroll
      for (int t = 0; t < TPS; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = ws.row(v, lane), q = ws.col(t, lane);
          drm[r * D + col0 + q] = dr[t][v];
          if (r < rows)
            p.dv[(static_cast<size_t>(ts + r) * p.Hv + h) * D + col0 + q] =
                rf.beta[r] * dr[t][v];
          sR[r * LDV + q] = -rf.beta[r] * rf.eG[r] * dr[t][v];
        }
    }
    for (int idx = tid; idx < BC * CW; idx += BT) {
      const int r = idx / CW, q = idx % CW;
      sO[r * LDV + q] *= p.scale * rf.eG[r];
    }
    __syncthreads();
    // dH <- e^{G_n} dH + Q^T (diag(scale e^G) dO) + K^T (-diag(beta e^G) dR)
    {
      const float en = rf.eG[BC - 1];
#pragma unroll
      for (int t = 0; t < TPH; ++t) dh[t] *= en;
      mmf(dh, wh, sQ, 1, LDQ, sO, LDV, 1, BC, lane);
      mmf(dh, wh, sK, 1, LDK, sR, LDV, 1, BC, lane);
    }
    __syncthreads();
  }
  if (p.d_initial_state) {
    float *s = p.d_initial_state + (static_cast<size_t>(n) * p.Hv + h) * ss;
#pragma unroll
    for (int t = 0; t < TPH; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) s[wh.row(v, lane) * D + col0 + wh.col(t, lane)] = dh[t][v];
  }
  }
}

// Per (chunk, value head): the gradients of q, k (per value head), beta and g.
//   phase 1 (over 32-column slices of V): dA = -(dR D^T), dP = dO D^T,
//     U1 = dO H0^T, Ua = dR H0^T, Ub = D dH_n^T, dR_r . v_r and <dH_n, H0>;
//   phase 2: dAs, dPs, E + F = dA * A + dP * P, dA * Araw (masked to the triangles);
//   phase 3: dQ = dPs K + diag(scale e^G) U1,
//            dK = dAs K + dAs^T K + dPs^T Q - diag(beta e^G) Ua + diag(e^{G_n - G}) Ub,
//            dbeta_r = (dA * Araw) row sum + dR_r . v_r - e^{G_r} k_r . Ua_r,
//            dG_r = rowsum(E + F) - colsum(E + F) + scale e^{G_r} q_r . U1_r
//                   - beta_r e^{G_r} k_r . Ua_r - w_r,  w_r = e^{G_n - G_r} k_r . Ub_r,
//            plus e^{G_n} <dH_n, H0> + sum w on the last row; dg = reverse cumsum.
template <typename TIn, typename TQK, int D>
__global__ void __launch_bounds__(BT) bwd_grads_kernel(const BackwardParams p) {
  constexpr int LDV = ld_row_read(32);   // phase 1 slices: by rows
  constexpr int LDG = ld_any_read(BC);   // dAs, dPs: by rows and by columns
  constexpr int LDD = ld_col_read(D);    // K, Q: by columns
  constexpr int TPC = (BC / 16) * (BC / 16) / NW;   // 64 x 64 tiles per wave
  constexpr int TPD = (BC / 16) * (D / 16) / NW;    // 64 x D tiles per wave
  constexpr int HALVES = NW / (BC / 16);            // waves sharing one tile row of 64 x D
  static_assert(BT == 8 * BC, "row sums and dots: eight threads per row");
  // phase 1 and phases 2-3 share one LDS arena
  // bf16 inputs run phase 1's products on the fp16 matrix cores (float32 inputs keep
  // the fp32 ones, whose 1e-5 bound fp16 operands would not meet)
  constexpr bool H16 = sizeof(TIn) == 2;
  constexpr int LDH = 40;   // fp16 slice rows: 16-byte reads on 16 rows, conflict-free
  // phase 3 on the fp16 matrix cores too when q and k are bf16 (exact in fp16): dAs and
  // dPs as fp16 hi/lo pairs.  Then the local pass keeps no D either: phase 1 forms each
  // slice of D = T R from K, H0, V and T (K and T staged once, in LDS of their own
  // for K, which phase 3 reads too)
  constexpr bool H16Q = H16 && sizeof(TQK) == 2;
  constexpr int LDS64 = BC + 8;   // fp16 64 x 64 rows: conflict-free 8-byte and transposed reads
  constexpr int LDKH = D + 8;     // fp16 K, Q rows
  constexpr int P1 = H16 ? (5 * BC * LDH + 4 * D * LDH) / 2 + 2 * BC * LDV +
                               (H16Q ? (2 * BC * LDH + 2 * BC * LDS64) / 2 : 0)
                         : 4 * BC * LDV + 2 * D * LDV;
  constexpr int P23 = H16Q ? (4 * BC * LDS64 + BC * LDKH) / 2 + 2 * BC * LDC
                           : 2 * BC * LDG + 2 * BC * LDC + 2 * BC * LDD;
  constexpr int ARENA = P1 > P23 ? P1 : P23;
  __shared__ __align__(16) float arena[ARENA];
  __shared__ __align__(16) _Float16 hK1[H16Q ? BC * LDKH : 8];   // K (fp16) for phases 1 and 3
  __shared__ RowFactors rf;
  __shared__ float srow[3][BC];         // row sums of E + F, column sums of E + F, row sums of dA * Araw
  __shared__ float sdot[3][HALVES][BC]; // q.U1, k.Ua, k.Ub per row, one partial per wave of a tile row
  __shared__ float srv[BC];             // dR . v per row
  __shared__ float sred[NW];

  const int c = blockIdx.x, h = blockIdx.y;
  if (c >= p.cb[p.num_seqs]) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = chunk_seq(p.cb, p.num_seqs, c);
  const int j = c - p.cb[n];
  int t0, t1;
  seq_span(p, n, t0, t1);
  const int ts = t0 + BC * j, rows = min(BC, t1 - ts);
  const int hk = h / (p.Hv / p.Hk);
  const size_t cc = static_cast<size_t>(c) * p.Hv + h;
  const size_t ss = static_cast<size_t>(D) * D;
  row_factors(rf, p, h, ts, rows, tid);

  const float *h0 = entry_state(p, n, j, h, D);
  const float *dhn = p.dhn + cc * ss;
  const float *dm = p.dmat + cc * BC * D;
  const float *drm = p.drmat + cc * BC * D;

  const WTile<BC, TPC> wc(wave);
  const WTile<D, TPD> wd(wave);
  f32x4 dA[TPC], dP[TPC], U1[TPD], Ua[TPD], Ub[TPD];
  zero(dA);
  zero(dP);
  zero(U1);
  zero(Ua);
  zero(Ub);
  float hh = 0.0f, rv = 0.0f;
  // phase 2's inputs (K, Q rows and the chunk's Araw, P entries of this thread's
  // tiles) are fetched during the last slice of phase 1; fp32 K, Q rows at D = 128
  // would not fit the registers and are loaded when needed
  constexpr bool kPreKQ = sizeof(TQK) == 2 || D <= 64;
  RowsRegs<TQK, D, D> fk, fq;
  float ar[TPC][4], pv[TPC][4];
  if constexpr (H16) {
    // bf16 inputs: the slices as fp16 for the matrix cores (k contiguous in every
    // operand), dR and V also as fp32 for the row dots, <dH_n, H0> from the fp32
    // registers before they are refilled
    _Float16 *hD = reinterpret_cast<_Float16 *>(arena), *hR = hD + BC * LDH, *hO = hR + BC * LDH;
    _Float16 *hDl = hO + BC * LDH, *hRl = hDl + BC * LDH;   // low parts of D and dR
    _Float16 *hH = hRl + BC * LDH, *hG = hH + D * LDH;
    _Float16 *hHl = hG + D * LDH, *hGl = hHl + D * LDH;     // low parts of the states
    float *sRb = reinterpret_cast<float *>(hGl + D * LDH), *svb = sRb + BC * LDV;
    // H16Q: R = diag(beta) (V - diag(e^G) K H0) of the slice and T, as fp16 pairs
    _Float16 *hY = reinterpret_cast<_Float16 *>(svb + BC * LDV), *hYl = hY + BC * LDH;
    _Float16 *hTh = hYl + BC * LDH, *hTl = hTh + BC * LDS64;
    MatRegs<BC, 32> fD, fR;
    RowsRegs<TIn, D, 32> fO, fV;
    MatRegs<D, 32> fH, fG;
    auto fetch = [&](int vb) {
      if constexpr (!H16Q) fD.fetch(dm + vb, D, tid);
      fR.fetch(drm + vb, D, tid);
      fO.fetch(static_cast<const TIn *>(p.d_out), p.Hv, h, ts, rows, vb, tid, p.nh);
      fV.fetch(static_cast<const TIn *>(p.v), p.Hv, h, ts, rows, vb, tid);
      fH.fetch(h0 ? h0 + vb : nullptr, D, tid);
      fG.fetch(dhn + vb, D, tid);
    };
    if constexpr (H16Q) {
      fk.fetch(static_cast<const TQK *>(p.k), p.Hk, hk, ts, rows, 0, tid);
      MatRegs<BC, BC> ft;
      ft.fetch(p.tmat + cc * BC * BC, BC, tid);
      fk.store_h(hK1, LDKH, rows, tid);
      ft.store_hl(hTh, hTl, LDS64, tid);
    }
    fetch(0);
    for (int vb = 0; vb < D; vb += 32) {
      __syncthreads();
      if constexpr (!H16Q) fD.store_hl(hD, hDl, LDH, tid);
      fR.store_hl(hR, hRl, LDH, tid);
      fR.store(sRb, LDV, tid);
      fO.store_h(hO, LDH, rows, tid, ts, p.nh);
      fV.store(svb, LDV, rows, tid);
      fH.store_hl(hH, hHl, LDH, tid);
      fG.store_hl(hG, hGl, LDH, tid);
      hh += fH.dot(fG);
      if (vb + 32 < D) {
        fetch(vb + 32);
      } else {
        if constexpr (kPreKQ) {
          if constexpr (!H16Q) fk.fetch(static_cast<const TQK *>(p.k), p.Hk, hk, ts, rows, 0, tid);
          fq.fetch(static_cast<const TQK *>(p.q), p.Hk, hk, ts, rows, 0, tid, p.nh);
        }
        const float *araw = p.araw + cc * BC * BC;
        const float *pm = p.pmat + cc * BC * BC;
#pragma unroll
        for (int t = 0; t < TPC; ++t)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int r = wc.row(v, lane), q = wc.col(t, lane);
            ar[t][v] = araw[r * BC + q];
            pv[t][v] = pm[r * BC + q];
          }
      }
      __syncthreads();
      if constexpr (H16Q) {
        // this slice of D = T R, R = diag(beta) (V - diag(e^G) K H0): one 16 x 16 tile of
        // the 64 x 32 slice per wave; K exact, H0, R and T as pairs
        using M = Mma<false>;
        const WTile<32, 1> wx(wave);
        const int l16 = lane & 15;
        f32x4 x = zero4();
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += 32) {
          const M::frag ka = M::load(hK1, LDKH, wx.r0 + l16, k0, lane);
          const M::frag bh = frag_tr(hH, LDH, k0, wx.c0, lane);
          const M::frag bl = frag_tr(hHl, LDH, k0, wx.c0, lane);
          x = M::mma(ka, bl, M::mma(ka, bh, x));
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = wx.row(v, lane), q = wx.col(0, lane);
          const float y = rf.beta[r] * (svb[r * LDV + q] - rf.eG[r] * x[v]);
          const _Float16 a = static_cast<_Float16>(y);
          hY[r * LDH + q] = a;
          hYl[r * LDH + q] = static_cast<_Float16>(y - static_cast<float>(a));
        }
        __syncthreads();
        f32x4 d = zero4();
#pragma unroll
        for (int k0 = 0; k0 < BC; k0 += 32) {
          const M::frag th = M::load(hTh, LDS64, wx.r0 + l16, k0, lane);
          const M::frag tl = M::load(hTl, LDS64, wx.r0 + l16, k0, lane);
          const M::frag rh = frag_tr(hY, LDH, k0, wx.c0, lane);
          const M::frag rl = frag_tr(hYl, LDH, k0, wx.c0, lane);
          d = M::mma(tl, rh, M::mma(th, rl, M::mma(th, rh, d)));
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = wx.row(v, lane), q = wx.col(0, lane);
          const _Float16 a = static_cast<_Float16>(d[v]);
          hD[r * LDH + q] = a;
          hDl[r * LDH + q] = static_cast<_Float16>(d[v] - static_cast<float>(a));
        }
        __syncthreads();
      }
      // x y with x = xh + xl, y = yh + yl (dO is exact in fp16): xh yh + xh yl + xl yh
      {
        f32x4 *const acc[2] = {dA, dP};
        const _Float16 *const X[2] = {hR, hO};
        mmh_xyt<2>(acc, wc, X, LDH, hD, LDH, 32, lane);
        mmh_xyt<2>(acc, wc, X, LDH, hDl, LDH, 32, lane);
        f32x4 *const acc1[1] = {dA};
        const _Float16 *const X1[1] = {hRl};
        mmh_xyt<1>(acc1, wc, X1, LDH, hD, LDH, 32, lane);
      }
      {
        f32x4 *const acc[2] = {U1, Ua};
        const _Float16 *const X[2] = {hO, hR};
        mmh_xyt<2>(acc, wd, X, LDH, hH, LDH, 32, lane);
        mmh_xyt<2>(acc, wd, X, LDH, hHl, LDH, 32, lane);
        f32x4 *const acc1[1] = {Ua};
        const _Float16 *const X1[1] = {hRl};
        mmh_xyt<1>(acc1, wd, X1, LDH, hH, LDH, 32, lane);
      }
      {
        f32x4 *const acc[1] = {Ub};
        const _Float16 *const X[1] = {hD};
        mmh_xyt<1>(acc, wd, X, LDH, hG, LDH, 32, lane);
        mmh_xyt<1>(acc, wd, X, LDH, hGl, LDH, 32, lane);
        const _Float16 *const X1[1] = {hDl};
        mmh_xyt<1>(acc, wd, X1, LDH, hG, LDH, 32, lane);
      }
      {
        // dR . v of row tid / 8, this thread's 4 columns of the slice
        const int r = tid >> 3, q0 = 4 * (tid & 7);
#pragma unroll
        for (int e = 0; e < 4; ++e) rv = fmaf(sRb[r * LDV + q0 + e], svb[r * LDV + q0 + e], rv);
      }
    }
  } else
  {
    float *sDb = arena, *sRb = sDb + BC * LDV, *sOb = sRb + BC * LDV, *svb = sOb + BC * LDV;
    float *sHb = svb + BC * LDV, *sGb = sHb + D * LDV;
    // the next slice is fetched into registers while this one's products run
    MatRegs<BC, 32> fD, fR;
    RowsRegs<TIn, D, 32> fO, fV;
    MatRegs<D, 32> fH, fG;
    auto fetch = [&](int vb) {
      fD.fetch(dm + vb, D, tid);
      fR.fetch(drm + vb, D, tid);
      fO.fetch(static_cast<const TIn *>(p.d_out), p.Hv, h, ts, rows, vb, tid, p.nh);
      fV.fetch(static_cast<const TIn *>(p.v), p.Hv, h, ts, rows, vb, tid);
      fH.fetch(h0 ? h0 + vb : nullptr, D, tid);
      fG.fetch(dhn + vb, D, tid);
    };
    fetch(0);
    for (int vb = 0; vb < D; vb += 32) {
      __syncthreads();
      fD.store(sDb, LDV, tid);
      fR.store(sRb, LDV, tid);
      fO.store(sOb, LDV, rows, tid, ts, p.nh);
      fV.store(svb, LDV, rows, tid);
      fH.store(sHb, LDV, tid);
      fG.store(sGb, LDV, tid);
      if (vb + 32 < D) {
        fetch(vb + 32);
      } else {
        if constexpr (kPreKQ) {
          fk.fetch(static_cast<const TQK *>(p.k), p.Hk, hk, ts, rows, 0, tid);
          fq.fetch(static_cast<const TQK *>(p.q), p.Hk, hk, ts, rows, 0, tid, p.nh);
        }
        const float *araw = p.araw + cc * BC * BC;
        const float *pm = p.pmat + cc * BC * BC;
#pragma unroll
        for (int t = 0; t < TPC; ++t)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int r = wc.row(v, lane), q = wc.col(t, lane);
            ar[t][v] = araw[r * BC + q];
            pv[t][v] = pm[r * BC + q];
          }
      }
      __syncthreads();
      // <dH_n, H0> over this slice (each thread its share of the elements)
      for (int idx = tid; idx < D * 32; idx += BT) {
        const int r = idx / 32, q = idx % 32;
        hh = fmaf(sHb[r * LDV + q], sGb[r * LDV + q], hh);
      }
      mmf2(dA, dP, wc, sRb, LDV, 1, sOb, LDV, 1, sDb, 1, LDV, 32, lane);
      mmf2(U1, Ua, wd, sOb, LDV, 1, sRb, LDV, 1, sHb, 1, LDV, 32, lane);
      mmf(Ub, wd, sDb, LDV, 1, sGb, 1, LDV, 32, lane);
      {
        // dR . v of row tid / 8, this thread's 4 columns of the slice
        const int r = tid >> 3, q0 = 4 * (tid & 7);
#pragma unroll
        for (int e = 0; e < 4; ++e) rv = fmaf(sRb[r * LDV + q0 + e], svb[r * LDV + q0 + e], rv);
      }
    }
  }
  // the 8 partial row dots of a row sit in 8 consecutive lanes
#pragma unroll
  for (int o = 4; o > 0; o >>= 1) rv += __shfl_xor(rv, o, 64);
  __syncthreads();

  float *sdAs = arena, *sdPs = sdAs + BC * LDG, *sM1 = sdPs + BC * LDG, *sM2 = sM1 + BC * LDC;
  float *sK = sM2 + BC * LDC, *sQ = sK + BC * LDD;
  // the fp16 layout of the same arena
  _Float16 *hA = reinterpret_cast<_Float16 *>(arena), *hAl = hA + BC * LDS64;
  _Float16 *hP = hAl + BC * LDS64, *hPl = hP + BC * LDS64;
  _Float16 *hQ = hPl + BC * LDS64;
  const _Float16 *hK = hK1;   // staged before phase 1
  if constexpr (H16Q) {
    sM1 = reinterpret_cast<float *>(hQ + BC * LDKH);
    sM2 = sM1 + BC * LDC;
  }
  // x -> fp16 hi, lo with hi + lo carrying ~22 bits of x
  auto put_hl = [](_Float16 *hi, _Float16 *lo, int i, float x) {
    const _Float16 a = static_cast<_Float16>(x);
    hi[i] = a;
    lo[i] = static_cast<_Float16>(x - static_cast<float>(a));
  };
#pragma unroll
  for (int t = 0; t < TPC; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = wc.row(v, lane), q = wc.col(t, lane);
      const float gam = q <= r ? expf(static_cast<float>(rf.G[r] - rf.G[q])) : 0.0f;
      const float a = q < r ? -dA[t][v] : 0.0f;
      const float pp = q <= r ? dP[t][v] : 0.0f;
      if constexpr (H16Q) {
        put_hl(hA, hAl, r * LDS64 + q, a * rf.beta[r] * gam);
        put_hl(hP, hPl, r * LDS64 + q, p.scale * pp * gam);
      } else {
        sdAs[r * LDG + q] = a * rf.beta[r] * gam;
        sdPs[r * LDG + q] = p.scale * pp * gam;
      }
      sM1[r * LDC + q] = a * rf.beta[r] * ar[t][v] + pp * pv[t][v];
      sM2[r * LDC + q] = a * ar[t][v];
    }
  if constexpr (H16Q) {
    fq.store_h(hQ, LDKH, rows, tid, ts, p.nh);
  } else if constexpr (kPreKQ) {
    fk.store(sK, LDD, rows, tid);
    fq.store(sQ, LDD, rows, tid, ts, p.nh);
  } else {
    load_rows<TQK, D, D>(sK, LDD, static_cast<const TQK *>(p.k), p.Hk, hk, ts, rows, 0, tid);
    load_rows<TQK, D, D>(sQ, LDD, static_cast<const TQK *>(p.q), p.Hk, hk, ts, rows, 0, tid,
                         p.nh);
  }
  if ((tid & 7) == 0) srv[tid >> 3] = rv;
  // <dH_n, H0>: wave sums, then across waves
  {
    float s = hh;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    if (lane == 0) sred[wave] = s;
  }
  __syncthreads();

  {
    // row and column sums of E + F and row sums of dA * Araw: row (column) tid / 8,
    // 8 of its entries per thread, then a sum over the 8 consecutive lanes
    const int r = tid >> 3, q0 = 8 * (tid & 7);
    float rs = 0.0f, cs = 0.0f, r2 = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      rs += sM1[r * LDC + q0 + e];
      cs += sM1[(q0 + e) * LDC + r];
      r2 += sM2[r * LDC + q0 + e];
    }
#pragma unroll
    for (int o = 4; o > 0; o >>= 1) {
      rs += __shfl_xor(rs, o, 64);
      cs += __shfl_xor(cs, o, 64);
      r2 += __shfl_xor(r2, o, 64);
    }
    if ((tid & 7) == 0) {
      srow[0][r] = rs;
      srow[1][r] = cs;
      srow[2][r] = r2;
    }
  }
  // row dots of U1, Ua, Ub with the rows of Q and K: the 16 lanes of a lane group
  // hold one row's columns of a tile; the HALVES waves of a tile row add in LDS
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int r = wd.row(v, lane);
    float s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll
    for (int t = 0; t < TPD; ++t) {
      const int col = wd.col(t, lane);
      float qv, kv;
      if constexpr (H16Q) {
        qv = static_cast<float>(hQ[r * LDKH + col]);
        kv = static_cast<float>(hK[r * LDKH + col]);
      } else {
        qv = sQ[r * LDD + col];
        kv = sK[r * LDD + col];
      }
      s1 = fmaf(qv, U1[t][v], s1);
      s2 = fmaf(kv, Ua[t][v], s2);
      s3 = fmaf(kv, Ub[t][v], s3);
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) {
      s1 += __shfl_xor(s1, o, 64);
      s2 += __shfl_xor(s2, o, 64);
      s3 += __shfl_xor(s3, o, 64);
    }
    if ((lane & 15) == 0) {
      const int half = wave % HALVES;
      sdot[0][half][r] = s1;
      sdot[1][half][r] = s2;
      sdot[2][half][r] = s3;
    }
  }

  // dQ = dPs K + diag(scale e^G) U1,
  // dK = dAs K + dAs^T K + dPs^T Q - diag(beta e^G) Ua + diag(e^{G_n - G}) Ub
  f32x4 dq[TPD], dk[TPD];
  zero(dq);
  zero(dk);
  if constexpr (H16Q) {
    // A fragments of dPs, dAs (this wave's rows) and of dAs^T, dPs^T (transposed reads),
    // B fragments of K, Q (transposed reads), 32 chunk rows per step
    using M = Mma<false>;
    const int i = lane & 15;
#pragma unroll
    for (int k0 = 0; k0 < BC; k0 += 32) {
      const M::frag aP = M::load(hP, LDS64, wd.r0 + i, k0, lane);
      const M::frag aPl = M::load(hPl, LDS64, wd.r0 + i, k0, lane);
      const M::frag aA = M::load(hA, LDS64, wd.r0 + i, k0, lane);
      const M::frag aAl = M::load(hAl, LDS64, wd.r0 + i, k0, lane);
      const M::frag tA = frag_tr(hA, LDS64, k0, wd.r0, lane);
      const M::frag tAl = frag_tr(hAl, LDS64, k0, wd.r0, lane);
      const M::frag tP = frag_tr(hP, LDS64, k0, wd.r0, lane);
      const M::frag tPl = frag_tr(hPl, LDS64, k0, wd.r0, lane);
#pragma unroll
      for (int t = 0; t < TPD; ++t) {
        const M::frag bK = frag_tr(hK, LDKH, k0, wd.c0 + 16 * t, lane);
        const M::frag bQ = frag_tr(hQ, LDKH, k0, wd.c0 + 16 * t, lane);
        dq[t] = M::mma(aPl, bK, M::mma(aP, bK, dq[t]));
        dk[t] = M::mma(aAl, bK, M::mma(aA, bK, dk[t]));
        dk[t] = M::mma(tAl, bK, M::mma(tA, bK, dk[t]));
        dk[t] = M::mma(tPl, bQ, M::mma(tP, bQ, dk[t]));
      }
    }
  } else {
    mmf3(dq, dk, dk, wd, sdPs, LDG, 1, sdAs, LDG, 1, sdAs, 1, LDG, sK, LDD, 1, BC, lane);
    mmf(dk, wd, sdPs, 1, LDG, sQ, LDD, 1, BC, lane);
  }
  {
    float *dst;
    size_t rs;
    if (p.Hk == p.Hv) {
      dst = p.dq + static_cast<size_t>(hk) * D;
      rs = static_cast<size_t>(p.Hk) * D;
    } else {
      dst = p.dq_h + static_cast<size_t>(h) * D;
      rs = static_cast<size_t>(p.Hv) * D;
    }
#pragma unroll
    for (int t = 0; t < TPD; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = wd.row(v, lane);
        if (r < rows && (ts + r) % p.nh == p.nh - 1)   // query rows: one per token
          dst[static_cast<size_t>((ts + r) / p.nh) * rs + wd.col(t, lane)] =
              dq[t][v] + p.scale * rf.eG[r] * U1[t][v];
      }
  }
  {
    float *dst;
    size_t rs;
    if (p.Hk == p.Hv) {
      dst = p.dk + static_cast<size_t>(hk) * D;
      rs = static_cast<size_t>(p.Hk) * D;
    } else {
      dst = p.dk_h + static_cast<size_t>(h) * D;
      rs = static_cast<size_t>(p.Hv) * D;
    }
#pragma unroll
    for (int t = 0; t < TPD; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = wd.row(v, lane);
        if (r < rows)
          dst[static_cast<size_t>(ts + r) * rs + wd.col(t, lane)] =
              dk[t][v] - rf.beta[r] * rf.eG[r] * Ua[t][v] + rf.eGl[r] * Ub[t][v];
      }
  }
  __syncthreads();

  // dbeta and dG per row, then dg = reverse cumulative sum of dG (wave 0)
  if (tid < BC) {
    const int r = tid;
    float d0 = 0.0f, x = 0.0f, wb = 0.0f;
#pragma unroll
    for (int m = 0; m < HALVES; ++m) {
      d0 += sdot[0][m][r];
      x += sdot[1][m][r];
      wb += sdot[2][m][r];
    }
    const float w = rf.eGl[r] * wb;
    float dG = srow[0][r] - srow[1][r] + p.scale * rf.eG[r] * d0 - rf.beta[r] * rf.eG[r] * x - w;
    float wsum = w;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) wsum += __shfl_xor(wsum, o, 64);
    if (r == BC - 1) {
      float hsum = 0.0f;
#pragma unroll
      for (int m = 0; m < NW; ++m) hsum += sred[m];
      dG += rf.eG[BC - 1] * hsum + wsum;
    }
    const float db = srow[2][r] + srv[r] - rf.eG[r] * x;
    // reverse inclusive scan: dg_r = sum_{r' >= r} dG_r'
    float s = dG;
#pragma unroll
    for (int o = 1; o < BC; o <<= 1) {
      const float y = __shfl_down(s, o, 64);
      if (r + o < BC) s += y;
    }
    if (r < rows) {
      p.dbeta[static_cast<size_t>(ts + r) * p.Hv + h] = db;
      // g_t sits on the token's first row: dg_t = sum of dG over the rows from there
      if ((ts + r) % p.nh == 0) p.dg[static_cast<size_t>((ts + r) / p.nh) * p.Hv + h] = s;
    }
  }
}

// grouped heads: dq[t, hk] = sum of the group's per-value-head dq (tokens), and
// the same for dk (rows)
template <int D>
__global__ void bwd_group_sum_kernel(const BackwardParams p, long total_q, long total_k) {
  const long i = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total_k) return;
  const int e = static_cast<int>(i % D);
  const long th = i / D;                 // row * Hk + hk
  const int hk = static_cast<int>(th % p.Hk);
  const long t = th / p.Hk;
  const int grp = p.Hv / p.Hk;
  float sq = 0.0f, sk = 0.0f;
  for (int m = 0; m < grp; ++m) {
    const size_t src = (static_cast<size_t>(t) * p.Hv + hk * grp + m) * D + e;
    if (i < total_q) sq += p.dq_h[src];
    sk += p.dk_h[src];
  }
  if (i < total_q) p.dq[i] = sq;
  p.dk[i] = sk;
}

// ---- in-kernel L2 norm and gates from raw projections ------------------------------

// The rows of D elements of the L2 norm kernels: eight consecutive elements per lane
// (one 16-byte load of bf16), D / 8 lanes per row, 64 / (D / 8) rows per wave; a row's
// sums are reduced over its lane group.  Rows past the end load zeros and store nothing,
// so that every lane takes part in the shuffles.
template <int D>
struct L2Rows {
  static constexpr int LPR = D / 8, RPW = 64 / LPR, RPB = 4 * RPW;   // 256 threads
  static __device__ __forceinline__ float sum(float x) {
#pragma unroll
    for (int o = LPR / 2; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
  }
};

// (token, q/k head) rows of D: x / sqrt(sum x^2 + 1e-6) into fp32 copies
template <typename TIn, int D>
__global__ void __launch_bounds__(256) bwd_l2norm_kernel(const BackwardParams p, float *qn,
                                                         float *kn, long rows_q, long rows) {
  using R = L2Rows<D>;
  const int lane = threadIdx.x & 63;
  const long row = (static_cast<long>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * R::RPW +
                   lane / R::LPR;
  const int c0 = 8 * (lane % R::LPR);
  for (int w = 0; w < 2; ++w) {   // q rows exist below rows_q, k rows below rows
    const bool has = row < (w ? rows : rows_q);
    Seg8<TIn> in;
    if (has)
      in.load(static_cast<const TIn *>(w ? p.k_raw : p.q_raw) + row * D + c0);
    else
      in.zero();
    float x[8], ss = 0.0f;
    in.get(x);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
    const float rn = 1.0f / sqrtf(R::sum(ss) + 1e-6f);
    if (has) {
      float *dst = (w ? kn : qn) + row * D + c0;
      *reinterpret_cast<float4 *>(dst) = make_float4(x[0] * rn, x[1] * rn, x[2] * rn, x[3] * rn);
      *reinterpret_cast<float4 *>(dst + 4) =
          make_float4(x[4] * rn, x[5] * rn, x[6] * rn, x[7] * rn);
    }
  }
}

// g = -exp(A_log) softplus(alpha + dt_bias) per (token, value head) and
// beta = sigmoid(b) per (row, value head)
__global__ void bwd_gates_kernel(const BackwardParams p, float *g, float *beta, long n_tok,
                                 long n_row) {
  const long i = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n_row) return;
  const int h = static_cast<int>(i % p.Hv);
  if (i < n_tok) g[i] = gate_decay(p.alpha_raw[i], expf(p.A_log[h]), p.dt_bias[h]);
  beta[i] = gate_beta(p.b_raw[i]);
}

// dx = (dx^ - x^ (x^ . dx^)) / n with n = sqrt(sum x^2 + 1e-6), x^ = x / n, in place
// on dq and dk (rows as in the norm kernel above)
template <typename TIn, int D>
__global__ void __launch_bounds__(256) bwd_l2norm_grad_kernel(const BackwardParams p, long rows_q,
                                                              long rows) {
  using R = L2Rows<D>;
  const int lane = threadIdx.x & 63;
  const long row = (static_cast<long>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * R::RPW +
                   lane / R::LPR;
  const int c0 = 8 * (lane % R::LPR);
  for (int w = 0; w < 2; ++w) {   // q rows exist below rows_q, k rows below rows
    const bool has = row < (w ? rows : rows_q);
    float *dx = (w ? p.dk : p.dq) + row * D + c0;
    Seg8<TIn> in;
    Seg8<float> din;
    if (has) {
      in.load(static_cast<const TIn *>(w ? p.k_raw : p.q_raw) + row * D + c0);
      din.load(dx);
    } else {
      in.zero();
      din.zero();
    }
    float x[8], d[8], ss = 0.0f;
    in.get(x);
    din.get(d);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
    const float rn = 1.0f / sqrtf(R::sum(ss) + 1e-6f);
    float dot = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) dot = fmaf(x[e] * rn, d[e], dot);
    dot = R::sum(dot);
    if (has) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (d[e] - x[e] * rn * dot) * rn;
      *reinterpret_cast<float4 *>(dx) = make_float4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<float4 *>(dx + 4) = make_float4(o[4], o[5], o[6], o[7]);
    }
  }
}

// Chain rule through the gates, one workgroup per value head (a fixed-order sum over
// tokens): dalpha = dg * dg/dalpha = -dg A sigmoid(alpha + dt_bias), db = dbeta
// beta (1 - beta), both in place; dA_log = sum_t dg g (dg/dA_log = g) and
// ddt_bias = sum_t dalpha.
__global__ void __launch_bounds__(256) bwd_gates_grad_kernel(const BackwardParams p) {
  __shared__ float red[2][256];
  const int h = blockIdx.x, tid = threadIdx.x;
  const float A = expf(p.A_log[h]), dtb = p.dt_bias[h];
  float sa = 0.0f, sd = 0.0f;
  for (long t = tid; t < p.tokens; t += 256) {
    const size_t i = static_cast<size_t>(t) * p.Hv + h;
    const float x = p.alpha_raw[i] + dtb;
    const float dg = p.dg[i];
    const float g = -A * softplus_f32(x);
    const float da = -dg * A / (1.0f + expf(-x));
    p.dg[i] = da;
    sa = fmaf(dg, g, sa);
    sd += da;
  }
  for (long t = tid; t < p.tokens * p.nh; t += 256) {
    const size_t i = static_cast<size_t>(t) * p.Hv + h;
    const float b = gate_beta(p.b_raw[i]);
    p.dbeta[i] *= b * (1.0f - b);
  }
  red[0][tid] = sa;
  red[1][tid] = sd;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) {
      red[0][tid] += red[0][tid + o];
      red[1][tid] += red[1][tid + o];
    }
    __syncthreads();
  }
  if (tid == 0) {
    p.dA_log[h] = red[0][0];
    p.ddt_bias[h] = red[1][0];
  }
}

namespace {

template <typename TIn, typename TQK, int D>
hipError_t launch_bwd_qk(const BackwardParams &p, int max_chunks, hipStream_t s) {
  if (max_chunks > 0)
    hipLaunchKernelGGL((bwd_local_kernel<TIn, TQK, D>), dim3(max_chunks, p.Hv), dim3(BT), 0, s,
                       p);
  // every (sequence, head) runs the sweep: an empty sequence passes dH_T to dH0;
  // 16-column tiles when 32-column ones leave compute units idle
  const int rounds = (p.num_seqs * p.Hv + 7) / 8;   // XCD rounds of (sequence, head) groups
  bool narrow = false;
  if constexpr (D == 128) {
    narrow = static_cast<long>(p.num_seqs) * p.Hv * (D / 32) < kCUs;
    if (narrow)
      hipLaunchKernelGGL((bwd_sweep_kernel<TIn, TQK, D, 16>), dim3(8 * (D / 16) * rounds),
                         dim3(BT), 0, s, p);
  }
  if (!narrow)
    hipLaunchKernelGGL((bwd_sweep_kernel<TIn, TQK, D, 32>), dim3(8 * (D / 32) * rounds),
                       dim3(BT), 0, s, p);
  if (max_chunks > 0)
    hipLaunchKernelGGL((bwd_grads_kernel<TIn, TQK, D>), dim3(max_chunks, p.Hv), dim3(BT), 0, s,
                       p);
  return hipSuccess;
}

template <typename TIn, int D>
hipError_t launch_bwd_d(const BackwardParams &p, int max_chunks, long tokens, hipStream_t s) {
  // with the in-kernel L2 norm the kernels read the normalised fp32 copies of q, k
  if (p.q_raw)
    launch_bwd_qk<TIn, float, D>(p, max_chunks, s);
  else
    launch_bwd_qk<TIn, TIn, D>(p, max_chunks, s);
  if (p.Hv != p.Hk && tokens > 0) {
    const long total_q = tokens * p.Hk * D, total_k = total_q * p.nh;
    hipLaunchKernelGGL((bwd_group_sum_kernel<D>), dim3((total_k + 255) / 256), dim3(256), 0, s,
                       p, total_q, total_k);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward_table(const BackwardParams &p, hipStream_t stream) {
  hipLaunchKernelGGL(bwd_table_kernel, dim3(1), dim3(64), 0, stream, p);
  return hipGetLastError();
}

template <typename TIn, int D>
hipError_t launch_pro_d(const BackwardParams &p, hipStream_t s) {
  const long rows_q = p.tokens * p.Hk, rows = rows_q * p.nh;
  if (p.q_raw && rows > 0) {   // (an empty grid is a launch error)
    constexpr long RPB = L2Rows<D>::RPB;
    hipLaunchKernelGGL((bwd_l2norm_kernel<TIn, D>), dim3((rows + RPB - 1) / RPB), dim3(256), 0, s,
                       p, const_cast<float *>(static_cast<const float *>(p.q)),
                       const_cast<float *>(static_cast<const float *>(p.k)), rows_q, rows);
  }
  const long n_tok = p.tokens * p.Hv, n_row = n_tok * p.nh;
  if (p.alpha_raw && n_row > 0) {
    hipLaunchKernelGGL(bwd_gates_kernel, dim3((n_row + 255) / 256), dim3(256), 0, s, p,
                       const_cast<float *>(p.g), const_cast<float *>(p.beta), n_tok, n_row);
  }
  return hipGetLastError();
}

template <typename TIn, int D>
hipError_t launch_epi_d(const BackwardParams &p, hipStream_t s) {
  const long rows_q = p.tokens * p.Hk, rows = rows_q * p.nh;
  constexpr long RPB = L2Rows<D>::RPB;
  if (p.q_raw && rows > 0)
    hipLaunchKernelGGL((bwd_l2norm_grad_kernel<TIn, D>), dim3((rows + RPB - 1) / RPB), dim3(256),
                       0, s, p, rows_q, rows);
  // gate mode (dA_log is set exactly then): runs with no tokens too, so that dA_log and
  // ddt_bias are written (zeros) even when the projections are empty
  if (p.dA_log) hipLaunchKernelGGL(bwd_gates_grad_kernel, dim3(p.Hv), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_backward_prologue(const BackwardParams &p, int qkv_f32, int head,
                                    hipStream_t stream) {
  if (p.tokens == 0) return hipSuccess;
  if (head == 64) return qkv_f32 ? launch_pro_d<float, 64>(p, stream)
                                 : launch_pro_d<uint16_t, 64>(p, stream);
  if (head == 128) return qkv_f32 ? launch_pro_d<float, 128>(p, stream)
                                  : launch_pro_d<uint16_t, 128>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_backward_epilogue(const BackwardParams &p, int qkv_f32, int head,
                                    hipStream_t stream) {
  if (p.dA_log == nullptr && p.q_raw == nullptr) return hipSuccess;   // no norm, no gate mode
  if (head == 64) return qkv_f32 ? launch_epi_d<float, 64>(p, stream)
                                 : launch_epi_d<uint16_t, 64>(p, stream);
  if (head == 128) return qkv_f32 ? launch_epi_d<float, 128>(p, stream)
                                  : launch_epi_d<uint16_t, 128>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_backward(const BackwardParams &p, int qkv_f32, int head, int max_chunks,
                           long tokens, hipStream_t stream) {
  if (head == 64)
    return qkv_f32 ? launch_bwd_d<float, 64>(p, max_chunks, tokens, stream)
                   : launch_bwd_d<uint16_t, 64>(p, max_chunks, tokens, stream);
  if (head == 128)
    return qkv_f32 ? launch_bwd_d<float, 128>(p, max_chunks, tokens, stream)
                   : launch_bwd_d<uint16_t, 128>(p, max_chunks, tokens, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdr
