// Chunked prefill of the gated delta rule on 64-row chunks (bf16 inputs, fp16
// matrix-core operands with fp32 accumulation, fp32 state).
//
// Same chunk algebra as prefill.hip (Megatron Core API page
// "core.ssm.gated_delta_net.gdn", torch_chunk_gated_delta_rule; n_h Householder
// sub-steps per token, page "core.ssm.gated_delta_product"): with H = S^T (K x V),
// inside one chunk entering with state H0,
//   A = strict_lower(diag(beta) K K^T * Gamma),  R = diag(beta) (V - diag(exp G) K H0),
//   D = (I + A)^-1 R,
//   O = scale (diag(exp G) Q H0 + (Q K^T * Gamma) D),
//   H_n = exp(G_last) H0 + K^T diag(exp(G_last - G)) D.
// A chunk here is 64 rows (64 / n_h tokens).  (I + A)^-1 R is evaluated by block
// forward substitution over the four 16-row blocks with the inverses of the
// diagonal blocks only:  D_b = T_bb (R_b - sum_{c<b} A_bc D_c),  T_bb = (I + A_bb)^-1.
//
// Why 64 rows: the work that does not grow with the rows of a chunk (scaling the
// state by exp(G_last), converting it to fp16 operands, the workgroup barriers, the
// sixteen-step back substitution of the diagonal inverses, which inverts all four
// blocks at once in the 64 lanes of one wave) is spread over twice the rows of a
// 32-row chunk.
//
// Layout in LDS: K, Q (fp16, converted from bf16 and optionally L2-normalised) and V
// (the workgroup's value columns, raw bf16) are stored row-major only.  The products
// that need them transposed (K^T as the A operand of the state update, V in the
// accumulator layout of R) read them with the gfx950 LDS transpose load
// (ds_read_b64_tr_b16): within each 16-lane group, lane s names 8 bytes at row
// r0 + 4g + s/4, column c0 + 4 (s % 4); lane j of the group then receives
// M[r0 + 4g + e][c0 + j], e = 0..3 (the layout of a 16x16 accumulator tile, and,
// two reads stacked, of a 32-deep operand fragment).
//
// Work decomposition: one workgroup per (sequence, value head, tile of 32 NS value
// columns), with NS state waves (32 columns of H each, in registers for the whole
// sequence) and four producer waves.  Each chunk interval has two phases separated
// by workgroup barriers:
//   phase A: state waves  X = K H0, R and D of chunk i;
//            producers    stage chunk i+1 (K in the layout of an operand of the
//                         producer's own 16-row block, whose diagonal block of A each
//                         producer then forms from registers), fetch chunk i+2;
//   phase B: state waves  O and the state update of chunk i; the next chunk's
//                         values into the wave's own LDS columns;
//            producers    solve chunk i+1: the inverses of the diagonal blocks, A_32
//                         and the decay scan of chunk i+2 (wave 0), the other
//                         off-diagonal blocks of A (wave 1), the causal tiles of
//                         P = scale (Q K^T * Gamma) (waves 2 and 3).
// Staged chunks and solved operands are double-buffered in LDS, the per-row decay
// factors triple-buffered (written two phases before their interval), the values
// single-buffered (each state wave reads only the columns it wrote).  Inputs and
// outputs go through range-checked buffer resources that end at the sequence's last
// row: rows past it read as zero and are never written, with no clamps or branches.

#include "chunk_helpers.hpp"
#include "common.hpp"
#include "gdr_internal.hpp"

namespace gdr {

typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Word 3 of a raw buffer resource (32-bit data format, no swizzle, no stride): loads
// and stores at offsets past the resource's byte count are dropped.
constexpr int kBufferWord3 = 0x00020000;

// four consecutive outputs at a byte offset of a buffer resource (dropped past its end)
template <typename TOut>
__device__ __forceinline__ void store4_rsrc(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 o) {
  if constexpr (sizeof(TOut) == 4) {
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, o), r, off, 0, 0);
  } else {
    typedef int i32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    const bf16x4 h = __builtin_convertvector(o, bf16x4);
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, h), r, off, 0, 0);
  }
}

// two floats -> two fp16 in one word (one v_cvt_pk_f16_f32, round to nearest even)
__device__ __forceinline__ uint32_t pk_f16(float a, float b) {
  const f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, h16x2));
}
// eight bf16 (raw bits) -> eight fp16 in LDS with one 16-byte store
__device__ __forceinline__ void store8_bf16_as_f16(_Float16 *dst, const uint4 &u) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  uint32_t r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pk_f16(__uint_as_float(w[i] << 16), __uint_as_float(w[i] & 0xffff0000u));
  *reinterpret_cast<uint4 *>(dst) = make_uint4(r[0], r[1], r[2], r[3]);
}
// eight floats -> eight fp16 in LDS with one 16-byte store
__device__ __forceinline__ void store8_pk(_Float16 *dst, const float (&x)[8]) {
  *reinterpret_cast<uint4 *>(dst) =
      make_uint4(pk_f16(x[0], x[1]), pk_f16(x[2], x[3]), pk_f16(x[4], x[5]), pk_f16(x[6], x[7]));
}

// Buffer resource over rows [r0, r0 + nrows) of a row-major 16-bit matrix with `stride`
// elements per row: loads past those rows read as zero.
// The arguments are uniform across the wave; the read-first-lane tells the compiler so
// (a resource it takes for divergent would be applied lane group by lane group).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t *base, int r0,
                                                            int nrows, uint32_t stride) {
  const uint64_t a = reinterpret_cast<uint64_t>(base + static_cast<size_t>(r0) * stride);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  const int bytes = __builtin_amdgcn_readfirstlane(
      static_cast<int>(static_cast<uint32_t>(max(nrows, 0)) * stride * 2));
  return __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void *>((static_cast<uint64_t>(hi) << 32) | lo), 0, bytes, kBufferWord3);
}
// Gates from raw projections (g = -A softplus(alpha + dt_bias), beta = sigmoid(b)) on
// the hardware exp2, log2 and reciprocal, each within about 1 ulp: this kernel's
// inputs are bf16, whose rounding is far coarser.  softplus(x) = max(x, 0) +
// log1p(e^-|x|), with log1p(y) = ln(u) y / (u - 1) for u = 1 + y (u - 1 is exact;
// y itself when u rounds to 1), so that exp never overflows and small y keep their
// relative accuracy.
__device__ __forceinline__ float softplus_hw(float x) {
  const float y = __builtin_amdgcn_exp2f(-fabsf(x) * 1.4426950408889634f);
  const float u = 1.0f + y;
  const float l = u == 1.0f ? y
                            : __builtin_amdgcn_logf(u) * 0.6931471805599453f * y *
                                  __builtin_amdgcn_rcpf(u - 1.0f);
  return fmaxf(x, 0.0f) + l;
}
__device__ __forceinline__ float sigmoid_hw(float b) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-b * 1.4426950408889634f));
}

// sixteen bytes at a byte offset of a buffer resource
__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

template <int DK_, int NH_, int NS_>
struct P64 {
  using M = Mma<false>;
  using frag = M::frag;
  static constexpr int DK = DK_, NH = NH_, NS = NS_;
  static constexpr int CR = 64;                 // rows per chunk
  static constexpr int NP = 4;                  // producer waves
  static constexpr int NW = NS + NP;
  static constexpr int NT = 64 * NW;
  static constexpr int ST = 64 * NP;            // staging threads
  static constexpr int CQ = CR / NH;            // query rows per chunk
  static constexpr int NQB = CQ / 16;
  static constexpr int DVT = 32 * NS;           // value columns per workgroup
  static constexpr int LDK = DK + 8;            // K, Q row stride (elements)
  static constexpr int LDV = DVT + 8;           // V row stride
  static constexpr int LDA = CR + 8;            // A (64 x 64) and P (CQ x 64) row stride
  static constexpr int LDT = 32 + 8;            // T rows: T_bb in columns 0..15, zeros after
  static constexpr int LDR = 20;                // fp32 diagonal blocks for the inversion
  static constexpr int ARB = 16 * LDR + 4;
  static constexpr int KS = DK / 32;            // 32-deep slices over keys
  static constexpr int KM = DK / 16;            // 16-row blocks of H
  static constexpr int SEG = DK / 8;            // 8-element segments per K / Q row
  static constexpr int KPT = CR * SEG / ST;     // K segments per staging thread
  static constexpr int QPT = CQ * SEG / ST;
  static_assert(KPT * ST == CR * SEG && QPT * ST == CQ * SEG, "staging split");
  static_assert(QPT >= 1 && NQB >= 1, "staging split");
};

template <class Tr>
struct alignas(16) Stage64 {
  _Float16 K[Tr::CR * Tr::LDK];
  _Float16 Q[Tr::CQ * Tr::LDK];
  float G2[Tr::CR];               // G_r log2(e): exponent base of the solve's columns
  float GB[Tr::CR];               // G_r log2(e) + log2(beta_r): base of A's rows
};
// the per-row factors the state waves read (a chunk's are written two phases before its
// interval, and read through all of it: three buffers)
template <class Tr>
struct alignas(16) Fac64 {
  float eG[Tr::CR];               // exp(G_r)
  float eGl[Tr::CR];              // exp(G_last - G_r)
  float B[Tr::CR];                // beta
};
template <class Tr>
struct alignas(16) Solve64 {
  _Float16 T[Tr::CR * Tr::LDT];   // rows 16b..16b+15: -T_bb in columns 0..15
  _Float16 A[Tr::CR * Tr::LDA];   // A_bc, b > c; diagonal and upper blocks zero
  _Float16 P[Tr::CQ * Tr::LDA];   // scale (Q K^T * Gamma), causal
};
template <class Tr>
struct Smem64 {
  Stage64<Tr> st[2];
  Solve64<Tr> sv[2];
  Fac64<Tr> fac[3];
  float AR[4][Tr::ARB];
  uint16_t V[Tr::CR * Tr::LDV];   // the chunk's values (raw bf16), 32 columns per state wave
};

// the producer wave that loads the gates and runs the per-chunk decay scan (with outputs;
// without them, producer 3, which then has no tiles of P to form)
template <bool OUT>
constexpr int scan_producer() { return OUT ? 0 : 3; }

struct Scan64 {
  float g2, gb, eg, egl, b;
};

template <class Tr>
struct Regs64 {
  Seg8<uint16_t> k[Tr::KPT], q[Tr::QPT];
  float g, b;     // gates of the chunk the decay scan reads next
};

// ---- the solve of one chunk (producer waves, phase B) --------------------------------
//
// Every tile is formed transposed (K_c X_b^T, X = K or Q), so that a lane holds four
// consecutive columns of one row and writes them with one store.  Its entries are
// scaled by exp(G_r - G_c) times beta_r (A) or the output scale (P), evaluated as
// exp2 of a difference of per-row bases in log2 units (GB = G log2 e + log2 beta, G2 =
// G log2 e); entries at or above the diagonal are masked before the exponential
// (there G_r - G_c may be large and positive).  Each wave loads the K row blocks it
// needs once and reuses them across its tiles.

// operand fragments of the 16-row block b of a row-major fp16 matrix (all KS slices)
template <class Tr>
__device__ __forceinline__ void p64_block(const _Float16 *X, int b, int lane,
                                          typename Tr::M::frag (&f)[Tr::KS]) {
#pragma unroll
  for (int sl = 0; sl < Tr::KS; ++sl)
    f[sl] = Tr::M::load(X, Tr::LDK, 16 * b + (lane & 15), 32 * sl, lane);
}

// one tile: acc = (K_c X_q^T) -> row q0 + l16, columns 16 c + 4 g4 + i of `dst`,
// scaled by exp2(base - G2[col]); with MASK, columns past `rmax(q)` are zero
template <class Tr, bool MASK>
__device__ __forceinline__ void p64_tile_out(const Stage64<Tr> &s, f32x4 acc, float base,
                                             int rlast, _Float16 *dst, int c, int lane) {
  const int g4 = lane >> 4;
  const float4 gc = *reinterpret_cast<const float4 *>(s.G2 + 16 * c + 4 * g4);
  const float gcv[4] = {gc.x, gc.y, gc.z, gc.w};
  float x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float d = base - gcv[i];
    if constexpr (MASK) {
      const int col = 16 * c + 4 * g4 + i;
      x[i] = acc[i] * __builtin_amdgcn_exp2f(col <= rlast ? d : -INFINITY);
    } else {
      x[i] = acc[i] * __builtin_amdgcn_exp2f(d);
    }
  }
  store4e(dst + 16 * c + 4 * g4, x);
}

// Diagonal block b of A from the raw product K_b K_b^T (accumulator layout): fp32 in
// AR[b].  The product is symmetric, so its accumulator tile also gives lane (l16, g4)
// row l16, columns 4 g4 .. 4 g4 + 3: entries left of the diagonal are scaled by
// exp2(GB_row - G2_col), the rest masked to zero before the exponential.
struct DiagBases {
  float base;
  float4 gc;
};
template <class Tr>
__device__ __forceinline__ DiagBases p64_diag_bases(const Stage64<Tr> &s, int b, int lane) {
  const int l16 = lane & 15, g4 = lane >> 4;
  return {s.GB[16 * b + l16], *reinterpret_cast<const float4 *>(s.G2 + 16 * b + 4 * g4)};
}
template <class Tr>
__device__ __forceinline__ void p64_diag_put(const DiagBases &d, f32x4 acc, int b,
                                             float (*AR)[Tr::ARB], int lane) {
  const int l16 = lane & 15, g4 = lane >> 4;
  const float gcv[4] = {d.gc.x, d.gc.y, d.gc.z, d.gc.w};
  float a[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    a[i] = acc[i] * __builtin_amdgcn_exp2f(4 * g4 + i < l16 ? d.base - gcv[i] : -INFINITY);
  *reinterpret_cast<float4 *>(AR[b] + l16 * Tr::LDR + 4 * g4) = make_float4(a[0], a[1], a[2], a[3]);
}
template <class Tr>
__device__ __forceinline__ void p64_diag_store(const Stage64<Tr> &s, f32x4 acc, int b,
                                               float (*AR)[Tr::ARB], int lane) {
  p64_diag_put<Tr>(p64_diag_bases<Tr>(s, b, lane), acc, b, AR, lane);
}

// All four diagonal blocks from the staged K (the first chunk of a sequence; later
// chunks' blocks are formed by the producers from registers while staging).  The
// operands are read in the staging registers' layout (lane: row l16, contraction
// indices 32 sl + 8 g4 .. + 7), so that both ways give the same bits.
template <class Tr>
__device__ __forceinline__ void p64_diag_lds(const Stage64<Tr> &s, float (*AR)[Tr::ARB],
                                             int lane) {
  using M = typename Tr::M;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    if (b == 2) __builtin_amdgcn_sched_barrier(0);   // two blocks' operands at a time
    typename M::frag f[Tr::KS];
#pragma unroll
    for (int sl = 0; sl < Tr::KS; ++sl)
      f[sl].v = *reinterpret_cast<const f16x8 *>(s.K + (16 * b + (lane & 15)) * Tr::LDK +
                                                  32 * sl + 8 * (lane >> 4));
    f32x4 acc = zero4();
#pragma unroll
    for (int sl = 0; sl < Tr::KS; ++sl) acc = M::mma(f[sl], f[sl], acc);
    p64_diag_store<Tr>(s, acc, b, AR, lane);
  }
}

// The inverses T_bb = (I + A_bb)^-1 of the four diagonal blocks in AR.  Row j of T_bb
// solves the upper triangular system (I + A_bb)^T t = e_j by back substitution; lane
// 16 b + j does it for block b, so one pass over the 64 lanes inverts all four.
template <class Tr>
__device__ __forceinline__ void p64_invert(Solve64<Tr> &v, float (*AR)[Tr::ARB], int lane) {
  constexpr int LDT = Tr::LDT, LDR = Tr::LDR;
  const int bk = lane >> 4, j = lane & 15;
  const float *Ab = AR[bk];
  float t[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) t[r] = (r == j) ? 1.0f : 0.0f;
  // step c subtracts row c of A_bb (left of its diagonal) times t_c; the rows are read
  // in three batches, each ahead of its steps
  auto steps = [&](auto first, auto count) __attribute__((always_inline)) {
    constexpr int C0 = decltype(first)::value, NC = decltype(count)::value;
    float4 row[NC][4];
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
#pragma unroll
      for (int qd = 0; qd <= (C0 - cc - 1) / 4; ++qd)
        row[cc][qd] = *reinterpret_cast<const float4 *>(Ab + (C0 - cc) * LDR + 4 * qd);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      const int c = C0 - cc;
#pragma unroll
      for (int r = 0; r < c; ++r) {
        const float4 q = row[cc][r / 4];
        const float acr = (r & 3) == 0 ? q.x : (r & 3) == 1 ? q.y : (r & 3) == 2 ? q.z : q.w;
        t[r] -= acr * t[c];
      }
    }
  };
  steps(std::integral_constant<int, 15>(), std::integral_constant<int, 5>());
  steps(std::integral_constant<int, 10>(), std::integral_constant<int, 5>());
  steps(std::integral_constant<int, 5>(), std::integral_constant<int, 5>());
  // stored negated: the state waves' substitution steps take -T_bb (see there)
  _Float16 *trow = v.T + (16 * bk + j) * LDT;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float x[4] = {-t[4 * q], -t[4 * q + 1], -t[4 * q + 2], -t[4 * q + 3]};
    store4e(trow + 4 * q, x);
  }
}

// The off-diagonal blocks A_bc, b > c (no mask: every column is left of the diagonal).
// Producer 1 forms all but A_32, which producer 0 forms beside the inversion.
template <class Tr>
__device__ __forceinline__ void p64_offdiag(const Stage64<Tr> &s, Solve64<Tr> &v, int lane) {
  using M = typename Tr::M;
  constexpr int KS = Tr::KS;
  const int l16 = lane & 15;
  typename M::frag f[4][KS];
#pragma unroll
  for (int b = 0; b < 4; ++b) p64_block<Tr>(s.K, b, lane, f[b]);
#pragma unroll
  for (int b = 1; b < 4; ++b) {
    const int q = 16 * b + l16;
    const float base = s.GB[q];
#pragma unroll
    for (int c = 0; c < (b == 3 ? 2 : b); ++c) {
      f32x4 acc = zero4();
#pragma unroll
      for (int sl = 0; sl < KS; ++sl) acc = M::mma(f[c][sl], f[b][sl], acc);
      p64_tile_out<Tr, false>(s, acc, base, 0, v.A + q * Tr::LDA, c, lane);
    }
  }
}

// The causal tiles of P = scale (Q K^T * Gamma) for query blocks MQ0 and MQ1 (-1: none):
// query row q reads key row r = n_h q + n_h - 1 and keys 0 .. r.
template <class Tr, int MQ0, int MQ1>
__device__ __forceinline__ void p64_prows(const Stage64<Tr> &s, Solve64<Tr> &v, float scale,
                                          int lane) {
  using M = typename Tr::M;
  constexpr int KS = Tr::KS, NH = Tr::NH;
  // last key block of query block mq
  constexpr auto kmax = [](int mq) { return (NH * (16 * mq + 16) - 1) / 16; };
  constexpr int NK = 1 + (kmax(MQ0) > (MQ1 >= 0 ? kmax(MQ1) : 0) ? kmax(MQ0) : kmax(MQ1));
  const int l16 = lane & 15;
  const float lscale = __builtin_amdgcn_logf(fabsf(scale));   // log2 |scale|
  const float sgn = scale < 0.0f ? -1.0f : 1.0f;
  typename M::frag fk[NK][KS];
#pragma unroll
  for (int ni = 0; ni < NK; ++ni) p64_block<Tr>(s.K, ni, lane, fk[ni]);
  auto row = [&](auto mqc) __attribute__((always_inline)) {
    constexpr int mq = decltype(mqc)::value;
    typename M::frag fq[KS];
    p64_block<Tr>(s.Q, mq, lane, fq);
    const int q = 16 * mq + l16;
    const int r = NH * q + NH - 1;
    const float base = s.G2[r] + lscale;
#pragma unroll
    for (int ni = 0; ni <= kmax(mq); ++ni) {
      f32x4 acc = zero4();
#pragma unroll
      for (int sl = 0; sl < KS; ++sl) acc = M::mma(fk[ni][sl], fq[sl], acc);
      acc *= sgn;
      // keys of this block can pass the query's own row only near the diagonal
      if (16 * ni + 15 > NH * (16 * mq) + NH - 1)
        p64_tile_out<Tr, true>(s, acc, base, r, v.P + q * Tr::LDA, ni, lane);
      else
        p64_tile_out<Tr, false>(s, acc, base, r, v.P + q * Tr::LDA, ni, lane);
    }
  };
  row(std::integral_constant<int, MQ0>());
  if constexpr (MQ1 >= 0) {
    __builtin_amdgcn_sched_barrier(0);
    row(std::integral_constant<int, (MQ1 >= 0 ? MQ1 : 0)>());
  }
}

// A_32 on its own (the pass that writes no outputs)
template <class Tr>
__device__ __forceinline__ void p64_a32(const Stage64<Tr> &s, Solve64<Tr> &v, int lane) {
  using M = typename Tr::M;
  typename M::frag f2[Tr::KS], f3[Tr::KS];
  p64_block<Tr>(s.K, 2, lane, f2);
  p64_block<Tr>(s.K, 3, lane, f3);
  const int q = 48 + (lane & 15);
  f32x4 acc = zero4();
#pragma unroll
  for (int sl = 0; sl < Tr::KS; ++sl) acc = M::mma(f2[sl], f3[sl], acc);
  p64_tile_out<Tr, false>(s, acc, s.GB[q], 0, v.A + q * Tr::LDA, 2, lane);
}

// The solve of one chunk; the diagonal blocks of A are in AR already.  Without
// outputs there is no P to form, and the producers share the rest: the inversions (0),
// five off-diagonal blocks (1), A_32 (2); producer 3 runs the decay scan.
template <class Tr, bool OUT>
__device__ __forceinline__ void p64_solve(const Stage64<Tr> &s, Solve64<Tr> &v,
                                          float (*AR)[Tr::ARB], int pw, float scale, int lane) {
  if constexpr (!OUT) {
    if (pw == 0)
      p64_invert<Tr>(v, AR, lane);
    else if (pw == 1)
      p64_offdiag<Tr>(s, v, lane);
    else if (pw == 2)
      p64_a32<Tr>(s, v, lane);
    return;
  }
  if (pw == 0) {
    // A_32 beside the inversion: its operands are read first, its products issued after
    using M = typename Tr::M;
    typename M::frag f2[Tr::KS], f3[Tr::KS];
    p64_block<Tr>(s.K, 2, lane, f2);
    p64_block<Tr>(s.K, 3, lane, f3);
    const int q = 48 + (lane & 15);
    const float base = s.GB[q];
    p64_invert<Tr>(v, AR, lane);
    f32x4 acc = zero4();
#pragma unroll
    for (int sl = 0; sl < Tr::KS; ++sl) acc = M::mma(f2[sl], f3[sl], acc);
    p64_tile_out<Tr, false>(s, acc, base, 0, v.A + q * Tr::LDA, 2, lane);
  } else if (pw == 1) {
    p64_offdiag<Tr>(s, v, lane);
  } else if constexpr (Tr::NQB == 4) {   // one token per row: 1 + 4 and 2 + 3 tiles
    if (pw == 2)
      p64_prows<Tr, 0, 3>(s, v, scale, lane);
    else
      p64_prows<Tr, 1, 2>(s, v, scale, lane);
  } else {                                // two sub-steps per token: 4 and 2 tiles
    if (pw == 2)
      p64_prows<Tr, 1, -1>(s, v, scale, lane);
    else
      p64_prows<Tr, 0, -1>(s, v, scale, lane);
  }
}

// OUT = false: the call writes no outputs (out == NULL: the passes of a long sequence in
// segments that only carry states, the backward's forward recompute).  Then neither Q
// nor P is needed: Q is neither fetched nor staged, P not formed, and the state waves
// skip the output products.
template <typename TOut, int DK, int NH, int NS, bool OUT>
__global__ void __launch_bounds__(64 * (NS + 4))
prefill64_kernel(const PrefillParams p) {
  using Tr = P64<DK, NH, NS>;
  using M = typename Tr::M;
  using frag = typename M::frag;
  constexpr int CR = Tr::CR, CQ = Tr::CQ, NQB = Tr::NQB, DVT = Tr::DVT, SEG = Tr::SEG;
  constexpr int LDK = Tr::LDK, LDV = Tr::LDV, LDA = Tr::LDA, LDT = Tr::LDT, NT = Tr::NT;
  constexpr int ST = Tr::ST, KS = Tr::KS, KM = Tr::KM, KPT = Tr::KPT, QPT = Tr::QPT;

  __shared__ Smem64<Tr> sm;

  const int w_item = xcd_work_item(blockIdx.x, p.group_size, p.num_groups);
  if (w_item < 0) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const bool is_state = wave < NS;
  const int pw = wave - NS;            // producer wave index (state waves: negative)
  const int stid = tid - 64 * NS;      // staging thread index
  const int l16 = lane & 15;
  const int g4 = lane >> 4;

  // work item -> (sequence, query/key head, value head, column tile)
  const int group = w_item / p.group_size;
  const int member = w_item % p.group_size;
  const int n = group / p.Hk;
  const int hk = group % p.Hk;
  const int h = hk * (p.Hv / p.Hk) + member / p.num_vtiles;
  const int vt = member % p.num_vtiles;
  const int col0 = vt * DVT + 32 * wave;   // first value column of a state wave

  int t0, t1;
  if (p.cu_seqlens) {
    t0 = p.cu_seqlens[n];
    t1 = p.cu_seqlens[n + 1];
  } else {
    t0 = n * p.seqlen;
    t1 = t0 + p.seqlen;
  }
  int bnd_rows = 0, bnd_base = 0;
  if (p.boundary_states) {
    const int iv = p.boundary_interval;
    bnd_rows = iv * NH;
    if (p.cu_seqlens) {
      for (int m = 0; m < n; ++m) bnd_base += (p.cu_seqlens[m + 1] - p.cu_seqlens[m]) / iv;
    } else {
      bnd_base = n * (p.seqlen / iv);
    }
  }
  int src = n, dst = n;
  if (p.state_indices) {
    const int idx = p.state_indices[n];
    src = idx < 0 ? 0 : idx;
    dst = idx;
  }

  // uniform bases; every element offset below fits in 32 bits (checked on the host)
  const uint16_t *__restrict__ kb = static_cast<const uint16_t *>(p.k) + hk * DK;
  const uint16_t *__restrict__ qb = static_cast<const uint16_t *>(p.q) + hk * DK;
  const uint16_t *__restrict__ vrow =
      p.v ? static_cast<const uint16_t *>(p.v) + h * p.DV + vt * DVT : nullptr;
  const float *__restrict__ gb = p.g + h;
  const float *__restrict__ bb = p.beta + h;
  float gate_A = 0.0f, gate_dt = 0.0f;
  if (p.gate_mode) {
    gate_A = expf(p.A_log[h]);
    gate_dt = p.dt_bias[h];
  }
  TOut *__restrict__ ob = p.out ? static_cast<TOut *>(p.out) + h * p.DV + col0 : nullptr;
  const uint32_t kstride = p.Hk * DK;
  const uint32_t vstride = p.Hv * p.DV;
  const size_t state_stride = static_cast<size_t>(DK) * p.DV;

  // the solve buffers' parts that no chunk writes (T columns 16..31, the diagonal and
  // upper blocks of A, the P tiles above the causal boundary) must read as zero
  {
    _Float16 *z = reinterpret_cast<_Float16 *>(&sm.sv[0]);
    constexpr int nz = static_cast<int>(sizeof(sm.sv)) / static_cast<int>(sizeof(_Float16));
    for (int i = tid; i < nz; i += NT) z[i] = static_cast<_Float16>(0.0f);
  }

  const int row_begin = t0 * NH, row_end = t1 * NH;
  const int nchunks = (row_end - row_begin + CR - 1) / CR;

  Regs64<Tr> rg;   // producer registers: the inputs of one chunk between fetch and staging
  frag kh[KPT];    // producer registers: its staged K block as fp16 operand fragments

  // inputs of the chunk starting at row c -> producer registers (addresses clamped to
  // the sequence, also past its end; validity is applied at staging)
  // inputs of the chunk starting at row c -> producer registers, through buffer
  // resources that end at the sequence's last row: rows past it read as zero, which is
  // what the chunk algebra needs of them (no clamps, no masks), and the per-lane offsets
  // stay the same from chunk to chunk
  auto k_rsrc = [&](int c) __attribute__((always_inline)) {
    return rows_rsrc(kb, c, min(CR, row_end - c), kstride);
  };
  auto q_rsrc = [&](int c) __attribute__((always_inline)) {
    const int tq = c / NH;
    return rows_rsrc(qb, tq, min(CQ, t1 - tq), kstride);
  };
  auto k_off = [&](int j) __attribute__((always_inline)) {
    return static_cast<uint32_t>(((16 * pw + l16) * kstride + (4 * j + g4) * 8) * 2);
  };
  auto q_off = [&](int j) __attribute__((always_inline)) {
    const int u = stid + j * ST, r = u / SEG, sg = u % SEG;
    return static_cast<uint32_t>((r * kstride + sg * 8) * 2);
  };
  auto fetch = [&](Regs64<Tr> &cr, int c) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rk = k_rsrc(c), rq = q_rsrc(c);
#pragma unroll
    for (int j = 0; j < KPT; ++j) cr.k[j].u = load16(rk, k_off(j));
    if constexpr (OUT) {
#pragma unroll
      for (int j = 0; j < QPT; ++j) cr.q[j].u = load16(rq, q_off(j));
    }
  };
  // the gates of the chunk starting at row c (producer 0; requested a whole interval
  // before the decay scan reads them)
  auto fetch_gates = [&](Regs64<Tr> &cr, int c) __attribute__((always_inline)) {
    const int row = min(c + lane, row_end - 1);
    cr.g = gb[static_cast<uint32_t>(row / NH) * p.Hv];
    cr.b = bb[static_cast<uint32_t>(row) * p.Hv];
  };
  // producer registers (a chunk; rows past the sequence hold zeros) -> staged LDS
  // buffer.  The L2 norm is a compile-time choice, so that no branch splits the
  // conversions.  Each register is refilled with chunk cn's inputs as soon as it has
  // been consumed, so that those loads have almost a whole interval to land (they
  // take longer than what is left of it after the staging; a chunk past the sequence's
  // end reads zeros).
  auto stage = [&](Regs64<Tr> &cr, Stage64<Tr> &s, auto l2c, int cn) __attribute__((always_inline)) {
    constexpr bool L2 = decltype(l2c)::value;
    const __amdgpu_buffer_rsrc_t rk = k_rsrc(cn), rq = q_rsrc(cn);
    // L2 factor of a row from this lane's partial sum of squares: the lanes that hold
    // the row's other segments are xor 16 and 32 away (K) or xor 1 .. SEG / 2 (Q)
    auto rnorm = [&](float ss, auto krows) __attribute__((always_inline)) {
      if constexpr (decltype(krows)::value) {
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
      } else {
#pragma unroll
        for (int o = SEG / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
      }
      return 1.0f / sqrtf(ss + 1e-6f);
    };
    {   // K: row 16 pw + l16, segments 4 j + g4 (the row's KPT segments in lanes l16,
        // l16 + 16, l16 + 32, l16 + 48)
      float x[KPT][8];
#pragma unroll
      for (int j = 0; j < KPT; ++j) cr.k[j].get(x[j]);
      if constexpr (L2) {
        float ss = 0.0f;
#pragma unroll
        for (int j = 0; j < KPT; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e) ss += x[j][e] * x[j][e];
        const float rn = rnorm(ss, std::true_type());
#pragma unroll
        for (int j = 0; j < KPT; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e) x[j][e] *= rn;
      }
      const int r = 16 * pw + l16;
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const uint4 w = make_uint4(pk_f16(x[j][0], x[j][1]), pk_f16(x[j][2], x[j][3]),
                                   pk_f16(x[j][4], x[j][5]), pk_f16(x[j][6], x[j][7]));
        *reinterpret_cast<uint4 *>(s.K + r * LDK + (4 * j + g4) * 8) = w;
        kh[j].v = __builtin_bit_cast(f16x8, w);
        cr.k[j].u = load16(rk, k_off(j));
      }
    }
    // Q: segment u % SEG of row u / SEG, u = stid + j ST (a row's SEG segments in
    // consecutive lanes); only with outputs
#pragma unroll
    for (int j = 0; j < (OUT ? QPT : 0); ++j) {
      const int u = stid + j * ST, r = u / SEG, sg = u % SEG;
      if constexpr (L2) {
        float x[8];
        cr.q[j].get(x);
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
        const float rn = rnorm(ss, std::false_type());
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= rn;
        store8_pk(s.Q + r * LDK + sg * 8, x);
      } else {
        store8_bf16_as_f16(s.Q + r * LDK + sg * 8, cr.q[j].u);
      }
      cr.q[j].u = load16(rq, q_off(j));
    }
  };
  // Per-row decay factors of the chunk starting at row c (producer 0, from the gates
  // it fetched): the inclusive prefix sum of the per-row decay in fp64 (a token's g
  // sits on its first sub-step) and the factors derived from it; gates formed here
  // from raw projections when asked.  Evaluated one phase before the chunk's staging
  // writes them, where producer 0 has room.
  auto scan = [&](const Regs64<Tr> &cr, int c) __attribute__((always_inline)) {
    const bool ok = lane < min(CR, row_end - c);
    float gv = cr.g;
    float bv = cr.b;
    if (p.gate_mode) {
      gv = -gate_A * softplus_hw(cr.g + gate_dt);
      bv = sigmoid_hw(cr.b);
    }
    const double gr = prefix_sum64((ok && (c + lane) % NH == 0) ? gv : 0.0);
    bv = ok ? bv : 0.0f;
    const double glast = readlane_f64(gr, CR - 1);
    Scan64 sc;
    sc.g2 = static_cast<float>(gr) * 1.4426950408889634f;
    sc.gb = sc.g2 + __builtin_amdgcn_logf(bv);   // log2(0) = -inf: beta 0 rows vanish
    sc.eg = fexp(static_cast<float>(gr));
    sc.egl = fexp(static_cast<float>(glast - gr));
    sc.b = bv;
    return sc;
  };
  // the exponent bases, which the producers read (into the chunk's stage buffer, whose
  // previous chunk no longer needs them), and the factors the state waves read (into
  // the chunk's factor buffer); both stored as soon as evaluated
  auto put_bases = [&](const Scan64 &sc, Stage64<Tr> &s) __attribute__((always_inline)) {
    s.G2[lane] = sc.g2;
    s.GB[lane] = sc.gb;
  };
  auto put_factors = [&](const Scan64 &sc, Fac64<Tr> &f) __attribute__((always_inline)) {
    f.eG[lane] = sc.eg;
    f.eGl[lane] = sc.egl;
    f.B[lane] = sc.b;
  };

  // Each role runs its own code (its registers stay out of the other's): the prologue's
  // two barriers, then two barriers per chunk interval, in both.
  if (is_state) {
    // ---- initial state -> registers of the state waves ------------------------------
    f32x4 H[2][KM];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int m = 0; m < KM; ++m) H[ct][m] = zero4();
    if (p.initial_state) {
      const float *s0 = p.initial_state + (static_cast<size_t>(src) * p.Hv + h) * state_stride;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int m = 0; m < KM; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            H[ct][m][i] = s0[static_cast<size_t>(16 * m + 4 * g4 + i) * p.DV + col0 + 16 * ct + l16];
    }

    auto store_state = [&](float *s1) __attribute__((always_inline)) {
      uint32_t lane_off = static_cast<uint32_t>(4 * g4 * p.DV + col0 + l16);
      asm volatile("" : "+v"(lane_off));
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int m = 0; m < KM; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float *row = s1 + static_cast<size_t>(16 * m + i) * p.DV + 16 * ct;
            row[lane_off] = H[ct][m][i];
          }
    };

    // The chunk's values: each state wave brings in its own 32 columns (rows
    // 16 j + lane / 4, columns 8 (lane % 4) .. + 7 of its tile) through a resource that
    // ends at the sequence's last row (rows past it read as zero; no values: all zero).
    // They are only ever read by the wave that wrote them, so one LDS buffer serves:
    // a chunk's values are written in the phase B before its interval, after the wave's
    // reads of the previous chunk's, from registers loaded an interval earlier.
    // (Branch-free: without values, and past the sequence's end, the resource holds no
    // rows and the loads return zeros.)
    uint4 vr[4];
    auto load_v = [&](int c) __attribute__((always_inline)) {
      const __amdgpu_buffer_rsrc_t rv =
          rows_rsrc(vrow ? vrow + 32 * wave : kb, c, vrow ? min(CR, row_end - c) : 0, vstride);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        vr[j] = load16(rv, ((16 * j + (lane >> 2)) * vstride + 8 * (lane & 3)) * 2);
    };
    auto put_v = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<uint4 *>(sm.V + (16 * j + (lane >> 2)) * LDV + 32 * wave +
                                   8 * (lane & 3)) = vr[j];
    };
    load_v(row_begin);
    put_v();
    load_v(row_begin + CR);

    // the initial state has landed before the pipeline starts
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();   // prologue: producers stage chunk 0
    __syncthreads();   // prologue: producers solve chunk 0
    for (int ci = 0; ci < nchunks; ++ci) {
      const int c0 = row_begin + ci * CR;
      const Stage64<Tr> &s = sm.st[ci & 1];
      const Solve64<Tr> &v = sm.sv[ci & 1];
      const Fac64<Tr> &f = sm.fac[ci % 3];
      const int tq0 = c0 / NH;

      // ---- phase A: X = K H0, R, D ----------------------------------------------
      frag hb[2][KS];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int sl = 0; sl < KS; ++sl) hb[ct][sl] = M::from_acc(H[ct][2 * sl], H[ct][2 * sl + 1]);
      // Block by block: X_b = K_b H0, then -R_b = diag(beta) (diag(exp G) X_b - V_b) (V in
      // the accumulator layout by transposed reads of the row-major bf16 values), then
      // the substitution step D_b = T_bb (R_b - sum_{c<b} A_bc D_c).  The solve stores
      // -T_bb, and -R_b enters the products of A as their accumulator, so the step is
      // two matrix-core products with no vector work between them; each block's step
      // overlaps the next block's X.
      const frag tf0 = M::load(v.T, LDT, l16, 0, lane);
      const frag tf1 = M::load(v.T, LDT, 16 + l16, 0, lane);
      const frag tf2 = M::load(v.T, LDT, 32 + l16, 0, lane);
      const frag tf3 = M::load(v.T, LDT, 48 + l16, 0, lane);
      const frag af1 = M::load(v.A, LDA, 16 + l16, 0, lane);
      const frag af2 = M::load(v.A, LDA, 32 + l16, 0, lane);
      const frag af3a = M::load(v.A, LDA, 48 + l16, 0, lane);
      const frag af3b = M::load(v.A, LDA, 48 + l16, 32, lane);
      f32x4 D[2][4];
      frag d01[2];
      // the operands of block mk + 1 are read while block mk's products run
      frag kf[2][KS];
      s16x4 vv[2][2];
      float4 b4[2], e4[2];
      auto load_k = [&](int mk) __attribute__((always_inline)) {
#pragma unroll
        for (int sl = 0; sl < KS; ++sl) kf[mk & 1][sl] = M::load(s.K, LDK, 16 * mk + l16, 32 * sl, lane);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
          vv[mk & 1][ct] = read_tr(sm.V, LDV, 16 * mk, 32 * wave + 16 * ct, lane);
        b4[mk & 1] = *reinterpret_cast<const float4 *>(f.B + 16 * mk + 4 * g4);
        e4[mk & 1] = *reinterpret_cast<const float4 *>(f.eG + 16 * mk + 4 * g4);
      };
      load_k(0);
#pragma unroll
      for (int mk = 0; mk < 4; ++mk) {
        if (mk + 1 < 4) load_k(mk + 1);
        const float br[4] = {b4[mk & 1].x, b4[mk & 1].y, b4[mk & 1].z, b4[mk & 1].w};
        const float er[4] = {e4[mk & 1].x, e4[mk & 1].y, e4[mk & 1].z, e4[mk & 1].w};
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          f32x4 x = zero4();
#pragma unroll
          for (int sl = 0; sl < KS; ++sl) x = M::mma(kf[mk & 1][sl], hb[ct][sl], x);
          f32x4 rn;   // -R_b
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float vx =
                __uint_as_float(static_cast<uint32_t>(static_cast<uint16_t>(vv[mk & 1][ct][i])) << 16);
            rn[i] = br[i] * (er[i] * x[i] - vx);
          }
          if (mk == 0) {
            D[ct][0] = M::mma(tf0, M::from_acc(rn, zero4()), zero4());
          } else if (mk == 1) {
            const f32x4 z = M::mma(af1, M::from_acc(D[ct][0], zero4()), rn);
            D[ct][1] = M::mma(tf1, M::from_acc(z, zero4()), zero4());
            d01[ct] = M::from_acc(D[ct][0], D[ct][1]);
          } else if (mk == 2) {
            const f32x4 z = M::mma(af2, d01[ct], rn);
            D[ct][2] = M::mma(tf2, M::from_acc(z, zero4()), zero4());
          } else {
            const f32x4 z = M::mma(af3b, M::from_acc(D[ct][2], zero4()), M::mma(af3a, d01[ct], rn));
            D[ct][3] = M::mma(tf3, M::from_acc(z, zero4()), zero4());
          }
        }
      }
      // D as the operands of phase B: db = D (for O), dk = diag(exp(G_last - G)) D (for
      // the state update), both fp16
      frag db[2][2], dk[2][2];   // db unused without outputs
#pragma unroll
      for (int sk = 0; sk < 2; ++sk) {
        const float4 l0 = *reinterpret_cast<const float4 *>(f.eGl + 32 * sk + 4 * g4);
        const float4 l1 = *reinterpret_cast<const float4 *>(f.eGl + 32 * sk + 16 + 4 * g4);
        const f32x4 e0 = {l0.x, l0.y, l0.z, l0.w};
        const f32x4 e1 = {l1.x, l1.y, l1.z, l1.w};
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          if constexpr (OUT) db[ct][sk] = M::from_acc(D[ct][2 * sk], D[ct][2 * sk + 1]);
          dk[ct][sk] = M::from_acc(D[ct][2 * sk] * e0, D[ct][2 * sk + 1] * e1);
        }
      }
      __syncthreads();

      // ---- phase B: O and the state update ----------------------------------------
      // (first, the next chunk's values replace this chunk's, which this wave has read,
      // and the one after is requested)
      put_v();
      load_v(c0 + 2 * CR);
      if constexpr (OUT) {
        // O^T = scale H0^T Q^T diag(exp G) + D^T P^T (P carries the scale): a lane holds
        // output columns 4 g4 .. 4 g4 + 3 of token l16 of each query block.
        float sx[NQB];
  #pragma unroll
        for (int mq = 0; mq < NQB; ++mq) sx[mq] = p.scale * f.eG[NH * (16 * mq + l16) + NH - 1];
        // this chunk's output rows through a buffer resource whose range ends at the
        // sequence's last token (no rows at all without outputs): stores to rows past it
        // are dropped by the range check, with no branch around them
        const int orows = ob ? min(CQ, t1 - tq0) : 0;
        const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
            ob ? ob + static_cast<size_t>(tq0) * vstride : nullptr, 0,
            orows * static_cast<int>(vstride * sizeof(TOut)), kBufferWord3);
        // operand reads are issued one block ahead of the products that use them
        frag qf[2][KS], pf[2][2];
        auto load_qp = [&](int mq) __attribute__((always_inline)) {
          const int nsk = (NH * (16 * mq + 16) - 1) / 32 + 1;   // key slices reaching the block
  #pragma unroll
          for (int sl = 0; sl < KS; ++sl) qf[mq & 1][sl] = M::load(s.Q, LDK, 16 * mq + l16, 32 * sl, lane);
  #pragma unroll
          for (int sk = 0; sk < 2; ++sk)
            if (sk < nsk) pf[mq & 1][sk] = M::load(v.P, LDA, 16 * mq + l16, 32 * sk, lane);
        };
        load_qp(0);
  #pragma unroll
        for (int mq = 0; mq < NQB; ++mq) {
          if (mq + 1 < NQB) load_qp(mq + 1);
          const int nsk = (NH * (16 * mq + 16) - 1) / 32 + 1;
  #pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            f32x4 xo = zero4();
  #pragma unroll
            for (int sl = 0; sl < KS; ++sl) xo = M::mma(hb[ct][sl], qf[mq & 1][sl], xo);
            f32x4 yo = M::mma(db[ct][0], pf[mq & 1][0], zero4());
            if (nsk > 1) yo = M::mma(db[ct][1], pf[mq & 1][1], yo);
            store4_rsrc<TOut>(orsrc, ((16 * mq + l16) * vstride + 16 * ct + 4 * g4) * sizeof(TOut),
                              sx[mq] * xo + yo);
          }
        }
      }
      // H <- exp(G_last) H0 + K^T diag(exp(G_last - G)) D
      const float dl = f.eG[CR - 1];
      frag kt[2][2];
      auto load_kt = [&](int m) __attribute__((always_inline)) {
        kt[m & 1][0] = frag_tr(s.K, LDK, 0, 16 * m, lane);
        kt[m & 1][1] = frag_tr(s.K, LDK, 32, 16 * m, lane);
      };
      load_kt(0);
#pragma unroll
      for (int m = 0; m < KM; ++m) {
        if (m + 1 < KM) load_kt(m + 1);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
          H[ct][m] = M::mma(kt[m & 1][1], dk[ct][1], M::mma(kt[m & 1][0], dk[ct][0], H[ct][m] * dl));
      }
      // a boundary state after every bnd_rows rows (boundaries fall on chunk ends)
      if (bnd_rows && ((ci + 1) * CR) % bnd_rows == 0 && (ci + 1) * CR <= row_end - row_begin) {
        const int e = bnd_base + (ci + 1) * CR / bnd_rows - 1;
        store_state(p.boundary_states + (static_cast<size_t>(e) * p.Hv + h) * state_stride);
      }
      __syncthreads();
    }
    // ---- final state ---------------------------------------------------------
    if (p.final_state && dst >= 0)
      store_state(p.final_state + (static_cast<size_t>(dst) * p.Hv + h) * state_stride);
  } else {
    // ---- producers ---------------------------------------------------------------
    // prologue: chunk 0 staged and solved, chunk 1 fetched.  Interval ci: stage chunk
    // ci+1, each register refilled with chunk ci+2's inputs as soon as it is staged
    // (phase A); solve chunk ci+1 (phase B).  The loads have almost an interval to land.
    // The decay scan of a chunk runs in the phase B two phases before the chunk's solve
    // (on producer 0 with outputs, on producer 3 without), and each producer forms its
    // diagonal block of A from its staged K registers in the phase A before the solve, so
    // that producer 0's share of the solve is the inversion, one off-diagonal block and
    // the scan.  Without outputs no Q is loaded or staged and no P is formed.
    // The producer that runs the decay scan (SCAN) has its own copy of the loop, so the
    // gate loads and the scan are compiled only there.
    auto run = [&](auto l2c, auto scanc) __attribute__((always_inline)) {
      constexpr bool SCAN = decltype(scanc)::value;
      Scan64 sc{};   // the scan producer: the decay factors of one chunk
      if (nchunks > 0) {
        fetch(rg, row_begin);
        if (SCAN) {
          fetch_gates(rg, row_begin);
          sc = scan(rg, row_begin);
          put_bases(sc, sm.st[0]);
          put_factors(sc, sm.fac[0]);
          if (nchunks > 1) fetch_gates(rg, row_begin + CR);
        }
        stage(rg, sm.st[0], l2c, row_begin + CR);
      }
      __syncthreads();
      if (nchunks > 0) {
        if (pw == 0) p64_diag_lds<Tr>(sm.st[0], sm.AR, lane);
        p64_solve<Tr, OUT>(sm.st[0], sm.sv[0], sm.AR, pw, p.scale, lane);
      }
      if (SCAN && nchunks > 1) {
        sc = scan(rg, row_begin + CR);
        put_bases(sc, sm.st[1]);
        put_factors(sc, sm.fac[1]);
        if (nchunks > 2) fetch_gates(rg, row_begin + 2 * CR);
      }
      __syncthreads();
      for (int ci = 0; ci < nchunks; ++ci) {
        const bool next = ci + 1 < nchunks;
        // the scan producer requests the gates of chunk ci + 3 first (rows clamped to
        // the sequence), into registers of their own that take the place of the current
        // ones after this interval's scan: issued before the staging and unconditionally,
        // they are counted in the staging's waits, which then no longer wait for them
        float gnext = 0.0f, bnext = 0.0f;
        if constexpr (SCAN) {
          const int row = min(row_begin + (ci + 3) * CR + lane, row_end - 1);
          gnext = gb[static_cast<uint32_t>(row / NH) * p.Hv];
          bnext = bb[static_cast<uint32_t>(row) * p.Hv];
        }
        if (next) {
          Stage64<Tr> &sn = sm.st[(ci + 1) & 1];
          // this producer's diagonal block K_pw K_pw^T of chunk ci + 1 is formed after
          // the staging; its exponent bases (stored in the previous phase B) are read
          // first
          const DiagBases db = p64_diag_bases<Tr>(sn, pw, lane);
          stage(rg, sn, l2c, row_begin + (ci + 2) * CR);
          f32x4 acc = zero4();
#pragma unroll
          for (int sl = 0; sl < KS; ++sl) acc = M::mma(kh[sl], kh[sl], acc);
          p64_diag_put<Tr>(db, acc, pw, sm.AR, lane);
        }
        __syncthreads();
        if (next)
          p64_solve<Tr, OUT>(sm.st[(ci + 1) & 1], sm.sv[(ci + 1) & 1], sm.AR, pw, p.scale, lane);
        if constexpr (SCAN) {
          if (ci + 2 < nchunks) {
            sc = scan(rg, row_begin + (ci + 2) * CR);
            put_bases(sc, sm.st[ci & 1]);   // chunk ci + 2 takes chunk ci's buffer
            put_factors(sc, sm.fac[(ci + 2) % 3]);
          }
          rg.g = gnext;
          rg.b = bnext;
        }
        __syncthreads();
      }
    };
    if (pw == scan_producer<OUT>()) {
      if (p.l2norm)
        run(std::true_type(), std::true_type());
      else
        run(std::false_type(), std::true_type());
    } else {
      if (p.l2norm)
        run(std::true_type(), std::false_type());
      else
        run(std::false_type(), std::false_type());
    }
  }
}

// ---- dispatch --------------------------------------------------------------------

namespace {

template <int DK, int NH, int NS>
hipError_t launch64_one(const PrefillParams &p, int grid, hipStream_t stream) {
  constexpr int threads = 64 * P64<DK, NH, NS>::NW;
  if (!p.out)
    hipLaunchKernelGGL((prefill64_kernel<__bf16, DK, NH, NS, false>), dim3(grid), dim3(threads),
                       0, stream, p);
  else if (p.out_bf16)
    hipLaunchKernelGGL((prefill64_kernel<__bf16, DK, NH, NS, true>), dim3(grid), dim3(threads), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((prefill64_kernel<float, DK, NH, NS, true>), dim3(grid), dim3(threads), 0,
                       stream, p);
  return hipGetLastError();
}

template <int DK, int NH>
hipError_t launch64_ns(const PrefillParams &p, int ns, int grid, hipStream_t s) {
  if (ns == 1) return launch64_one<DK, NH, 1>(p, grid, s);
  if (ns == 2) return launch64_one<DK, NH, 2>(p, grid, s);
  if (ns == 4) return launch64_one<DK, NH, 4>(p, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill64(const PrefillParams &p, int head_k, int nh, int state_waves,
                            int grid, hipStream_t stream) {
  if (head_k == 64) {
    if (nh == 1) return launch64_ns<64, 1>(p, state_waves, grid, stream);
    if (nh == 2) return launch64_ns<64, 2>(p, state_waves, grid, stream);
  } else if (head_k == 128) {
    if (nh == 1) return launch64_ns<128, 1>(p, state_waves, grid, stream);
    if (nh == 2) return launch64_ns<128, 2>(p, state_waves, grid, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdr
