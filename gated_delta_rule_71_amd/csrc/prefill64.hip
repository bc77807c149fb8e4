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
//            producers    fetch chunk i+2 into registers, stage chunk i+1 into LDS;
//   phase B: state waves  O and the state update of chunk i;
//            producers    solve chunk i+1: diagonal blocks and their inverses
//                         (wave 0), off-diagonal blocks of A (wave 1), the causal
//                         tiles of P = scale (Q K^T * Gamma) (waves 2 and 3).
// Staged chunks and solved operands are double-buffered in LDS.

#include "chunk_helpers.hpp"
#include "common.hpp"
#include "gdr_internal.hpp"

namespace gdr {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

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

// Lane j of 16-lane group g receives M[r0 + 4g + e][c0 + j], e = 0..3, of a row-major
// 16-bit matrix M in LDS (leading dimension ld elements).
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
  static constexpr int VSEG = DVT / 8;
  static constexpr int VPT = CR * VSEG / ST;
  static_assert(KPT * ST == CR * SEG && QPT * ST == CQ * SEG && VPT * ST == CR * VSEG,
                "staging split");
  static_assert(QPT >= 1 && VPT >= 1 && NQB >= 1, "staging split");
};

template <class Tr>
struct alignas(16) Stage64 {
  _Float16 K[Tr::CR * Tr::LDK];
  _Float16 Q[Tr::CQ * Tr::LDK];
  uint16_t V[Tr::CR * Tr::LDV];   // raw bf16
  float G2[Tr::CR];               // G_r log2(e): exponent base of the solve's columns
  float GB[Tr::CR];               // G_r log2(e) + log2(beta_r): base of A's rows
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
  float AR[4][Tr::ARB];
};

template <class Tr>
struct Regs64 {
  Seg8<uint16_t> k[Tr::KPT], q[Tr::QPT], v[Tr::VPT];
  float g, b;
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

// The four diagonal blocks A_bb and their inverses T_bb = (I + A_bb)^-1.  Row j of
// T_bb solves the upper triangular system (I + A_bb)^T t = e_j by back substitution;
// lane 16 b + j does it for block b, so one pass over the 64 lanes inverts all four.
template <class Tr>
__device__ __forceinline__ void p64_diag(const Stage64<Tr> &s, Solve64<Tr> &v,
                                         float (*AR)[Tr::ARB], int lane) {
  using M = typename Tr::M;
  constexpr int KS = Tr::KS, LDT = Tr::LDT, LDR = Tr::LDR;
  const int l16 = lane & 15, g4 = lane >> 4;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    if (b == 2) __builtin_amdgcn_sched_barrier(0);   // two blocks' operands at a time
    typename M::frag f[KS];
    p64_block<Tr>(s.K, b, lane, f);
    f32x4 acc = zero4();
#pragma unroll
    for (int sl = 0; sl < KS; ++sl) acc = M::mma(f[sl], f[sl], acc);
    // K_b K_b^T is symmetric: its accumulator tile also gives lane (l16, g4) row l16,
    // columns 4 g4 .. 4 g4 + 3
    const float base = s.GB[16 * b + l16];
    const float4 gc = *reinterpret_cast<const float4 *>(s.G2 + 16 * b + 4 * g4);
    const float gcv[4] = {gc.x, gc.y, gc.z, gc.w};
    float a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = acc[i] * __builtin_amdgcn_exp2f(4 * g4 + i < l16 ? base - gcv[i] : -INFINITY);
    *reinterpret_cast<float4 *>(AR[b] + l16 * LDR + 4 * g4) = make_float4(a[0], a[1], a[2], a[3]);
  }
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
    for (int c = 0; c < b; ++c) {
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

template <class Tr>
__device__ __forceinline__ void p64_solve(const Stage64<Tr> &s, Solve64<Tr> &v,
                                          float (*AR)[Tr::ARB], int pw, float scale, int lane) {
  if (pw == 0) {
    p64_diag<Tr>(s, v, AR, lane);
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

template <typename TOut, int DK, int NH, int NS>
__global__ void __launch_bounds__(64 * (NS + 4))
prefill64_kernel(const PrefillParams p) {
  using Tr = P64<DK, NH, NS>;
  using M = typename Tr::M;
  using frag = typename M::frag;
  constexpr int CR = Tr::CR, CQ = Tr::CQ, NQB = Tr::NQB, DVT = Tr::DVT, SEG = Tr::SEG;
  constexpr int LDK = Tr::LDK, LDV = Tr::LDV, LDA = Tr::LDA, LDT = Tr::LDT, NT = Tr::NT;
  constexpr int ST = Tr::ST, KS = Tr::KS, KM = Tr::KM, KPT = Tr::KPT, QPT = Tr::QPT;
  constexpr int VPT = Tr::VPT, VSEG = Tr::VSEG;

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
    constexpr int nz = static_cast<int>(sizeof(sm.sv) / sizeof(_Float16));
    for (int i = tid; i < nz; i += NT) z[i] = static_cast<_Float16>(0.0f);
  }

  const int row_begin = t0 * NH, row_end = t1 * NH;
  const int nchunks = (row_end - row_begin + CR - 1) / CR;

  Regs64<Tr> rg;   // producer registers: the inputs of one chunk between fetch and staging

  // inputs of the chunk starting at row c -> producer registers (addresses clamped to
  // the sequence, also past its end; validity is applied at staging)
  auto fetch = [&](Regs64<Tr> &cr, int c) __attribute__((always_inline)) {
    const int last = row_end - 1;
    const int tq = c / NH, tlast = t1 - 1;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int u = stid + j * ST, r = u / SEG, sg = u % SEG;
      cr.k[j].load(kb + (static_cast<uint32_t>(min(c + r, last)) * kstride + sg * 8));
    }
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const int u = stid + j * ST, r = u / SEG, sg = u % SEG;
      cr.q[j].load(qb + (static_cast<uint32_t>(min(tq + r, tlast)) * kstride + sg * 8));
    }
    if (vrow) {   // one uniform branch around all value loads
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        const int u = stid + j * ST, r = u / VSEG, sg = u % VSEG;
        cr.v[j].load(vrow + (static_cast<uint32_t>(min(c + r, last)) * vstride + sg * 8));
      }
    } else {
#pragma unroll
      for (int j = 0; j < VPT; ++j) cr.v[j].zero();
    }
    if (pw == 3) {
      const int row = min(c + lane, last);
      cr.g = gb[static_cast<uint32_t>(row / NH) * p.Hv];
      cr.b = bb[static_cast<uint32_t>(row) * p.Hv];
    }
  };
  // producer registers (chunk starting at row c) -> staged LDS buffer.  The L2 norm and
  // whether every row of the chunk is valid are compile-time choices, so that no
  // branch splits the conversions and full chunks skip the row masks.
  auto stage = [&](const Regs64<Tr> &cr, int c, Stage64<Tr> &s, auto l2c) __attribute__((always_inline)) {
    constexpr bool L2 = decltype(l2c)::value;
    const int nrow = min(CR, row_end - c);          // valid rows
    const int nq = min(CQ, t1 - c / NH);            // valid query rows
    auto rows = [&](auto fullc) __attribute__((always_inline)) {
      constexpr bool FULL = decltype(fullc)::value;
      auto masked = [&](const uint4 &u, bool ok) __attribute__((always_inline)) {
        if constexpr (FULL) return u;
        return make_uint4(ok ? u.x : 0u, ok ? u.y : 0u, ok ? u.z : 0u, ok ? u.w : 0u);
      };
      // one 8-element segment of a K or Q row -> fp16 in LDS, L2-normalised over the row
      // (the SEG lanes holding a row are consecutive)
      auto segment = [&](const Seg8<uint16_t> &in, bool ok, _Float16 *dst) __attribute__((always_inline)) {
        const uint4 u = masked(in.u, ok);
        if constexpr (L2) {
          Seg8<uint16_t> t;
          t.u = u;
          float x[8];
          t.get(x);
          float ss = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
#pragma unroll
          for (int o = SEG / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
          const float rn = 1.0f / sqrtf(ss + 1e-6f);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] *= rn;
          store8_pk(dst, x);
        } else {
          store8_bf16_as_f16(dst, u);
        }
      };
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const int u = stid + j * ST, r = u / SEG, sg = u % SEG;
        segment(cr.k[j], r < nrow, s.K + r * LDK + sg * 8);
      }
#pragma unroll
      for (int j = 0; j < QPT; ++j) {
        const int u = stid + j * ST, r = u / SEG, sg = u % SEG;
        segment(cr.q[j], r < nq, s.Q + r * LDK + sg * 8);
      }
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        const int u = stid + j * ST, r = u / VSEG, sg = u % VSEG;
        *reinterpret_cast<uint4 *>(s.V + r * LDV + sg * 8) = masked(cr.v[j].u, r < nrow);
      }
    };
    if (nrow == CR && nq == CQ)
      rows(std::true_type());
    else
      rows(std::false_type());
    if (pw == 3) {
      // inclusive prefix sum of the per-row decay in fp64 (a token's g sits on its
      // first sub-step), and the per-row factors; gates formed here from raw
      // projections when asked
      const bool ok = lane < nrow;
      float gv = cr.g;
      float bv = cr.b;
      if (p.gate_mode) {
        gv = gate_decay(cr.g, gate_A, gate_dt);
        bv = gate_beta(cr.b);
      }
      const double gr = prefix_sum64((ok && (c + lane) % NH == 0) ? gv : 0.0);
      bv = ok ? bv : 0.0f;
      const double glast = readlane_f64(gr, CR - 1);
      const float g2 = static_cast<float>(gr) * 1.4426950408889634f;
      s.G2[lane] = g2;
      s.GB[lane] = g2 + __builtin_amdgcn_logf(bv);   // log2(0) = -inf: beta 0 rows vanish
      s.eG[lane] = fexp(static_cast<float>(gr));
      s.eGl[lane] = fexp(static_cast<float>(glast - gr));
      s.B[lane] = bv;
    }
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

    // the initial state has landed before the pipeline starts
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();   // prologue: producers stage chunk 0
    __syncthreads();   // prologue: producers solve chunk 0
    for (int ci = 0; ci < nchunks; ++ci) {
      const int c0 = row_begin + ci * CR;
      const Stage64<Tr> &s = sm.st[ci & 1];
      const Solve64<Tr> &v = sm.sv[ci & 1];
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
#pragma unroll
      for (int mk = 0; mk < 4; ++mk) {
        frag kf[KS];
#pragma unroll
        for (int sl = 0; sl < KS; ++sl) kf[sl] = M::load(s.K, LDK, 16 * mk + l16, 32 * sl, lane);
        const int r0 = 16 * mk + 4 * g4;
        const float4 b4 = *reinterpret_cast<const float4 *>(s.B + r0);
        const float4 e4 = *reinterpret_cast<const float4 *>(s.eG + r0);
        const float br[4] = {b4.x, b4.y, b4.z, b4.w};
        const float er[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const s16x4 vv = read_tr(s.V, LDV, 16 * mk, 32 * wave + 16 * ct, lane);
          f32x4 x = zero4();
#pragma unroll
          for (int sl = 0; sl < KS; ++sl) x = M::mma(kf[sl], hb[ct][sl], x);
          f32x4 rn;   // -R_b
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float vx = __uint_as_float(static_cast<uint32_t>(static_cast<uint16_t>(vv[i])) << 16);
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
      frag db[2][2], dk[2][2];
#pragma unroll
      for (int sk = 0; sk < 2; ++sk) {
        const float4 l0 = *reinterpret_cast<const float4 *>(s.eGl + 32 * sk + 4 * g4);
        const float4 l1 = *reinterpret_cast<const float4 *>(s.eGl + 32 * sk + 16 + 4 * g4);
        const f32x4 e0 = {l0.x, l0.y, l0.z, l0.w};
        const f32x4 e1 = {l1.x, l1.y, l1.z, l1.w};
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          db[ct][sk] = M::from_acc(D[ct][2 * sk], D[ct][2 * sk + 1]);
          dk[ct][sk] = M::from_acc(D[ct][2 * sk] * e0, D[ct][2 * sk + 1] * e1);
        }
      }
      __syncthreads();

      // ---- phase B: O and the state update ----------------------------------------
      // O^T = scale H0^T Q^T diag(exp G) + D^T P^T (P carries the scale): a lane holds
      // output columns 4 g4 .. 4 g4 + 3 of token l16 of each query block
#pragma unroll
      for (int mq = 0; mq < NQB; ++mq) {
        frag qf[KS];
#pragma unroll
        for (int sl = 0; sl < KS; ++sl) qf[sl] = M::load(s.Q, LDK, 16 * mq + l16, 32 * sl, lane);
        // key slices (32 rows) reaching this query block's last row
        const int nsk = (NH * (16 * mq + 16) - 1) / 32 + 1;
        frag pf[2];
#pragma unroll
        for (int sk = 0; sk < 2; ++sk)
          if (sk < nsk) pf[sk] = M::load(v.P, LDA, 16 * mq + l16, 32 * sk, lane);
        const float sx = p.scale * s.eG[NH * (16 * mq + l16) + NH - 1];
        f32x4 xo[2], yo[2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          xo[ct] = zero4();
#pragma unroll
          for (int sl = 0; sl < KS; ++sl) xo[ct] = M::mma(hb[ct][sl], qf[sl], xo[ct]);
          yo[ct] = M::mma(db[ct][0], pf[0], zero4());
          if (nsk > 1) yo[ct] = M::mma(db[ct][1], pf[1], yo[ct]);
        }
        const int tok = tq0 + 16 * mq + l16;
        if (p.out && tok < t1) {
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            float o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = sx * xo[ct][i] + yo[ct][i];
            store4(ob + (static_cast<uint32_t>(tok) * vstride + 16 * ct + 4 * g4), o);
          }
        }
      }
      // H <- exp(G_last) H0 + K^T diag(exp(G_last - G)) D
      const float dl = s.eG[CR - 1];
#pragma unroll
      for (int m = 0; m < KM; ++m) {
        const frag k0 = frag_tr(s.K, LDK, 0, 16 * m, lane);
        const frag k1 = frag_tr(s.K, LDK, 32, 16 * m, lane);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
          H[ct][m] = M::mma(k1, dk[ct][1], M::mma(k0, dk[ct][0], H[ct][m] * dl));
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
    // ci+1, then fetch chunk ci+2 into the same registers (phase A); solve chunk ci+1
    // (phase B).  The loads have the rest of the interval to land before their staging.
    auto run = [&](auto l2c) __attribute__((always_inline)) {
      if (nchunks > 0) {
        fetch(rg, row_begin);
        stage(rg, row_begin, sm.st[0], l2c);
        if (nchunks > 1) fetch(rg, row_begin + CR);
      }
      __syncthreads();
      if (nchunks > 0) p64_solve<Tr>(sm.st[0], sm.sv[0], sm.AR, pw, p.scale, lane);
      __syncthreads();
      for (int ci = 0; ci < nchunks; ++ci) {
        const bool next = ci + 1 < nchunks;
        if (next) stage(rg, row_begin + (ci + 1) * CR, sm.st[(ci + 1) & 1], l2c);
        if (ci + 2 < nchunks) fetch(rg, row_begin + (ci + 2) * CR);
        __syncthreads();
        if (next) p64_solve<Tr>(sm.st[(ci + 1) & 1], sm.sv[(ci + 1) & 1], sm.AR, pw, p.scale, lane);
        __syncthreads();
      }
    };
    if (p.l2norm)
      run(std::true_type());
    else
      run(std::false_type());
  }
}

// ---- dispatch --------------------------------------------------------------------

namespace {

template <int DK, int NH, int NS>
hipError_t launch64_one(const PrefillParams &p, int grid, hipStream_t stream) {
  constexpr int threads = 64 * P64<DK, NH, NS>::NW;
  if (p.out_bf16)
    hipLaunchKernelGGL((prefill64_kernel<__bf16, DK, NH, NS>), dim3(grid), dim3(threads), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((prefill64_kernel<float, DK, NH, NS>), dim3(grid), dim3(threads), 0,
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
