// Chunked prefill of the gated delta rule on gfx950 matrix cores.
//
// The recurrence S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
// o_t = scale S_t q_t (Gated DeltaNet, Megatron Core API page
// "core.ssm.gated_delta_net.gdn", torch_chunk_gated_delta_rule; with n_h
// Householder sub-steps per token, page "core.ssm.gated_delta_product",
// GatedDeltaProductMixer) is evaluated chunk by chunk.  With the state kept as
// H = S^T (K x V) and, inside one chunk of n rows entering with state H0,
//   G_r     = g_0 + ... + g_r          (a token's g sits on its first sub-step)
//   Gamma   = [exp(G_r - G_i)]_{i<=r}  (masked before the exponential)
//   A       = strict_lower(diag(beta) K K^T * Gamma),  T = (I + A)^-1
//   R       = diag(beta) V - diag(beta exp(G)) (K H0)
//   D       = T R
//   O       = scale (diag(exp(G)) (Q H0) + (Q K^T * Gamma) D)      (query rows)
//   H_n     = exp(G_{n-1}) H0 + (diag(exp(G_{n-1} - G)) K)^T D
// which equals the per-token recurrence exactly in real arithmetic.
//
// Work decomposition: one workgroup per (sequence, value head, tile of 32*NS value
// columns), with two kinds of waves.
//   * NS state waves each own 32 columns of H (two 16-column matrix-core tiles
//     that share every operand fragment they read) for the whole sequence, in
//     accumulator registers, and run only the state-dependent products of each
//     chunk: X = K H0, R, D = T R, O and the state update.  H and D pass between
//     products in registers.  O is formed transposed (O^T = H0^T Q^T + D^T P^T),
//     which puts four consecutive output columns of one token in each lane.
//   * NP producer waves prepare the chunks ahead of them: they solve chunk i+1
//     (the 16x16 diagonal blocks of A on the matrix cores and the inverses of
//     I + A_bb by column substitution, one block per wave; the off-diagonal block
//     A_10; P = Q K^T * Gamma; and the decayed, transposed keys K~^T of the state
//     update), stage chunk i+2 (K, Q, optionally L2-normalised, the workgroup's V
//     columns transposed, the cumulative decay and per-row factors) from registers
//     into LDS, and fetch the inputs of chunk i+3 into registers.
// Both kinds work at once and meet at one workgroup barrier per chunk, so a chunk
// interval costs the longer of the two instead of their sum.  With the diagonal
// inverses T_bb the chunk's delta follows by block forward substitution,
// D_0 = T_00 R_0, D_1 = T_11 (R_1 - A_10 D_0); the off-diagonal block of
// (I + A)^-1 is never formed.  Staged inputs are triple-buffered, solved operands
// double-buffered; none of them leave LDS.  HBM sees q, k, v, g, beta once per
// column tile (the tiles of one head share them through L2), o once and the state
// once in each direction.
//
// Operand precision: bf16 inputs run with fp16 operands (bf16 values convert
// exactly; T, P, H and D are rounded to fp16, 11 significant bits) and fp32
// accumulation; fp32 inputs run every product with fp32 operands.

#include "common.hpp"
#include "gdr_internal.hpp"

namespace gdr {

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

// Element e of two 8-element segments (rows r and r+1 of V) as one pair, written
// to VT[e][r..r+1]: the transpose of a 2 x 8 block, in input precision.
__device__ __forceinline__ void store_vt_pairs(uint16_t *dst, int ld, const Seg8<uint16_t> &a,
                                               const Seg8<uint16_t> &b) {
  const uint32_t wa[4] = {a.u.x, a.u.y, a.u.z, a.u.w};
  const uint32_t wb[4] = {b.u.x, b.u.y, b.u.z, b.u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    *reinterpret_cast<uint32_t *>(dst + (2 * i) * ld) = (wa[i] & 0xffffu) | (wb[i] << 16);
    *reinterpret_cast<uint32_t *>(dst + (2 * i + 1) * ld) = (wa[i] >> 16) | (wb[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void store_vt_pairs(float *dst, int ld, const Seg8<float> &a,
                                               const Seg8<float> &b) {
  float x[8], y[8];
  a.get(x);
  b.get(y);
#pragma unroll
  for (int e = 0; e < 8; ++e) *reinterpret_cast<float2 *>(dst + e * ld) = make_float2(x[e], y[e]);
}

template <typename TIn_, int DK_, int CR_, int NH_, int NS_, bool F32_>
struct PrefillTraits {
  using TIn = TIn_;
  using M = Mma<F32_>;
  using elem = typename M::elem;
  static constexpr bool F32 = F32_;
  static constexpr int DK = DK_, CR = CR_, NH = NH_, NS = NS_;
  static constexpr int NP = 4;                       // producer waves
  static constexpr int NW = NS + NP;                 // waves per workgroup
  static constexpr int NT = 64 * NW;                 // threads
  static constexpr int PT = 64 * NP;                 // producer threads
  static constexpr int CQ = CR / NH;                 // query rows per chunk
  static constexpr int NB = CR / 16;                 // 16-row blocks
  static constexpr int NQB = CQ / 16;                // 16-row query blocks
  static constexpr int DVT = 32 * NS;                // value columns per workgroup
  static constexpr int PAD = F32 ? 4 : 8;            // elements of row padding
  static constexpr int LDK = DK + PAD;               // K, Q leading dimension
  static constexpr int LDC = 32 + PAD;               // T, A10, P, KT leading dimension
  static constexpr int LDA = 20;                     // AT (fp32 16x16, column-major) leading dim.
  static constexpr int LDVT = CR + 4;                // VT (value column major) leading dim.
  static constexpr int KS = DK / 32;                 // 32-deep slices over keys
  static constexpr int KM = DK / 16;                 // 16-row blocks of H
  static constexpr int SEG = DK / 8;                 // 8-element segments per row
  static constexpr int KPT = (CR * SEG + PT - 1) / PT;
  static constexpr int QPT = (CQ * SEG + PT - 1) / PT;
  static constexpr int VSEG = DVT / 8;               // 8-element segments per V row
  static constexpr int VUNITS = (CR / 2) * VSEG;     // (row pair, segment) units of V
  static constexpr int VPT = (VUNITS + PT - 1) / PT;
  static_assert(CR == 16 || CR == 32, "chunk rows");
  static_assert(CQ % 16 == 0, "query rows");
  static_assert(DK % 32 == 0, "head_k");
  static_assert(NP >= 2 && NP >= NB + 1, "producer waves");
};

// one staged chunk
template <class Tr>
struct alignas(16) StageBuf {
  typename Tr::elem K[Tr::CR * Tr::LDK];
  typename Tr::elem Q[Tr::CQ * Tr::LDK];
  typename Tr::TIn VT[Tr::DVT * Tr::LDVT];   // the workgroup's value columns, transposed
  double G[Tr::CR];     // cumulative decay (fp64: differences of large sums stay exact)
  float eG[Tr::CR];     // exp(G_r)
  float eGl[Tr::CR];    // exp(G_last - G_r)
  float B[Tr::CR];      // beta
};
// the solved operands of one chunk
template <class Tr>
struct alignas(16) SolveBuf {
  typename Tr::elem T[Tr::CR * Tr::LDC];    // diag(T_00, T_11), T_bb = (I + A_bb)^-1
  typename Tr::elem A10[16 * Tr::LDC];      // A_10 in columns 0..15 (32-row chunks)
  typename Tr::elem P[Tr::CQ * Tr::LDC];    // Q K^T * Gamma, causal
  typename Tr::elem KT[Tr::DK * Tr::LDC];   // (diag(exp(G_last - G)) K)^T
};
template <class Tr>
struct PrefillSmem {
  StageBuf<Tr> st[3];
  SolveBuf<Tr> sv[2];
  float AT[2][16 * Tr::LDA];   // per diagonal block: A_bb column-major, for its inverting wave
};

// Inputs of one chunk held in a producer thread's registers between their fetch
// and their staging.  They are loaded raw from clamped addresses; rows past the
// sequence end are zeroed only when the values are consumed, so that no
// instruction waits on a load before the data is needed.
template <class Tr>
struct ChunkRegs {
  Seg8<typename Tr::TIn> k[Tr::KPT], q[Tr::QPT], v[Tr::VPT][2];
  float g, b;   // producer wave 0: decay and write strength of row `lane`
  int c;        // first row of the chunk these registers hold
};

// ---- solve one chunk: T_bb, A_10, P and K~^T (producer waves) ------------------
// producer wave b < NB: A_bb and its inverse; the other producer waves: A_10 and
// the P tiles round-robin, then the decayed, transposed keys.
template <class Tr>
__device__ __forceinline__ void solve_chunk(const StageBuf<Tr> &s, SolveBuf<Tr> &v,
                                            float (*AT)[16 * Tr::LDA], int pw, int lane) {
  using M = typename Tr::M;
  constexpr int NB = Tr::NB, NH = Tr::NH, LDK = Tr::LDK, LDC = Tr::LDC, LDA = Tr::LDA;
  const int l16 = lane & 15, g4 = lane >> 4;
  // one 16x16 tile of diag(beta) K K^T * Gamma (rows mi, columns ni), strict lower
  auto a_tile = [&](int mi, int ni, float (&out)[4]) {
    f32x4 acc = zero4();
#pragma unroll
    for (int sl = 0; sl < Tr::KS; ++sl)
      acc = M::mma(M::load(s.K, LDK, 16 * mi + l16, 32 * sl, lane),
                   M::load(s.K, LDK, 16 * ni + l16, 32 * sl, lane), acc);
    const int c = 16 * ni + l16;
    const double gc = s.G[c];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * mi + 4 * g4 + i;
      // mask before the exponential: G_r - G_c may be large positive above
      const float d = c < r ? static_cast<float>(s.G[r] - gc) : 0.0f;
      out[i] = c < r ? s.B[r] * acc[i] * fexp(d) : 0.0f;
    }
  };
  if (pw < NB) {
    const int bk = pw;
    float a[4];
    a_tile(bk, bk, a);
    // column-major: column c of A_bb is 16 contiguous floats (one 16-byte store
    // per lane here, four 16-byte loads per column below)
    float *Ab = AT[bk];
    *reinterpret_cast<float4 *>(Ab + l16 * LDA + 4 * g4) = make_float4(a[0], a[1], a[2], a[3]);
    // column substitution: lanes 0..15 keep column j of (I + A_bb)^-1 in registers;
    // step i eliminates entry i from the rows below it, with column i+1 already
    // being loaded while step i computes
    if (lane < 16) {
      const int j = lane;
      float t[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) t[r] = (r == j) ? 1.0f : 0.0f;
      float4 cur[4], nxt[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) cur[q] = *reinterpret_cast<const float4 *>(Ab + 4 * q);
#pragma unroll
      for (int i = 0; i < 15; ++i) {
        if (i + 1 < 15) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            nxt[q] = *reinterpret_cast<const float4 *>(Ab + (i + 1) * LDA + 4 * q);
        }
        const float col[16] = {cur[0].x, cur[0].y, cur[0].z, cur[0].w, cur[1].x, cur[1].y,
                               cur[1].z, cur[1].w, cur[2].x, cur[2].y, cur[2].z, cur[2].w,
                               cur[3].x, cur[3].y, cur[3].z, cur[3].w};
#pragma unroll
        for (int r = i + 1; r < 16; ++r) t[r] -= col[r] * t[i];
#pragma unroll
        for (int q = 0; q < 4; ++q) cur[q] = nxt[q];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) v.T[(16 * bk + r) * LDC + 16 * bk + j] = M::cvt(t[r]);
    }
    return;
  }
  // tiles: A_10 (32-row chunks), then the P tiles on or below the causal boundary
  constexpr int nwk = Tr::NP - NB;
  constexpr int NA = NB == 2 ? 1 : 0;
  constexpr int NPT = Tr::NQB * NB;
  for (int ti = pw - NB; ti < NA + NPT; ti += nwk) {
    if (NA == 1 && ti == 0) {
      float a[4];
      a_tile(1, 0, a);
#pragma unroll
      for (int i = 0; i < 4; ++i) v.A10[(4 * g4 + i) * LDC + l16] = M::cvt(a[i]);
      continue;
    }
    const int pt = ti - NA;
    const int mq = pt / NB, ni = pt % NB;
    if (16 * ni > NH * (16 * mq + 15) + NH - 1) continue;   // above the boundary: zero
    f32x4 acc = zero4();
#pragma unroll
    for (int sl = 0; sl < Tr::KS; ++sl)
      acc = M::mma(M::load(s.Q, LDK, 16 * mq + l16, 32 * sl, lane),
                   M::load(s.K, LDK, 16 * ni + l16, 32 * sl, lane), acc);
    const int c = 16 * ni + l16;
    const double gc = s.G[c];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = 16 * mq + 4 * g4 + i;
      const int r = NH * q + NH - 1;
      const float d = c <= r ? static_cast<float>(s.G[r] - gc) : 0.0f;
      v.P[q * LDC + c] = M::cvt(c <= r ? acc[i] * fexp(d) : 0.0f);
    }
  }
  // K~^T[d][r] = exp(G_last - G_r) K[r][d]: a lane takes two rows and 8 keys and
  // writes 8 row pairs (one 32-bit store each for fp16 operands)
  {
    constexpr int UNITS = (Tr::CR / 2) * Tr::SEG;  // (row pair, segment) units
    for (int u = (pw - NB) * 64 + lane; u < UNITS; u += nwk * 64) {
      const int rp = u % (Tr::CR / 2), sg = u / (Tr::CR / 2);
      const int r0 = 2 * rp;
      const float d0 = s.eGl[r0], d1 = s.eGl[r0 + 1];
      float x0[8], x1[8];
      load8(s.K + r0 * LDK + 8 * sg, x0);
      load8(s.K + (r0 + 1) * LDK + 8 * sg, x1);
#pragma unroll
      for (int e = 0; e < 8; ++e) store2(v.KT + (8 * sg + e) * LDC + r0, x0[e] * d0, x1[e] * d1);
    }
  }
}

template <typename TIn, typename TOut, int DK, int CR, int NH, int NS, bool F32>
__global__ void __launch_bounds__(64 * (NS + 4))
prefill_kernel(const PrefillParams p) {
  using Tr = PrefillTraits<TIn, DK, CR, NH, NS, F32>;
  using M = typename Tr::M;
  using elem = typename Tr::elem;
  using frag = typename M::frag;
  constexpr int CQ = Tr::CQ, NB = Tr::NB, NQB = Tr::NQB, DVT = Tr::DVT, SEG = Tr::SEG;
  constexpr int LDK = Tr::LDK, LDC = Tr::LDC, LDVT = Tr::LDVT, NT = Tr::NT, PT = Tr::PT;
  constexpr int KS = Tr::KS, KM = Tr::KM, KPT = Tr::KPT, QPT = Tr::QPT;

  __shared__ PrefillSmem<Tr> sm;

  const int w_item = xcd_work_item(blockIdx.x, p.group_size, p.num_groups);
  if (w_item < 0) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const bool is_state = wave < NS;
  const int pw = wave - NS;            // producer wave index (state waves: negative)
  const int ptid = tid - 64 * NS;      // producer thread index
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
  int src = n, dst = n;
  if (p.state_indices) {
    const int idx = p.state_indices[n];
    src = idx < 0 ? 0 : idx;
    dst = idx;
  }

  // uniform bases; every element offset below fits in 32 bits (checked on the host)
  const TIn *__restrict__ kb = static_cast<const TIn *>(p.k) + hk * DK;
  const TIn *__restrict__ qb = static_cast<const TIn *>(p.q) + hk * DK;
  const TIn *__restrict__ vrow = static_cast<const TIn *>(p.v) + h * p.DV + vt * DVT;
  const float *__restrict__ gb = p.g + h;
  const float *__restrict__ bb = p.beta + h;
  TOut *__restrict__ ob = static_cast<TOut *>(p.out) + h * p.DV + col0;   // + token, lane
  const uint32_t kstride = p.Hk * DK;        // elements between key rows (and query rows)
  const uint32_t vstride = p.Hv * p.DV;      // elements between value / output rows
  const size_t state_stride = static_cast<size_t>(DK) * p.DV;

  // parts of the solve buffers no chunk writes must read as zero
  {
    elem *z = reinterpret_cast<elem *>(&sm.sv[0]);
    constexpr int nz = static_cast<int>(sizeof(sm.sv) / (sizeof(elem)));
    for (int i = tid; i < nz; i += NT) z[i] = M::cvt(0.0f);
  }

  // ---- initial state -> registers of the state waves --------------------------
  // H[ct][m]: rows 16m.. of H, columns col0 + 16ct + (0..15)
  f32x4 H[2][KM];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int m = 0; m < KM; ++m) H[ct][m] = zero4();
  if (is_state && p.initial_state) {
    const float *s0 = p.initial_state + (static_cast<size_t>(src) * p.Hv + h) * state_stride;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int m = 0; m < KM; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          H[ct][m][i] = s0[static_cast<size_t>(16 * m + 4 * g4 + i) * p.DV + col0 + 16 * ct + l16];
  }

  const int row_begin = t0 * NH, row_end = t1 * NH;
  const int nchunks = (row_end - row_begin + CR - 1) / CR;

  ChunkRegs<Tr> cra, crb;   // producer registers: two chunks' inputs

  // inputs of the chunk starting at row c -> producer registers (addresses clamped
  // to the sequence and the column tile, also for chunks past the end; validity is
  // applied where the values are consumed)
  auto fetch = [&](ChunkRegs<Tr> &cr, int c) {
    const int last = row_end - 1;
    const int tq = c / NH, tlast = t1 - 1;
    cr.c = c;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int idx = ptid + j * PT, r = idx / SEG, sg = idx % SEG;
      const int row = min(c + r, last);
      cr.k[j].load(kb + (static_cast<uint32_t>(row) * kstride + sg * 8));
    }
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const int idx = ptid + j * PT, r = idx / SEG, sg = idx % SEG;
      const int t = min(tq + r, tlast);
      cr.q[j].load(qb + (static_cast<uint32_t>(t) * kstride + sg * 8));
    }
#pragma unroll
    for (int j = 0; j < Tr::VPT; ++j) {
      const int u = ptid + j * PT;
      const int rp = u % (CR / 2), sg = min(u / (CR / 2), Tr::VSEG - 1);
      const int ra = min(c + 2 * rp, last), rb = min(c + 2 * rp + 1, last);
      cr.v[j][0].load(vrow + (static_cast<uint32_t>(ra) * vstride + sg * 8));
      cr.v[j][1].load(vrow + (static_cast<uint32_t>(rb) * vstride + sg * 8));
    }
    if (pw == 0) {
      const int row = min(c + lane, last);
      cr.g = gb[static_cast<uint32_t>(row / NH) * p.Hv];
      cr.b = bb[static_cast<uint32_t>(row) * p.Hv];
    }
  };
  // producer registers -> staged LDS buffer
  auto stage = [&](const ChunkRegs<Tr> &cr, StageBuf<Tr> &s) {
    const int nrow = min(CR, row_end - cr.c);              // valid key rows
    const int nq = min(CQ, t1 - cr.c / NH);                // valid query rows
    auto rows = [&](const Seg8<TIn> *srcr, int count, int nrows, int nvalid, elem *dstm) {
#pragma unroll
      for (int j = 0; j < count; ++j) {
        const int idx = ptid + j * PT, r = idx / SEG, sg = idx % SEG;
        float x[8];
        srcr[j].get(x);
        if (nvalid < nrows && r >= nvalid) {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = 0.0f;
        }
        if (p.l2norm) {
          float ss = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
#pragma unroll
          for (int o = SEG / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
          const float rn = 1.0f / sqrtf(ss + 1e-6f);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] *= rn;
        }
        if (r < nrows) store8(dstm + r * LDK + sg * 8, x);
      }
    };
    rows(cr.k, KPT, CR, nrow, s.K);
    rows(cr.q, QPT, CQ, nq, s.Q);
#pragma unroll
    for (int j = 0; j < Tr::VPT; ++j) {
      const int u = ptid + j * PT;
      const int rp = u % (CR / 2), sg = u / (CR / 2);
      Seg8<TIn> a = cr.v[j][0], b = cr.v[j][1];
      if (nrow < CR) {
        if (2 * rp >= nrow) a.zero();
        if (2 * rp + 1 >= nrow) b.zero();
      }
      if (sg < Tr::VSEG) store_vt_pairs(s.VT + (8 * sg) * LDVT + 2 * rp, LDVT, a, b);
    }
    if (pw == 0) {
      // inclusive prefix sum of the per-row decay, in fp64, and per-row factors
      const bool ok = lane < nrow;
      const double gr = prefix_sum32((ok && (cr.c + lane) % NH == 0) ? cr.g : 0.0);
      const float bv = ok ? cr.b : 0.0f;
      const double glast = readlane_f64(gr, CR - 1);
      if (lane < CR) {
        s.G[lane] = gr;
        s.eG[lane] = fexp(static_cast<float>(gr));
        s.eGl[lane] = fexp(static_cast<float>(glast - gr));
        s.B[lane] = bv;
      }
    }
  };

  // the initial state has landed before the pipeline starts: no wait for it can be
  // left inside the loop
  __builtin_amdgcn_s_waitcnt(0);

  // ---- prologue ---------------------------------------------------------------------
  if (!is_state && nchunks > 0) {
    fetch(cra, row_begin);
    stage(cra, sm.st[0]);
    fetch(crb, row_begin + CR);
  }
  __syncthreads();
  if (!is_state && nchunks > 0) {
    solve_chunk<Tr>(sm.st[0], sm.sv[0], sm.AT, pw, lane);
    if (nchunks > 1) stage(crb, sm.st[1]);
    fetch(cra, row_begin + 2 * CR);
  }
  __syncthreads();

  // ---- pipelined chunk loop ---------------------------------------------------------
  // Each role runs its own loop; both pass one workgroup barrier per chunk, so
  // chunk ci's state products (state waves) overlap the solve of chunk ci+1, the
  // staging of chunk ci+2 and the fetch of chunk ci+3 (producer waves).
  if (is_state) {
    for (int ci = 0; ci < nchunks; ++ci) {
      const int c0 = row_begin + ci * CR;
      // ---- state-dependent products of chunk ci (this wave's 32 columns) ----
      const StageBuf<Tr> &s = sm.st[ci % 3];
      const SolveBuf<Tr> &v = sm.sv[ci & 1];
      const int tq0 = c0 / NH;
      const bool full = tq0 + CQ <= t1;   // every query row of the chunk is in the sequence

      frag hb[2][KS];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int sl = 0; sl < KS; ++sl) hb[ct][sl] = M::from_acc(H[ct][2 * sl], H[ct][2 * sl + 1]);

      // R = diag(beta) (V - diag(exp G) K H0)
      f32x4 R[2][2];
#pragma unroll
      for (int mk = 0; mk < NB; ++mk) {
        f32x4 a0 = zero4(), a1 = zero4();
#pragma unroll
        for (int sl = 0; sl < KS; ++sl) {
          const frag kf = M::load(s.K, LDK, 16 * mk + l16, 32 * sl, lane);
          a0 = M::mma(kf, hb[0][sl], a0);
          a1 = M::mma(kf, hb[1][sl], a1);
        }
        const int r0 = 16 * mk + 4 * g4;
        const float4 b4 = *reinterpret_cast<const float4 *>(s.B + r0);
        const float4 e4 = *reinterpret_cast<const float4 *>(s.eG + r0);
        const float bq[4] = {b4.x, b4.y, b4.z, b4.w}, eq[4] = {e4.x, e4.y, e4.z, e4.w};
        float v0[4], v1[4];
        load4(s.VT + (32 * wave + l16) * LDVT + r0, v0);
        load4(s.VT + (32 * wave + 16 + l16) * LDVT + r0, v1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          R[0][mk][i] = bq[i] * (v0[i] - eq[i] * a0[i]);
          R[1][mk][i] = bq[i] * (v1[i] - eq[i] * a1[i]);
        }
      }
      if constexpr (NB == 1) R[0][1] = R[1][1] = zero4();

      // D_0 = T_00 R_0;  D_1 = T_11 (R_1 - A_10 D_0)   (T rows hold diag(T_00, T_11))
      f32x4 D[2][2];
      {
        const frag tf0 = M::load(v.T, LDC, l16, 0, lane);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) D[ct][0] = M::mma(tf0, M::from_acc(R[ct][0], zero4()), zero4());
      }
      if constexpr (NB == 2) {
        const frag af = M::load(v.A10, LDC, l16, 0, lane);
        const frag tf1 = M::load(v.T, LDC, 16 + l16, 0, lane);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const f32x4 z = M::mma(af, M::from_acc(D[ct][0], zero4()), zero4());
          const f32x4 y = R[ct][1] - z;
          D[ct][1] = M::mma(tf1, M::from_acc(zero4(), y), zero4());
        }
      } else {
        D[0][1] = D[1][1] = zero4();
      }
      const frag db[2] = {M::from_acc(D[0][0], D[0][1]), M::from_acc(D[1][0], D[1][1])};

      // O^T = scale (H0^T Q^T diag(exp G) + D^T P^T): lane holds output columns
      // 4*g4 .. 4*g4+3 of token l16 of the query block
#pragma unroll
      for (int mq = 0; mq < NQB; ++mq) {
        f32x4 x0 = zero4(), x1 = zero4();
#pragma unroll
        for (int sl = 0; sl < KS; ++sl) {
          const frag qf = M::load(s.Q, LDK, 16 * mq + l16, 32 * sl, lane);
          x0 = M::mma(hb[0][sl], qf, x0);
          x1 = M::mma(hb[1][sl], qf, x1);
        }
        const frag pf = M::load(v.P, LDC, 16 * mq + l16, 0, lane);
        const f32x4 y0 = M::mma(db[0], pf, zero4());
        const f32x4 y1 = M::mma(db[1], pf, zero4());
        const int q = 16 * mq + l16;
        const float sx = p.scale * s.eG[NH * q + NH - 1];
        float o0[4], o1[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o0[i] = sx * x0[i] + p.scale * y0[i];
          o1[i] = sx * x1[i] + p.scale * y1[i];
        }
        const int tok = tq0 + q;
        if (full || tok < t1) {
          TOut *o = ob + (static_cast<uint32_t>(tok) * vstride + 4 * g4);
          store4(o, o0);
          store4(o + 16, o1);
        }
      }

      // H <- exp(G_last) H0 + K~^T D
      const float dl = s.eG[CR - 1];
#pragma unroll
      for (int m = 0; m < KM; ++m) {
        const frag kt = M::load(v.KT, LDC, 16 * m + l16, 0, lane);
        H[0][m] = M::mma(kt, db[0], H[0][m] * dl);
        H[1][m] = M::mma(kt, db[1], H[1][m] * dl);
      }
      __syncthreads();
    }
  } else if (nchunks > 0) {
    // two register sets alternate between fetch and staging (the loop is unrolled
    // by two): the set fetched in one interval is staged in the next, and the set
    // carried around the loop stays in place
    auto produce = [&](int ci, const ChunkRegs<Tr> &from, ChunkRegs<Tr> &into) {
      if (ci + 1 < nchunks)
        solve_chunk<Tr>(sm.st[(ci + 1) % 3], sm.sv[(ci + 1) & 1], sm.AT, pw, lane);
      if (ci + 2 < nchunks) stage(from, sm.st[(ci + 2) % 3]);
      fetch(into, row_begin + (ci + 3) * CR);
      __syncthreads();
    };
    for (int ci = 0;; ci += 2) {
      produce(ci, cra, crb);
      if (ci + 1 >= nchunks) break;
      produce(ci + 1, crb, cra);
      if (ci + 2 >= nchunks) break;
    }
  }

  // ---- final state ---------------------------------------------------------------
  if (is_state && p.final_state && dst >= 0) {
    float *s1 = p.final_state + (static_cast<size_t>(dst) * p.Hv + h) * state_stride;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int m = 0; m < KM; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s1[static_cast<size_t>(16 * m + 4 * g4 + i) * p.DV + col0 + 16 * ct + l16] = H[ct][m][i];
  }
}

// ---- dispatch --------------------------------------------------------------------

namespace {

template <typename TIn, int DK, int CR, int NH, int NS, bool F32>
hipError_t launch_one(const PrefillParams &p, int grid, hipStream_t stream) {
  constexpr int threads = 64 * PrefillTraits<TIn, DK, CR, NH, NS, F32>::NW;
  if (p.out_bf16)
    hipLaunchKernelGGL((prefill_kernel<TIn, __bf16, DK, CR, NH, NS, F32>), dim3(grid),
                       dim3(threads), 0, stream, p);
  else
    hipLaunchKernelGGL((prefill_kernel<TIn, float, DK, CR, NH, NS, F32>), dim3(grid),
                       dim3(threads), 0, stream, p);
  return hipGetLastError();
}

template <typename TIn, int DK, int NS, bool F32>
hipError_t launch_rows(const PrefillParams &p, int rows, int nh, int grid, hipStream_t s) {
  constexpr bool kRows32 = !(F32 && DK > 64);
  if (nh == 1) {
    if (rows == 16) return launch_one<TIn, DK, 16, 1, NS, F32>(p, grid, s);
    if constexpr (kRows32)
      if (rows == 32) return launch_one<TIn, DK, 32, 1, NS, F32>(p, grid, s);
  } else if (nh == 2) {
    if constexpr (kRows32)
      if (rows == 32) return launch_one<TIn, DK, 32, 2, NS, F32>(p, grid, s);
  }
  return hipErrorInvalidValue;
}

template <typename TIn, int NS, bool F32>
hipError_t launch_dk(const PrefillParams &p, int head_k, int rows, int nh, int grid,
                     hipStream_t s) {
  if (head_k == 64) return launch_rows<TIn, 64, NS, F32>(p, rows, nh, grid, s);
  if (head_k == 128) return launch_rows<TIn, 128, NS, F32>(p, rows, nh, grid, s);
  return hipErrorInvalidValue;
}

template <typename TIn, bool F32>
hipError_t launch_ns(const PrefillParams &p, int head_k, int rows, int nh, int ns, int grid,
                     hipStream_t s) {
  if (ns == 1) return launch_dk<TIn, 1, F32>(p, head_k, rows, nh, grid, s);
  if (ns == 2) return launch_dk<TIn, 2, F32>(p, head_k, rows, nh, grid, s);
  if (ns == 4) return launch_dk<TIn, 4, F32>(p, head_k, rows, nh, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace

int prefill_chunk_rows(int chunk_size, int nh, int qkv_f32, int head_k) {
  // fp32 operands with K = 128 only fit 16-row chunks in LDS
  const int cap = (qkv_f32 && head_k > 64) ? 16 : 32;
  const int rows = chunk_size * nh;
  return rows < cap ? rows : cap;
}

int prefill_state_waves(int head_v, int num_seqs, int num_v_heads) {
  // State waves (32 value columns each) per workgroup: the widest tile that still
  // gives every compute unit a workgroup; with fewer sequence-head pairs than
  // that, narrower tiles put more compute units to work on each head.
  constexpr long kComputeUnits = 256;
  const long pairs = static_cast<long>(num_seqs) * num_v_heads;
  for (int ns = head_v / 32; ns > 1; ns >>= 1)
    if (pairs * (head_v / (32 * ns)) >= kComputeUnits) return ns;
  return 1;
}

hipError_t launch_prefill(const PrefillParams &p, int qkv_f32, int head_k, int rows, int nh,
                          int state_waves, hipStream_t stream) {
  const int items_per_xcd_round = 8 * p.group_size;
  const int rounds = (p.num_groups + 7) / 8;
  const int grid = items_per_xcd_round * rounds;
  if (grid == 0) return hipSuccess;
  return qkv_f32 ? launch_ns<float, true>(p, head_k, rows, nh, state_waves, grid, stream)
                 : launch_ns<uint16_t, false>(p, head_k, rows, nh, state_waves, grid, stream);
}

}  // namespace gdr
