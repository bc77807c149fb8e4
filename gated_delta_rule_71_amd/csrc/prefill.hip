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
//     I + A_bb by back substitution, both blocks on one wave; the off-diagonal
//     block A_10; P = scale (Q K^T * Gamma)), stage chunk i+2 (K and K^T, Q,
//     optionally L2-normalised, the workgroup's V columns transposed, the
//     cumulative decay and per-row factors) from registers into LDS, and fetch the
//     inputs of chunk i+3 into registers.
// Both kinds work at once and meet at one workgroup barrier per chunk, so a chunk
// interval costs the longer of the two instead of their sum.  With the diagonal
// inverses T_bb the chunk's delta follows by block forward substitution,
// D_0 = T_00 R_0, D_1 = T_11 (R_1 - A_10 D_0); the off-diagonal block of
// (I + A)^-1 is never formed.  Staged inputs are triple-buffered, solved operands
// double-buffered; none of them leave LDS.  HBM sees q, k, v, g, beta once per
// column tile (the tiles of one head share them through L2), o once and the state
// once in each direction.
//
// Operand precision: bf16 inputs run with fp16 operands and fp32 accumulation;
// fp32 inputs run every product with fp32 operands.  On the fp16 path q, k and v
// (after the optional L2 norm), and the in-kernel T, P, H and D, are rounded to
// fp16 (11 significant bits).  bf16 values of magnitude in [2^-14, 65504) convert
// exactly; smaller ones become fp16 subnormals and lose low bits (negligible
// against the unit-norm rows they sit in), and entries of magnitude >= 65504
// (inputs, the state, or the in-kernel deltas) overflow to infinity.

#include <type_traits>

#include "chunk_helpers.hpp"
#include "common.hpp"
#include "gdr_internal.hpp"

namespace gdr {

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
  static constexpr int ST = 64 * NP;                 // staging threads (all producer waves)
  static constexpr int CQ = CR / NH;                 // query rows per chunk
  static constexpr int NB = CR / 16;                 // 16-row blocks
  static constexpr int NQB = CQ / 16;                // 16-row query blocks
  static constexpr int DVT = 32 * NS;                // value columns per workgroup
  static constexpr int PAD = F32 ? 4 : 8;            // elements of row padding
  static constexpr int LDK = DK + PAD;               // K, Q leading dimension
  static constexpr int LDC = 32 + PAD;               // T, A10, P, KT leading dimension
  static constexpr int LDA = 20;                     // AR (fp32 16x16 blocks) leading dim.
  // VT (value column major) leading dimension: with 8 elements of padding the
  // bf16 rows sit 20 LDS words apart, where a wave's 8-byte reads of them do not
  // collide in the banks (fp32 keeps 4: its largest tile would not fit otherwise)
  static constexpr int LDVT = CR + (F32 ? 4 : 8);
  // AR block stride: four words past 16 rows, so that the two blocks' rows read
  // together during the inversion fall in different banks
  static constexpr int ARB = 16 * LDA + 4;
  static constexpr int KS = DK / 32;                 // 32-deep slices over keys
  static constexpr int KM = DK / 16;                 // 16-row blocks of H
  static constexpr int SEG = DK / 8;                 // 8-element segments per row
  static constexpr int KUNITS = (CR / 2) * SEG;      // (row pair, segment) units of K
  static constexpr int KPT = (KUNITS + ST - 1) / ST;
  static constexpr int QPT = (CQ * SEG + ST - 1) / ST;
  static constexpr int VSEG = DVT / 8;               // 8-element segments per V row
  static constexpr int VUNITS = (CR / 2) * VSEG;     // (row pair, segment) units of V
  static constexpr int VPT = (VUNITS + ST - 1) / ST;
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
  typename Tr::elem KT[Tr::DK * Tr::LDC];   // K^T (keys by rows)
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
  typename Tr::elem P[Tr::CQ * Tr::LDC];    // scale (Q K^T * Gamma), causal
};
template <class Tr>
struct PrefillSmem {
  StageBuf<Tr> st[3];
  SolveBuf<Tr> sv[2];
  float AR[2][Tr::ARB];   // the diagonal blocks A_bb (fp32, row-major) for the inversion
};

// Inputs of one chunk held in a producer thread's registers between their fetch
// and their staging.  They are loaded raw from clamped addresses; rows past the
// sequence end are zeroed only when the values are consumed, so that no
// instruction waits on a load before the data is needed.
template <class Tr>
struct ChunkRegs {
  Seg8<typename Tr::TIn> k[Tr::KPT][2], q[Tr::QPT], v[Tr::VPT][2];
  float g, b;   // producer wave 0: decay and write strength of row `lane`
  int c;        // first row of the chunk these registers hold
};

// ---- solve one chunk (producer waves) ---------------------------------------------
// Each task issues all of its LDS reads first, then its matrix-core products, then
// its epilogue and stores, so that no read has to wait behind a store.
//   producer wave 0: the diagonal blocks A_bb and their inverses T_bb;
//   producer waves 1 and 2: A_10 and the P tiles on or below the causal boundary.
// Every producer wave also stages and fetches; wave 3 runs the decay scan.

// Tile j of the off-diagonal work: A_10 first (32-row chunks), then the nonzero P
// tiles.  Encoded as 4*row_block + col_block, plus 16 for P tiles; -1 past the end.
template <class Tr>
__device__ __forceinline__ constexpr int tile_job(int j) {
  if (Tr::NB == 2) {
    if (j == 0) return 4;
    --j;
  }
  for (int mq = 0; mq < Tr::NQB; ++mq)
    for (int ni = 0; ni < Tr::NB; ++ni)
      if (16 * ni <= Tr::NH * (16 * mq + 15) + Tr::NH - 1) {
        if (j == 0) return 16 + 4 * mq + ni;
        --j;
      }
  return -1;
}
template <class Tr>
__device__ __forceinline__ constexpr int tile_job_count() {
  int n = 0;
  while (tile_job<Tr>(n) >= 0) ++n;
  return n;
}

// Off-diagonal tiles J0 .. J1-1: A_10 = strict_lower(diag(beta) K_1 K_0^T * Gamma) and
// P tiles = scale (Q K^T * Gamma) on or below the causal boundary.  Each is formed
// transposed (K_ni X^T), so that a lane holds four consecutive columns of one row
// and writes them with one store.
template <class Tr, int J0, int J1>
__device__ __forceinline__ void run_tiles(const StageBuf<Tr> &s, SolveBuf<Tr> &v, float scale,
                                          int lane) {
  constexpr int N = J1 - J0;
  if constexpr (N > 0) {
    using M = typename Tr::M;
    using frag = typename M::frag;
    constexpr int KS = Tr::KS, LDK = Tr::LDK, LDC = Tr::LDC, NH = Tr::NH;
    const int l16 = lane & 15, g4 = lane >> 4;
    frag fk[N][KS], fx[N][KS];
    double gr[N], gc[N][4];
    float br[N];
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int code = tile_job<Tr>(J0 + j);
      const bool is_p = code >= 16;
      const int mi = (code & 15) >> 2, ni = code & 3;
      const typename Tr::elem *xrows = is_p ? s.Q : s.K;
#pragma unroll
      for (int sl = 0; sl < KS; ++sl) {
        fk[j][sl] = M::load(s.K, LDK, 16 * ni + l16, 32 * sl, lane);
        fx[j][sl] = M::load(xrows, LDK, 16 * mi + l16, 32 * sl, lane);
      }
      const int q = 16 * mi + l16;               // row of A_10 / P held by this lane
      const int r = is_p ? NH * q + NH - 1 : q;  // its key row
      gr[j] = s.G[r];
      br[j] = is_p ? scale : s.B[r];
#pragma unroll
      for (int i = 0; i < 4; ++i) gc[j][i] = s.G[16 * ni + 4 * g4 + i];
    }
    f32x4 acc[N];
#pragma unroll
    for (int j = 0; j < N; ++j) {
      acc[j] = zero4();
#pragma unroll
      for (int sl = 0; sl < KS; ++sl) acc[j] = M::mma(fk[j][sl], fx[j][sl], acc[j]);
    }
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int code = tile_job<Tr>(J0 + j);
      const bool is_p = code >= 16;
      const int mi = (code & 15) >> 2, ni = code & 3;
      const int q = 16 * mi + l16;
      const int r = is_p ? NH * q + NH - 1 : q;
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 16 * ni + 4 * g4 + i;
        // mask before the exponential: G_r - G_c may be large positive above
        const bool keep = is_p ? c <= r : c < r;
        const float d = keep ? static_cast<float>(gr[j] - gc[j][i]) : 0.0f;
        x[i] = keep ? br[j] * acc[j][i] * fexp(d) : 0.0f;
      }
      if (is_p)
        store4e(v.P + q * LDC + 16 * ni + 4 * g4, x);
      else
        store4e(v.A10 + l16 * LDC + 4 * g4, x);
    }
  }
}

// The diagonal blocks A_bb = strict_lower(diag(beta) K_b K_b^T * Gamma) and their
// inverses T_bb = (I + A_bb)^-1.  K_b K_b^T is symmetric, so its accumulator tile
// also gives lane (l16, g4) row l16, columns 4*g4 .. 4*g4+3 of A_bb, written to LDS
// row-major with one store.  Row j of T_bb solves (I + A_bb)^T t = e_j, an upper
// triangular system: lanes 16b .. 16b+15 solve it for block b by back
// substitution (lane j keeps row j of T_bb in registers, step c subtracts row c of
// A_bb times t_c) and write the row with two or four 16-byte stores.
template <class Tr>
__device__ __forceinline__ void diag_blocks(const StageBuf<Tr> &s, SolveBuf<Tr> &v,
                                            float (*AR)[Tr::ARB], int lane) {
  using M = typename Tr::M;
  using frag = typename M::frag;
  constexpr int NB = Tr::NB, KS = Tr::KS, LDK = Tr::LDK, LDC = Tr::LDC, LDA = Tr::LDA;
  const int l16 = lane & 15, g4 = lane >> 4;
  frag f[NB][KS];
  double gr[NB], gc[NB][4];
  float br[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int sl = 0; sl < KS; ++sl) f[b][sl] = M::load(s.K, LDK, 16 * b + l16, 32 * sl, lane);
    gr[b] = s.G[16 * b + l16];
    br[b] = s.B[16 * b + l16];
#pragma unroll
    for (int i = 0; i < 4; ++i) gc[b][i] = s.G[16 * b + 4 * g4 + i];
  }
  f32x4 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    acc[b] = zero4();
#pragma unroll
    for (int sl = 0; sl < KS; ++sl) acc[b] = M::mma(f[b][sl], f[b][sl], acc[b]);
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 4 * g4 + i;   // column within the block; the row is l16
      const bool keep = c < l16;
      const float d = keep ? static_cast<float>(gr[b] - gc[b][i]) : 0.0f;
      a[i] = keep ? br[b] * acc[b][i] * fexp(d) : 0.0f;
    }
    *reinterpret_cast<float4 *>(AR[b] + l16 * LDA + 4 * g4) = make_float4(a[0], a[1], a[2], a[3]);
  }
  if (lane < 16 * NB) {
    const int bk = lane >> 4, j = lane & 15;
    const float *Ab = AR[bk];
    float t[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) t[r] = (r == j) ? 1.0f : 0.0f;
    // step c needs row c of A_bb left of its diagonal (quads 0 .. (c-1)/4); the rows
    // are read in three batches, each ahead of its steps
    auto steps = [&](auto first, auto count) {
      constexpr int C0 = decltype(first)::value, NC = decltype(count)::value;
      float4 row[NC][4];
#pragma unroll
      for (int cc = 0; cc < NC; ++cc)
#pragma unroll
        for (int qd = 0; qd <= (C0 - cc - 1) / 4; ++qd)
          row[cc][qd] = *reinterpret_cast<const float4 *>(Ab + (C0 - cc) * LDA + 4 * qd);
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
    typename Tr::elem *trow = v.T + (16 * bk + j) * LDC + 16 * bk;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float x[4] = {t[4 * q], t[4 * q + 1], t[4 * q + 2], t[4 * q + 3]};
      store4e(trow + 4 * q, x);
    }
  }
}

template <class Tr>
__device__ __forceinline__ void solve_chunk(const StageBuf<Tr> &s, SolveBuf<Tr> &v,
                                            float (*AR)[Tr::ARB], int pw, float scale,
                                            int lane) {
  static_assert(Tr::NP == 4, "four producer waves");
  constexpr int NJ = tile_job_count<Tr>();
  constexpr int H1 = (NJ + 1) / 2;
  if (pw == 0)
    diag_blocks<Tr>(s, v, AR, lane);
  else if (pw == 1)
    run_tiles<Tr, 0, H1>(s, v, scale, lane);
  else if (pw == 2)
    run_tiles<Tr, H1, NJ>(s, v, scale, lane);
}

template <typename TIn, typename TOut, int DK, int CR, int NH, int NS, bool F32>
__global__ void __launch_bounds__(64 * (NS + 4))
prefill_kernel(const PrefillParams p) {
  using Tr = PrefillTraits<TIn, DK, CR, NH, NS, F32>;
  using M = typename Tr::M;
  using elem = typename Tr::elem;
  using frag = typename M::frag;
  constexpr int CQ = Tr::CQ, NB = Tr::NB, NQB = Tr::NQB, DVT = Tr::DVT, SEG = Tr::SEG;
  constexpr int LDK = Tr::LDK, LDC = Tr::LDC, LDVT = Tr::LDVT, NT = Tr::NT, ST = Tr::ST;
  constexpr int KS = Tr::KS, KM = Tr::KM, KPT = Tr::KPT, QPT = Tr::QPT;

  __shared__ PrefillSmem<Tr> sm;

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
  // boundary states: rows between entries, and the first entry of this sequence
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
  const TIn *__restrict__ kb = static_cast<const TIn *>(p.k) + hk * DK;
  const TIn *__restrict__ qb = static_cast<const TIn *>(p.q) + hk * DK;
  const TIn *__restrict__ vrow =
      p.v ? static_cast<const TIn *>(p.v) + h * p.DV + vt * DVT : nullptr;
  const float *__restrict__ gb = p.g + h;
  const float *__restrict__ bb = p.beta + h;
  // gate parameters of this value head when g and beta hold raw projections
  float gate_A = 0.0f, gate_dt = 0.0f;
  if (p.gate_mode) {
    gate_A = expf(p.A_log[h]);
    gate_dt = p.dt_bias[h];
  }
  TOut *__restrict__ ob =
      p.out ? static_cast<TOut *>(p.out) + h * p.DV + col0 : nullptr;   // + token, lane
  const uint32_t kstride = p.Hk * DK;        // elements between key rows (and query rows)
  const uint32_t vstride = p.Hv * p.DV;      // elements between value / output rows
  const size_t state_stride = static_cast<size_t>(DK) * p.DV;

  // parts of the solve buffers and of K^T (columns past a 16-row chunk) that no
  // chunk writes must read as zero
  {
    elem *z = reinterpret_cast<elem *>(&sm.sv[0]);
    constexpr int nz = static_cast<int>(sizeof(sm.sv) / (sizeof(elem)));
    for (int i = tid; i < nz; i += NT) z[i] = M::cvt(0.0f);
    if constexpr (CR < 32) {
      constexpr int nkt = Tr::DK * LDC;
#pragma unroll
      for (int b = 0; b < 3; ++b)
        for (int i = tid; i < nkt; i += NT) sm.st[b].KT[i] = M::cvt(0.0f);
    }
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

  // this state wave's 32 columns of H -> a [K, V] state at s1 (uniform): each store
  // is a uniform row pointer plus one per-lane offset, kept opaque so that the
  // compiler does not precompute (and hold) 64 separate lane addresses
  auto store_state = [&](float *s1) {
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

  const int row_begin = t0 * NH, row_end = t1 * NH;
  const int nchunks = (row_end - row_begin + CR - 1) / CR;

  ChunkRegs<Tr> cra, crb;   // producer registers: two chunks' inputs

  // K unit u -> (row pair, segment).  With L2 normalisation the SEG units of a row
  // pair sit in consecutive lanes (the norm is a reduction over them); without it
  // consecutive lanes take consecutive row pairs, so that the transposed stores
  // of a wave fall in distinct banks.
  auto k_unit = [&](int u, int &rp, int &sg) {
    if (p.l2norm) {
      rp = u / SEG;
      sg = u % SEG;
    } else {
      rp = u % (CR / 2);
      sg = u / (CR / 2);
    }
  };

  // inputs of the chunk starting at row c -> producer registers (addresses clamped
  // to the sequence and the column tile, also for chunks past the end; validity is
  // applied where the values are consumed)
  auto fetch = [&](ChunkRegs<Tr> &cr, int c) {
    const int last = row_end - 1;
    const int tq = c / NH, tlast = t1 - 1;
    cr.c = c;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      int rp, sg;
      k_unit(stid + j * ST, rp, sg);
      rp = min(rp, CR / 2 - 1);
      sg = min(sg, SEG - 1);
      const int ra = min(c + 2 * rp, last), rb = min(c + 2 * rp + 1, last);
      cr.k[j][0].load(kb + (static_cast<uint32_t>(ra) * kstride + sg * 8));
      cr.k[j][1].load(kb + (static_cast<uint32_t>(rb) * kstride + sg * 8));
    }
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const int idx = stid + j * ST, r = idx / SEG, sg = idx % SEG;
      const int t = min(tq + r, tlast);
      cr.q[j].load(qb + (static_cast<uint32_t>(t) * kstride + sg * 8));
    }
#pragma unroll
    for (int j = 0; j < Tr::VPT; ++j) {
      const int u = stid + j * ST;
      const int rp = u % (CR / 2), sg = min(u / (CR / 2), Tr::VSEG - 1);
      const int ra = min(c + 2 * rp, last), rb = min(c + 2 * rp + 1, last);
      if (p.v) {
        cr.v[j][0].load(vrow + (static_cast<uint32_t>(ra) * vstride + sg * 8));
        cr.v[j][1].load(vrow + (static_cast<uint32_t>(rb) * vstride + sg * 8));
      } else {   // no values: the state's own evolution (a transition operator)
        cr.v[j][0].zero();
        cr.v[j][1].zero();
      }
    }
    if (pw == 3) {
      const int row = min(c + lane, last);
      cr.g = gb[static_cast<uint32_t>(row / NH) * p.Hv];
      cr.b = bb[static_cast<uint32_t>(row) * p.Hv];
    }
  };
  // producer registers -> staged LDS buffer
  auto stage = [&](const ChunkRegs<Tr> &cr, StageBuf<Tr> &s) {
    const int nrow = min(CR, row_end - cr.c);              // valid key rows
    const int nq = min(CQ, t1 - cr.c / NH);                // valid query rows
    // one 8-element segment of a row: zero past the valid rows, optionally divided
    // by the row's L2 norm (the SEG lanes holding a row are consecutive)
    auto segment = [&](const Seg8<TIn> &src, bool valid, float (&x)[8]) {
      src.get(x);
      if (!valid) {
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
    };
    // K rows 2rp, 2rp+1: row-major, and transposed as row pairs
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      int rp, sg;
      k_unit(stid + j * ST, rp, sg);
      float x0[8], x1[8];
      segment(cr.k[j][0], nrow == CR || 2 * rp < nrow, x0);
      segment(cr.k[j][1], nrow == CR || 2 * rp + 1 < nrow, x1);
      if (Tr::KUNITS % ST == 0 || (rp < CR / 2 && sg < SEG)) {
        store8(s.K + (2 * rp) * LDK + sg * 8, x0);
        store8(s.K + (2 * rp + 1) * LDK + sg * 8, x1);
#pragma unroll
        for (int e = 0; e < 8; ++e) store2(s.KT + (8 * sg + e) * LDC + 2 * rp, x0[e], x1[e]);
      }
    }
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const int idx = stid + j * ST, r = idx / SEG, sg = idx % SEG;
      float x[8];
      segment(cr.q[j], nq == CQ || r < nq, x);
      if (r < CQ) store8(s.Q + r * LDK + sg * 8, x);
    }
#pragma unroll
    for (int j = 0; j < Tr::VPT; ++j) {
      const int u = stid + j * ST;
      const int rp = u % (CR / 2), sg = u / (CR / 2);
      Seg8<TIn> a = cr.v[j][0], b = cr.v[j][1];
      if (nrow < CR) {
        if (2 * rp >= nrow) a.zero();
        if (2 * rp + 1 >= nrow) b.zero();
      }
      if (sg < Tr::VSEG) store_vt_pairs(s.VT + (8 * sg) * LDVT + 2 * rp, LDVT, a, b);
    }
    if (pw == 3) {
      // inclusive prefix sum of the per-row decay, in fp64, and per-row factors
      // (the gates are formed here first when g and beta hold raw projections)
      const bool ok = lane < nrow;
      float gv = cr.g;
      float bv = cr.b;
      if (p.gate_mode) {
        gv = gate_decay(cr.g, gate_A, gate_dt);
        bv = gate_beta(cr.b);
      }
      const double gr = prefix_sum32((ok && (cr.c + lane) % NH == 0) ? gv : 0.0);
      bv = ok ? bv : 0.0f;
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
  const bool stager = !is_state;   // producer waves that stage and fetch
  if (stager && nchunks > 0) {
    fetch(cra, row_begin);
    stage(cra, sm.st[0]);
    fetch(crb, row_begin + CR);
  }
  __syncthreads();
  if (stager && nchunks > 0) {
    solve_chunk<Tr>(sm.st[0], sm.sv[0], sm.AR, pw, p.scale, lane);
    if (nchunks > 1) stage(crb, sm.st[1]);
    fetch(cra, row_begin + 2 * CR);
  }
  __syncthreads();

  // ---- pipelined chunk loop ---------------------------------------------------------
  // Each role runs its own loop; both pass one workgroup barrier per chunk, so
  // chunk ci's state products (state waves) overlap the solve of chunk ci+1, the
  // staging of chunk ci+2 and the fetch of chunk ci+3 (producer waves).
  if (is_state) {
    // Software pipeline of the state waves: the operands of R for chunk ci+1 (its
    // K fragments, V columns, beta and exp(G) rows; staged an interval earlier) are
    // read at the end of interval ci, so they arrive while the wave waits at the
    // barrier; the solved operands and Q are read behind the products of R, the
    // decayed keys behind those of Q H0.
    frag kf[NB][KS];
    float vr[2][NB][4], br[NB][4], er[NB][4];
    auto load_r = [&](const StageBuf<Tr> &s) {
#pragma unroll
      for (int mk = 0; mk < NB; ++mk) {
#pragma unroll
        for (int sl = 0; sl < KS; ++sl) kf[mk][sl] = M::load(s.K, LDK, 16 * mk + l16, 32 * sl, lane);
        const int r0 = 16 * mk + 4 * g4;
        const float4 b4 = *reinterpret_cast<const float4 *>(s.B + r0);
        const float4 e4 = *reinterpret_cast<const float4 *>(s.eG + r0);
        br[mk][0] = b4.x; br[mk][1] = b4.y; br[mk][2] = b4.z; br[mk][3] = b4.w;
        er[mk][0] = e4.x; er[mk][1] = e4.y; er[mk][2] = e4.z; er[mk][3] = e4.w;
        load4(s.VT + (32 * wave + l16) * LDVT + r0, vr[0][mk]);
        load4(s.VT + (32 * wave + 16 + l16) * LDVT + r0, vr[1][mk]);
      }
    };
    if (nchunks > 0) load_r(sm.st[0]);
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

      // X = K H0 (both column tiles)
      f32x4 X[2][2];
#pragma unroll
      for (int mk = 0; mk < NB; ++mk) {
        X[0][mk] = zero4();
        X[1][mk] = zero4();
#pragma unroll
        for (int sl = 0; sl < KS; ++sl) {
          X[0][mk] = M::mma(kf[mk][sl], hb[0][sl], X[0][mk]);
          X[1][mk] = M::mma(kf[mk][sl], hb[1][sl], X[1][mk]);
        }
      }
      // the operands of D and O, read while those products run
      const frag tf0 = M::load(v.T, LDC, l16, 0, lane);
      frag af, tf1;
      if constexpr (NB == 2) {
        af = M::load(v.A10, LDC, l16, 0, lane);
        tf1 = M::load(v.T, LDC, 16 + l16, 0, lane);
      }
      frag qf[NQB][KS], pf[NQB];
      float sx[NQB];
#pragma unroll
      for (int mq = 0; mq < NQB; ++mq) {
#pragma unroll
        for (int sl = 0; sl < KS; ++sl) qf[mq][sl] = M::load(s.Q, LDK, 16 * mq + l16, 32 * sl, lane);
        pf[mq] = M::load(v.P, LDC, 16 * mq + l16, 0, lane);
        sx[mq] = p.scale * s.eG[NH * (16 * mq + l16) + NH - 1];
      }
      const float dl = s.eG[CR - 1];

      // R = diag(beta) (V - diag(exp G) X)
      f32x4 R[2][2];
#pragma unroll
      for (int mk = 0; mk < NB; ++mk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          R[0][mk][i] = br[mk][i] * (vr[0][mk][i] - er[mk][i] * X[0][mk][i]);
          R[1][mk][i] = br[mk][i] * (vr[1][mk][i] - er[mk][i] * X[1][mk][i]);
        }
      if constexpr (NB == 1) R[0][1] = R[1][1] = zero4();

      // D_0 = T_00 R_0;  D_1 = T_11 (R_1 - A_10 D_0)   (T rows hold diag(T_00, T_11))
      f32x4 D[2][2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) D[ct][0] = M::mma(tf0, M::from_acc(R[ct][0], zero4()), zero4());
      if constexpr (NB == 2) {
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

      // O^T = scale H0^T Q^T diag(exp G) + D^T P^T (P carries the scale): lane holds
      // output columns 4*g4 .. 4*g4+3 of token l16 of each query block
      f32x4 xo[NQB][2], yo[NQB][2];
#pragma unroll
      for (int mq = 0; mq < NQB; ++mq) {
        xo[mq][0] = zero4();
        xo[mq][1] = zero4();
#pragma unroll
        for (int sl = 0; sl < KS; ++sl) {
          xo[mq][0] = M::mma(hb[0][sl], qf[mq][sl], xo[mq][0]);
          xo[mq][1] = M::mma(hb[1][sl], qf[mq][sl], xo[mq][1]);
        }
      }
      // the keys of the update, read while those products run
      frag kt[KM];
#pragma unroll
      for (int m = 0; m < KM; ++m) kt[m] = M::load(s.KT, LDC, 16 * m + l16, 0, lane);
      // D~ = diag(exp(G_last - G)) D: the decay of the update, on its B operand
      frag dk[2];
      {
        const float4 l0 = *reinterpret_cast<const float4 *>(s.eGl + 4 * g4);
        f32x4 e0 = {l0.x, l0.y, l0.z, l0.w}, e1 = zero4();
        if constexpr (NB == 2) {
          const float4 l1 = *reinterpret_cast<const float4 *>(s.eGl + 16 + 4 * g4);
          e1 = f32x4{l1.x, l1.y, l1.z, l1.w};
        }
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) dk[ct] = M::from_acc(D[ct][0] * e0, D[ct][1] * e1);
      }
#pragma unroll
      for (int mq = 0; mq < NQB; ++mq) {
        yo[mq][0] = M::mma(db[0], pf[mq], zero4());
        yo[mq][1] = M::mma(db[1], pf[mq], zero4());
      }

      // H <- exp(G_last) H0 + K^T D~
#pragma unroll
      for (int m = 0; m < KM; ++m) {
        H[0][m] = M::mma(kt[m], dk[0], H[0][m] * dl);
        H[1][m] = M::mma(kt[m], dk[1], H[1][m] * dl);
      }

#pragma unroll
      for (int mq = 0; mq < NQB; ++mq) {
        float o0[4], o1[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o0[i] = sx[mq] * xo[mq][0][i] + yo[mq][0][i];   // P carries the scale
          o1[i] = sx[mq] * xo[mq][1][i] + yo[mq][1][i];
        }
        const int tok = tq0 + 16 * mq + l16;
        if (p.out && (full || tok < t1)) {
          TOut *o = ob + (static_cast<uint32_t>(tok) * vstride + 4 * g4);
          store4(o, o0);
          store4(o + 16, o1);
        }
      }
      // a boundary state after every bnd_rows rows (boundaries fall on chunk ends)
      if (bnd_rows && ((ci + 1) * CR) % bnd_rows == 0 && (ci + 1) * CR <= row_end - row_begin) {
        const int e = bnd_base + (ci + 1) * CR / bnd_rows - 1;
        store_state(p.boundary_states + (static_cast<size_t>(e) * p.Hv + h) * state_stride);
      }
      // the R operands of the next chunk (staged an interval ago; read past the end
      // of the sequence they are never used)
      load_r(sm.st[(ci + 1) % 3]);
      __syncthreads();
    }
  } else if (nchunks > 0) {
    // two register sets alternate between fetch and staging (the loop is unrolled
    // by two): the set fetched in one interval is staged in the next, and the set
    // carried around the loop stays in place
    auto produce = [&](int ci, const ChunkRegs<Tr> &from, ChunkRegs<Tr> &into) {
      if (ci + 1 < nchunks)
        solve_chunk<Tr>(sm.st[(ci + 1) % 3], sm.sv[(ci + 1) & 1], sm.AR, pw, p.scale, lane);
      if (stager) {
        if (ci + 2 < nchunks) stage(from, sm.st[(ci + 2) % 3]);
        fetch(into, row_begin + (ci + 3) * CR);
      }
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
  if (is_state && p.final_state && dst >= 0)
    store_state(p.final_state + (static_cast<size_t>(dst) * p.Hv + h) * state_stride);
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

bool prefill_variant_exists(int qkv_f32, int head_k, int rows, int nh, int ns) {
  // mirrors launch_prefill64 (64-row chunks of bf16 inputs) and launch_ns / launch_dk /
  // launch_rows above
  if (ns != 1 && ns != 2 && ns != 4) return false;
  if (head_k != 64 && head_k != 128) return false;
  if (rows == 64) return !qkv_f32 && (nh == 1 || nh == 2);
  const bool rows32 = !(qkv_f32 && head_k > 64);
  if (nh == 1) return rows == 16 || (rows32 && rows == 32);
  if (nh == 2) return rows32 && rows == 32;
  return false;
}

int prefill_chunk_rows(int chunk_size, int nh, int qkv_f32, int head_k) {
  // bf16 inputs run 64-row chunks (prefill64.hip) when the chunk size reaches them;
  // fp32 operands fit 32-row chunks in LDS, 16-row chunks with K = 128
  const int cap = !qkv_f32 ? 64 : head_k > 64 ? 16 : 32;
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
  if (rows == 64) return launch_prefill64(p, head_k, nh, state_waves, grid, stream);
  return qkv_f32 ? launch_ns<float, true>(p, head_k, rows, nh, state_waves, grid, stream)
                 : launch_ns<uint16_t, false>(p, head_k, rows, nh, state_waves, grid, stream);
}

}  // namespace gdr
