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
// Work decomposition: one workgroup per (sequence, value head, tile of 16*NW value
// columns).  Columns of H evolve independently, so each wave owns 16 columns of
// H for the whole sequence, in matrix-core accumulator registers, and walks the
// sequence's chunks (32 rows) in order.  The per-chunk work is software
// pipelined over three chunks so that one workgroup barrier per chunk suffices:
// in interval i the workgroup
//   * runs the state-dependent products of chunk i (every wave, its columns):
//     X = [Q; K] H0, R, D = T R, O and the state update, on the matrix cores,
//     with H and D passed between products in registers and the decayed keys
//     of the update read straight from the row-major K tile;
//   * solves chunk i+1: two waves form the 16x16 diagonal blocks of A on the
//     matrix cores and invert I + A_bb by column substitution (one block each, no
//     synchronisation); another forms the off-diagonal block A_10; the rest form
//     P = Q K^T * Gamma and the decayed, transposed keys K~^T used by the state
//     update.  With the diagonal inverses T_bb the chunk's delta follows by block
//     forward substitution, D_0 = T_00 R_0, D_1 = T_11 (R_1 - A_10 D_0), so the
//     off-diagonal block of (I + A)^-1 is never formed;
//   * stages chunk i+2 (K, Q, optionally L2-normalised, the workgroup's V
//     columns, the cumulative decay and per-row decay factors) from registers
//     into LDS and fetches the inputs of chunk i+3 into registers.
// Staged inputs are triple-buffered, T and P double-buffered.  T and P never
// leave LDS; HBM sees q, k, v, g, beta once per column tile (the tiles of one
// head share them through L2), o once and the state once in each direction.
//
// Operand precision: bf16 inputs run with fp16 operands (bf16 values convert
// exactly; T, P, H and D are rounded to fp16, 11 significant bits) and fp32
// accumulation; fp32 inputs run every product with fp32 operands.

#include "common.hpp"
#include "gdr_internal.hpp"

namespace gdr {

// contraction index held in fragment element e by lane group g (see common.hpp)
__device__ __forceinline__ constexpr int kidx(int g, int e) {
  return e < 4 ? 4 * g + e : 12 + 4 * g + e;
}

// exp(x) on the hardware base-2 exponential
__device__ __forceinline__ float fexp(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

template <typename TIn_, int DK_, int CR_, int NH_, int NW_, bool F32_>
struct PrefillTraits {
  using TIn = TIn_;
  using M = Mma<F32_>;
  using elem = typename M::elem;
  static constexpr bool F32 = F32_;
  static constexpr int DK = DK_, CR = CR_, NH = NH_, NW = NW_;
  static constexpr int CQ = CR / NH;                 // query rows per chunk
  static constexpr int NB = CR / 16;                 // 16-row blocks
  static constexpr int NQB = CQ / 16;                // 16-row query blocks
  static constexpr int DVT = 16 * NW;                // value columns per workgroup
  static constexpr int PAD = F32 ? 4 : 8;            // elements of row padding
  static constexpr int LDK = DK + PAD;               // K, Q leading dimension
  static constexpr int LDC = 32 + PAD;               // T, A10, P, KT leading dimension
  static constexpr int LDA = 20;                     // AT (fp32 16x16, column-major) leading dim.
  static constexpr int NT = 64 * NW;                 // threads
  static constexpr int KS = DK / 32;                 // 32-deep slices over keys
  static constexpr int KM = DK / 16;                 // 16-row blocks of H
  static constexpr int SEG = DK / 8;                 // 8-element segments per row
  static constexpr int KPT = (CR * SEG + NT - 1) / NT;
  static constexpr int QPT = (CQ * SEG + NT - 1) / NT;
  static constexpr int VSEG = DVT / 8;               // 8-element segments per V row
  static constexpr int VPT = (CR * VSEG + NT - 1) / NT;
  static constexpr int LDV = DVT + 8;                // V leading dimension
  static_assert(CR == 16 || CR == 32, "chunk rows");
  static_assert(CQ % 16 == 0, "query rows");
  static_assert(DK % 32 == 0, "head_k");
  static_assert(NW >= 2, "waves");
};

// one staged chunk
template <class Tr>
struct StageBuf {
  typename Tr::elem K[Tr::CR * Tr::LDK];
  typename Tr::elem Q[Tr::CQ * Tr::LDK];
  typename Tr::TIn V[Tr::CR * Tr::LDV];   // the workgroup's value columns, input type
  double G[Tr::CR];     // cumulative decay (fp64: differences of large sums stay exact)
  float eG[Tr::CR];     // exp(G_r)
  float eGl[Tr::CR];    // exp(G_last - G_r)
  float B[Tr::CR];      // beta
};
// the solved operands of one chunk
template <class Tr>
struct SolveBuf {
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

// Inputs of one chunk held in registers between their fetch and their staging.
// They are loaded raw from clamped addresses; rows past the sequence end are
// zeroed only when the values are consumed, so that no instruction waits on a
// load before the data is needed.
template <class Tr>
struct ChunkRegs {
  Seg8<typename Tr::TIn> k[Tr::KPT], q[Tr::QPT], v[Tr::VPT];
  float g, b;   // wave 0: decay and write strength of row `lane`
  int c;        // first row of the chunk these registers hold
};

// ---- solve one chunk: T_bb, A_10, P and K~^T ------------------------------------
// wave b < NB: A_bb and its inverse; wave NB (32-row chunks): A_10; the remaining
// waves: P tiles and the decayed, transposed keys.
template <class Tr>
__device__ __forceinline__ void solve_chunk(const StageBuf<Tr> &s, SolveBuf<Tr> &v,
                                            float (*AT)[16 * Tr::LDA], int wave, int lane) {
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
  if (wave < NB) {
    const int bk = wave;
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
  if (NB == 2 && wave == NB) {
    float a[4];
    a_tile(1, 0, a);
#pragma unroll
    for (int i = 0; i < 4; ++i) v.A10[(4 * g4 + i) * LDC + l16] = M::cvt(a[i]);
  }
  // the remaining work is spread over waves first = NB + (NB == 2) .. NW-1
  constexpr int first = NB + (NB == 2 ? 1 : 0);
  constexpr int nwk = Tr::NW - first;
  static_assert(nwk >= 1, "waves");
  // waves >= first take P tiles round-robin (the A_10 wave joins the K~^T work)
  if (wave >= first) {
    constexpr int NPT = Tr::NQB * NB;
    for (int ti = wave - first; ti < NPT; ti += nwk) {
      const int mq = ti / NB, ni = ti % NB;
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
  }
  // K~^T[d][r] = exp(G_last - G_r) K[r][d]: a lane takes two rows and 8 keys and
  // writes 8 row pairs (one 32-bit store each for fp16 operands)
  {
    constexpr int kfirst = NB;                     // the A_10 wave helps here too
    constexpr int nkw = Tr::NW - kfirst;
    constexpr int UNITS = (Tr::CR / 2) * Tr::SEG;  // (row pair, segment) units
    for (int u = (wave - kfirst) * 64 + lane; u < UNITS; u += nkw * 64) {
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

template <typename TIn, typename TOut, int DK, int CR, int NH, int NW, bool F32>
__global__ void __launch_bounds__(64 * NW)
prefill_kernel(const PrefillParams p) {
  using Tr = PrefillTraits<TIn, DK, CR, NH, NW, F32>;
  using M = typename Tr::M;
  using elem = typename Tr::elem;
  using frag = typename M::frag;
  constexpr int CQ = Tr::CQ, NB = Tr::NB, NQB = Tr::NQB, DVT = Tr::DVT, SEG = Tr::SEG;
  constexpr int LDK = Tr::LDK, LDC = Tr::LDC, NT = Tr::NT, KS = Tr::KS, KM = Tr::KM;
  constexpr int KPT = Tr::KPT, QPT = Tr::QPT;

  __shared__ PrefillSmem<Tr> sm;

  const int w_item = xcd_work_item(blockIdx.x, p.group_size, p.num_groups);
  if (w_item < 0) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int l16 = lane & 15;
  const int g4 = lane >> 4;

  // work item -> (sequence, query/key head, value head, column tile)
  const int group = w_item / p.group_size;
  const int member = w_item % p.group_size;
  const int n = group / p.Hk;
  const int hk = group % p.Hk;
  const int h = hk * (p.Hv / p.Hk) + member / p.num_vtiles;
  const int vt = member % p.num_vtiles;
  const int col0 = vt * DVT + 16 * wave;   // first value column of this wave

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
  TOut *__restrict__ ob = static_cast<TOut *>(p.out) + h * p.DV + col0;   // + row, lane
  const uint32_t kstride = p.Hk * DK;        // elements between key rows (and query rows)
  const uint32_t vstride = p.Hv * p.DV;      // elements between value / output rows
  const size_t state_stride = static_cast<size_t>(DK) * p.DV;

  // parts of the solve buffers no chunk writes must read as zero
  {
    elem *z = reinterpret_cast<elem *>(&sm.sv[0]);
    constexpr int nz = static_cast<int>(sizeof(sm.sv) / sizeof(elem));
    for (int i = tid; i < nz; i += NT) z[i] = M::cvt(0.0f);
  }

  // ---- initial state -> registers ---------------------------------------------
  f32x4 H[KM];
  if (p.initial_state) {
    const float *s0 = p.initial_state + (static_cast<size_t>(src) * p.Hv + h) * state_stride;
#pragma unroll
    for (int m = 0; m < KM; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        H[m][i] = s0[static_cast<size_t>(16 * m + 4 * g4 + i) * p.DV + col0 + l16];
  } else {
#pragma unroll
    for (int m = 0; m < KM; ++m) H[m] = zero4();
  }

  const int row_begin = t0 * NH, row_end = t1 * NH;
  const int nchunks = (row_end - row_begin + CR - 1) / CR;

  ChunkRegs<Tr> cr;

  // inputs of the chunk starting at row c -> registers (addresses clamped to the
  // sequence; validity is applied where the values are consumed)
  auto fetch_kq = [&](int c) {
    const int last = row_end - 1;
    const int tq = c / NH, tlast = t1 - 1;
    cr.c = c;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int idx = tid + j * NT, r = idx / SEG, sg = idx % SEG;
      const int row = min(c + r, last);
      cr.k[j].load(kb + (static_cast<uint32_t>(row) * kstride + sg * 8));
    }
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const int idx = tid + j * NT, r = idx / SEG, sg = idx % SEG;
      const int t = min(tq + r, tlast);
      cr.q[j].load(qb + (static_cast<uint32_t>(t) * kstride + sg * 8));
    }
#pragma unroll
    for (int j = 0; j < Tr::VPT; ++j) {
      const int idx = tid + j * NT, r = idx / Tr::VSEG, sg = idx % Tr::VSEG;
      const int row = min(c + r, last);
      cr.v[j].load(vrow + (static_cast<uint32_t>(row) * vstride + sg * 8));
    }
    if (wave == 0) {
      const int row = min(c + lane, last);
      cr.g = gb[static_cast<uint32_t>(row / NH) * p.Hv];
      cr.b = bb[static_cast<uint32_t>(row) * p.Hv];
    }
  };
  // registers -> staged LDS buffer
  auto stage = [&](StageBuf<Tr> &s) {
    const int nrow = min(CR, row_end - cr.c);              // valid key rows
    const int nq = min(CQ, t1 - cr.c / NH);                // valid query rows
    auto rows = [&](const Seg8<TIn> *src, int count, int nrows, int nvalid, elem *dstm) {
#pragma unroll
      for (int j = 0; j < count; ++j) {
        const int idx = tid + j * NT, r = idx / SEG, sg = idx % SEG;
        float x[8];
        src[j].get(x);
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
      const int idx = tid + j * NT, r = idx / Tr::VSEG, sg = idx % Tr::VSEG;
      Seg8<TIn> x = cr.v[j];
      if (nrow < CR && r >= nrow) x.zero();
      if (r < CR) x.store(s.V + r * Tr::LDV + sg * 8);
    }
    if (wave == 0) {
      // inclusive prefix sum of the per-row decay, in fp64, and per-row factors
      const bool ok = lane < nrow;
      double gr = (ok && (cr.c + lane) % NH == 0) ? cr.g : 0.0f;
      const float bv = ok ? cr.b : 0.0f;
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) {
        const double y = __shfl_up(gr, o);
        if (lane >= o) gr += y;
      }
      const double glast = __shfl(gr, CR - 1);
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
  if (nchunks > 0) {
    fetch_kq(row_begin);
    stage(sm.st[0]);
    if (nchunks > 1) fetch_kq(row_begin + CR);
  }
  __syncthreads();
  if (nchunks > 0) {
    solve_chunk<Tr>(sm.st[0], sm.sv[0], sm.AT, wave, lane);
    if (nchunks > 1) stage(sm.st[1]);
    if (nchunks > 2) fetch_kq(row_begin + 2 * CR);
  }
  __syncthreads();

  // ---- pipelined chunk loop ---------------------------------------------------------
  for (int ci = 0; ci < nchunks; ++ci) {
    const int c0 = row_begin + ci * CR;
    const int tq0 = c0 / NH;
    const bool full = tq0 + CQ <= t1;   // every query row of the chunk is in the sequence
    const StageBuf<Tr> &s = sm.st[ci % 3];
    const SolveBuf<Tr> &v = sm.sv[ci & 1];

    // ---- state-dependent products of chunk ci (each wave: its 16 columns) ----
    {
      frag hb[KS];
#pragma unroll
      for (int sl = 0; sl < KS; ++sl) hb[sl] = M::from_acc(H[2 * sl], H[2 * sl + 1]);

      // R = diag(beta) V - diag(beta exp(G)) K H0
      f32x4 R[2];
#pragma unroll
      for (int mk = 0; mk < NB; ++mk) {
        f32x4 acc = zero4();
#pragma unroll
        for (int sl = 0; sl < KS; ++sl)
          acc = M::mma(M::load(s.K, LDK, 16 * mk + l16, 32 * sl, lane), hb[sl], acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * mk + 4 * g4 + i;
          const float vv = to_f32(s.V[r * Tr::LDV + 16 * wave + l16]);
          R[mk][i] = s.B[r] * (vv - s.eG[r] * acc[i]);
        }
      }
      if constexpr (NB == 1) R[1] = zero4();
      // D_0 = T_00 R_0;  D_1 = T_11 (R_1 - A_10 D_0)   (T rows hold diag(T_00, T_11))
      f32x4 D[2];
      D[0] = M::mma(M::load(v.T, LDC, l16, 0, lane), M::from_acc(R[0], zero4()), zero4());
      if constexpr (NB == 2) {
        const f32x4 z = M::mma(M::load(v.A10, LDC, l16, 0, lane), M::from_acc(D[0], zero4()),
                               zero4());
        const f32x4 y = R[1] - z;
        D[1] = M::mma(M::load(v.T, LDC, 16 + l16, 0, lane), M::from_acc(zero4(), y), zero4());
      } else {
        D[1] = zero4();
      }
      const frag db = M::from_acc(D[0], D[1]);

      // O = scale (diag(exp(G)) Q H0 + P D)
#pragma unroll
      for (int mq = 0; mq < NQB; ++mq) {
        f32x4 xq = zero4();
#pragma unroll
        for (int sl = 0; sl < KS; ++sl)
          xq = M::mma(M::load(s.Q, LDK, 16 * mq + l16, 32 * sl, lane), hb[sl], xq);
        const f32x4 pd = M::mma(M::load(v.P, LDC, 16 * mq + l16, 0, lane), db, zero4());
        const int tb = tq0 + 16 * mq + 4 * g4;
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int q = 16 * mq + 4 * g4 + i;
          o[i] = p.scale * (s.eG[NH * q + NH - 1] * xq[i] + pd[i]);
        }
        const uint32_t off = static_cast<uint32_t>(tb) * vstride + l16;
        if (full) {
#pragma unroll
          for (int i = 0; i < 4; ++i) ob[off + i * vstride] = static_cast<TOut>(o[i]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (tb + i < t1) ob[off + i * vstride] = static_cast<TOut>(o[i]);
        }
      }

      // H <- exp(G_last) H0 + K~^T D
      const float dl = s.eG[CR - 1];
#pragma unroll
      for (int m = 0; m < KM; ++m)
        H[m] = M::mma(M::load(v.KT, LDC, 16 * m + l16, 0, lane), db, H[m] * dl);
    }

    // ---- solve chunk ci+1, stage chunk ci+2, fetch chunk ci+3 -------------------
    if (ci + 1 < nchunks) solve_chunk<Tr>(sm.st[(ci + 1) % 3], sm.sv[(ci + 1) & 1], sm.AT, wave, lane);
    if (ci + 2 < nchunks) stage(sm.st[(ci + 2) % 3]);
    if (ci + 3 < nchunks) fetch_kq(c0 + 3 * CR);
    __syncthreads();
  }

  // ---- final state ---------------------------------------------------------------
  if (p.final_state && dst >= 0) {
    float *s1 = p.final_state + (static_cast<size_t>(dst) * p.Hv + h) * state_stride;
#pragma unroll
    for (int m = 0; m < KM; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        s1[static_cast<size_t>(16 * m + 4 * g4 + i) * p.DV + col0 + l16] = H[m][i];
  }
}

// ---- dispatch --------------------------------------------------------------------

namespace {

template <typename TIn, int DK, int CR, int NH, int NW, bool F32>
hipError_t launch_one(const PrefillParams &p, int grid, hipStream_t stream) {
  if (p.out_bf16)
    hipLaunchKernelGGL((prefill_kernel<TIn, __bf16, DK, CR, NH, NW, F32>), dim3(grid),
                       dim3(64 * NW), 0, stream, p);
  else
    hipLaunchKernelGGL((prefill_kernel<TIn, float, DK, CR, NH, NW, F32>), dim3(grid),
                       dim3(64 * NW), 0, stream, p);
  return hipGetLastError();
}

template <typename TIn, int DK, int NW, bool F32>
hipError_t launch_rows(const PrefillParams &p, int rows, int nh, int grid, hipStream_t s) {
  constexpr bool kRows32 = !(F32 && DK > 64);
  if (nh == 1) {
    if (rows == 16) return launch_one<TIn, DK, 16, 1, NW, F32>(p, grid, s);
    if constexpr (kRows32)
      if (rows == 32) return launch_one<TIn, DK, 32, 1, NW, F32>(p, grid, s);
  } else if (nh == 2) {
    if constexpr (kRows32)
      if (rows == 32) return launch_one<TIn, DK, 32, 2, NW, F32>(p, grid, s);
  }
  return hipErrorInvalidValue;
}

template <typename TIn, bool F32>
hipError_t launch_waves(const PrefillParams &p, int head_k, int rows, int nh, int waves, int grid,
                        hipStream_t s) {
  if (waves == 4) {
    if (head_k == 64) return launch_rows<TIn, 64, 4, F32>(p, rows, nh, grid, s);
    if (head_k == 128) return launch_rows<TIn, 128, 4, F32>(p, rows, nh, grid, s);
  } else if (waves == 8) {
    if (head_k == 64) return launch_rows<TIn, 64, 8, F32>(p, rows, nh, grid, s);
    if (head_k == 128) return launch_rows<TIn, 128, 8, F32>(p, rows, nh, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int prefill_chunk_rows(int chunk_size, int nh, int qkv_f32, int head_k) {
  // fp32 operands with K = 128 only fit 16-row chunks in LDS
  const int cap = (qkv_f32 && head_k > 64) ? 16 : 32;
  const int rows = chunk_size * nh;
  return rows < cap ? rows : cap;
}

int prefill_waves(int head_v, int num_seqs, int num_v_heads) {
  // Value columns per workgroup: a whole 128-column head (8 waves) when there are
  // enough sequence-head pairs to fill the chip, else 64 columns (4 waves) so that
  // two workgroups share each head.
  if (head_v == 128 && static_cast<long>(num_seqs) * num_v_heads >= 256) return 8;
  return 4;
}

hipError_t launch_prefill(const PrefillParams &p, int qkv_f32, int head_k, int rows, int nh,
                          int waves, hipStream_t stream) {
  const int items_per_xcd_round = 8 * p.group_size;
  const int rounds = (p.num_groups + 7) / 8;
  const int grid = items_per_xcd_round * rounds;
  if (grid == 0) return hipSuccess;
  return qkv_f32 ? launch_waves<float, true>(p, head_k, rows, nh, waves, grid, stream)
                 : launch_waves<uint16_t, false>(p, head_k, rows, nh, waves, grid, stream);
}

}  // namespace gdr
