// Single-token decode of the gated delta rule over a slot-indexed fp32 state cache.
//
// One step of S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
// o_t = scale S_t q_t per (request, value head), in place on the cache slot the
// request names (ssm_decode on the Megatron Core API pages
// "core.ssm.gated_delta_net.gdn" and "core.ssm.gated_delta_product").  Padding
// rows (batch_indices[i] = -1) read slot 0 and write nothing (PR "Add GDN dynamic
// inference #6499", review thread on padding).
//
// With H = S^T ([K, V] as stored), alpha = exp(g) and n_h Householder sub-steps
// (n_h = 1 for the plain rule), every quantity the step needs from the old state
// is a matrix-vector product with H^T, so H is read once and written once:
//   a_s = H^T k_s,  y = H^T q                              (one pass over H)
//   u_s = alpha a_s + sum_{s'<s} (k_s'.k_s) d_s',  d_s = beta_s (v_s - u_s)
//   o   = scale (alpha y + sum_s (k_s.q) d_s)
//   H'  = alpha H + sum_s k_s d_s^T                        (same registers)
// Several tokens per request repeat the step with H in registers; the slot is
// read once and written once.
//
// Layout: one 256-thread workgroup per (request, value head).  Thread t owns four
// adjacent value columns (16-byte accesses; a 128-column row is read by 32
// consecutive lanes, fully coalesced) in every (256/(V/4))-th key row, so the
// whole 64 KiB state sits in registers between the read and the write.  Column
// sums over the key dimension reduce across lanes with shuffles, then across the
// four waves through LDS.

#include "common.hpp"
#include "gdr_internal.hpp"

namespace gdr {

template <typename TIn, int DK, int DV, int NH>
__global__ void __launch_bounds__(256)
decode_kernel(const DecodeParams p) {
  constexpr int NT = 256;
  constexpr int CG = DV / 4;          // column groups of 4
  constexpr int RG = NT / CG;         // row groups
  constexpr int RPT = DK / RG;        // rows per thread
  constexpr int NV = NH + 1;          // vectors multiplied by H^T: k_0..k_{NH-1}, q
  constexpr int WAVES = NT / kWave;
  static_assert(DK % RG == 0, "rows");

  __shared__ float qs[DK];
  __shared__ float ks[NH][DK];
  __shared__ float dots[NV * NH];     // k_s'.k_s and k_s.q
  __shared__ float red[WAVES][NV][DV];

  const int i = blockIdx.x / p.Hv;
  const int h = blockIdx.x % p.Hv;
  const int hk = h / (p.Hv / p.Hk);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int cg = tid % CG, rg = tid / CG;

  const int r = p.batch_indices ? p.batch_indices[i] : i;
  const int slot = r < 0 ? 0 : r;
  const size_t state_size = static_cast<size_t>(DK) * DV;
  float *st = p.state + (static_cast<size_t>(slot) * p.Hv + h) * state_size;

  // issue the state reads first: they are the bulk of the traffic
  float4 Hr[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m)
    Hr[m] = *reinterpret_cast<const float4 *>(st + static_cast<size_t>(rg + RG * m) * DV + 4 * cg);

  const TIn *qg = static_cast<const TIn *>(p.q);
  const TIn *kg = static_cast<const TIn *>(p.k);
  const TIn *vg = static_cast<const TIn *>(p.v);
  const float gate_A = p.gate_mode ? expf(p.A_log[h]) : 0.0f;

  // this thread's rows of H -> a [K, V] state at dst
  auto store_state = [&](float *dst) {
#pragma unroll
    for (int m = 0; m < RPT; ++m)
      *reinterpret_cast<float4 *>(dst + static_cast<size_t>(rg + RG * m) * DV + 4 * cg) = Hr[m];
  };

  // the request's tokens one after another; the state stays in registers
  for (int t = 0; t < p.num_tokens; ++t) {
    const size_t tok = static_cast<size_t>(i) * p.num_tokens + t;   // token row
    // q and k rows (optionally L2-normalised) -> LDS
    if (wave <= NH) {
      const TIn *src = (wave < NH) ? kg + ((tok * NH + wave) * p.Hk + hk) * DK
                                   : qg + (tok * p.Hk + hk) * DK;
      float x[DK / 64];
      float ss = 0.0f;
#pragma unroll
      for (int e = 0; e < DK / 64; ++e) {
        x[e] = load_f32(src + lane + 64 * e);
        ss += x[e] * x[e];
      }
      if (p.l2norm) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
        const float rn = 1.0f / sqrtf(ss + 1e-6f);
#pragma unroll
        for (int e = 0; e < DK / 64; ++e) x[e] *= rn;
      }
      float *dstv = (wave < NH) ? ks[wave] : qs;
#pragma unroll
      for (int e = 0; e < DK / 64; ++e) dstv[lane + 64 * e] = x[e];
    }
    __syncthreads();
    // dot products among the sub-step keys and the query (one wave per product)
    for (int d = wave; d < NV * NH; d += WAVES) {
      const int s = d / NV, o = d % NV;   // k_s . (k_o or q when o == NH)
      const float *b = (o < NH) ? ks[o] : qs;
      float acc = 0.0f;
      for (int e = lane; e < DK; e += 64) acc += ks[s][e] * b[e];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
      if (lane == 0) dots[d] = acc;
    }

    // partial H^T x for x in {k_0.., q}: this thread's rows, its 4 columns
    float part[NV][4];
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int c = 0; c < 4; ++c) part[v][c] = 0.0f;
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      const int row = rg + RG * m;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const float xv = (v < NH) ? ks[v][row] : qs[row];
        part[v][0] += Hr[m].x * xv;
        part[v][1] += Hr[m].y * xv;
        part[v][2] += Hr[m].z * xv;
        part[v][3] += Hr[m].w * xv;
      }
    }
    // reduce over the row groups inside the wave (lanes CG apart)
#pragma unroll
    for (int off = CG; off < 64; off <<= 1)
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int c = 0; c < 4; ++c) part[v][c] += __shfl_xor(part[v][c], off);
    if (lane < CG) {
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int c = 0; c < 4; ++c) red[wave][v][4 * cg + c] = part[v][c];
    }
    __syncthreads();

    // the gates (formed here from the raw projections when gate_mode is set)
    float alpha, bet[NH];
    {
      const float gin = p.g[tok * p.Hv + h];
      alpha = p.gate_mode ? expf(gate_decay(gin, gate_A, p.dt_bias[h])) : expf(gin);
#pragma unroll
      for (int s = 0; s < NH; ++s) {
        const float b = p.beta[(tok * NH + s) * p.Hv + h];
        bet[s] = p.gate_mode ? gate_beta(b) : b;
      }
    }
    // per-column step (every thread, for its own 4 columns)
    float dlt[NH][4];
    float out[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int col = 4 * cg + c;
      float a[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) s += red[w][v][col];
        a[v] = s;
      }
      float o = alpha * a[NH];
#pragma unroll
      for (int s = 0; s < NH; ++s) {
        float u = alpha * a[s];
#pragma unroll
        for (int s2 = 0; s2 < s; ++s2) u += dots[s2 * NV + s] * dlt[s2][c];
        const size_t row = tok * NH + s;
        const float vv = load_f32(vg + (row * p.Hv + h) * DV + col);
        dlt[s][c] = bet[s] * (vv - u);
        o += dots[s * NV + NH] * dlt[s][c];
      }
      out[c] = p.scale * o;
    }
    if (rg == 0) {
      const size_t off = (tok * p.Hv + h) * DV + 4 * cg;
      if (p.out_bf16) {
        uint16_t *op = static_cast<uint16_t *>(p.out) + off;
        const uint2 pk = {static_cast<uint32_t>(f32_to_bf16(out[0])) |
                              (static_cast<uint32_t>(f32_to_bf16(out[1])) << 16),
                          static_cast<uint32_t>(f32_to_bf16(out[2])) |
                              (static_cast<uint32_t>(f32_to_bf16(out[3])) << 16)};
        *reinterpret_cast<uint2 *>(op) = pk;
      } else {
        *reinterpret_cast<float4 *>(static_cast<float *>(p.out) + off) =
            make_float4(out[0], out[1], out[2], out[3]);
      }
    }

    // H' = alpha H + sum_s k_s d_s^T, in registers
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      const int row = rg + RG * m;
      float4 hn;
      hn.x = alpha * Hr[m].x;
      hn.y = alpha * Hr[m].y;
      hn.z = alpha * Hr[m].z;
      hn.w = alpha * Hr[m].w;
#pragma unroll
      for (int s = 0; s < NH; ++s) {
        const float kv = ks[s][row];
        hn.x += kv * dlt[s][0];
        hn.y += kv * dlt[s][1];
        hn.z += kv * dlt[s][2];
        hn.w += kv * dlt[s][3];
      }
      Hr[m] = hn;
    }
    if (p.intermediate_state && r >= 0)
      store_state(p.intermediate_state + (tok * p.Hv + h) * state_size);
    // the next token rewrites qs, ks, dots and red
    if (t + 1 < p.num_tokens) __syncthreads();
  }
  if (r >= 0) store_state(st);   // padding: no state write
}

namespace {
template <typename TIn, int DK, int DV>
hipError_t launch_nh(const DecodeParams &p, int nh, hipStream_t s) {
  const dim3 grid(p.batch * p.Hv), block(256);
  if (nh == 1) hipLaunchKernelGGL((decode_kernel<TIn, DK, DV, 1>), grid, block, 0, s, p);
  else if (nh == 2) hipLaunchKernelGGL((decode_kernel<TIn, DK, DV, 2>), grid, block, 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}
template <typename TIn>
hipError_t launch_dims(const DecodeParams &p, int dk, int dv, int nh, hipStream_t s) {
  if (dk == 128 && dv == 128) return launch_nh<TIn, 128, 128>(p, nh, s);
  if (dk == 64 && dv == 64) return launch_nh<TIn, 64, 64>(p, nh, s);
  if (dk == 128 && dv == 64) return launch_nh<TIn, 128, 64>(p, nh, s);
  if (dk == 64 && dv == 128) return launch_nh<TIn, 64, 128>(p, nh, s);
  return hipErrorInvalidValue;
}
}  // namespace

hipError_t launch_decode(const DecodeParams &p, int qkv_f32, int dk, int dv, int nh,
                         hipStream_t stream) {
  if (p.batch == 0) return hipSuccess;
  return qkv_f32 ? launch_dims<float>(p, dk, dv, nh, stream)
                 : launch_dims<uint16_t>(p, dk, dv, nh, stream);
}

}  // namespace gdr
