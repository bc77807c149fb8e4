// Host side of the C ABI declared in include/gdr.h: argument checks (pure host
// code, no HIP calls), launch-shape selection and kernel dispatch.

#include <math.h>
#include <stdint.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "gdr.h"
#include "gdr_internal.hpp"

namespace {

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool dtype_ok(int32_t d) { return d == GDR_DTYPE_F32 || d == GDR_DTYPE_BF16; }
bool head_ok(int32_t d) { return d == 64 || d == 128; }
bool pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

constexpr int64_t kMaxRows = (int64_t{1} << 31) - 1024;

}  // namespace

extern "C" {

int gdr_abi_version(void) { return GDR_ABI_VERSION; }

const char *gdr_status_string(int status) {
  switch (status) {
    case GDR_OK: return "GDR_OK";
    case GDR_ERR_INVALID_ARG: return "GDR_ERR_INVALID_ARG";
    case GDR_ERR_UNSUPPORTED: return "GDR_ERR_UNSUPPORTED";
    case GDR_ERR_WORKSPACE: return "GDR_ERR_WORKSPACE";
    case GDR_ERR_HIP: return "GDR_ERR_HIP";
    default: return "GDR_ERR_UNKNOWN";
  }
}

int gdr_validate_prefill(const gdr_prefill_args *a) {
  if (!a) return GDR_ERR_INVALID_ARG;
  if (a->batch < 0 || a->seqlen < 0 || a->num_seqs < 0) return GDR_ERR_INVALID_ARG;
  if (a->num_qk_heads <= 0 || a->num_v_heads <= 0) return GDR_ERR_INVALID_ARG;
  if (a->num_v_heads % a->num_qk_heads != 0) return GDR_ERR_INVALID_ARG;
  if (a->head_k <= 0 || a->head_v <= 0 || a->num_householder <= 0 || a->chunk_size <= 0)
    return GDR_ERR_INVALID_ARG;
  if (!dtype_ok(a->qkv_dtype) || !dtype_ok(a->out_dtype)) return GDR_ERR_INVALID_ARG;
  if (a->use_qk_l2norm != 0 && a->use_qk_l2norm != 1) return GDR_ERR_INVALID_ARG;
  if (isinf(a->scale)) return GDR_ERR_INVALID_ARG;
  if (a->gate_mode != 0 && a->gate_mode != 1) return GDR_ERR_INVALID_ARG;
  if (a->cu_seqlens) {
    if (a->batch != 1) return GDR_ERR_INVALID_ARG;
  } else if (a->num_seqs != a->batch) {
    return GDR_ERR_INVALID_ARG;
  }
  if (a->state_indices && a->num_slots <= 0) return GDR_ERR_INVALID_ARG;
  const int64_t tokens = int64_t{a->batch} * a->seqlen;
  if (tokens * a->num_householder > kMaxRows) return GDR_ERR_UNSUPPORTED;
  // the prefill kernels form element offsets within q, k, v and out as 32-bit
  // unsigned values: rows * (heads * head size) must stay below 2^32
  {
    const int64_t kw = int64_t{a->num_qk_heads} * a->head_k;
    const int64_t vw = int64_t{a->num_v_heads} * a->head_v;
    if (tokens * a->num_householder * (kw > vw ? kw : vw) >= (int64_t{1} << 32))
      return GDR_ERR_UNSUPPORTED;
  }
  if (!head_ok(a->head_k) || !head_ok(a->head_v)) return GDR_ERR_UNSUPPORTED;
  if (a->num_householder > 2) return GDR_ERR_UNSUPPORTED;
  if (!pow2(a->chunk_size) || a->chunk_size < 16 || a->chunk_size > 256)
    return GDR_ERR_UNSUPPORTED;
  // the chunk shape the kernels would run must be instantiated (float32 inputs with
  // K = 128 fit only 16-row chunks in LDS, which the two-sub-step rows do not use)
  {
    const int f32 = a->qkv_dtype == GDR_DTYPE_F32;
    const int rows = gdr::prefill_chunk_rows(a->chunk_size, a->num_householder, f32, a->head_k);
    if (!gdr::prefill_variant_exists(f32, a->head_k, rows, a->num_householder, 1))
      return GDR_ERR_UNSUPPORTED;
  }
  if (tokens > 0) {
    if (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->out) return GDR_ERR_INVALID_ARG;
    if (a->gate_mode == 1 && (!a->A_log || !a->dt_bias)) return GDR_ERR_INVALID_ARG;
    if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->out))
      return GDR_ERR_INVALID_ARG;
  }
  if ((a->initial_state && !aligned16(a->initial_state)) ||
      (a->final_state && !aligned16(a->final_state)))
    return GDR_ERR_INVALID_ARG;
  // boundary states every multiple of 64 rows (64 / n_h tokens)
  if (a->boundary_states &&
      (!aligned16(a->boundary_states) || a->boundary_interval <= 0 ||
       (int64_t{a->boundary_interval} * a->num_householder) % 64 != 0))
    return GDR_ERR_INVALID_ARG;
  return GDR_OK;
}

int gdr_validate_decode(const gdr_decode_args *a) {
  if (!a) return GDR_ERR_INVALID_ARG;
  if (a->batch < 0 || a->num_qk_heads <= 0 || a->num_v_heads <= 0) return GDR_ERR_INVALID_ARG;
  if (a->num_v_heads % a->num_qk_heads != 0) return GDR_ERR_INVALID_ARG;
  if (a->head_k <= 0 || a->head_v <= 0 || a->num_householder <= 0) return GDR_ERR_INVALID_ARG;
  if (!dtype_ok(a->qkv_dtype) || !dtype_ok(a->out_dtype)) return GDR_ERR_INVALID_ARG;
  if (a->use_qk_l2norm != 0 && a->use_qk_l2norm != 1) return GDR_ERR_INVALID_ARG;
  if (isinf(a->scale)) return GDR_ERR_INVALID_ARG;
  if (a->gate_mode != 0 && a->gate_mode != 1) return GDR_ERR_INVALID_ARG;
  if (a->num_tokens < 1) return GDR_ERR_INVALID_ARG;
  if (!head_ok(a->head_k) || !head_ok(a->head_v)) return GDR_ERR_UNSUPPORTED;
  if (a->num_householder > 2) return GDR_ERR_UNSUPPORTED;
  if (a->num_tokens > (1 << 16)) return GDR_ERR_UNSUPPORTED;
  if (a->batch > 0) {
    if (a->intermediate_state && !aligned16(a->intermediate_state)) return GDR_ERR_INVALID_ARG;
    if (a->gate_mode == 1 && (!a->A_log || !a->dt_bias)) return GDR_ERR_INVALID_ARG;
    if (a->num_slots <= 0) return GDR_ERR_INVALID_ARG;
    if (!a->batch_indices && a->batch > a->num_slots) return GDR_ERR_INVALID_ARG;
    if (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->state || !a->out)
      return GDR_ERR_INVALID_ARG;
    if (!aligned16(a->state) || !aligned16(a->out)) return GDR_ERR_INVALID_ARG;
    if (int64_t{a->batch} * a->num_v_heads > kMaxRows) return GDR_ERR_UNSUPPORTED;
    // token-row offsets (request * T + t) times heads x head size stay 64-bit in the
    // kernel; the row count itself must fit an int
    if (int64_t{a->batch} * a->num_tokens * a->num_householder > kMaxRows)
      return GDR_ERR_UNSUPPORTED;
  }
  return GDR_OK;
}

// ---- long batched sequences in segments ------------------------------------------

namespace {

constexpr int kComputeUnits = 256;

// Segment plan for a prefill: S > 1 segments per batch row (or S segment slots shared
// by packed sequences) when the sequences alone leave most compute units idle (fewer
// workgroups than compute units even with 32 value columns each) and are long enough
// for segments of >= 2048 tokens.
struct SegPlan {
  int S = 1, seg_len = 0;
  bool packed = false;      // segments of packed sequences, planned on the device
  size_t cu = 0, first = 0, ident = 0, F = 0, A = 0, H_in = 0, total = 0;
};

// workspace layout of a plan with `nseq` segments (and `nfirst` entries of the packed
// plan's first-segment table)
void seg_layout(SegPlan &sp, const gdr_prefill_args *a, size_t nseq, size_t nfirst) {
  const size_t Hv = a->num_v_heads;
  const size_t kk = static_cast<size_t>(a->head_k) * a->head_k;
  const size_t kv = static_cast<size_t>(a->head_k) * a->head_v;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += round_up(bytes);
    return at;
  };
  sp.cu = take((nseq + 1) * sizeof(int32_t));
  sp.first = nfirst ? take(nfirst * sizeof(int32_t)) : 0;
  sp.ident = take(nseq * Hv * kk * 4);
  sp.A = take(nseq * Hv * kk * 4);
  sp.F = take(nseq * Hv * kv * 4);
  sp.H_in = take(nseq * Hv * kv * 4);
  sp.total = off;
}

// Packed sequences whose (sequence, value head) pairs leave compute units idle.  Their
// lengths live on the device, so the plan is sized from the total: S = 256 / Hv
// segment slots (one workgroup per slot and head at four state waves), segments of
// seg_len >= 2048 tokens such that sum_n max(1, ceil(L_n / seg_len)) <= S.  It is taken
// only where it pays whatever the lengths: seg_len <= T_tot / (4 N), so the longest
// sequence (at least T_tot / N tokens) is at least four segments long and its chain
// shortens more than the three passes cost.  Boundary states keep the single pass.
SegPlan seg_plan_packed(const gdr_prefill_args *a) {
  SegPlan sp;
  if (a->boundary_states || a->num_seqs < 1) return sp;
  const long N = a->num_seqs, Hv = a->num_v_heads, T = a->seqlen;
  if (N * Hv * (a->head_v / 32) >= kComputeUnits) return sp;
  const long S = kComputeUnits / Hv;
  if (S < 5 * N) return sp;
  long seg_len = ((T + (S - N) - 1) / (S - N) + 63) / 64 * 64;
  if (seg_len < 2048) seg_len = 2048;
  if (seg_len * 4 * N > T) return sp;
  sp.S = static_cast<int>(S);
  sp.seg_len = static_cast<int>(seg_len);
  sp.packed = true;
  seg_layout(sp, a, static_cast<size_t>(S), static_cast<size_t>(N) + 1);
  return sp;
}

SegPlan seg_plan(const gdr_prefill_args *a) {
  SegPlan sp;
  if (!a || a->batch < 1 || a->num_v_heads < 1 || a->head_v < 32 || a->head_k < 1) return sp;
  if (a->cu_seqlens) return seg_plan_packed(a);
  if (a->state_indices) return sp;
  const long pairs = static_cast<long>(a->batch) * a->num_v_heads;
  if (pairs * (a->head_v / 32) >= kComputeUnits) return sp;
  int S = 1;
  while (2 * S * pairs <= kComputeUnits && a->seqlen / (2 * S) >= 2048) S *= 2;
  if (S < 2) return sp;
  sp.S = S;
  sp.seg_len = ((a->seqlen + S - 1) / S + 63) / 64 * 64;
  if (static_cast<long>(S - 1) * sp.seg_len >= a->seqlen) {   // last segment empty
    sp.S = 1;
    return sp;
  }
  // boundary states (written by the last pass) keep their order when every
  // segment but a row's last is a whole number of intervals
  if (a->boundary_states &&
      (a->boundary_interval <= 0 || sp.seg_len % a->boundary_interval != 0)) {
    sp.S = 1;
    return sp;
  }
  seg_layout(sp, a, static_cast<size_t>(a->batch) * S, 0);
  return sp;
}

}  // namespace

size_t gdr_prefill_workspace_bytes(const gdr_prefill_args *a) {
  // the single-pass chunked prefill keeps every intermediate on chip; long batched
  // sequences that leave compute units idle may also run in segments, which needs
  // the workspace below (optional: without it the single pass runs)
  return seg_plan(a).total;
}

namespace {

// Enqueue a validated prefill.  ws, ws_bytes: device memory for the segment path of
// long batched rows (NULL: the single pass runs).
int enqueue_prefill(const gdr_prefill_args *a, hipStream_t s, void *ws_base, size_t ws_bytes) {
  if (a->num_seqs == 0) return GDR_OK;
  gdr::PrefillParams p;
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.g = a->g;
  p.beta = a->beta;
  p.cu_seqlens = a->cu_seqlens;
  p.state_indices = a->state_indices;
  p.initial_state = a->initial_state;
  p.final_state = a->final_state;
  p.out = a->out;
  p.seqlen = a->seqlen;
  p.num_seqs = a->num_seqs;
  p.Hk = a->num_qk_heads;
  p.Hv = a->num_v_heads;
  p.DV = a->head_v;
  const int state_waves = gdr::prefill_state_waves(a->head_v, a->num_seqs, a->num_v_heads);
  p.num_vtiles = a->head_v / (32 * state_waves);
  p.group_size = p.num_vtiles * (a->num_v_heads / a->num_qk_heads);
  p.num_groups = a->num_seqs * a->num_qk_heads;
  p.l2norm = a->use_qk_l2norm;
  p.out_bf16 = a->out_dtype == GDR_DTYPE_BF16;
  p.scale = isnan(a->scale) ? 1.0f / sqrtf(static_cast<float>(a->head_k)) : a->scale;
  p.gate_mode = a->gate_mode;
  p.A_log = a->A_log;
  p.dt_bias = a->dt_bias;
  p.boundary_states = a->boundary_states;
  p.boundary_interval = a->boundary_interval;
  const int f32 = a->qkv_dtype == GDR_DTYPE_F32;
  const int rows = gdr::prefill_chunk_rows(a->chunk_size, a->num_householder, f32, a->head_k);
  const SegPlan sp = seg_plan(a);
  const bool aligned = (reinterpret_cast<uintptr_t>(ws_base) & (kAlign - 1)) == 0;
  if (sp.S > 1 && ws_base && aligned && ws_bytes >= sp.total) {
    // long rows in segments: the passes are prefills over the segments as packed
    // sequences (see segments.hip)
    char *ws = static_cast<char *>(ws_base);
    gdr::SegmentParams g{};
    g.batch = a->batch;
    g.seqlen = a->seqlen;
    g.S = sp.S;
    g.seg_len = sp.seg_len;
    g.Hv = a->num_v_heads;
    g.DK = a->head_k;
    g.DV = a->head_v;
    g.cu = reinterpret_cast<int32_t *>(ws + sp.cu);
    g.ident = reinterpret_cast<float *>(ws + sp.ident);
    g.F = reinterpret_cast<float *>(ws + sp.F);
    g.A = reinterpret_cast<float *>(ws + sp.A);
    g.initial_state = a->initial_state;
    g.H_in = reinterpret_cast<float *>(ws + sp.H_in);
    g.final_state = a->final_state;
    if (sp.packed) {   // the caller's sequences, planned into the S slots on the device
      g.batch = a->num_seqs;
      g.src_cu = a->cu_seqlens;
      g.first = reinterpret_cast<int32_t *>(ws + sp.first);
      g.state_indices = a->state_indices;
    }
    const int nseq = sp.packed ? sp.S : a->batch * sp.S;
    auto run = [&](gdr::PrefillParams q, int dv) {
      q.cu_seqlens = g.cu;
      q.seqlen = a->batch * a->seqlen;
      q.num_seqs = nseq;
      q.DV = dv;
      const int ns = gdr::prefill_state_waves(dv, nseq, a->num_v_heads);
      q.num_vtiles = dv / (32 * ns);
      q.group_size = q.num_vtiles * (a->num_v_heads / a->num_qk_heads);
      q.num_groups = nseq * a->num_qk_heads;
      return gdr::launch_prefill(q, f32, a->head_k, rows, a->num_householder, ns, s);
    };
    // every pass's launch shape exists before anything is enqueued
    for (const int dv : {a->head_v, a->head_k})
      if (!gdr::prefill_variant_exists(f32, a->head_k, rows, a->num_householder,
                                       gdr::prefill_state_waves(dv, nseq, a->num_v_heads)))
        return GDR_ERR_UNSUPPORTED;
    if (gdr::launch_segment_setup(g, s) != hipSuccess) return GDR_ERR_HIP;
    gdr::PrefillParams pf = p;          // 1: from zero, final states F, no outputs
    pf.state_indices = nullptr;         // the passes' states are per segment
    pf.initial_state = nullptr;
    pf.final_state = const_cast<float *>(g.F);
    pf.out = nullptr;
    pf.boundary_states = nullptr;       // boundary states come from the last pass
    if (run(pf, a->head_v) != hipSuccess) return GDR_ERR_HIP;
    gdr::PrefillParams pa = pf;         // 2: no values, from the identity: transitions
    pa.v = nullptr;
    pa.initial_state = g.ident;
    pa.final_state = const_cast<float *>(g.A);
    if (run(pa, a->head_k) != hipSuccess) return GDR_ERR_HIP;
    if (gdr::launch_segment_combine(g, s) != hipSuccess) return GDR_ERR_HIP;   // 3
    gdr::PrefillParams po = p;          // 4: from the entering states, outputs (and
    po.state_indices = nullptr;         //    boundary states)
    po.initial_state = g.H_in;
    po.final_state = nullptr;
    return run(po, a->head_v) == hipSuccess ? GDR_OK : GDR_ERR_HIP;
  }
  if (!gdr::prefill_variant_exists(f32, a->head_k, rows, a->num_householder, state_waves))
    return GDR_ERR_UNSUPPORTED;
  const hipError_t e = gdr::launch_prefill(p, f32, a->head_k, rows, a->num_householder,
                                           state_waves, s);
  return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

}  // namespace

int gdr_chunk_gated_delta_rule(const gdr_prefill_args *a, void *stream) {
  const int st = gdr_validate_prefill(a);
  if (st != GDR_OK) return st;
  return enqueue_prefill(a, static_cast<hipStream_t>(stream), a->workspace, a->workspace_bytes);
}

// ---- prefill without allocation -----------------------------------------------------

// Scratch of gdr_chunk_gated_delta_rule_noalloc: the segment path's workspace in a
// file-scope device array, which every GPU the library runs on holds until the
// process ends.  Every segment plan keeps its segment count (batch rows x segments,
// or packed segment slots) x value heads <= 256, so its four float32 matrices per
// segment and head (identity and transition K x K, zero-start and entering states
// K x V, with K, V <= 128) take at most 4 x 16 MiB; the segment boundaries (<= 257
// int32), the packed plan's first-slot table (<= 53 int32) and the 256-byte
// alignment of each part fit in the rest.
constexpr size_t kScratchBytes = (size_t{64} << 20) + 4096;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up on the first call
// made with that device current (each GPU holds its own copy of the array).  Host code
// uses only this address, never the array's name.
int scratch_address(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GDR_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GDR_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GDR_OK;
}

}  // namespace

int gdr_chunk_gated_delta_rule_noalloc(const gdr_prefill_args *a, void *stream) {
  const int st = gdr_validate_prefill(a);
  if (st != GDR_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const SegPlan sp = seg_plan(a);
  if (sp.S <= 1) return enqueue_prefill(a, s, nullptr, 0);   // no scratch needed
  if (sp.total > kScratchBytes) return GDR_ERR_WORKSPACE;
  void *ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc != GDR_OK) return rc;
  return enqueue_prefill(a, s, ws, kScratchBytes);
}

int gdr_ssm_decode(const gdr_decode_args *a, void *stream) {
  const int st = gdr_validate_decode(a);
  if (st != GDR_OK) return st;
  if (a->batch == 0) return GDR_OK;
  gdr::DecodeParams p;
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.g = a->g;
  p.beta = a->beta;
  p.state = a->state;
  p.batch_indices = a->batch_indices;
  p.out = a->out;
  p.batch = a->batch;
  p.Hk = a->num_qk_heads;
  p.Hv = a->num_v_heads;
  p.l2norm = a->use_qk_l2norm;
  p.out_bf16 = a->out_dtype == GDR_DTYPE_BF16;
  p.scale = isnan(a->scale) ? 1.0f / sqrtf(static_cast<float>(a->head_k)) : a->scale;
  p.gate_mode = a->gate_mode;
  p.A_log = a->A_log;
  p.dt_bias = a->dt_bias;
  p.num_tokens = a->num_tokens;
  p.intermediate_state = a->intermediate_state;
  const hipError_t e = gdr::launch_decode(p, a->qkv_dtype == GDR_DTYPE_F32, a->head_k,
                                          a->head_v, a->num_householder,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

// ---- backward ------------------------------------------------------------------

namespace {

// Workspace carve-up of the backward (byte offsets from the base, each aligned).
struct BwdLayout {
  size_t tab, states, dhn, araw, pmat, tmat, dmat, drmat, dqh, dkh, qn, kn, gg, gb, fwd, total;
  size_t fwd_bytes;   // workspace of the forward recompute (long rows in segments)
  int max_chunks;
};

// the forward recompute's prefill arguments (boundary state every 64 rows); the
// pointers are left NULL except a stand-in for boundary_states, as only the sizes
// matter to the segment plan
gdr_prefill_args bwd_forward_args(const gdr_backward_args *a) {
  gdr_prefill_args f{};
  f.batch = a->batch;
  f.seqlen = a->seqlen;
  f.num_seqs = a->num_seqs;
  f.num_qk_heads = a->num_qk_heads;
  f.num_v_heads = a->num_v_heads;
  f.head_k = a->head_k;
  f.head_v = a->head_v;
  f.num_householder = a->num_householder;
  f.chunk_size = 64 / (a->num_householder > 0 ? a->num_householder : 1);
  f.qkv_dtype = a->qkv_dtype;
  f.out_dtype = a->qkv_dtype;
  f.use_qk_l2norm = a->use_qk_l2norm;
  f.scale = a->scale;
  f.cu_seqlens = a->cu_seqlens;
  f.gate_mode = a->gate_mode;
  f.A_log = a->A_log;
  f.dt_bias = a->dt_bias;
  f.boundary_states = reinterpret_cast<float *>(kAlign);   // stand-in, replaced at the call
  f.boundary_interval = f.chunk_size;
  return f;
}

BwdLayout bwd_layout(const gdr_backward_args *a) {
  BwdLayout L{};
  const size_t tokens = static_cast<size_t>(a->batch) * a->seqlen;
  const size_t nh = static_cast<size_t>(a->num_householder);
  const size_t rows = tokens * nh;   // one row per Householder sub-step
  const size_t N = static_cast<size_t>(a->num_seqs);
  const size_t D = static_cast<size_t>(a->head_k);
  const size_t Hv = static_cast<size_t>(a->num_v_heads);
  // 64-row chunks: sum of ceil(R_n / 64) <= (rows + 63 N) / 64; boundary states:
  // sum of floor(R_n / 64) <= rows / 64
  const size_t chunks = (rows + 63 * N) / 64;
  const size_t entries = rows / 64;
  L.max_chunks = static_cast<int>(chunks);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += round_up(bytes);
    return at;
  };
  L.tab = take(2 * (N + 1) * sizeof(int32_t));
  L.states = take(entries * Hv * D * D * 4);
  L.dhn = take(chunks * Hv * D * D * 4);
  L.araw = take(chunks * Hv * 64 * 64 * 4);
  L.pmat = take(chunks * Hv * 64 * 64 * 4);
  L.tmat = take(chunks * Hv * 64 * 64 * 4);
  // bf16 q, k (no in-kernel norm): the gradient kernel forms D itself
  const bool d_kept = a->qkv_dtype == GDR_DTYPE_F32 || a->use_qk_l2norm;
  L.dmat = take(d_kept ? chunks * Hv * 64 * D * 4 : 0);
  L.drmat = take(chunks * Hv * 64 * D * 4);
  const bool grouped = a->num_v_heads != a->num_qk_heads;
  L.dqh = take(grouped ? tokens * Hv * D * 4 : 0);
  L.dkh = take(grouped ? rows * Hv * D * 4 : 0);
  const size_t Hk = static_cast<size_t>(a->num_qk_heads);
  L.qn = take(a->use_qk_l2norm ? tokens * Hk * D * 4 : 0);
  L.kn = take(a->use_qk_l2norm ? rows * Hk * D * 4 : 0);
  L.gg = take(a->gate_mode ? tokens * Hv * 4 : 0);
  L.gb = take(a->gate_mode ? rows * Hv * 4 : 0);
  const gdr_prefill_args f = bwd_forward_args(a);
  L.fwd_bytes = gdr_prefill_workspace_bytes(&f);
  L.fwd = take(L.fwd_bytes);
  L.total = off;
  return L;
}

}  // namespace

int gdr_validate_backward(const gdr_backward_args *a) {
  if (!a) return GDR_ERR_INVALID_ARG;
  if (a->batch < 0 || a->seqlen < 0 || a->num_seqs < 0) return GDR_ERR_INVALID_ARG;
  if (a->num_qk_heads <= 0 || a->num_v_heads <= 0) return GDR_ERR_INVALID_ARG;
  if (a->num_v_heads % a->num_qk_heads != 0) return GDR_ERR_INVALID_ARG;
  if (a->head_k <= 0 || a->head_v <= 0) return GDR_ERR_INVALID_ARG;
  if (!dtype_ok(a->qkv_dtype)) return GDR_ERR_INVALID_ARG;
  if (isinf(a->scale)) return GDR_ERR_INVALID_ARG;
  if (a->use_qk_l2norm != 0 && a->use_qk_l2norm != 1) return GDR_ERR_INVALID_ARG;
  if (a->gate_mode != 0 && a->gate_mode != 1) return GDR_ERR_INVALID_ARG;
  if (a->gate_mode == 1 && (!a->A_log || !a->dt_bias || !a->dA_log || !a->ddt_bias))
    return GDR_ERR_INVALID_ARG;
  if (a->cu_seqlens) {
    if (a->batch != 1) return GDR_ERR_INVALID_ARG;
  } else if (a->num_seqs != a->batch) {
    return GDR_ERR_INVALID_ARG;
  }
  if (a->num_householder < 1) return GDR_ERR_INVALID_ARG;
  if (a->head_k != a->head_v || !head_ok(a->head_k)) return GDR_ERR_UNSUPPORTED;
  if (a->num_householder > 2) return GDR_ERR_UNSUPPORTED;
  // the forward recompute of the gated delta product has no float32 path at D = 128
  if (a->num_householder == 2 && a->qkv_dtype == GDR_DTYPE_F32 && a->head_k == 128)
    return GDR_ERR_UNSUPPORTED;
  const int64_t tokens = int64_t{a->batch} * a->seqlen;
  if (tokens * a->num_householder > kMaxRows) return GDR_ERR_UNSUPPORTED;
  {
    const int64_t kw = int64_t{a->num_qk_heads} * a->head_k;
    const int64_t vw = int64_t{a->num_v_heads} * a->head_v;
    if (tokens * a->num_householder * (kw > vw ? kw : vw) >= (int64_t{1} << 32))
      return GDR_ERR_UNSUPPORTED;
  }
  if (int64_t{a->num_seqs} * a->num_v_heads * (a->head_v / 32) > kMaxRows)
    return GDR_ERR_UNSUPPORTED;
  if (tokens > 0) {
    if (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->d_out) return GDR_ERR_INVALID_ARG;
    if (!a->dq || !a->dk || !a->dv || !a->dg || !a->dbeta) return GDR_ERR_INVALID_ARG;
    if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->d_out))
      return GDR_ERR_INVALID_ARG;
  }
  if ((a->initial_state && !aligned16(a->initial_state)) ||
      (a->d_final_state && !aligned16(a->d_final_state)))
    return GDR_ERR_INVALID_ARG;
  if (a->num_seqs > 0) {
    if (a->workspace_bytes < gdr_backward_workspace_bytes(a)) return GDR_ERR_WORKSPACE;
    if (!a->workspace || (reinterpret_cast<uintptr_t>(a->workspace) & (kAlign - 1)) != 0)
      return GDR_ERR_WORKSPACE;
  }
  return GDR_OK;
}

size_t gdr_backward_workspace_bytes(const gdr_backward_args *a) {
  if (!a || a->num_seqs <= 0 || a->batch < 0 || a->seqlen < 0 || a->head_k <= 0 ||
      a->num_v_heads <= 0 || a->num_qk_heads <= 0)
    return 0;
  return bwd_layout(a).total;
}

int gdr_chunk_gated_delta_rule_backward(const gdr_backward_args *a, void *stream) {
  const int st = gdr_validate_backward(a);
  if (st != GDR_OK) return st;
  if (a->num_seqs == 0) return GDR_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const BwdLayout L = bwd_layout(a);
  char *ws = static_cast<char *>(a->workspace);
  const long tokens = static_cast<long>(a->batch) * a->seqlen;

  gdr::BackwardParams p{};
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.g = a->g;
  p.beta = a->beta;
  p.cu_seqlens = a->cu_seqlens;
  p.initial_state = a->initial_state;
  p.d_out = a->d_out;
  p.d_final_state = a->d_final_state;
  p.dq = a->dq;
  p.dk = a->dk;
  p.dv = a->dv;
  p.dg = a->dg;
  p.dbeta = a->dbeta;
  p.d_initial_state = a->d_initial_state;
  p.seqlen = a->seqlen;
  p.num_seqs = a->num_seqs;
  p.Hk = a->num_qk_heads;
  p.Hv = a->num_v_heads;
  p.scale = isnan(a->scale) ? 1.0f / sqrtf(static_cast<float>(a->head_k)) : a->scale;
  p.cb = reinterpret_cast<int32_t *>(ws + L.tab);
  p.bb = p.cb + (a->num_seqs + 1);
  p.states = reinterpret_cast<float *>(ws + L.states);
  p.dhn = reinterpret_cast<float *>(ws + L.dhn);
  p.araw = reinterpret_cast<float *>(ws + L.araw);
  p.pmat = reinterpret_cast<float *>(ws + L.pmat);
  p.tmat = reinterpret_cast<float *>(ws + L.tmat);
  p.dmat = reinterpret_cast<float *>(ws + L.dmat);
  p.drmat = reinterpret_cast<float *>(ws + L.drmat);
  p.dq_h = reinterpret_cast<float *>(ws + L.dqh);
  p.dk_h = reinterpret_cast<float *>(ws + L.dkh);
  p.tokens = tokens;
  p.nh = a->num_householder;
  if (a->use_qk_l2norm) {
    // the backward kernels read the normalised copies; the raw inputs serve the
    // chain rule through the norm
    p.q_raw = a->q;
    p.k_raw = a->k;
    p.q = ws + L.qn;
    p.k = ws + L.kn;
  }
  if (a->gate_mode) {
    p.alpha_raw = a->g;
    p.b_raw = a->beta;
    p.A_log = a->A_log;
    p.dt_bias = a->dt_bias;
    p.dA_log = a->dA_log;
    p.ddt_bias = a->ddt_bias;
    p.g = reinterpret_cast<const float *>(ws + L.gg);
    p.beta = reinterpret_cast<const float *>(ws + L.gb);
  }
  const int f32 = a->qkv_dtype == GDR_DTYPE_F32;

  if (gdr::launch_backward_table(p, s) != hipSuccess) return GDR_ERR_HIP;
  if (gdr::launch_backward_prologue(p, f32, a->head_k, s) != hipSuccess) return GDR_ERR_HIP;
  if (tokens > 0) {
    // forward recompute: the state after every 64 rows of each sequence (long
    // batched rows run in segments with their workspace); its outputs are not needed,
    // so the kernels write none (the checks see a stand-in for them)
    gdr_prefill_args f = bwd_forward_args(a);
    f.q = a->q;
    f.k = a->k;
    f.v = a->v;
    f.g = a->g;
    f.beta = a->beta;
    f.initial_state = a->initial_state;
    f.out = const_cast<void *>(a->d_out);   // a stand-in for the checks only
    f.boundary_states = p.states;
    const int fv = gdr_validate_prefill(&f);
    if (fv != GDR_OK) return fv;
    f.out = nullptr;
    const int fs = enqueue_prefill(&f, s, L.fwd_bytes ? ws + L.fwd : nullptr, L.fwd_bytes);
    if (fs != GDR_OK) return fs;
  }
  if (gdr::launch_backward(p, f32, a->head_k, L.max_chunks, tokens, s) != hipSuccess)
    return GDR_ERR_HIP;
  const hipError_t e = gdr::launch_backward_epilogue(p, f32, a->head_k, s);
  return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

int gdr_validate_conv_prefill(const gdr_conv_prefill_args *a) {
  if (!a) return GDR_ERR_INVALID_ARG;
  if (a->tokens < 0 || a->num_seqs < 1 || a->channels <= 0 || a->channels % 4 != 0)
    return GDR_ERR_INVALID_ARG;
  if (!dtype_ok(a->dtype) || (a->activation != 0 && a->activation != 1))
    return GDR_ERR_INVALID_ARG;
  if (a->width < 2 || a->width > 4) return GDR_ERR_UNSUPPORTED;
  if (int64_t{a->tokens} * a->channels >= (int64_t{1} << 40)) return GDR_ERR_UNSUPPORTED;
  if (!a->weight || !a->cu_seqlens) return GDR_ERR_INVALID_ARG;
  if (a->tokens > 0 && (!a->x || !a->out || !aligned16(a->x) || !aligned16(a->out)))
    return GDR_ERR_INVALID_ARG;
  if (a->state_indices && (!a->conv_state || a->num_slots <= 0)) return GDR_ERR_INVALID_ARG;
  return GDR_OK;
}

int gdr_validate_conv_decode(const gdr_conv_decode_args *a) {
  if (!a) return GDR_ERR_INVALID_ARG;
  if (a->batch < 0 || a->num_tokens < 1 || a->channels <= 0 || a->channels % 4 != 0)
    return GDR_ERR_INVALID_ARG;
  if (!dtype_ok(a->dtype) || (a->activation != 0 && a->activation != 1))
    return GDR_ERR_INVALID_ARG;
  if (a->width < 2 || a->width > 4) return GDR_ERR_UNSUPPORTED;
  if (a->batch > 0) {
    if (!a->x || !a->out || !a->weight || !a->conv_state || a->num_slots <= 0)
      return GDR_ERR_INVALID_ARG;
    if (!aligned16(a->x) || !aligned16(a->out)) return GDR_ERR_INVALID_ARG;
    if (!a->batch_indices && a->batch > a->num_slots) return GDR_ERR_INVALID_ARG;
    if (int64_t{a->batch} * a->num_tokens * a->channels >= (int64_t{1} << 40))
      return GDR_ERR_UNSUPPORTED;
  }
  return GDR_OK;
}

int gdr_validate_gated_rmsnorm(const gdr_gated_rmsnorm_args *a) {
  if (!a) return GDR_ERR_INVALID_ARG;
  if (a->tokens < 0 || a->heads <= 0 || !dtype_ok(a->dtype)) return GDR_ERR_INVALID_ARG;
  if (a->norm_before_gate != 0 && a->norm_before_gate != 1) return GDR_ERR_INVALID_ARG;
  if (!(a->eps >= 0.0f) || isinf(a->eps)) return GDR_ERR_INVALID_ARG;
  if (a->group != 64 && a->group != 128 && a->group != 256) return GDR_ERR_UNSUPPORTED;
  if (a->tokens > 0) {
    if (!a->x || !a->z || !a->weight || !a->out) return GDR_ERR_INVALID_ARG;
    if (!aligned16(a->x) || !aligned16(a->z) || !aligned16(a->out) || !aligned16(a->weight))
      return GDR_ERR_INVALID_ARG;
  }
  return GDR_OK;
}

int gdr_causal_conv1d_prefill(const gdr_conv_prefill_args *a, void *stream) {
  const int st = gdr_validate_conv_prefill(a);
  if (st != GDR_OK) return st;
  gdr::ConvParams p{};
  p.x = a->x;
  p.weight = a->weight;
  p.bias = a->bias;
  p.cu_seqlens = a->cu_seqlens;
  p.state_indices = a->state_indices;
  p.conv_state = a->conv_state;
  p.out = a->out;
  p.tokens = a->tokens;
  p.num_seqs = a->num_seqs;
  p.C = a->channels;
  p.W = a->width;
  p.activation = a->activation;
  const hipError_t e = gdr::launch_conv(p, a->dtype == GDR_DTYPE_F32, 0,
                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

int gdr_causal_conv1d_decode(const gdr_conv_decode_args *a, void *stream) {
  const int st = gdr_validate_conv_decode(a);
  if (st != GDR_OK) return st;
  if (a->batch == 0) return GDR_OK;
  gdr::ConvParams p{};
  p.x = a->x;
  p.weight = a->weight;
  p.bias = a->bias;
  p.state_indices = a->batch_indices;
  p.conv_state = a->conv_state;
  p.intermediate_state = a->intermediate_state;
  p.out = a->out;
  p.batch = a->batch;
  p.num_tokens = a->num_tokens;
  p.C = a->channels;
  p.W = a->width;
  p.activation = a->activation;
  const hipError_t e = gdr::launch_conv(p, a->dtype == GDR_DTYPE_F32, 1,
                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

int gdr_gated_rmsnorm(const gdr_gated_rmsnorm_args *a, void *stream) {
  const int st = gdr_validate_gated_rmsnorm(a);
  if (st != GDR_OK) return st;
  gdr::NormParams p{};
  p.x = a->x;
  p.z = a->z;
  p.weight = a->weight;
  p.out = a->out;
  p.rows = static_cast<long>(a->tokens) * a->heads;
  p.heads = a->heads;
  p.group = a->group;
  p.norm_before_gate = a->norm_before_gate;
  p.eps = a->eps;
  const hipError_t e = gdr::launch_gated_rmsnorm(p, a->dtype == GDR_DTYPE_F32,
                                                 static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

}  // extern "C"
