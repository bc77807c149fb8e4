// Internal launch interface between the host API (gdr_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

struct PrefillParams {
  const void *q;
  const void *k;
  const void *v;                 // NULL: values read as zero
  const float *g;
  const float *beta;
  const int32_t *cu_seqlens;     // NULL: batched, sequence n = tokens [n*seqlen, (n+1)*seqlen)
  const int32_t *state_indices;  // NULL: dense states
  const float *initial_state;    // NULL: zeros
  float *final_state;            // NULL: not written
  void *out;                     // NULL: outputs not written
  int seqlen;
  int num_seqs;
  int Hk;
  int Hv;
  int DV;
  int num_vtiles;                // DV / value columns per workgroup
  int group_size;                // work items sharing one (sequence, q/k head)
  int num_groups;                // num_seqs * Hk
  int l2norm;
  int out_bf16;
  float scale;
  int gate_mode;                 // 1: g, beta hold raw projections (gates computed here)
  const float *A_log;            // [Hv] (gate_mode 1)
  const float *dt_bias;          // [Hv] (gate_mode 1)
  float *boundary_states;        // NULL, or [entries, Hv, K, V]
  int boundary_interval;         // tokens between boundary states
};

struct DecodeParams {
  const void *q;
  const void *k;
  const void *v;
  const float *g;
  const float *beta;
  float *state;
  const int32_t *batch_indices;  // NULL: request i uses slot i
  void *out;
  int batch;
  int Hk;
  int Hv;
  int l2norm;
  int out_bf16;
  float scale;
  int gate_mode;
  const float *A_log;
  const float *dt_bias;
  int num_tokens;                // tokens per request (>= 1)
  float *intermediate_state;     // NULL, or [batch, num_tokens, Hv, K, V]
};

struct ConvParams {
  const void *x;                 // [tokens, C] (prefill) or [batch, num_tokens, C] (decode)
  const float *weight;           // [C, W]
  const float *bias;             // [C] or NULL
  const int32_t *cu_seqlens;     // prefill: [num_seqs + 1]
  const int32_t *state_indices;  // prefill: per sequence; decode: per request; NULL: identity
  float *conv_state;             // [rows, C, W - 1] or NULL (prefill only)
  float *intermediate_state;     // decode: [batch, num_tokens, C, W - 1] or NULL
  void *out;
  int tokens;
  int num_seqs;
  int batch;
  int num_tokens;
  int C;
  int W;
  int activation;                // 0: none, 1: SiLU
};

struct NormParams {
  const void *x;                 // [rows, group]
  const void *z;                 // [rows, group]
  const float *weight;           // [heads * group]
  void *out;
  long rows;                     // tokens * heads
  int heads;
  int group;
  int norm_before_gate;
  float eps;
};

struct BackwardParams {
  const void *q;                 // [Tt, Hk, D]
  const void *k;                 // [Tt * n_h, Hk, D]
  const void *v;                 // [Tt * n_h, Hv, D]
  const float *g;                // [Tt, Hv]
  const float *beta;             // [Tt * n_h, Hv]
  const int32_t *cu_seqlens;     // NULL: batched
  const float *initial_state;    // [N, Hv, D, D] or NULL (zeros)
  const void *d_out;             // [Tt, Hv, D], q's dtype
  const float *d_final_state;    // [N, Hv, D, D] or NULL (zeros)
  float *dq;                     // [Tt, Hk, D]
  float *dk;                     // [Tt * n_h, Hk, D]
  float *dv;                     // [Tt * n_h, Hv, D]
  float *dg;                     // [Tt, Hv]
  float *dbeta;                  // [Tt * n_h, Hv]
  float *d_initial_state;        // [N, Hv, D, D] or NULL (not written)
  int seqlen;
  int num_seqs;
  int Hk;
  int Hv;
  float scale;
  // workspace
  int32_t *cb;                   // [N + 1] first chunk of each sequence
  int32_t *bb;                   // [N + 1] first boundary state of each sequence
  float *states;                 // [E, Hv, D, D] forward state after every 64 tokens
  float *dhn;                    // [chunks, Hv, D, D] gradient of the state leaving a chunk
  float *araw;                   // [chunks, Hv, 64, 64] strict_lower((K K^T) * Gamma)
  float *pmat;                   // [chunks, Hv, 64, 64] scale (Q K^T) * Gamma, causal
  float *tmat;                   // [chunks, Hv, 64, 64] (I + A)^-1
  float *dmat;                   // [chunks, Hv, 64, D] D = T R
  float *drmat;                  // [chunks, Hv, 64, D] dR = T^T dD
  float *dq_h;                   // [Tt, Hv, D] per value head (grouped heads only)
  float *dk_h;                   // [Tt * n_h, Hv, D]
  // in-kernel L2 norm: q, k above point at the normalised fp32 copies, these at the
  // raw inputs (NULL without the norm)
  const void *q_raw;
  const void *k_raw;
  // gates formed from raw projections: g, beta above point at the formed gates,
  // these at the projections and per-head parameters (NULL in gate mode 0)
  const float *alpha_raw;        // [Tt, Hv]
  const float *b_raw;            // [Tt, Hv]
  const float *A_log;            // [Hv]
  const float *dt_bias;          // [Hv]
  float *dA_log;                 // [Hv]
  float *ddt_bias;               // [Hv]
  long tokens;
  int nh;                        // Householder sub-steps per token (rows per token)
};

// Segments of long sequences (the prefill's workspace).
//  * Batched rows (src_cu NULL): segment s of batch row b covers tokens
//    [s * seg_len, min((s + 1) * seg_len, seqlen)) and is packed sequence b * S + s of
//    the internal passes.
//  * Packed sequences (src_cu = the caller's cu_seqlens): the S segment slots are
//    planned on the device; sequence n owns slots first[n] .. first[n+1]-1, each of
//    seg_len tokens but its last (every sequence at least one, possibly empty); the
//    slots past the last sequence's are empty segments at the end of the tokens.
struct SegmentParams {
  int batch;                     // batch rows, or packed sequences
  int seqlen;
  int S;                         // segments per batch row; segment slots when packed
  int seg_len;                   // tokens per segment (a multiple of 64)
  int Hv;
  int DK;
  int DV;
  int32_t *cu;                   // [batch * S + 1] (packed: [S + 1])
  float *ident;                  // [segments, Hv, DK, DK] identity states
  const float *F;                // [segments, Hv, DK, DV] final states from zero
  const float *A;                // [segments, Hv, DK, DK] transitions
  const float *initial_state;    // [batch, Hv, DK, DV], a slot cache, or NULL
  float *H_in;                   // [segments, Hv, DK, DV] entering states
  float *final_state;            // [batch, Hv, DK, DV], a slot cache, or NULL
  const int32_t *src_cu;         // packed: [batch + 1] the caller's cu_seqlens
  int32_t *first;                // packed: [batch + 1] first segment slot of each sequence
  const int32_t *state_indices;  // packed: slot of each sequence (NULL: dense states)
};
hipError_t launch_segment_setup(const SegmentParams &p, hipStream_t stream);
hipError_t launch_segment_combine(const SegmentParams &p, hipStream_t stream);

// Whether a prefill kernel is instantiated for this launch shape (host only).
bool prefill_variant_exists(int qkv_f32, int head_k, int rows, int nh, int ns);
// Rows per chunk the prefill kernels run for a requested chunk size (tokens).
int prefill_chunk_rows(int chunk_size, int nh, int qkv_f32, int head_k);
// State waves (32 value columns each) per prefill workgroup.
int prefill_state_waves(int head_v, int num_seqs, int num_v_heads);

hipError_t launch_prefill(const PrefillParams &p, int qkv_f32, int head_k, int rows, int nh,
                          int state_waves, hipStream_t stream);
// 64-row chunks of bf16 inputs (launched by launch_prefill)
hipError_t launch_prefill64(const PrefillParams &p, int head_k, int nh, int state_waves, int grid,
                            hipStream_t stream);
hipError_t launch_decode(const DecodeParams &p, int qkv_f32, int dk, int dv, int nh,
                         hipStream_t stream);
// mode 0: prefill (outputs, then conv states); mode 1: decode
hipError_t launch_conv(const ConvParams &p, int f32, int mode, hipStream_t stream);
hipError_t launch_gated_rmsnorm(const NormParams &p, int f32, hipStream_t stream);
// the chunk table of the backward, then its kernels (after the forward recompute)
hipError_t launch_backward_table(const BackwardParams &p, hipStream_t stream);
hipError_t launch_backward(const BackwardParams &p, int qkv_f32, int head, int max_chunks,
                           long tokens, hipStream_t stream);
// the normalised q, k and the formed gates the backward kernels read (before the
// forward recompute), and the chain rule through both (after the backward kernels)
hipError_t launch_backward_prologue(const BackwardParams &p, int qkv_f32, int head,
                                    hipStream_t stream);
hipError_t launch_backward_epilogue(const BackwardParams &p, int qkv_f32, int head,
                                    hipStream_t stream);

}  // namespace gdr
