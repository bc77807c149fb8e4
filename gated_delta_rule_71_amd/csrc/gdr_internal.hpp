// Internal launch interface between the host API (gdr_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

struct PrefillParams {
  const void *q;
  const void *k;
  const void *v;
  const float *g;
  const float *beta;
  const int32_t *cu_seqlens;     // NULL: batched, sequence n = tokens [n*seqlen, (n+1)*seqlen)
  const int32_t *state_indices;  // NULL: dense states
  const float *initial_state;    // NULL: zeros
  float *final_state;            // NULL: not written
  void *out;
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

// Rows per chunk the prefill kernels run for a requested chunk size (tokens).
int prefill_chunk_rows(int chunk_size, int nh, int qkv_f32, int head_k);
// State waves (32 value columns each) per prefill workgroup.
int prefill_state_waves(int head_v, int num_seqs, int num_v_heads);

hipError_t launch_prefill(const PrefillParams &p, int qkv_f32, int head_k, int rows, int nh,
                          int state_waves, hipStream_t stream);
hipError_t launch_decode(const DecodeParams &p, int qkv_f32, int dk, int dv, int nh,
                         hipStream_t stream);

}  // namespace gdr
