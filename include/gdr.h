/*
 * gdr.h — C ABI of the MI355X (gfx950) gated delta rule library (libgdr.so).
 *
 * The library computes the gated delta rule
 *
 *     S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = scale S_t q_t,
 *
 * the recurrence of Megatron Core's Gated DeltaNet (API page
 * "core.ssm.gated_delta_net.gdn", function torch_chunk_gated_delta_rule) and,
 * with several Householder sub-steps per token, of its Gated Delta Product
 * mixer (API page "core.ssm.gated_delta_product", class GatedDeltaProductMixer).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor arguments are DEVICE pointers to row-major arrays whose innermost
 *    dimension is contiguous; base addresses must be 16-byte aligned.
 *  - The state S of one (sequence, value head) is stored as a [K, V] float32
 *    matrix holding S transposed: element [i][j] is S[j][i].
 *  - Value head h reads query/key head floor(h * Hk / Hv) (Hv a multiple of Hk).
 *  - q/k/v share one input dtype; g, beta and all states are float32.
 *  - Gates (gate_mode): with gate_mode 0 the g and beta arguments hold the gates
 *    themselves, the per-token log-decay g_t and the write strength beta_t.  With
 *    gate_mode 1 they hold the raw per-token projections the gates are computed
 *    from inside the kernels (the "alpha" and "beta" outputs of the fused input
 *    projection, GatedDeltaNet.forward_pre_attn_and_core_attn and
 *    _prepare_inference_inputs on page "core.ssm.gated_delta_net.gdn", which leave
 *    the gates to the kernel), together with the per-value-head parameters A_log
 *    and dt_bias of GatedDeltaNet._compute_gates:
 *        g_t    = -exp(A_log[h]) * softplus(alpha_t + dt_bias[h]),
 *        beta_t = sigmoid(b_t),      softplus(x) = log(1 + exp(x)).
 *    The pages name the parameters (A_log, dt_bias; A_init_range, dt_min, dt_max
 *    on page "core.ssm.gated_delta_product") but print no formula; this is the
 *    decay parametrisation those names denote (A = exp(A_log) > 0 times a
 *    softplus time step).  The gates are evaluated in float32 (the library's
 *    expf / log1pf; softplus split at 0 so that exp never overflows).
 *  - Calls only enqueue work on `stream` (a hipStream_t passed as void*; NULL is
 *    the default stream).  They never allocate, free or synchronise, keep no
 *    mutable global state, and their launch shapes depend only on the sizes in
 *    the argument struct, so they can be captured in a HIP graph.
 *  - Errors: arguments are checked on the host before anything is launched; on
 *    any error nothing is enqueued and no buffer is touched.  Preconditions on
 *    device-resident data (monotone cu_seqlens, 0 <= index < num_slots, unique
 *    non-negative indices, value ranges below) are documented, not checked:
 *    checking them would need a device synchronisation.  Violating them gives
 *    undefined results.
 *  - Value range of bf16 inputs: the prefill's matrix-core products take fp16
 *    operands.  q, k (after the optional L2 norm) and v, the state, and the
 *    in-kernel per-chunk values (the inverse T, the decayed scores P and the
 *    deltas D = T beta (v - exp(G) k^T S)) are rounded to fp16 there, so every
 *    such entry must stay below 65504 in magnitude (larger ones overflow to
 *    infinity); bf16 entries below 2^-14 become fp16 subnormals and keep fewer
 *    significant bits.  Unit-norm keys, states of moderate size and values of
 *    order one are far inside this range.  F32 inputs use fp32 operands
 *    throughout and have no such limit.
 */
#ifndef GDR_H
#define GDR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDR_ABI_VERSION 4

/* Status codes returned by every entry point. */
typedef enum {
  GDR_OK = 0,
  GDR_ERR_INVALID_ARG = 1, /* NULL where a pointer is required, bad size, misaligned */
  GDR_ERR_UNSUPPORTED = 2, /* valid but not implemented (head size, dtype, n_h, ...) */
  GDR_ERR_WORKSPACE = 3,   /* workspace smaller than gdr_backward_workspace_bytes()  */
  GDR_ERR_HIP = 4          /* the HIP runtime reported a launch error                 */
} gdr_status;

/* Element types of q/k/v and of the output. */
typedef enum { GDR_DTYPE_F32 = 0, GDR_DTYPE_BF16 = 1 } gdr_dtype;

/*
 * Chunked prefill over packed or batched sequences.  Mirrors
 * torch_chunk_gated_delta_rule(q, k, v, g, beta, scale=None, chunk_size=64,
 * initial_state=None, output_final_state=False, use_qk_l2norm_in_kernel=False,
 * cu_seqlens=None) -> (o, final_state) (page "core.ssm.gated_delta_net.gdn"),
 * with the slot-indexed state of ssm_prefill (page "core.ssm.gated_delta_product":
 * each request enters with whatever its cache slot holds and writes the slot back;
 * padding requests carry slot -1).
 *
 * Shapes (Tt = batch * seqlen tokens; with cu_seqlens, batch must be 1):
 *   q    [Tt, Hk, K]            k    [Tt, n_h, Hk, K]     v [Tt, n_h, Hv, V]
 *   g    [Tt, Hv]   float32     beta [Tt, n_h, Hv] float32
 *   out  [Tt, Hv, V]  (out_dtype)
 *   cu_seqlens    int32 [num_seqs + 1] or NULL.  NULL: num_seqs = batch and
 *                 sequence n is tokens [n*seqlen, (n+1)*seqlen).
 *   state_indices int32 [num_seqs] or NULL.
 *     NULL:  sequence n starts from initial_state[n] ([num_seqs, Hv, K, V]; NULL
 *            means zeros) and, if final_state != NULL, ends in final_state[n].
 *     given: initial_state and final_state are slot caches [num_slots, Hv, K, V]
 *            (usually the same pointer).  Sequence n reads slot max(idx, 0)
 *            (zeros if initial_state is NULL) and writes slot idx only when
 *            idx >= 0; -1 marks padding.  Slots no sequence writes are left
 *            byte-identical.
 *   final_state may equal initial_state (in place).
 *
 * scale: NaN selects the default 1/sqrt(K).
 * use_qk_l2norm: nonzero divides each q and k row by sqrt(sum x^2 + 1e-6).
 * num_householder: n_h (1 = gated delta rule; 2 = gated delta product with two
 *   Householder sub-steps per token; the decay exp(g_t) is applied once per
 *   token, before the first sub-step, and o_t is read after the last one).
 * chunk_size: tokens per chunk, a power of two in [16, 256].  Chunking does not
 *   change the result beyond rounding; the kernels evaluate chunks of
 *   min(chunk_size * n_h, 32) rows (16 rows for float32 inputs with K = 128).
 * boundary_states (optional, for prefix caching; the per-chunk states of page
 *   "core.ssm.gated_delta_product", ssm_prefill): the state of every sequence
 *   after each whole multiple of boundary_interval tokens from its start
 *   (boundary_interval * n_h a positive multiple of 64).
 *   Sequence n of L_n tokens writes floor(L_n / boundary_interval) entries, at
 *   rows off_n + j, off_n = sum over m < n of floor(L_m / boundary_interval);
 *   entry j holds the state after the sequence's first (j + 1) * boundary_interval
 *   tokens, in the [K, V] layout of final states.  E = sum of the counts.  Every
 *   sequence writes its entries, padding sequences (state index -1) included.
 * Supported: K in {64, 128}, V in {64, 128}, n_h in {1, 2}, q/k/v F32 or BF16,
 *   except n_h = 2 with F32 inputs and K = 128 (GDR_ERR_UNSUPPORTED: its chunks do
 *   not fit on chip), out F32 or BF16, Tt * n_h < 2^31 - 1024 rows and
 *   Tt * n_h * max(Hk * K, Hv * V) < 2^32 (element offsets within q, k, v and out
 *   are 32-bit); larger inputs return GDR_ERR_UNSUPPORTED.
 */
typedef struct {
  int32_t batch;            /* B; 1 when cu_seqlens is given                        */
  int32_t seqlen;           /* tokens per batch row (total tokens with cu_seqlens)  */
  int32_t num_seqs;         /* N; must equal batch when cu_seqlens is NULL          */
  int32_t num_qk_heads;     /* Hk                                                   */
  int32_t num_v_heads;      /* Hv                                                   */
  int32_t head_k;           /* K                                                    */
  int32_t head_v;           /* V                                                    */
  int32_t num_householder;  /* n_h                                                  */
  int32_t chunk_size;       /* tokens                                               */
  int32_t qkv_dtype;        /* gdr_dtype                                            */
  int32_t out_dtype;        /* gdr_dtype                                            */
  int32_t use_qk_l2norm;    /* 0 or 1                                               */
  float scale;              /* NaN => 1/sqrt(head_k)                                */
  int32_t num_slots;        /* slot count when state_indices != NULL                */
  const void *q;
  const void *k;
  const void *v;
  const float *g;
  const float *beta;
  const int32_t *cu_seqlens;
  const int32_t *state_indices;
  const float *initial_state;
  float *final_state;
  void *out;
  void *workspace;          /* optional device memory (segment path, below) or NULL */
  size_t workspace_bytes;
  int32_t gate_mode;        /* 0: g, beta are the gates; 1: raw projections (above) */
  const float *A_log;       /* [Hv] float32, gate_mode 1 only (else ignored)        */
  const float *dt_bias;     /* [Hv] float32, gate_mode 1 only (else ignored)        */
  float *boundary_states;   /* [E, Hv, K, V] float32 or NULL (below)                */
  int32_t boundary_interval; /* tokens, times n_h a multiple of 64 (boundary_states)*/
} gdr_prefill_args;

/*
 * Single-token decode over a slot-indexed float32 state cache, updated in place.
 * Mirrors ssm_decode (pages "core.ssm.gated_delta_net.gdn" and
 * "core.ssm.gated_delta_product") and the padding rule of PR "Add GDN dynamic
 * inference #6499" (review thread): batch_indices[i] = -1 marks padding; its
 * read is clamped to slot 0 and its write is skipped, so its output is the
 * step computed from slot 0 (meaningless if slot 0 is written in the same call).
 * batch_indices NULL means static batching: request i uses slot i.
 *
 * Shapes (T = num_tokens tokens per request, 1 for the single-token step):
 *   q [n, T, Hk, K]; k [n, T, n_h, Hk, K]; v [n, T, n_h, Hv, V]; g [n, T, Hv]
 *   float32; beta [n, T, n_h, Hv] float32; state [num_slots, Hv, K, V] float32;
 *   batch_indices int32 [n] or NULL; out [n, T, Hv, V] (out_dtype).
 * Several tokens per request (the [n, seq_len, ...] form of ssm_decode on page
 *   "core.ssm.gated_delta_product", e.g. speculative tokens) advance the state
 *   token by token: the slot is read once, the T steps run in registers, and the
 *   slot is written once at the end.  intermediate_state ([n, T, Hv, K, V]
 *   float32, or NULL; the intermediate_ssm_state argument of ssm_decode) then
 *   receives the state after each token.  A padding request evolves its copy of
 *   slot 0 privately and writes neither the slot nor intermediate states.
 * Supported: K = 128 or 64, V = 128 or 64, n_h in {1, 2}, 1 <= T <= 2^16.
 */
typedef struct {
  int32_t batch;            /* n requests                                           */
  int32_t num_qk_heads;
  int32_t num_v_heads;
  int32_t head_k;
  int32_t head_v;
  int32_t num_householder;
  int32_t num_slots;
  int32_t qkv_dtype;
  int32_t out_dtype;
  int32_t use_qk_l2norm;
  float scale;              /* NaN => 1/sqrt(head_k)                                */
  const void *q;
  const void *k;
  const void *v;
  const float *g;
  const float *beta;
  float *state;
  const int32_t *batch_indices;
  void *out;
  int32_t gate_mode;        /* 0: g, beta are the gates; 1: raw projections (above) */
  const float *A_log;       /* [Hv] float32, gate_mode 1 only (else ignored)        */
  const float *dt_bias;     /* [Hv] float32, gate_mode 1 only (else ignored)        */
  int32_t num_tokens;       /* T >= 1 tokens per request                            */
  float *intermediate_state; /* [n, T, Hv, K, V] float32 or NULL                    */
} gdr_decode_args;

/*
 * Short depthwise causal convolution over a packed token stream (the conv on the
 * V/K/Q projection before the recurrence: GatedDeltaProductMixer d_conv = 4 and
 * _prepare_qkv with conv_initial_states on page "core.ssm.gated_delta_product").
 *
 *   y[t][c] = act(bias[c] + sum_{j<W} weight[c][j] * x[t - (W-1) + j][c])
 *
 * where inputs before a sequence's first token come from its conv state: row
 * [c][0 .. W-2] holds the W-1 inputs preceding the sequence, oldest first (zeros
 * when conv_state is NULL).  act is SiLU (activation = 1) or the identity (0);
 * the pages do not name the activation, and SiLU is the one of the Mamba-style
 * conv these layers use.
 * Prefill (gdr_causal_conv1d_prefill): x, out [tokens, C]; cu_seqlens int32
 *   [num_seqs + 1] (required; one sequence = [0, tokens]); conv_state float32
 *   [rows, C, W-1] or NULL, addressed by state_indices[n] (NULL: row n); -1 marks
 *   padding: it reads row 0 and writes nothing.  After the outputs, each sequence's
 *   row receives its last W-1 inputs (from the old row when the sequence is
 *   shorter than W-1), in place.  Rows must be distinct across sequences.
 * Decode (gdr_causal_conv1d_decode, _decode_conv): x, out [batch, num_tokens, C];
 *   conv_state [num_slots, C, W-1] in place, row batch_indices[i] (NULL: i; -1:
 *   padding reads row 0, writes nothing); intermediate_state [batch, num_tokens,
 *   C, W-1] float32 or NULL receives the window after each token.
 * Supported: C a multiple of 4, W in {2, 3, 4}, x/out F32 or BF16 (one dtype).
 */
typedef struct {
  int32_t tokens;             /* packed tokens                                     */
  int32_t num_seqs;
  int32_t channels;           /* C                                                 */
  int32_t width;              /* W                                                 */
  int32_t dtype;              /* gdr_dtype of x and out                            */
  int32_t activation;         /* 1: SiLU, 0: none                                  */
  int32_t num_slots;          /* rows of conv_state when state_indices is given    */
  const void *x;
  const float *weight;        /* [C, W]                                            */
  const float *bias;          /* [C] or NULL                                       */
  const int32_t *cu_seqlens;
  const int32_t *state_indices;
  float *conv_state;
  void *out;
} gdr_conv_prefill_args;

typedef struct {
  int32_t batch;              /* requests                                          */
  int32_t num_tokens;         /* tokens per request (>= 1)                         */
  int32_t channels;
  int32_t width;
  int32_t dtype;
  int32_t activation;
  int32_t num_slots;
  const void *x;
  const float *weight;
  const float *bias;
  const int32_t *batch_indices;
  float *conv_state;          /* [num_slots, C, W-1], in place                     */
  float *intermediate_state;  /* [batch, num_tokens, C, W-1] or NULL               */
  void *out;
} gdr_conv_decode_args;

/*
 * Gated RMS normalisation of the recurrence output (ExtendedRMSNorm, an
 * RMSNormGated, page "core.ssm.gated_delta_product"; norm_before_gate as in
 * GatedDeltaProductMixer).  For each token and head, over the group of `group`
 * elements:
 *   norm_before_gate = 0:  u = x * silu(z),  y = u / sqrt(mean(u^2) + eps) * w
 *   norm_before_gate = 1:  y = x / sqrt(mean(x^2) + eps) * w * silu(z)
 * x, z, out [tokens, heads, group] (one dtype, F32 or BF16); weight float32
 * [heads * group].  Supported: group in {64, 128, 256}.
 */
typedef struct {
  int32_t tokens;
  int32_t heads;
  int32_t group;
  int32_t dtype;
  int32_t norm_before_gate;
  float eps;
  const void *x;
  const void *z;
  const float *weight;
  void *out;
} gdr_gated_rmsnorm_args;

/*
 * Chunked backward of the gated delta rule (training through
 * torch_chunk_gated_delta_rule, page "core.ssm.gated_delta_net.gdn"; the chunked
 * training kernels of the Gated DeltaNet and Gated Delta Product pages).  Given
 * d_out = dL/do and d_final_state = dL/dS_T of some loss L of the forward call
 * with the same inputs, writes dL/dq, dL/dk, dL/dv, dL/dg, dL/dbeta and
 * dL/d(initial_state).  The forward states every 64 tokens are recomputed inside
 * the call (into the workspace), so nothing from the forward call is needed.
 *
 * Shapes (Tt = batch * seqlen tokens; with cu_seqlens, batch must be 1; n_h =
 * num_householder sub-steps per token, 1 for the gated delta rule, 2 for the
 * gated delta product as in the prefill):
 *   q [Tt, Hk, D]; k [Tt, n_h, Hk, D]; v [Tt, n_h, Hv, D]; d_out [Tt, Hv, D]
 *   (qkv_dtype, one dtype for all four); g [Tt, Hv] and beta [Tt, n_h, Hv]
 *   float32; initial_state, d_final_state [N, Hv, D, D] float32 (the [K, V]
 *   layout of states) or NULL (zeros);
 *   outputs, all float32, shaped like their inputs: dq, dk (a q/k head receives
 *   the sum over the value heads that read it), dv, dg, dbeta, and
 *   d_initial_state [N, Hv, D, D] or NULL (not written).
 * use_qk_l2norm = 1: the forward divided q and k by sqrt(sum x^2 + 1e-6) (the
 *   in-kernel norm of the prefill); dq, dk are the gradients of the raw q, k.
 * gate_mode = 1: g and beta hold the raw projections alpha and b, and A_log,
 *   dt_bias [Hv] the per-head parameters, as in the prefill (gates formed in the
 *   kernels); dg and dbeta then receive dL/dalpha and dL/db, and dA_log, ddt_bias
 *   ([Hv] float32, required) receive dL/dA_log and dL/ddt_bias (sums over all
 *   tokens in a fixed order).  gate_mode = 0: dg, dbeta are the gradients of the
 *   gate values given.
 * Workspace: gdr_backward_workspace_bytes(args) bytes of device memory, 256-byte
 *   aligned, owned by the caller; its contents on entry do not matter.  It holds
 *   per 64-token chunk and value head the entering state, the gradient of the
 *   leaving state and four 64 x 64 or 64 x D float32 matrices (about
 *   2 D^2 + 3 * 64^2 + 64 D floats, 176 KiB at D = 128; one more 64 x D matrix
 *   with F32 inputs or use_qk_l2norm), plus float32 copies of the normalised q, k
 *   (use_qk_l2norm) and of the formed gates (gate_mode 1).
 * Supported: head_k == head_v = D in {64, 128}; q/k/v/d_out F32 or BF16;
 *   n_h in {1, 2} (n_h = 2 with F32 inputs only at D = 64, as in the prefill).
 * The outputs must not alias the inputs or the workspace.
 */
typedef struct {
  int32_t batch;
  int32_t seqlen;
  int32_t num_seqs;
  int32_t num_qk_heads;     /* Hk                                                   */
  int32_t num_v_heads;      /* Hv                                                   */
  int32_t head_k;           /* D                                                    */
  int32_t head_v;           /* must equal head_k                                    */
  int32_t qkv_dtype;        /* gdr_dtype of q, k, v and d_out                       */
  float scale;              /* NaN => 1/sqrt(head_k)                                */
  const void *q;
  const void *k;
  const void *v;
  const float *g;
  const float *beta;
  const int32_t *cu_seqlens;
  const float *initial_state;
  const void *d_out;
  const float *d_final_state;
  float *dq;
  float *dk;
  float *dv;
  float *dg;
  float *dbeta;
  float *d_initial_state;
  void *workspace;
  size_t workspace_bytes;
  int32_t use_qk_l2norm;    /* 0 or 1                                               */
  int32_t gate_mode;        /* 0: g, beta are the gates; 1: raw projections         */
  const float *A_log;       /* [Hv], gate_mode 1                                    */
  const float *dt_bias;     /* [Hv], gate_mode 1                                    */
  float *dA_log;            /* [Hv] output, gate_mode 1                             */
  float *ddt_bias;          /* [Hv] output, gate_mode 1                             */
  int32_t num_householder;  /* n_h: 1 or 2                                          */
} gdr_backward_args;

/* Version of this ABI (GDR_ABI_VERSION). */
int gdr_abi_version(void);

/* Static, human-readable name of a status code. */
const char *gdr_status_string(int status);

/* Host-only argument checks (no HIP calls; usable without a GPU). */
int gdr_validate_prefill(const gdr_prefill_args *args);
int gdr_validate_decode(const gdr_decode_args *args);

/*
 * Optional device workspace of a prefill, in bytes (a host-only function of the
 * sizes; 256-byte aligned memory owned by the caller, contents irrelevant).  It is
 * nonzero only for long sequences whose (sequence, value head) pairs leave compute
 * units idle: given the workspace, such a call splits every sequence into segments
 * and runs three chunked passes over them (from zero, the transition from the
 * identity with zero values, and from the true entering states, combined in
 * between), which shortens the dependent chain by the segment count.  Without it
 * (NULL or smaller) the single pass runs; both give the same result up to rounding.
 *  - Batched rows (no cu_seqlens, dense states): S = 2^j segments of every row,
 *    each >= 2048 tokens.  Boundary states are allowed when boundary_interval
 *    divides the segment length (checked here: 0 otherwise).
 *  - Packed sequences (cu_seqlens, dense or slot states, no boundary states): the
 *    lengths live on the device, so the plan is sized from the total token count
 *    (seqlen): 256 / Hv segment slots, sequence n taking max(1, ceil(L_n / seg_len))
 *    of them, planned by a device kernel.  Taken when 256 / Hv >= 5 num_seqs and the
 *    segment length is at most seqlen / (4 num_seqs), so that it pays whatever the
 *    lengths.  cu_seqlens must satisfy the documented layout (0 = cu[0] <= ... <=
 *    cu[num_seqs] = seqlen); the device plan clamps its writes to the workspace
 *    whatever the values.
 */
size_t gdr_prefill_workspace_bytes(const gdr_prefill_args *args);

/* Enqueue a prefill / a decode step on `stream` (hipStream_t). */
int gdr_chunk_gated_delta_rule(const gdr_prefill_args *args, void *stream);
int gdr_ssm_decode(const gdr_decode_args *args, void *stream);

/*
 * The prefill for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same call and
 * result as gdr_chunk_gated_delta_rule given the workspace of
 * gdr_prefill_workspace_bytes, with that workspace taken from a scratch array the
 * library holds in device memory instead (args->workspace and workspace_bytes are
 * ignored).  The caller still passes every input and output.
 *  - Limit: the scratch is 64 MiB + 4 KiB per GPU, held from the library's load to
 *    the end of the process.  Every segment plan of the library fits (its segment
 *    count x value heads <= 256); a plan that did not would return
 *    GDR_ERR_WORKSPACE with nothing enqueued.  Calls that need no workspace use no
 *    scratch.
 *  - It calls no allocator.  The first call made with a given device current looks
 *    up that device's scratch address (a runtime query, not a stream operation);
 *    make that first call outside graph capture.  Later calls only enqueue.
 *  - Every call on one GPU shares that GPU's scratch, which keeps the last call's
 *    contents (each call rewrites all it reads, so nothing needs clearing).  Calls
 *    that overlap on one GPU (on different streams, or replays of graphs holding
 *    such calls that run concurrently) race on it: order them on one stream.
 *  - Errors as gdr_chunk_gated_delta_rule, plus GDR_ERR_HIP when the scratch
 *    address cannot be obtained.
 */
int gdr_chunk_gated_delta_rule_noalloc(const gdr_prefill_args *args, void *stream);

/* Host-only checks and enqueue of the causal conv and the gated RMS norm. */
int gdr_validate_conv_prefill(const gdr_conv_prefill_args *args);
int gdr_validate_conv_decode(const gdr_conv_decode_args *args);
int gdr_validate_gated_rmsnorm(const gdr_gated_rmsnorm_args *args);
int gdr_causal_conv1d_prefill(const gdr_conv_prefill_args *args, void *stream);
int gdr_causal_conv1d_decode(const gdr_conv_decode_args *args, void *stream);
int gdr_gated_rmsnorm(const gdr_gated_rmsnorm_args *args, void *stream);

/* Host-only checks, workspace size and enqueue of the chunked backward. */
int gdr_validate_backward(const gdr_backward_args *args);
size_t gdr_backward_workspace_bytes(const gdr_backward_args *args);
int gdr_chunk_gated_delta_rule_backward(const gdr_backward_args *args, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* GDR_H */
