/*
 * CPU oracle for the gated delta rule — TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  The GPU library never links, includes or calls it, and it
 * shares no code with the GPU library.
 *
 * What it computes (plain fp64, one token at a time, no chunking):
 *
 *   The method the pages centre on is the gated delta rule, the recurrence behind
 *   the "torch_chunk_gated_delta_rule" function (Megatron Core API page
 *   "core.ssm.gated_delta_net.gdn", section "torch_chunk_gated_delta_rule") and the
 *   "sequence of Householder updates" of the Gated Delta Product mixer (API page
 *   "core.ssm.gated_delta_product", class "GatedDeltaProductMixer").  For one
 *   sequence and one value head, with a matrix state S of shape V x K:
 *
 *       S_t = exp(g_t) * S_{t-1} * (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *       o_t = scale * S_t q_t
 *
 *   The product S (I - beta k k^T) is evaluated as S - beta (S k) k^T, which is
 *   the same matrix by distributivity and costs O(K V) instead of O(K^2 V).
 *
 *   Gated delta product (num_householder = n_h > 1): per token the decay exp(g_t)
 *   is applied once, before the first Householder sub-step; then sub-steps
 *   j = 0..n_h-1 apply S <- S (I - beta_{t,j} k_{t,j} k_{t,j}^T)
 *   + beta_{t,j} v_{t,j} k_{t,j}^T in index order, and the output is read after
 *   the last sub-step.  At n_h = 1 this is the recurrence above.
 *
 *   Boundary conventions (from the pages' statement of the interface):
 *     - scale: the caller passes it; the Python side turns "None" into
 *       1/sqrt(K) (page "core.ssm.gated_delta_net.gdn", torch_chunk_gated_delta_rule).
 *     - optional q/k L2 normalisation per head row: x / sqrt(sum x^2 + 1e-6)
 *       (the flag "use_qk_l2norm_in_kernel" on the same page; the epsilon is not
 *       stated there and is this library's reading).
 *     - packed variable-length sequences by cumulative token offsets
 *       ("cu_seqlens", same page); every sequence starts from its own state.
 *     - value head h uses query/key head floor(h * Hk / Hv) (grouped heads).
 *     - state arrays are stored [.., Hv, K, V]: element [i][j] holds S[j][i].
 *     - slot-indexed states (page "core.ssm.gated_delta_product", ssm_prefill /
 *       ssm_decode, and PR "Add GDN dynamic inference #6499", review thread on
 *       padding): index -1 marks padding; its read is clamped to slot 0 and its
 *       write is skipped.  All reads see the states as they were before the call.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (no fast-math: IEEE fp64 throughout).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#include "gdr_oracle.h"

/* ---- one recurrence step on S (V x K, row-major S[i*K + j]) ------------------ */

/* S <- a * S * (I - beta k k^T) + beta v k^T, using Sk = S k as scratch. */
static void householder_step(double *S, int64_t K, int64_t V, double a, double beta,
                             const double *k, const double *v, double *Sk) {
  for (int64_t i = 0; i < V; ++i) {
    double acc = 0.0;
    for (int64_t j = 0; j < K; ++j) acc += S[i * K + j] * k[j];
    Sk[i] = acc;
  }
  for (int64_t i = 0; i < V; ++i) {
    for (int64_t j = 0; j < K; ++j) {
      S[i * K + j] = a * (S[i * K + j] - beta * Sk[i] * k[j]) + beta * v[i] * k[j];
    }
  }
}

/* o = scale * S q */
static void read_out(const double *S, int64_t K, int64_t V, double scale,
                     const double *q, double *o) {
  for (int64_t i = 0; i < V; ++i) {
    double acc = 0.0;
    for (int64_t j = 0; j < K; ++j) acc += S[i * K + j] * q[j];
    o[i] = scale * acc;
  }
}

/* x / sqrt(sum x^2 + 1e-6), or a plain copy when the flag is off. */
static void maybe_l2norm(const double *x, int64_t n, int on, double *y) {
  if (!on) {
    memcpy(y, x, (size_t)n * sizeof(double));
    return;
  }
  double ss = 0.0;
  for (int64_t i = 0; i < n; ++i) ss += x[i] * x[i];
  const double r = 1.0 / sqrt(ss + 1e-6);
  for (int64_t i = 0; i < n; ++i) y[i] = x[i] * r;
}

/* state layout [.., K, V] (element [i][j] = S[j][i]) <-> S (V x K) */
static void load_state(const double *src, int64_t K, int64_t V, double *S) {
  for (int64_t i = 0; i < K; ++i)
    for (int64_t j = 0; j < V; ++j) S[j * K + i] = src[i * V + j];
}
static void store_state(const double *S, int64_t K, int64_t V, double *dst) {
  for (int64_t i = 0; i < K; ++i)
    for (int64_t j = 0; j < V; ++j) dst[i * V + j] = S[j * K + i];
}

static int resolve_threads(int threads) {
#ifdef _OPENMP
  return threads > 0 ? threads : omp_get_max_threads();
#else
  (void)threads;
  return 1;
#endif
}

int gdr_oracle_threads(int threads) { return resolve_threads(threads); }

/* ---- prefill over packed sequences ------------------------------------------ */

int gdr_oracle_prefill(int64_t num_seqs, const int64_t *cu_seqlens, int64_t Hk, int64_t Hv,
                       int64_t K, int64_t V, int64_t n_h, const double *q, const double *k,
                       const double *v, const double *g, const double *beta, double scale,
                       int use_qk_l2norm, const double *initial_state,
                       const int64_t *state_indices, double *final_state, double *out,
                       int threads) {
  if (num_seqs < 0 || Hk <= 0 || Hv <= 0 || K <= 0 || V <= 0 || n_h <= 0) return 1;
  if (Hv % Hk != 0) return 1;
  if (!cu_seqlens || !q || !k || !v || !g || !beta || !out) return 1;
  const int64_t group = Hv / Hk;
  const int64_t pairs = num_seqs * Hv;
  const int64_t SS = K * V;

  /* Every sequence's starting state is read before any is written, so reads
     see the states as they were before the call even when the arrays alias. */
  double *states = (double *)calloc((size_t)(pairs > 0 ? pairs : 1) * (size_t)SS, sizeof(double));
  if (!states) return 2;
  for (int64_t p = 0; p < pairs; ++p) {
    const int64_t n = p / Hv, h = p % Hv;
    if (!initial_state) continue; /* zeros */
    int64_t src = n;
    if (state_indices) src = state_indices[n] < 0 ? 0 : state_indices[n];
    load_state(initial_state + (src * Hv + h) * SS, K, V, states + p * SS);
  }

  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(resolve_threads(threads))
  for (int64_t p = 0; p < pairs; ++p) {
    const int64_t n = p / Hv, h = p % Hv, hk = h / group;
    double *S = states + p * SS;
    double *buf = (double *)malloc((size_t)(V + 2 * K) * sizeof(double));
    if (!buf) {
#pragma omp atomic write
      err = 2;
      continue;
    }
    double *Sk = buf, *qn = buf + V, *kn = buf + V + K;
    for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
      for (int64_t j = 0; j < n_h; ++j) {
        const int64_t row = t * n_h + j; /* k, v, beta rows carry the sub-step axis */
        const double a = (j == 0) ? exp(g[t * Hv + h]) : 1.0;
        maybe_l2norm(k + (row * Hk + hk) * K, K, use_qk_l2norm, kn);
        householder_step(S, K, V, a, beta[row * Hv + h], kn, v + (row * Hv + h) * V, Sk);
      }
      maybe_l2norm(q + (t * Hk + hk) * K, K, use_qk_l2norm, qn);
      read_out(S, K, V, scale, qn, out + (t * Hv + h) * V);
    }
    free(buf);
  }

  if (!err && final_state) {
    for (int64_t p = 0; p < pairs; ++p) {
      const int64_t n = p / Hv, h = p % Hv;
      int64_t dst = n;
      if (state_indices) {
        if (state_indices[n] < 0) continue; /* padding writes nothing */
        dst = state_indices[n];
      }
      store_state(states + p * SS, K, V, final_state + (dst * Hv + h) * SS);
    }
  }
  free(states);
  return err;
}

/* ---- one decode token per request over a slot-indexed state cache ----------- */

int gdr_oracle_decode(int64_t n, int64_t Hk, int64_t Hv, int64_t K, int64_t V, int64_t n_h,
                      const double *q, const double *k, const double *v, const double *g,
                      const double *beta, double scale, int use_qk_l2norm, double *cache,
                      int64_t num_slots, const int64_t *batch_indices, double *out,
                      int threads) {
  if (n < 0 || Hk <= 0 || Hv <= 0 || K <= 0 || V <= 0 || n_h <= 0 || num_slots <= 0) return 1;
  if (Hv % Hk != 0 || !q || !k || !v || !g || !beta || !cache || !out) return 1;
  const int64_t group = Hv / Hk;
  const int64_t pairs = n * Hv;
  const int64_t SS = K * V;
  double *states = (double *)malloc((size_t)(pairs > 0 ? pairs : 1) * (size_t)SS * sizeof(double));
  if (!states) return 2;
  for (int64_t p = 0; p < pairs; ++p) {
    const int64_t i = p / Hv, h = p % Hv;
    int64_t slot = batch_indices ? batch_indices[i] : i;
    if (slot < 0) slot = 0; /* padding reads slot 0 */
    load_state(cache + (slot * Hv + h) * SS, K, V, states + p * SS);
  }
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(resolve_threads(threads))
  for (int64_t p = 0; p < pairs; ++p) {
    const int64_t i = p / Hv, h = p % Hv, hk = h / group;
    double *S = states + p * SS;
    double *buf = (double *)malloc((size_t)(V + 2 * K) * sizeof(double));
    if (!buf) {
#pragma omp atomic write
      err = 2;
      continue;
    }
    double *Sk = buf, *qn = buf + V, *kn = buf + V + K;
    for (int64_t j = 0; j < n_h; ++j) {
      const int64_t row = i * n_h + j;
      const double a = (j == 0) ? exp(g[i * Hv + h]) : 1.0;
      maybe_l2norm(k + (row * Hk + hk) * K, K, use_qk_l2norm, kn);
      householder_step(S, K, V, a, beta[row * Hv + h], kn, v + (row * Hv + h) * V, Sk);
    }
    maybe_l2norm(q + (i * Hk + hk) * K, K, use_qk_l2norm, qn);
    read_out(S, K, V, scale, qn, out + (i * Hv + h) * V);
    free(buf);
  }
  if (!err) {
    for (int64_t p = 0; p < pairs; ++p) {
      const int64_t i = p / Hv, h = p % Hv;
      const int64_t slot = batch_indices ? batch_indices[i] : i;
      if (slot < 0) continue; /* padding writes nothing */
      store_state(states + p * SS, K, V, cache + (slot * Hv + h) * SS);
    }
  }
  free(states);
  return err;
}
