/*
 * CPU oracle for the gated delta rule — TEST INFRASTRUCTURE ONLY (see gdr_oracle.c).
 * Host fp64 arrays, row-major, innermost dimension contiguous.  Returns 0 on
 * success, 1 on an invalid argument, 2 on allocation failure.
 */
#ifndef GDR_ORACLE_H
#define GDR_ORACLE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

/* Number of threads a call with `threads` (<= 0: all available) would use. */
int gdr_oracle_threads(int threads);

/*
 * Packed prefill.  T = cu_seqlens[num_seqs] tokens; n_h Householder sub-steps.
 *   q    [T, Hk, K]          k    [T, n_h, Hk, K]     v [T, n_h, Hv, V]
 *   g    [T, Hv]             beta [T, n_h, Hv]        out [T, Hv, V]
 *   initial_state [S, Hv, K, V] or NULL (zeros); final_state [S, Hv, K, V] or NULL.
 *   state_indices [num_seqs] or NULL.  NULL: sequence n reads initial_state[n] and
 *   writes final_state[n].  Otherwise it reads slot max(idx, 0) and writes slot idx
 *   only when idx >= 0.  initial_state and final_state may alias.
 */
int gdr_oracle_prefill(int64_t num_seqs, const int64_t *cu_seqlens, int64_t Hk, int64_t Hv,
                       int64_t K, int64_t V, int64_t n_h, const double *q, const double *k,
                       const double *v, const double *g, const double *beta, double scale,
                       int use_qk_l2norm, const double *initial_state,
                       const int64_t *state_indices, double *final_state, double *out,
                       int threads);

/*
 * One token per request over a slot cache [num_slots, Hv, K, V], updated in place.
 *   q [n, Hk, K]  k [n, n_h, Hk, K]  v [n, n_h, Hv, V]  g [n, Hv]  beta [n, n_h, Hv]
 *   out [n, Hv, V].  batch_indices [n] or NULL (request i uses slot i).
 */
int gdr_oracle_decode(int64_t n, int64_t Hk, int64_t Hv, int64_t K, int64_t V, int64_t n_h,
                      const double *q, const double *k, const double *v, const double *g,
                      const double *beta, double scale, int use_qk_l2norm, double *cache,
                      int64_t num_slots, const int64_t *batch_indices, double *out,
                      int threads);

#ifdef __cplusplus
}
#endif
#endif
