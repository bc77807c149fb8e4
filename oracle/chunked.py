"""Chunked evaluation of the gated delta rule in fp64 NumPy — TEST INFRASTRUCTURE ONLY.

This is the chunk-parallel reformulation that the chunked kernels follow (the
"chunk_size" argument of torch_chunk_gated_delta_rule, Megatron Core API page
"core.ssm.gated_delta_net.gdn"; the chunk-based kernel of the page
"core.ssm.gated_delta_product").  It exists to show, on the CPU, that splitting a
sequence into chunks of any size leaves the result of the per-token recurrence
unchanged; it is checked against the C oracle, never against the GPU.

Derivation (state H = S^T, K x V; rows r = 0..n-1 of one chunk, entering state H0):
  per-row decay g_r (for several Householder sub-steps per token, the token's g
  sits on its first sub-step and the others carry 0);
  G_r = g_0 + ... + g_r;  Gamma[r, i] = exp(G_r - G_i) for i <= r, else 0;
  unrolling H_r = exp(G_r) H0 + sum_{i<=r} Gamma[r,i] k_i d_i^T into the delta
  d_r = beta_r (v_r - exp(g_r) H_{r-1}^T k_r) gives the unit lower-triangular system
      (I + A) D = diag(beta) V - diag(beta exp(G)) K H0,
      A = strict_lower(diag(beta) (K K^T) * Gamma);
  with T = (I + A)^-1, W = T diag(beta exp(G)) K and U = T diag(beta) V:
      D   = U - W H0
      O   = scale * (diag(exp(G)) Q H0 + (Q K^T * Gamma * [i <= r]) D)   (query rows)
      H_n = exp(G_{n-1}) H0 + (diag(exp(G_{n-1} - G)) K)^T D
"""
from __future__ import annotations

import numpy as np


def _l2norm(x):
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + 1e-6)


def chunk_step(H0, Kc, Vc, gc, bc, Qc, qrows, scale):
    """One chunk.  Kc [n,K], Vc [n,V], gc [n], bc [n], Qc [m,K] at chunk rows qrows.

    Returns (O [m,V], H_n [K,V]).
    """
    n = Kc.shape[0]
    G = np.cumsum(gc)
    # decay between rows, masked to the lower triangle before exponentiation
    diff = G[:, None] - G[None, :]
    lower = np.tril(np.ones((n, n), dtype=bool))
    Gamma = np.where(lower, np.exp(np.where(lower, diff, 0.0)), 0.0)
    A = np.tril(bc[:, None] * (Kc @ Kc.T) * Gamma, k=-1)
    Tm = np.linalg.inv(np.eye(n) + A)
    W = Tm @ ((bc * np.exp(G))[:, None] * Kc)
    U = Tm @ (bc[:, None] * Vc)
    D = U - W @ H0
    # queries sit on a subset of the rows
    P = (Qc @ Kc.T) * Gamma[qrows, :]
    O = scale * (np.exp(G[qrows])[:, None] * (Qc @ H0) + P @ D)
    Kt = np.exp(G[-1] - G)[:, None] * Kc
    Hn = np.exp(G[-1]) * H0 + Kt.T @ D
    return O, Hn


def chunked_sequence(q, k, v, g, beta, scale, chunk_rows, H0, n_h=1, use_qk_l2norm=False):
    """One sequence and head.  q [L,K]; k [L*n_h,K]; v [L*n_h,V]; g [L]; beta [L*n_h].

    ``chunk_rows`` counts rows (token sub-steps); a chunk may end between the
    sub-steps of one token.  Returns (o [L,V], H [K,V]).
    """
    L = q.shape[0]
    if use_qk_l2norm:
        q, k = _l2norm(q), _l2norm(k)
    R = L * n_h
    g_rows = np.zeros(R)
    g_rows[0::n_h] = g
    out = np.zeros((L, v.shape[1]))
    H = np.array(H0, dtype=np.float64, copy=True)
    for c0 in range(0, R, chunk_rows):
        c1 = min(c0 + chunk_rows, R)
        rows = np.arange(c0, c1)
        qmask = (rows % n_h) == (n_h - 1)
        qrows = np.nonzero(qmask)[0]
        toks = rows[qmask] // n_h
        O, H = chunk_step(H, k[c0:c1], v[c0:c1], g_rows[c0:c1], beta[c0:c1],
                          q[toks], qrows, scale)
        out[toks] = O
    return out, H


def chunked_prefill(q, k, v, g, beta, *, chunk_rows, scale=None, cu_seqlens=None,
                    initial_state=None, num_householder=1, use_qk_l2norm=False):
    """Same shapes as :func:`oracle.prefill` (dense states only).  Returns (o, final)."""
    q = np.asarray(q, dtype=np.float64)
    B, T, Hk, K = q.shape
    n_h = int(num_householder)
    Hv, V = v.shape[-2], v.shape[-1]
    k = np.asarray(k, dtype=np.float64).reshape(B, T * n_h, Hk, K)
    v = np.asarray(v, dtype=np.float64).reshape(B, T * n_h, Hv, V)
    g = np.asarray(g, dtype=np.float64).reshape(B, T, Hv)
    beta = np.asarray(beta, dtype=np.float64).reshape(B, T * n_h, Hv)
    if scale is None:
        scale = 1.0 / np.sqrt(K)
    if cu_seqlens is None:
        spans = [(b, 0, T) for b in range(B)]
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        spans = [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
    out = np.zeros((B, T, Hv, V))
    final = np.zeros((len(spans), Hv, K, V))
    group = Hv // Hk
    for n, (b, t0, t1) in enumerate(spans):
        for h in range(Hv):
            hk = h // group
            H0 = np.zeros((K, V)) if initial_state is None else initial_state[n, h]
            o, H = chunked_sequence(
                q[b, t0:t1, hk], k[b, t0 * n_h:t1 * n_h, hk], v[b, t0 * n_h:t1 * n_h, h],
                g[b, t0:t1, h], beta[b, t0 * n_h:t1 * n_h, h], scale, chunk_rows, H0,
                n_h=n_h, use_qk_l2norm=use_qk_l2norm)
            out[b, t0:t1, h] = o
            final[n, h] = H
    return out, final
