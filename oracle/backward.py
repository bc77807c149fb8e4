"""Gradients of the gated delta rule in fp64 on the CPU — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; the GPU library shares nothing with it.

Training through torch_chunk_gated_delta_rule (Megatron Core API page
"core.ssm.gated_delta_net.gdn") needs the gradients of the loss with respect to
q, k, v, g, beta and the initial state, given the gradients of the outputs o and
of the final state.  The chunked backward these pages point to (the chunked
training kernels of the Gated DeltaNet and Gated Delta Product pages) reaches the
gradient of the same function, so the oracle is that gradient, by definition:

* :func:`prefill_backward` runs the per-token recurrence (the definition, as in
  ``gdr_oracle.c``) in fp64 with torch CPU tensors and differentiates it with
  reverse-mode automatic differentiation.  Its forward pass is checked against the
  C oracle and its gradients against central finite differences and closed forms
  (tests/test_oracle_backward.py).
* With the in-kernel q/k L2 norm and the gates formed from raw projections (the
  module's defaults on the same page: use_qk_l2norm_in_kernel, _compute_gates),
  the same differentiation runs through those steps too (:func:`l2norm_torch`,
  :func:`gates_torch`, the definitions of ``oracle/gating.py``).
* :func:`chunked_backward` is the chunk-by-chunk evaluation of the same gradient
  (the algebra the GPU backward follows), in fp64 NumPy.  It is checked against
  :func:`prefill_backward`, never against the GPU.

Chunk algebra (one chunk of rows r = 0..n-1 entering with state H0 = S^T, K x V;
G_r the cumulative decay inside the chunk; Gamma[r, i] = exp(G_r - G_i)):
  forward:  A = strict_lower(diag(beta) (K K^T) * Gamma),  T = (I + A)^-1,
            R = diag(beta) V - diag(beta e^G) K H0,  D = T R,
            O = diag(scale e^G) Q H0 + P D,  P = scale (Q K^T) * Gamma * [i <= r],
            H_n = e^{G_n} H0 + K~^T D,  K~ = diag(e^{G_n - G}) K.
  backward, given dO and dH_n (the gradient of the state leaving the chunk):
            dD  = P^T dO + K~ dH_n,        dR = T^T dD,        dV = diag(beta) dR,
            dA  = -strict_lower(dR D^T),   dP = lower(dO D^T),
            dH0 = e^{G_n} dH_n + Q^T diag(scale e^G) dO - K^T diag(beta e^G) dR,
            dQ  = diag(scale e^G) dO H0^T + dPs K,
            dK  = dAs K + dAs^T K + dPs^T Q - diag(beta e^G) dR H0^T
                  + diag(e^{G_n - G}) D dH_n^T,
  with dAs = dA * diag(beta) Gamma and dPs = scale dP * Gamma;
            dbeta_r = sum_i dA_ri (k_r . k_i) Gamma_ri + dR_r . (v_r - e^{G_r} (K H0)_r),
            dG_r    = rowsum(E + F)_r - colsum(E + F)_r
                      + scale e^{G_r} dO_r . (Q H0)_r - beta_r e^{G_r} dR_r . (K H0)_r
                      - w_r  (+ e^{G_n} <dH_n, H0> + sum_i w_i  on the last row),
  where E = dA * A, F = dP * P, w_i = e^{G_n - G_i} k_i^T dH_n D_i, and finally
  dg_j = sum_{r >= j} dG_r inside the chunk.
"""
from __future__ import annotations

import numpy as np


def _spans(B, T, cu_seqlens):
    if cu_seqlens is None:
        return [(b, 0, T) for b in range(B)]
    assert B == 1, "packed sequences use batch size 1"
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    return [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]


def forward_torch(q, k, v, g, beta, scale, H0):
    """The per-token recurrence on torch tensors for one sequence, all value heads.

    q [L,Hk,K]; k [L,Hk,K] or [L,n_h,Hk,K]; v [L,Hv,V] or [L,n_h,Hv,V]; g [L,Hv];
    beta [L,Hv] or [L,n_h,Hv]; H0 [Hv,K,V] (state S^T per head).  Value head h reads
    q/k head h // (Hv // Hk).  With n_h Householder sub-steps per token (the gated
    delta product) the decay exp(g_t) is applied once, before the first sub-step,
    each sub-step j writes beta_j (v_j - H^T k_j) along k_j, and o_t is read after
    the last one.  Returns (o [L,Hv,V], H_L).
    """
    import torch
    if k.dim() == 3:
        k, v, beta = k[:, None], v[:, None], beta[:, None]
    L, Hk, _ = q.shape
    n_h, Hv = k.shape[1], v.shape[2]
    hk = torch.arange(Hv) // (Hv // Hk)
    H = H0
    outs = []
    for t in range(L):
        H = torch.exp(g[t])[:, None, None] * H           # decay once per token
        for j in range(n_h):
            kt = k[t, j, hk]                             # [Hv, K]
            u = torch.einsum("hkv,hk->hv", H, kt)        # H^T k
            d = beta[t, j][:, None] * (v[t, j] - u)      # delta
            H = H + kt[:, :, None] * d[:, None, :]
        outs.append(scale * torch.einsum("hkv,hk->hv", H, q[t, hk]))
    o = torch.stack(outs) if outs else torch.zeros((0, Hv, v.shape[-1]), dtype=v.dtype)
    return o, H


def l2norm_torch(x):
    """x / sqrt(sum x^2 + 1e-6) over the last axis (the in-kernel q/k norm)."""
    import torch
    return x / torch.sqrt((x * x).sum(-1, keepdim=True) + 1e-6)


def gates_torch(alpha, b, A_log, dt_bias):
    """g = -exp(A_log) softplus(alpha + dt_bias), beta = sigmoid(b) on torch tensors
    (the definitions of oracle/gating.py; A_log, dt_bias broadcast over the last axis)."""
    import torch
    x = alpha + dt_bias
    # log(1 + e^x) = max(x, 0) + log(1 + e^-|x|): exp of a non-positive number only
    softplus = torch.clamp(x, min=0.0) + torch.log1p(torch.exp(-torch.abs(x)))
    return -torch.exp(A_log) * softplus, 1.0 / (1.0 + torch.exp(-b))


def prefill_backward(q, k, v, g, beta, do, dht=None, *, scale=None, cu_seqlens=None,
                     initial_state=None, return_forward=False, use_qk_l2norm=False,
                     A_log=None, dt_bias=None):
    """fp64 gradients of  L = <o, do> + <H_final, dht>  for the GDN recurrence.

    Batched layout as in :func:`oracle.prefill`: q [B,T,Hk,K]; k [B,T,Hk,K] or
    [B,T,n_h,Hk,K]; v [B,T,Hv,V] or [B,T,n_h,Hv,V]; do [B,T,Hv,V]; g [B,T,Hv]; beta
    [B,T,Hv] or [B,T,n_h,Hv]; initial_state, dht [N,Hv,K,V] or None.  The gradients
    of k, v, beta have the shapes of k, v, beta.
    With ``use_qk_l2norm`` the recurrence reads q, k divided by their L2 norm and
    dq, dk are the gradients of the raw q, k.  With ``A_log`` and ``dt_bias`` ([Hv])
    g and beta hold the raw projections alpha and b, the gates are formed from them,
    dg and dbeta are the gradients of alpha and b, and dA_log, ddt_bias [Hv] are added.
    Returns dict dq, dk [B,T,Hk,K]; dv [B,T,Hv,V]; dg, dbeta [B,T,Hv];
    dh0 [N,Hv,K,V] (all fp64), plus o and final_state when ``return_forward``.
    """
    import torch
    q = np.asarray(q, dtype=np.float64)
    B, T, Hk, K = q.shape
    Hv, V = v.shape[-2], v.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(K)
    spans = _spans(B, T, cu_seqlens)
    N = len(spans)
    k, v, beta = np.asarray(k), np.asarray(v), np.asarray(beta)
    res = {"dq": np.zeros((B, T, Hk, K)), "dk": np.zeros(k.shape),
           "dv": np.zeros(v.shape), "dg": np.zeros((B, T, Hv)),
           "dbeta": np.zeros(beta.shape), "dh0": np.zeros((N, Hv, K, V))}
    if return_forward:
        res["o"] = np.zeros((B, T, Hv, V))
        res["final_state"] = np.zeros((N, Hv, K, V))

    def leaf(x):
        return torch.tensor(np.asarray(x, dtype=np.float64), requires_grad=True)

    raw_gates = A_log is not None
    if raw_gates:
        res["dA_log"] = np.zeros(Hv)
        res["ddt_bias"] = np.zeros(Hv)
    for n, (b, t0, t1) in enumerate(spans):
        qs, ks, vs = leaf(q[b, t0:t1]), leaf(np.asarray(k)[b, t0:t1]), leaf(np.asarray(v)[b, t0:t1])
        gs, bs = leaf(np.asarray(g)[b, t0:t1]), leaf(np.asarray(beta)[b, t0:t1])
        h0 = leaf(np.zeros((Hv, K, V)) if initial_state is None else initial_state[n])
        qe, ke, ge, be = qs, ks, gs, bs
        if use_qk_l2norm:
            qe, ke = l2norm_torch(qs), l2norm_torch(ks)
        if raw_gates:
            al, dtb = leaf(A_log), leaf(dt_bias)
            ge, be = gates_torch(gs, bs, al, dtb)
        o, H = forward_torch(qe, ke, vs, ge, be, float(scale), h0)
        loss = (o * torch.tensor(np.asarray(do, dtype=np.float64)[b, t0:t1])).sum()
        if dht is not None:
            loss = loss + (H * torch.tensor(np.asarray(dht[n], dtype=np.float64))).sum()
        if loss.requires_grad:
            loss.backward()
        for name, x in (("dq", qs), ("dk", ks), ("dv", vs), ("dg", gs), ("dbeta", bs)):
            if x.grad is not None:
                res[name][b, t0:t1] = x.grad.numpy()
        if h0.grad is not None:
            res["dh0"][n] = h0.grad.numpy()
        if raw_gates:
            for name, x in (("dA_log", al), ("ddt_bias", dtb)):
                if x.grad is not None:
                    res[name] += x.grad.numpy()
        if return_forward:
            res["o"][b, t0:t1] = o.detach().numpy()
            res["final_state"][n] = H.detach().numpy()
    return res


# ---- chunked form ---------------------------------------------------------------------

def _chunk_backward(H0, dHn, Kc, Qc, Vc, dOc, gc, bc, scale):
    """Gradients of one chunk (rows r = 0..n-1).  Returns (dQ, dK, dV, dg, dbeta, dH0)."""
    n = Kc.shape[0]
    G = np.cumsum(gc)
    lower = np.tril(np.ones((n, n), dtype=bool))
    strict = np.tril(np.ones((n, n), dtype=bool), k=-1)
    Gam = np.where(lower, np.exp(np.where(lower, G[:, None] - G[None, :], 0.0)), 0.0)
    eG = np.exp(G)
    eGl = np.exp(G[-1] - G)
    KK = Kc @ Kc.T
    Araw = np.where(strict, KK * Gam, 0.0)
    A = bc[:, None] * Araw
    Tm = np.linalg.inv(np.eye(n) + A)
    P = np.where(lower, scale * (Qc @ Kc.T) * Gam, 0.0)
    X = Kc @ H0
    R = bc[:, None] * (Vc - eG[:, None] * X)
    D = Tm @ R
    Kt = eGl[:, None] * Kc
    # backward
    dD = P.T @ dOc + Kt @ dHn
    dR = Tm.T @ dD
    dV = bc[:, None] * dR
    dA = -np.where(strict, dR @ D.T, 0.0)
    dP = np.where(lower, dOc @ D.T, 0.0)
    dAs = dA * bc[:, None] * Gam
    dPs = scale * dP * Gam
    dH0 = np.exp(G[-1]) * dHn + Qc.T @ ((scale * eG)[:, None] * dOc) \
        - Kc.T @ ((bc * eG)[:, None] * dR)
    dQ = (scale * eG)[:, None] * (dOc @ H0.T) + dPs @ Kc
    dK = dAs @ Kc + dAs.T @ Kc + dPs.T @ Qc - (bc * eG)[:, None] * (dR @ H0.T) \
        + eGl[:, None] * (D @ dHn.T)
    dbeta = np.sum(dA * Araw, axis=1) + np.sum(dR * (Vc - eG[:, None] * X), axis=1)
    EF = dA * A + dP * P
    w = eGl * np.sum((Kc @ dHn) * D, axis=1)
    dG = EF.sum(axis=1) - EF.sum(axis=0) + scale * eG * np.sum(dOc * (Qc @ H0), axis=1) \
        - bc * eG * np.sum(dR * X, axis=1) - w
    dG[-1] += np.exp(G[-1]) * np.sum(dHn * H0) + w.sum()
    dg = np.cumsum(dG[::-1])[::-1]
    return dQ, dK, dV, dg, dbeta, dH0


def chunked_backward(q, k, v, g, beta, do, dht=None, *, chunk_size, scale=None,
                     cu_seqlens=None, initial_state=None):
    """Same arguments and result as :func:`prefill_backward`, chunk by chunk.

    The forward states at the chunk starts are recomputed with the chunked
    forward; then each sequence's chunks are visited last to first, carrying dH.
    """
    from .chunked import chunk_step
    q = np.asarray(q, dtype=np.float64)
    k, v = np.asarray(k, dtype=np.float64), np.asarray(v, dtype=np.float64)
    g, beta = np.asarray(g, dtype=np.float64), np.asarray(beta, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, T, Hk, K = q.shape
    Hv, V = v.shape[-2], v.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(K)
    spans = _spans(B, T, cu_seqlens)
    N = len(spans)
    group = Hv // Hk
    res = {"dq": np.zeros((B, T, Hk, K)), "dk": np.zeros((B, T, Hk, K)),
           "dv": np.zeros((B, T, Hv, V)), "dg": np.zeros((B, T, Hv)),
           "dbeta": np.zeros((B, T, Hv)), "dh0": np.zeros((N, Hv, K, V))}
    C = int(chunk_size)
    for n, (b, t0, t1) in enumerate(spans):
        starts = list(range(t0, t1, C))
        for h in range(Hv):
            hk = h // group
            H = np.zeros((K, V)) if initial_state is None else np.array(initial_state[n, h])
            states = []
            for c0 in starts:
                c1 = min(c0 + C, t1)
                states.append(H)
                _, H = chunk_step(H, k[b, c0:c1, hk], v[b, c0:c1, h], g[b, c0:c1, h],
                                  beta[b, c0:c1, h], q[b, c0:c1, hk], np.arange(c1 - c0), scale)
            dH = np.zeros((K, V)) if dht is None else np.array(dht[n, h], dtype=np.float64)
            for c0, H0 in reversed(list(zip(starts, states))):
                c1 = min(c0 + C, t1)
                dQ, dK, dV, dg, db, dH = _chunk_backward(
                    H0, dH, k[b, c0:c1, hk], q[b, c0:c1, hk], v[b, c0:c1, h], do[b, c0:c1, h],
                    g[b, c0:c1, h], beta[b, c0:c1, h], scale)
                res["dq"][b, c0:c1, hk] += dQ
                res["dk"][b, c0:c1, hk] += dK
                res["dv"][b, c0:c1, h] = dV
                res["dg"][b, c0:c1, h] = dg
                res["dbeta"][b, c0:c1, h] = db
            res["dh0"][n, h] = dH
    return res
