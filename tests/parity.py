"""Helpers shared by the GPU parity tests: upload workloads, run both sides, compare.

Tolerances (written here once, used by every parity test):
  * float32 inputs:  max_i |x_i - r_i| / max(|r_i|, RMS(r)) <= 1e-5
  * bf16 inputs with float32 states: max_i (|x_i - r_i| - u_out |r_i|) <= 2e-2 RMS(r),
    where u_out is the unit roundoff of the output type (2^-8 for bf16 outputs,
    0 for float32).  Rounding the exact output to bf16 alone moves it by up to
    u_out |r_i|, so the bound is taken on top of that storage rounding.
RMS(r) is the root mean square of the whole reference tensor being compared.
"""
from __future__ import annotations

import numpy as np

from gated_delta_rule_71_amd import workloads as W

F32_TOL = 1e-5
BF16_TOL = 2e-2
U_BF16 = 2.0 ** -8


def rms(r):
    r = np.asarray(r, dtype=np.float64)
    return float(np.sqrt(np.mean(r * r))) if r.size else 0.0


def err_f32(x, r):
    """max |x - r| / max(|r|, RMS(r))."""
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if r.size == 0:
        return 0.0
    return float(np.max(np.abs(x - r) / np.maximum(np.abs(r), rms(r))))


def err_bf16(x, r, out_bf16):
    """max (|x - r| - u_out |r|) / RMS(r)."""
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if r.size == 0:
        return 0.0
    u = U_BF16 if out_bf16 else 0.0
    return float(np.max(np.abs(x - r) - u * np.abs(r)) / max(rms(r), 1e-300))


def check(x, r, *, f32_inputs, out_bf16, what):
    assert np.all(np.isfinite(x)), f"{what}: non-finite values"
    if f32_inputs:
        e = err_f32(x, r)
        assert e <= F32_TOL, f"{what}: fp32 error {e:.3e} > {F32_TOL}"
    else:
        e = err_bf16(x, r, out_bf16)
        assert e <= BF16_TOL, f"{what}: bf16 error {e:.3e} > {BF16_TOL}"
    return e


# ---- torch plumbing ---------------------------------------------------------------

def to_dev(a, dtype_tag=None):
    """numpy storage array -> GPU tensor (uint16 arrays become bfloat16)."""
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
            torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t):
    """GPU tensor -> float64 numpy (bf16 converted exactly)."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


# ---- oracle on a workload -------------------------------------------------------------

def gate_values(wl):
    """(g, beta) float64 the oracle runs on: the workload's own, or the oracle's gates
    of its raw projections when it carries A_log / dt_bias."""
    if getattr(wl, "A_log", None) is None:
        return np.asarray(wl.g, dtype=np.float64), np.asarray(wl.beta, dtype=np.float64)
    import oracle
    return oracle.gates(wl.g, wl.beta, wl.A_log, wl.dt_bias)


def oracle_prefill(wl: W.PrefillWorkload, *, seqs=None, heads=None, use_qk_l2norm=False,
                   scale=None, threads=0):
    """fp64 oracle on (a sample of) a prefill workload.

    Returns dict {(n, h): (o [L,V], state [K,V])} for the sampled sequences n and
    value heads h (all by default).  States follow the workload's slot rules.
    """
    import oracle
    B, T, Hk, Hv, K, V = wl.shape
    n_h = wl.num_householder
    N = wl.num_seqs
    seqs = range(N) if seqs is None else seqs
    heads = range(Hv) if heads is None else heads
    group = Hv // Hk
    if wl.cu_seqlens is None:
        spans = [(b, 0, T) for b in range(B)]
    else:
        spans = [(0, int(wl.cu_seqlens[i]), int(wl.cu_seqlens[i + 1])) for i in range(N)]
    qf = wl.q
    kf = wl.k.reshape(B, T, n_h, Hk, K)
    vf = wl.v.reshape(B, T, n_h, Hv, V)
    gv, bv = gate_values(wl)
    bf = bv.reshape(B, T, n_h, Hv)
    res = {}
    jobs = []
    for n in seqs:
        b, t0, t1 = spans[n]
        for h in heads:
            hk = h // group
            if wl.initial_state is None:
                s0 = None
            else:
                src = n if wl.state_indices is None else max(int(wl.state_indices[n]), 0)
                s0 = W.as_f64(wl.initial_state[src, h])[None, None]
            jobs.append((n, h, b, t0, t1, hk, s0))
    # one oracle call per (sequence, head); the oracle parallelises inside
    # over pairs, so batch the heads of one sequence together when they share q/k
    for (n, h, b, t0, t1, hk, s0) in jobs:
        q = W.as_f64(qf[b:b + 1, t0:t1, hk:hk + 1])
        k = W.as_f64(kf[b:b + 1, t0:t1, :, hk:hk + 1])
        v = W.as_f64(vf[b:b + 1, t0:t1, :, h:h + 1])
        g = gv[b:b + 1, t0:t1, h:h + 1]
        be = np.asarray(bf[b:b + 1, t0:t1, :, h:h + 1], dtype=np.float64)
        o, fs = oracle.prefill(q, k, v, g, be, scale=scale, initial_state=s0,
                               output_final_state=True, use_qk_l2norm=use_qk_l2norm,
                               num_householder=n_h, threads=threads)
        res[(n, h)] = (o[0, :, 0], fs[0, 0])
    return res


def oracle_prefill_batch(wl: W.PrefillWorkload, pairs, *, use_qk_l2norm=False, scale=None,
                         threads=0):
    """Like oracle_prefill for an explicit list of (n, h) pairs, one oracle call.

    Packs the sampled pairs as independent sequences with one head each so the
    oracle's OpenMP loop runs them in parallel.
    """
    import oracle
    B, T, Hk, Hv, K, V = wl.shape
    n_h = wl.num_householder
    group = Hv // Hk
    N = wl.num_seqs
    if wl.cu_seqlens is None:
        spans = [(b, 0, T) for b in range(B)]
    else:
        spans = [(0, int(wl.cu_seqlens[i]), int(wl.cu_seqlens[i + 1])) for i in range(N)]
    kf = wl.k.reshape(B, T, n_h, Hk, K)
    vf = wl.v.reshape(B, T, n_h, Hv, V)
    gv, bv = gate_values(wl)
    bf = bv.reshape(B, T, n_h, Hv)
    qs, ks, vs, gs, bs, s0s, lens = [], [], [], [], [], [], []
    for (n, h) in pairs:
        b, t0, t1 = spans[n]
        hk = h // group
        qs.append(W.as_f64(wl.q[b, t0:t1, hk:hk + 1]))
        ks.append(W.as_f64(kf[b, t0:t1, :, hk:hk + 1]))
        vs.append(W.as_f64(vf[b, t0:t1, :, h:h + 1]))
        gs.append(gv[b, t0:t1, h:h + 1])
        bs.append(np.asarray(bf[b, t0:t1, :, h:h + 1], dtype=np.float64))
        if wl.initial_state is None:
            s0s.append(np.zeros((1, K, V)))
        else:
            src = n if wl.state_indices is None else max(int(wl.state_indices[n]), 0)
            s0s.append(W.as_f64(wl.initial_state[src, h])[None])
        lens.append(t1 - t0)
    cu = np.zeros(len(pairs) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lens)
    o, fs = oracle.prefill(np.concatenate(qs)[None], np.concatenate(ks)[None],
                           np.concatenate(vs)[None], np.concatenate(gs)[None],
                           np.concatenate(bs)[None], scale=scale, cu_seqlens=cu,
                           initial_state=np.stack(s0s), output_final_state=True,
                           use_qk_l2norm=use_qk_l2norm, num_householder=n_h,
                           threads=threads)
    res = {}
    for i, p in enumerate(pairs):
        res[p] = (o[0, cu[i]:cu[i + 1], 0], fs[i, 0])
    return res


# ---- GPU run of a workload -----------------------------------------------------------

def gpu_prefill(wl: W.PrefillWorkload, *, out_dtype=None, chunk_size=None, use_qk_l2norm=False,
                scale=None):
    """Run the HIP prefill on a workload.  Returns (o, states, dev) with o/states on host.

    ``states``: final states [N,Hv,K,V] (dense) or the whole slot cache after the call.
    """
    import torch
    import gated_delta_rule_71_amd as gdr
    dev = {name: to_dev(getattr(wl, name)) for name in ("q", "k", "v", "g", "beta")}
    cu = None if wl.cu_seqlens is None else to_dev(wl.cu_seqlens)
    idx = None if wl.state_indices is None else to_dev(wl.state_indices)
    h0 = None if wl.initial_state is None else to_dev(wl.initial_state)
    od = {None: None, "f32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
    A_log = to_dev(getattr(wl, "A_log", None))
    dt_bias = to_dev(getattr(wl, "dt_bias", None))
    o, fs = gdr.chunk_gated_delta_rule(
        dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], scale=scale,
        chunk_size=chunk_size or wl.chunk_size, initial_state=h0, output_final_state=True,
        use_qk_l2norm_in_kernel=use_qk_l2norm, cu_seqlens=cu, state_indices=idx,
        out_dtype=od, A_log=A_log, dt_bias=dt_bias)
    torch.cuda.synchronize()
    return o, fs, dev
