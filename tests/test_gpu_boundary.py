"""Boundary states of the prefill (prefix caching), through the C ABI (marked gpu).

With ``boundary_states`` and ``boundary_interval`` the prefill also writes each
sequence's state after every whole multiple of the interval, sequences in order.
Each entry is compared with the fp64 oracle's final state of that prefix of the
sequence (same initial state), and the outputs and final states must be bitwise
those of the same call without boundary states.
"""
from __future__ import annotations

import numpy as np
import pytest

from gated_delta_rule_71_amd import workloads as W
from parity import check, gate_values, to_dev, to_host

pytestmark = pytest.mark.gpu


def _spans(wl):
    B, T = wl.q.shape[:2]
    if wl.cu_seqlens is None:
        return [(b, 0, T) for b in range(B)]
    return [(0, int(wl.cu_seqlens[i]), int(wl.cu_seqlens[i + 1])) for i in range(wl.num_seqs)]


def _run(wl, interval, *, with_boundary, out_dtype):
    import torch
    import gated_delta_rule_71_amd as gdr
    d = {n: to_dev(getattr(wl, n)) for n in ("q", "k", "v", "g", "beta")}
    cu = None if wl.cu_seqlens is None else to_dev(wl.cu_seqlens)
    idx = None if wl.state_indices is None else to_dev(wl.state_indices)
    h0 = None if wl.initial_state is None else to_dev(wl.initial_state)
    B, T, Hk, Hv, K, V = wl.shape
    kw = {}
    bs = None
    if with_boundary:
        E = gdr.boundary_count([t1 - t0 for (_, t0, t1) in _spans(wl)], interval)
        bs = torch.full((E, Hv, K, V), float("nan"), dtype=torch.float32, device="cuda")
        kw = dict(boundary_states=bs, boundary_interval=interval)
    od = {"f32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
    o, fs = gdr.chunk_gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                       chunk_size=wl.chunk_size, initial_state=h0,
                                       output_final_state=True, cu_seqlens=cu,
                                       state_indices=idx, out_dtype=od, **kw)
    torch.cuda.synchronize()
    return o, fs, bs


def _oracle_prefix_states(wl, interval):
    """[(n, j, state [Hv,K,V])] from the oracle on each prefix of each sequence."""
    import oracle
    B, T, Hk, Hv, K, V = wl.shape
    n_h = wl.num_householder
    gv, bv = gate_values(wl)
    kf = wl.k.reshape(B, T, n_h, Hk, K)
    vf = wl.v.reshape(B, T, n_h, Hv, V)
    bf = bv.reshape(B, T, n_h, Hv)
    out = []
    for n, (b, t0, t1) in enumerate(_spans(wl)):
        if wl.initial_state is None:
            s0 = None
        else:
            src = n if wl.state_indices is None else max(int(wl.state_indices[n]), 0)
            s0 = W.as_f64(wl.initial_state[src])[None]
        for j in range((t1 - t0) // interval):
            e = t0 + (j + 1) * interval
            _, fs = oracle.prefill(W.as_f64(wl.q[b:b + 1, t0:e]), W.as_f64(kf[b:b + 1, t0:e]),
                                   W.as_f64(vf[b:b + 1, t0:e]), gv[b:b + 1, t0:e],
                                   bf[b:b + 1, t0:e], initial_state=s0,
                                   output_final_state=True, num_householder=n_h)
            out.append((n, j, fs[0]))
    return out


def _check_case(wl, interval, out_dtype="f32"):
    o0, f0, _ = _run(wl, interval, with_boundary=False, out_dtype=out_dtype)
    o1, f1, bs = _run(wl, interval, with_boundary=True, out_dtype=out_dtype)
    assert np.array_equal(to_host(o0), to_host(o1)), "outputs changed by boundary states"
    assert np.array_equal(f0.cpu().numpy(), f1.cpu().numpy()), "final states changed"
    ref = _oracle_prefix_states(wl, interval)
    got = bs.cpu().numpy().astype(np.float64)
    assert got.shape[0] == len(ref), (got.shape, len(ref))
    if ref:
        check(got, np.stack([r[2] for r in ref]), f32_inputs=wl.dtype == W.F32,
              out_bf16=False, what=f"{wl.name} boundary states (interval {interval})")
    return len(ref)


def test_boundary_varlen_bf16_slots():
    """Ragged packed sequences (empty, shorter than, equal to and past multiples of
    the interval) with a slot cache and one padding sequence."""
    lengths = [0, 63, 64, 200, 130, 256, 1]
    wl = W.prefill_packed("bnd_varlen", 51, lengths, 2, 4, 128, 128, W.BF16, 64,
                          num_slots=10, slot_init="random")
    wl.state_indices = wl.state_indices.copy()
    wl.state_indices[3] = -1
    assert _check_case(wl, 64) == 10


def test_boundary_batched_interval_128():
    wl = W.prefill_dense("bnd_batched", 52, 2, 300, 2, 4, 128, 128, W.BF16, 64,
                         initial_state="random")
    assert _check_case(wl, 128) == 4


def test_boundary_fp32_16_row_chunks():
    """float32 inputs with K = 128 run 16-row chunks: four per 64-token entry."""
    wl = W.prefill_dense("bnd_f32", 53, 1, 200, 1, 2, 128, 128, W.F32, 64,
                         initial_state="random")
    assert _check_case(wl, 64) == 3


def test_boundary_product_two_householder():
    """GDP (n_h = 2): an entry every 64 tokens = 128 rows."""
    wl = W.config4(T=200, H=2)
    assert _check_case(wl, 64) == 3


def test_boundary_none_written():
    """An interval longer than every sequence: no entries, nothing else changes."""
    wl = W.prefill_dense("bnd_none", 54, 2, 100, 2, 2, 64, 64, W.BF16, 64)
    assert _check_case(wl, 128) == 0
