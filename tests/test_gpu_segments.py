"""Long batched rows in segments (marked gpu): three chunked passes over the
segments (zero start, transition from the identity with zero values, true entering
states) and the state combine, against the fp64 oracle, next to the single pass.

The segment path runs when the call gets a workspace and the rows alone leave
compute units idle; the single pass runs otherwise.  Both reach the same function,
so both are held to the oracle with the parity bounds of parity.py.
"""
from __future__ import annotations

import numpy as np
import pytest

from gated_delta_rule_71_amd import workloads as W
from parity import check, gate_values, to_dev, to_host

pytestmark = pytest.mark.gpu


def _run(wl, segments, **kw):
    import torch
    import gated_delta_rule_71_amd as gdr
    d = {n: to_dev(getattr(wl, n)) for n in ("q", "k", "v", "g", "beta")}
    o, fs = gdr.chunk_gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                       chunk_size=wl.chunk_size,
                                       initial_state=to_dev(wl.initial_state),
                                       output_final_state=True, segments=segments,
                                       A_log=to_dev(wl.A_log), dt_bias=to_dev(wl.dt_bias), **kw)
    torch.cuda.synchronize()
    return to_host(o), fs.cpu().numpy().astype(np.float64)


def _oracle(wl, use_qk_l2norm=False):
    import oracle
    g, beta = gate_values(wl)
    return oracle.prefill(W.as_f64(wl.q), W.as_f64(wl.k), W.as_f64(wl.v), g, beta,
                          initial_state=None if wl.initial_state is None
                          else wl.initial_state.astype(np.float64),
                          output_final_state=True, use_qk_l2norm=use_qk_l2norm,
                          num_householder=wl.num_householder)


def _segments_used(wl):
    import torch
    import gated_delta_rule_71_amd as gdr
    d = {n: to_dev(getattr(wl, n)) for n in ("q", "k", "v", "g", "beta")}
    out = torch.empty(wl.q.shape[:2] + wl.v.shape[-2:], dtype=torch.float32, device="cuda")
    a = gdr.prefill_args(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk_size=wl.chunk_size,
                         out=out)
    return int(gdr.library().gdr_prefill_workspace_bytes(a)) > 0


@pytest.mark.parametrize("case", ["gdn_bf16", "gdn_f32_ragged", "gdp_bf16_grouped_raw"])
def test_segments_match_oracle_and_single_pass(case):
    if case == "gdn_bf16":
        wl = W.prefill_dense("seg_gdn", 41, 1, 8192, 4, 4, 128, 128, W.BF16, 64,
                             decay="slow", initial_state="random")
        kw, f32, l2 = {}, False, False
    elif case == "gdn_f32_ragged":
        # 9000 tokens: segments of 2304 tokens, the last one 2088
        wl = W.prefill_dense("seg_f32", 42, 2, 9000, 2, 2, 64, 64, W.F32, 64, decay="slow",
                             initial_state="random")
        kw, f32, l2 = {}, True, False
    else:
        wl = W.with_raw_gates(
            W.prefill_dense("seg_gdp", 43, 1, 8192, 2, 4, 128, 128, W.BF16, 32, decay="slow",
                            initial_state="random", num_householder=2), 43)
        kw, f32, l2 = {"use_qk_l2norm_in_kernel": True}, False, True
    assert _segments_used(wl), "the shape should take the segment path"
    o_seg, s_seg = _run(wl, True, **kw)
    o_one, s_one = _run(wl, False, **kw)
    ro, rs = _oracle(wl, use_qk_l2norm=l2)
    out_bf16 = not f32
    for what, o, s in (("segments", o_seg, s_seg), ("single pass", o_one, s_one)):
        e_o = check(o, ro, f32_inputs=f32, out_bf16=out_bf16, what=f"{case} {what} outputs")
        e_s = check(s, rs, f32_inputs=f32, out_bf16=False, what=f"{case} {what} final states")
        print(f"{case} {what}: output err {e_o:.3e}, state err {e_s:.3e}", flush=True)


def test_segments_deterministic():
    wl = W.prefill_dense("seg_det", 44, 1, 8192, 4, 4, 128, 128, W.BF16, 64, decay="config",
                         initial_state="random")
    a, b = _run(wl, True), _run(wl, True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
