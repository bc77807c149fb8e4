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


def test_segments_with_boundary_states():
    """Boundary states (prefix caching) written by the last pass of the segment path,
    in the order of the unsplit call, against the single pass and the oracle."""
    import torch
    import gated_delta_rule_71_amd as gdr
    import oracle
    wl = W.prefill_dense("seg_bnd", 45, 2, 8192, 2, 2, 128, 128, W.BF16, 64, decay="slow",
                         initial_state="random")
    d = {n: to_dev(getattr(wl, n)) for n in ("q", "k", "v", "g", "beta")}
    iv = 1024
    res = {}
    for seg in (True, False):
        bs = torch.empty((2 * 8192 // iv, 2, 128, 128), dtype=torch.float32, device="cuda")
        o, fs = gdr.chunk_gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                           initial_state=to_dev(wl.initial_state),
                                           output_final_state=True, segments=seg,
                                           boundary_states=bs, boundary_interval=iv)
        torch.cuda.synchronize()
        res[seg] = (to_host(o), fs.cpu().numpy().astype(np.float64),
                    bs.cpu().numpy().astype(np.float64))
    assert _segments_used(wl)
    # entry j of row b is the state after (j + 1) * iv tokens: the oracle's final state
    # of that prefix
    for b in range(2):
        for j in (0, 3, 7):
            L = (j + 1) * iv
            _, ref = oracle.prefill(W.as_f64(wl.q[b:b + 1, :L]), W.as_f64(wl.k[b:b + 1, :L]),
                                    W.as_f64(wl.v[b:b + 1, :L]), wl.g[b:b + 1, :L],
                                    wl.beta[b:b + 1, :L],
                                    initial_state=wl.initial_state[b:b + 1].astype(np.float64),
                                    output_final_state=True)
            for seg in (True, False):
                check(res[seg][2][b * (8192 // iv) + j], ref[0], f32_inputs=False,
                      out_bf16=False, what=f"boundary b={b} j={j} segments={seg}")
    ro, rs = _oracle(wl)
    check(res[True][0], ro, f32_inputs=False, out_bf16=True, what="segments outputs")
    check(res[True][1], rs, f32_inputs=False, out_bf16=False, what="segments final states")


# ---- packed sequences -----------------------------------------------------------------

def _packed_segments_used(wl):
    """Whether the library plans segments for this packed call (host-only query)."""
    import torch
    import gated_delta_rule_71_amd as gdr
    d = {n: to_dev(getattr(wl, n)) for n in ("q", "k", "v", "g", "beta")}
    out = torch.empty(wl.q.shape[:2] + wl.v.shape[-2:], dtype=torch.float32, device="cuda")
    a = gdr.prefill_args(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk_size=wl.chunk_size,
                         out=out, cu_seqlens=to_dev(wl.cu_seqlens),
                         state_indices=to_dev(wl.state_indices),
                         initial_state=to_dev(wl.initial_state))
    return int(gdr.library().gdr_prefill_workspace_bytes(a)) > 0


def _packed_run(wl, segments, **kw):
    """(outputs, states after the call) — states: the slot cache, or the final states."""
    import torch
    import gated_delta_rule_71_amd as gdr
    d = {n: to_dev(getattr(wl, n)) for n in ("q", "k", "v", "g", "beta")}
    cache = to_dev(wl.initial_state)
    o, fs = gdr.chunk_gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                       chunk_size=wl.chunk_size, initial_state=cache,
                                       output_final_state=True, cu_seqlens=to_dev(wl.cu_seqlens),
                                       state_indices=to_dev(wl.state_indices), segments=segments,
                                       A_log=to_dev(wl.A_log), dt_bias=to_dev(wl.dt_bias), **kw)
    torch.cuda.synchronize()
    return to_host(o), fs.cpu().numpy()


def _packed_check(wl, res, *, f32, l2, what):
    from parity import oracle_prefill_batch
    pairs = [(n, h) for n in range(wl.num_seqs) for h in range(wl.v.shape[-2])]
    ref = oracle_prefill_batch(wl, pairs, use_qk_l2norm=l2)
    cu = wl.cu_seqlens
    for name, (o, st) in res.items():
        ox, orf, sx, srf = [], [], [], []
        for (n, h) in pairs:
            ox.append(o[0, cu[n]:cu[n + 1], h])
            orf.append(ref[(n, h)][0])
            slot = n if wl.state_indices is None else int(wl.state_indices[n])
            if slot >= 0:
                sx.append(st[slot, h].astype(np.float64))
                srf.append(ref[(n, h)][1])
        e_o = check(np.concatenate(ox), np.concatenate(orf), f32_inputs=f32, out_bf16=not f32,
                    what=f"{what} {name} outputs")
        e_s = check(np.stack(sx), np.stack(srf), f32_inputs=f32, out_bf16=False,
                    what=f"{what} {name} states")
        print(f"{what} {name}: output err {e_o:.3e}, state err {e_s:.3e}", flush=True)


def test_packed_segments_slot_cache():
    """Packed sequences with a slot cache: a long one (10 segments of 2048 tokens, the
    last ragged), an empty padding request (slot -1: reads slot 0, writes nothing), a
    medium one and an empty request with a slot (written back unchanged).  Segments
    and single pass against the oracle; slots no request writes stay byte-identical."""
    lengths = [20000, 0, 13000, 0]
    wl = W.prefill_packed("seg_packed", 46, lengths, 2, 4, 128, 128, W.BF16, 64, decay="slow",
                          num_slots=8, slot_init="random")
    idx = wl.state_indices.copy()
    idx[1] = -1
    from dataclasses import replace
    wl = replace(wl, state_indices=idx)
    assert _packed_segments_used(wl), "the shape should take the segment path"
    res = {"segments": _packed_run(wl, True), "single pass": _packed_run(wl, False)}
    _packed_check(wl, res, f32=False, l2=False, what="packed slots")
    written = [int(s) for s in idx if s >= 0]
    untouched = np.setdiff1d(np.arange(wl.initial_state.shape[0]), written)
    for name, (_, st) in res.items():
        assert np.array_equal(st[untouched].view(np.uint32),
                              wl.initial_state[untouched].view(np.uint32)), name
        # the empty request with a slot leaves its slot's state as it was
        assert np.array_equal(st[idx[3]].view(np.uint32),
                              wl.initial_state[idx[3]].view(np.uint32)), name


def test_packed_segments_gdp_raw_gates_dense_states():
    """The gated delta product (n_h = 2) on packed sequences with dense initial
    states, gates formed from raw projections and q/k normalised in the kernel."""
    from dataclasses import replace
    base = W.prefill_dense("seg_packed_gdp", 47, 1, 16384, 4, 8, 128, 128, W.BF16, 32,
                           decay="slow", num_householder=2)
    rng = np.random.default_rng(47)
    cu = np.array([0, 15000, 16384], dtype=np.int32)
    h0 = (0.1 * rng.standard_normal((2, 8, 128, 128))).astype(np.float32)
    wl = W.with_raw_gates(replace(base, cu_seqlens=cu, initial_state=h0), 47)
    assert _packed_segments_used(wl), "the shape should take the segment path"
    kw = {"use_qk_l2norm_in_kernel": True}
    res = {"segments": _packed_run(wl, True, **kw), "single pass": _packed_run(wl, False, **kw)}
    _packed_check(wl, res, f32=False, l2=True, what="packed gdp")


def test_packed_segments_deterministic():
    wl = W.prefill_packed("seg_packed_det", 48, [9000, 12000], 4, 4, 128, 128, W.BF16, 64,
                          decay="config", num_slots=4, slot_init="random")
    assert _packed_segments_used(wl)
    a, b = _packed_run(wl, True), _packed_run(wl, True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("entry", ["workspace", "noalloc"])
def test_packed_segments_graph_replay(entry):
    """The packed segment path (device plan, three passes, combine) captured in a HIP
    graph replays to the eager result every time, the slot cache carried from call
    to call; with a caller workspace, and on the allocation-free entry's scratch."""
    import torch
    import gated_delta_rule_71_amd as gdr
    wl = W.prefill_packed("seg_graph", 49, [12000, 5000], 2, 4, 128, 128, W.BF16, 64,
                          decay="slow", num_slots=4, slot_init="random")
    assert _packed_segments_used(wl)
    dev = [to_dev(getattr(wl, n)) for n in ("q", "k", "v", "g", "beta")]
    cu, idx = to_dev(wl.cu_seqlens), to_dev(wl.state_indices)
    cache0 = to_dev(wl.initial_state)
    out = torch.empty(wl.q.shape[:2] + wl.v.shape[-2:], dtype=torch.bfloat16, device="cuda")
    probe = gdr.prefill_args(*dev, cu_seqlens=cu, state_indices=idx, initial_state=cache0,
                             out=out)
    ws = torch.empty(int(gdr.library().gdr_prefill_workspace_bytes(probe)), dtype=torch.uint8,
                     device="cuda")

    def call(cache):
        if entry == "workspace":
            gdr.chunk_gated_delta_rule(*dev, initial_state=cache, cu_seqlens=cu,
                                       state_indices=idx, out=out, workspace=ws)
        else:
            gdr.chunk_gated_delta_rule_noalloc(*dev, out=out, initial_state=cache,
                                               final_state=cache, cu_seqlens=cu,
                                               state_indices=idx)

    eager_c = cache0.clone()
    eager = []
    for _ in range(3):
        call(eager_c)
        eager.append((out.clone(), eager_c.clone()))
    torch.cuda.synchronize()
    graph_c = cache0.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(graph_c.clone())
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(graph_c)
    torch.cuda.synchronize()
    for step in range(3):
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager[step][0]), f"replay {step}: outputs differ"
        assert torch.equal(graph_c, eager[step][1]), f"replay {step}: slot cache differs"
        _ = torch.ones(1, device="cuda").sum().item()
    print(f"packed segments in a graph ({entry}): 3 replays bitwise", flush=True)
