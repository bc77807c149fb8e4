"""One layer step captured in a HIP graph (marked gpu): the causal conv over the
packed V/K/Q projection, the chunked recurrence with gates formed in the kernel
from raw projections and a slot cache, and the gated RMS norm of its output.
Every replay equals the eager run of the same step, bitwise (the pages require
the inference steps to be graph-capturable)."""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def test_layer_step_graph_replay():
    import torch
    import gated_delta_rule_71_amd as gdr
    rng = np.random.default_rng(81)
    dev = "cuda"
    lengths = [70, 3, 129]
    T = sum(lengths)
    Hk, Hv, K, V, Wd = 2, 4, 128, 128, 4
    C = 2 * Hk * K + Hv * V
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device=dev)
    idx = torch.tensor([2, 0, 5], dtype=torch.int32, device=dev)
    x = torch.randn((T, C), device=dev).to(torch.bfloat16)
    w = torch.randn((C, Wd), device=dev) * 0.3
    b = torch.randn(C, device=dev) * 0.1
    alpha = torch.randn((1, T, Hv), device=dev)
    braw = torch.randn((1, T, Hv), device=dev)
    A_log = torch.log(torch.empty(Hv, device=dev).uniform_(1, 16))
    dt_bias = torch.log(torch.expm1(torch.empty(Hv, device=dev).uniform_(0.001, 0.1)))
    z = torch.randn((T, Hv, V), device=dev).to(torch.bfloat16)
    wn = torch.empty(Hv * V, device=dev).uniform_(0.5, 1.5)
    conv0 = torch.randn((6, C, Wd - 1), device=dev) * 0.1
    ssm0 = torch.randn((6, Hv, K, V), device=dev) * 0.1

    def step(conv_state, ssm_state, outs):
        y = gdr.causal_conv1d(x, w, b, cu_seqlens=cu, conv_state=conv_state,
                              state_indices=idx, out=outs["y"])
        q = y[:, :Hk * K].reshape(1, T, Hk, K).contiguous()
        k = y[:, Hk * K:2 * Hk * K].reshape(1, T, Hk, K).contiguous()
        v = y[:, 2 * Hk * K:].reshape(1, T, Hv, V).contiguous()
        o, _ = gdr.chunk_gated_delta_rule(q, k, v, alpha, braw, initial_state=ssm_state,
                                          cu_seqlens=cu, state_indices=idx,
                                          use_qk_l2norm_in_kernel=True, A_log=A_log,
                                          dt_bias=dt_bias, out=outs["o"])
        gdr.gated_rmsnorm(o.reshape(T, Hv, V), z, wn, out=outs["n"])

    def fresh_outs():
        return {"y": torch.empty_like(x), "o": torch.empty((1, T, Hv, V), device=dev,
                                                           dtype=torch.bfloat16),
                "n": torch.empty((T, Hv, V), device=dev, dtype=torch.bfloat16)}

    ec, es, eo = conv0.clone(), ssm0.clone(), fresh_outs()
    eager = []
    for _ in range(3):
        step(ec, es, eo)
        eager.append({k: t.clone() for k, t in eo.items()} | {"conv": ec.clone(), "ssm": es.clone()})
    torch.cuda.synchronize()

    gc, gs, go = conv0.clone(), ssm0.clone(), fresh_outs()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm-up on side copies (allocator and library load)
        step(gc.clone(), gs.clone(), fresh_outs())
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(gc, gs, go)
    torch.cuda.synchronize()
    for r in range(3):
        graph.replay()
        torch.cuda.synchronize()
        for key in ("y", "o", "n"):
            assert torch.equal(go[key], eager[r][key]), f"replay {r}: {key} differs"
        assert torch.equal(gc, eager[r]["conv"]), f"replay {r}: conv states differ"
        assert torch.equal(gs, eager[r]["ssm"]), f"replay {r}: ssm states differ"
        _ = torch.ones(1, device=dev).sum().item()   # eager work between replays
