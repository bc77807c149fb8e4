"""Every prefill kernel variant the library routes real inputs to, against the
fp64 oracle through the C ABI (marked gpu).

The prefill picks the number of state waves per workgroup (NS, 32 value columns
each) from the count of (sequence, value head) pairs: the widest tile that still
gives each of the 256 compute units a workgroup.  For V = 128 that is NS = 4 at
256 pairs or more, NS = 2 at 128..255 and NS = 1 below; for V = 64, NS = 2 at 256
pairs or more.  The cases here reach the NS = 2 variants (packed and batched,
V = 128 and V = 64) and, at the packed workload's full shape (NS = 4), boundary
states and gates formed from raw projections, each entry checked against the
oracle's state of that prefix.
"""
from __future__ import annotations

import numpy as np
import pytest

from gated_delta_rule_71_amd import workloads as W
from parity import check, gate_values, gpu_prefill, oracle_prefill_batch, to_dev, to_host

pytestmark = pytest.mark.gpu


def _state_waves(head_v, pairs):
    """The documented tile rule (mirrors the host's choice)."""
    ns = head_v // 32
    while ns > 1:
        if pairs * (head_v // (32 * ns)) >= 256:
            return ns
        ns //= 2
    return 1


def _spans(wl):
    B, T = wl.q.shape[:2]
    if wl.cu_seqlens is None:
        return [(b, 0, T) for b in range(B)]
    return [(0, int(wl.cu_seqlens[i]), int(wl.cu_seqlens[i + 1])) for i in range(wl.num_seqs)]


def _compare(wl, o, states, pairs, *, out_bf16, what):
    ref = oracle_prefill_batch(wl, pairs)
    spans = _spans(wl)
    oh = to_host(o)
    sh = states.cpu().numpy().astype(np.float64)
    ox, orf, sx, srf = [], [], [], []
    for (n, h) in pairs:
        b, t0, t1 = spans[n]
        ox.append(oh[b, t0:t1, h])
        orf.append(ref[(n, h)][0])
        slot = n if wl.state_indices is None else int(wl.state_indices[n])
        if slot >= 0:
            sx.append(sh[slot, h])
            srf.append(ref[(n, h)][1])
    f32 = wl.dtype == W.F32
    e_o = check(np.concatenate(ox), np.concatenate(orf), f32_inputs=f32, out_bf16=out_bf16,
                what=f"{what} outputs")
    e_s = check(np.stack(sx), np.stack(srf), f32_inputs=f32, out_bf16=False,
                what=f"{what} states")
    print(f"{what}: output err {e_o:.3e}, state err {e_s:.3e}", flush=True)


def _all_pairs(wl):
    return [(n, h) for n in range(wl.num_seqs) for h in range(wl.v.shape[-2])]


@pytest.mark.parametrize("decay", ["config", "slow"])
def test_ns2_packed_4seqs_Hk16_Hv32(decay):
    """4 packed sequences x 32 value heads = 128 pairs: two state waves per workgroup.
    Ragged lengths around the chunk size, slot cache with untouched sentinel slots."""
    lengths = [700, 1301, 257, 64]
    wl = W.prefill_packed("ns2_packed", 61, lengths, 16, 32, 128, 128, W.BF16, 64, decay=decay,
                          num_slots=8, slot_init="random")
    assert _state_waves(128, wl.num_seqs * 32) == 2
    before = wl.initial_state.copy()
    o, st, _ = gpu_prefill(wl)
    _compare(wl, o, st, _all_pairs(wl), out_bf16=True, what=f"NS=2 packed {decay}")
    written = [int(s) for s in wl.state_indices if s >= 0]
    untouched = np.setdiff1d(np.arange(before.shape[0]), written)
    assert np.array_equal(st.cpu().numpy()[untouched].view(np.uint32),
                          before[untouched].view(np.uint32))


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_ns2_batched_B8_T512_H16(out_dtype):
    """B = 8, H = 16: 128 pairs, two state waves; random initial state."""
    wl = W.prefill_dense("ns2_batched", 62, 8, 512, 16, 16, 128, 128, W.BF16, 64,
                         decay="slow", initial_state="random")
    assert _state_waves(128, 8 * 16) == 2
    o, st, _ = gpu_prefill(wl, out_dtype=out_dtype)
    _compare(wl, o, st, _all_pairs(wl), out_bf16=out_dtype == "bf16", what="NS=2 batched")


@pytest.mark.parametrize("dims,dtype", [((128, 64), W.BF16), ((64, 64), W.BF16),
                                        ((64, 64), W.F32)])
def test_ns2_value_dim_64_256_pairs(dims, dtype):
    """V = 64 with 256 pairs (B = 16, H = 16): both 32-column state waves of a head in
    one workgroup."""
    K, V = dims
    wl = W.prefill_dense("ns2_v64", 63, 16, 150, 16, 16, K, V, dtype, 64, decay="slow",
                         initial_state="random")
    assert _state_waves(V, 16 * 16) == 2
    o, st, _ = gpu_prefill(wl, out_dtype="f32")
    _compare(wl, o, st, _all_pairs(wl), out_bf16=False, what=f"NS=2 K{K} V{V} {dtype}")


def _oracle_boundaries(wl, pairs, interval):
    """{(n, h): [state after each whole interval]} from the oracle, walking each
    sequence one interval at a time (prefill(L) then prefill of the rest equals the
    whole prefill, an oracle pin), all sampled pairs in one call per step."""
    import oracle
    B, T, Hk, Hv, K, V = wl.shape
    group = Hv // Hk
    gv, bv = gate_values(wl)
    spans = _spans(wl)
    cur = {}
    for (n, h) in pairs:
        src = n if wl.state_indices is None else max(int(wl.state_indices[n]), 0)
        cur[(n, h)] = W.as_f64(wl.initial_state[src, h]).copy()
    out = {p: [] for p in pairs}
    j = 0
    while True:
        live = [(n, h) for (n, h) in pairs
                if (j + 1) * interval <= spans[n][2] - spans[n][1]]
        if not live:
            return out
        qs, ks, vs, gs, bs, s0 = [], [], [], [], [], []
        for (n, h) in live:
            b, t0, _ = spans[n]
            a, e = t0 + j * interval, t0 + (j + 1) * interval
            hk = h // group
            qs.append(W.as_f64(wl.q[b, a:e, hk:hk + 1]))
            ks.append(W.as_f64(wl.k[b, a:e, hk:hk + 1]))
            vs.append(W.as_f64(wl.v[b, a:e, h:h + 1]))
            gs.append(gv[b, a:e, h:h + 1])
            bs.append(bv[b, a:e, h:h + 1])
            s0.append(cur[(n, h)])
        cu = np.arange(len(live) + 1, dtype=np.int64) * interval
        _, fs = oracle.prefill(np.concatenate(qs)[None], np.concatenate(ks)[None],
                               np.concatenate(vs)[None], np.concatenate(gs)[None],
                               np.concatenate(bs)[None], cu_seqlens=cu,
                               initial_state=np.stack(s0)[:, None], output_final_state=True)
        for i, p in enumerate(live):
            cur[p] = fs[i, 0]
            out[p].append(fs[i, 0])
        j += 1


@pytest.mark.parametrize("raw_gates", [False, True])
def test_ns4_full_varlen_boundary_states(raw_gates):
    """The packed workload at full size (8 sequences, 36 112 tokens, 32 value heads:
    four state waves) with a boundary state every 1024 tokens, optionally with the
    gates formed in the kernel from raw projections.  Outputs and final states are
    bitwise those of the call without boundary states and match the oracle on
    sampled heads; every boundary entry of those heads matches the oracle's prefix
    state."""
    import torch
    import gated_delta_rule_71_amd as gdr
    wl = W.config2()
    if raw_gates:
        wl = W.with_raw_gates(wl, 71)
    B, T, Hk, Hv, K, V = wl.shape
    assert _state_waves(V, wl.num_seqs * Hv) == 4
    interval = 1024
    d = {n: to_dev(getattr(wl, n)) for n in ("q", "k", "v", "g", "beta")}
    cu, idx = to_dev(wl.cu_seqlens), to_dev(wl.state_indices)
    gate = dict(A_log=to_dev(getattr(wl, "A_log", None)),
                dt_bias=to_dev(getattr(wl, "dt_bias", None)))
    lens = [t1 - t0 for (_, t0, t1) in _spans(wl)]
    E = gdr.boundary_count(lens, interval)
    runs = []
    for with_b in (False, True):
        cache = to_dev(wl.initial_state)
        kw = dict(gate)
        bs = None
        if with_b:
            bs = torch.full((E, Hv, K, V), float("nan"), dtype=torch.float32, device="cuda")
            kw.update(boundary_states=bs, boundary_interval=interval)
        o, _ = gdr.chunk_gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                          initial_state=cache, cu_seqlens=cu,
                                          state_indices=idx, **kw)
        torch.cuda.synchronize()
        runs.append((o, cache, bs))
    (o0, c0, _), (o1, c1, bs) = runs
    assert torch.equal(o0, o1), "outputs changed by boundary states"
    assert torch.equal(c0, c1), "final states changed by boundary states"
    rng = np.random.default_rng(72)
    pairs = [(n, int(h)) for n in range(wl.num_seqs) for h in rng.permutation(Hv)[:2]]
    _compare(wl, o1, c1, pairs, out_bf16=True,
             what=f"NS=4 full varlen{' raw gates' if raw_gates else ''}")
    ref = _oracle_boundaries(wl, pairs, interval)
    offs = np.concatenate([[0], np.cumsum([L // interval for L in lens])])
    got = bs.cpu().numpy().astype(np.float64)
    gx, rx = [], []
    for (n, h) in pairs:
        assert len(ref[(n, h)]) == offs[n + 1] - offs[n]
        for j, r in enumerate(ref[(n, h)]):
            gx.append(got[offs[n] + j, h])
            rx.append(r)
    e = check(np.stack(gx), np.stack(rx), f32_inputs=False, out_bf16=False,
              what="NS=4 boundary states")
    print(f"NS=4 boundary entries ({len(rx)} sampled): err {e:.3e}", flush=True)
    # entries of heads that were not sampled are written too (no NaN left)
    assert np.all(np.isfinite(got)), "a boundary entry was not written"


def test_packed_all_empty_slots_l2norm_raw_gates():
    """Every packed sequence empty (no tokens at all) over a slot cache with one padding
    entry, with the in-kernel norm and raw gates: each sequence's state passes through
    its slot and the padding slot is not written, so the cache is bitwise unchanged."""
    wl = W.with_raw_gates(W.prefill_packed("none", 71, [0, 0, 0], 2, 4, 128, 128, W.BF16, 64,
                                           num_slots=6, slot_init="random"), 71)
    wl.state_indices = wl.state_indices.copy()
    wl.state_indices[1] = -1
    before = wl.initial_state.copy()
    o, st, _ = gpu_prefill(wl, out_dtype="bf16", use_qk_l2norm=True)
    assert o.numel() == 0
    assert np.array_equal(to_host(st), before)
