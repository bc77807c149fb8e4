"""The allocation-free prefill entry point (gdr_chunk_gated_delta_rule_noalloc)
through the C ABI, against the entry point that takes a caller workspace (marked
gpu).

Long batched rows with few (row, value head) pairs take the segment path, whose
workspace the allocation-free entry point takes from the library's per-GPU
scratch.  Two calls in a row, the second on a smaller input, each equal the
workspace entry point's result bit for bit (same kernels, same plan) and the fp64
oracle within the bf16 bound; a call that needs no scratch is checked too.
"""
from __future__ import annotations

import numpy as np
import pytest

from gated_delta_rule_71_amd import workloads as W
from parity import check, oracle_prefill_batch, to_dev, to_host

pytestmark = pytest.mark.gpu


def _run_both(wl):
    import torch
    import gated_delta_rule_71_amd as gdr
    d = [to_dev(getattr(wl, n)) for n in ("q", "k", "v", "g", "beta")]
    h0 = to_dev(wl.initial_state)
    lib = gdr.library()
    probe = gdr.prefill_args(*d, chunk_size=wl.chunk_size, initial_state=h0, final_state=h0,
                             out=torch.empty(1, dtype=torch.bfloat16, device="cuda"))
    seg_bytes = int(lib.gdr_prefill_workspace_bytes(probe))
    # the entry point with a caller workspace (allocated by the binding)
    o_ws, s_ws = gdr.chunk_gated_delta_rule(*d, chunk_size=wl.chunk_size, initial_state=h0,
                                            output_final_state=True)
    # the allocation-free entry point: outputs preallocated, nothing else
    o = torch.full_like(o_ws, float("nan"))
    fs = torch.full_like(s_ws, float("nan"))
    r = gdr.chunk_gated_delta_rule_noalloc(*d, out=o, chunk_size=wl.chunk_size,
                                           initial_state=h0, final_state=fs)
    torch.cuda.synchronize()
    assert r is o
    return seg_bytes, (o_ws, s_ws), (o, fs)


@pytest.mark.parametrize("decay", ["config", "slow"])
def test_noalloc_two_calls_second_smaller(decay):
    cases = [("noalloc_a", 81, 1, 8192, 2, 4), ("noalloc_b", 82, 1, 4096, 1, 2)]
    for name, seed, B, T, Hk, Hv in cases:
        wl = W.prefill_dense(name, seed, B, T, Hk, Hv, 128, 128, W.BF16, 64, decay=decay,
                             initial_state="random")
        seg_bytes, (o_ws, s_ws), (o, fs) = _run_both(wl)
        assert seg_bytes > 0, f"{name}: expected the segment path"
        assert np.array_equal(to_host(o), to_host(o_ws)), f"{name}: outputs differ"
        assert np.array_equal(fs.cpu().numpy(), s_ws.cpu().numpy()), f"{name}: states differ"
        pairs = [(0, h) for h in range(Hv)]
        ref = oracle_prefill_batch(wl, pairs)
        oh = to_host(o)
        ox = np.concatenate([oh[0, :, h] for (_, h) in pairs])
        orf = np.concatenate([ref[p][0] for p in pairs])
        e_o = check(ox, orf, f32_inputs=False, out_bf16=True, what=f"{name} outputs")
        e_s = check(fs.cpu().numpy()[0].astype(np.float64), np.stack([ref[p][1] for p in pairs]),
                    f32_inputs=False, out_bf16=False, what=f"{name} states")
        print(f"{name} ({decay}): segment workspace {seg_bytes} B; err o {e_o:.2e}, "
              f"state {e_s:.2e}", flush=True)


def test_noalloc_without_segments():
    """A call the single pass serves (no scratch): same result as the other entry."""
    wl = W.prefill_dense("noalloc_c", 83, 2, 300, 2, 4, 128, 128, W.BF16, 64, decay="slow",
                         initial_state="random")
    seg_bytes, (o_ws, s_ws), (o, fs) = _run_both(wl)
    assert seg_bytes == 0
    assert np.array_equal(to_host(o), to_host(o_ws))
    assert np.array_equal(fs.cpu().numpy(), s_ws.cpu().numpy())


def test_noalloc_packed_slot_cache_two_calls():
    """Packed sequences on a slot cache (the device-planned segment path): each call
    equals the workspace entry point's bit for bit, the second on fewer tokens."""
    import torch
    import gated_delta_rule_71_amd as gdr
    for name, seed, lengths in (("noalloc_p1", 84, [15000, 9000]), ("noalloc_p2", 85, [9000])):
        wl = W.prefill_packed(name, seed, lengths, 2, 4, 128, 128, W.BF16, 64, decay="slow",
                              num_slots=4, slot_init="random")
        d = [to_dev(getattr(wl, n)) for n in ("q", "k", "v", "g", "beta")]
        cu, idx = to_dev(wl.cu_seqlens), to_dev(wl.state_indices)
        probe = gdr.prefill_args(*d, cu_seqlens=cu, state_indices=idx,
                                 initial_state=to_dev(wl.initial_state),
                                 out=torch.empty(1, dtype=torch.bfloat16, device="cuda"))
        assert int(gdr.library().gdr_prefill_workspace_bytes(probe)) > 0, name
        c_ws = to_dev(wl.initial_state)
        o_ws, _ = gdr.chunk_gated_delta_rule(*d, initial_state=c_ws, cu_seqlens=cu,
                                             state_indices=idx)
        c = to_dev(wl.initial_state)
        o = torch.full_like(o_ws, float("nan"))
        gdr.chunk_gated_delta_rule_noalloc(*d, out=o, initial_state=c, final_state=c,
                                           cu_seqlens=cu, state_indices=idx)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(o), to_host(o_ws)), f"{name}: outputs differ"
        assert torch.equal(c, c_ws), f"{name}: slot caches differ"
        print(f"{name}: packed noalloc equals the workspace entry", flush=True)
