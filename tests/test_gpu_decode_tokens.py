"""Several decode tokens per request (speculative tokens) with intermediate
states, through the C ABI (marked gpu).  Compared with the oracle's token-by-token
decode (oracle.decode_tokens, pinned to the prefill of the same tokens)."""
from __future__ import annotations

import numpy as np
import pytest

from gated_delta_rule_71_amd import workloads as W
from parity import check, gate_values, to_dev, to_host

pytestmark = pytest.mark.gpu


def _workload(seed, *, n=16, T=5, slots=24, Hk=2, Hv=4, K=128, V=128, n_h=1, dtype=W.BF16,
              pad=3):
    rng = np.random.default_rng(seed)
    ax = (n, T) + ((n_h,) if n_h > 1 else ())
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    q = unit(rng.standard_normal((n, T, Hk, K), dtype=np.float32))
    k = unit(rng.standard_normal(ax + (Hk, K), dtype=np.float32))
    v = rng.standard_normal(ax + (Hv, V), dtype=np.float32)
    g = (-rng.uniform(0, 1, (n, T, Hv))).astype(np.float32)
    beta = rng.uniform(0, 1, ax + (Hv,)).astype(np.float32)
    cache = (0.1 * rng.standard_normal((slots, Hv, K, V))).astype(np.float32)
    idx = (1 + rng.permutation(slots - 1)[:n]).astype(np.int32)   # slot 0 not written
    idx[rng.permutation(n)[:pad]] = -1
    return W.DecodeWorkload("tokens", dtype, W.store(q, dtype), W.store(k, dtype),
                            W.store(v, dtype), g, beta, cache, idx)


def _run(wl, *, intermediate=True, out_dtype="f32"):
    import torch
    import gated_delta_rule_71_amd as gdr
    n, T = wl.q.shape[:2]
    Hv, K, V = wl.cache.shape[1:]
    cache = to_dev(wl.cache)
    inter = (torch.full((n, T, Hv, K, V), float("nan"), device="cuda") if intermediate
             else None)
    od = {"f32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
    o = gdr.ssm_decode(to_dev(wl.q), to_dev(wl.k), to_dev(wl.v), to_dev(wl.g), to_dev(wl.beta),
                       cache, batch_indices=to_dev(wl.batch_indices), out_dtype=od,
                       A_log=to_dev(wl.A_log), dt_bias=to_dev(wl.dt_bias),
                       intermediate_ssm_state=inter)
    torch.cuda.synchronize()
    return o, cache, inter


def _check(wl, o, cache, inter, *, n_h=1, out_bf16=False):
    import oracle
    f32 = wl.dtype == W.F32
    ref_cache = W.as_f64(wl.cache).copy()
    g, beta = gate_values(wl)
    n, T = wl.q.shape[:2]
    k = W.as_f64(wl.k).reshape((n, T, n_h) + wl.k.shape[-2:])
    v = W.as_f64(wl.v).reshape((n, T, n_h) + wl.v.shape[-2:])
    ro, rs = oracle.decode_tokens(W.as_f64(wl.q), k, v, g, beta.reshape(n, T, n_h, -1),
                                  ref_cache, batch_indices=wl.batch_indices,
                                  num_householder=n_h)
    check(to_host(o), ro, f32_inputs=f32, out_bf16=out_bf16, what="outputs (all tokens)")
    real = wl.batch_indices >= 0
    written = wl.batch_indices[real]
    after = cache.cpu().numpy()
    check(after[written].astype(np.float64), ref_cache[written], f32_inputs=f32, out_bf16=False,
          what="final slot states")
    untouched = np.setdiff1d(np.arange(wl.cache.shape[0]), written)
    assert np.array_equal(after[untouched].view(np.uint32), wl.cache[untouched].view(np.uint32))
    if inter is not None:
        ih = inter.cpu().numpy()
        check(ih[real].astype(np.float64), rs[real], f32_inputs=f32, out_bf16=False,
              what="intermediate states")
        assert np.all(np.isnan(ih[~real])), "padding requests write no intermediate state"


@pytest.mark.parametrize("case", [dict(dtype=W.BF16), dict(dtype=W.F32), dict(dtype=W.BF16, n_h=2),
                                  dict(dtype=W.F32, K=64, V=64, T=9)],
                         ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_decode_tokens(case):
    wl = _workload(61, **case)
    o, cache, inter = _run(wl)
    _check(wl, o, cache, inter, n_h=case.get("n_h", 1))


def test_decode_tokens_raw_gates_bf16_out():
    wl = W.with_raw_gates(_workload(62, T=4), 62)
    o, cache, inter = _run(wl, out_dtype="bf16")
    _check(wl, o, cache, inter, out_bf16=True)


def test_decode_tokens_without_intermediate():
    wl = _workload(63, T=3)
    o, cache, _ = _run(wl, intermediate=False)
    _check(wl, o, cache, None)


def test_decode_one_token_form_is_the_single_step():
    """[n, 1, ...] inputs give bitwise the outputs and slots of the [n, ...] call."""
    import torch
    import gated_delta_rule_71_amd as gdr
    wl = _workload(64, T=1)
    o1, c1, _ = _run(wl, intermediate=False)
    c2 = to_dev(wl.cache)
    o2 = gdr.ssm_decode(to_dev(wl.q[:, 0]), to_dev(wl.k[:, 0]), to_dev(wl.v[:, 0]),
                        to_dev(wl.g[:, 0]), to_dev(wl.beta[:, 0]), c2,
                        batch_indices=to_dev(wl.batch_indices), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, 0], o2) and torch.equal(c1, c2)
