"""The oracle's several-tokens decode against the recurrence run as a prefill:
T decode tokens from a slot equal a T-token prefill from that slot's state, and
one token equals the single-token decode."""
from __future__ import annotations

import numpy as np

import oracle


def _inputs(seed, n=4, T=6, Hk=1, Hv=2, D=8, n_h=1):
    r = np.random.default_rng(seed)
    unit = lambda s: (lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True))(
        r.standard_normal(s))
    q = unit((n, T, Hk, D))
    k = unit((n, T, n_h, Hk, D))
    v = r.standard_normal((n, T, n_h, Hv, D))
    g = -r.uniform(0, 1, (n, T, Hv))
    beta = r.uniform(0, 1, (n, T, n_h, Hv))
    cache = r.standard_normal((7, Hv, D, D))
    return q, k, v, g, beta, cache


def _close(a, b, tol, what):
    err = float(np.max(np.abs(a - b) / np.maximum(1.0, np.abs(b))))
    assert err <= tol, f"{what}: {err:.3e}"


def test_tokens_equal_prefill():
    for n_h in (1, 2):
        q, k, v, g, beta, cache = _inputs(31 + n_h, n_h=n_h)
        idx = np.array([5, -1, 2, 0])
        before = cache.copy()
        o, states = oracle.decode_tokens(q, k, v, g, beta, cache, batch_indices=idx,
                                         num_householder=n_h)
        for i, r in enumerate(idx):
            s0 = before[max(r, 0)][None]
            op, fp = oracle.prefill(q[i:i + 1], k[i:i + 1], v[i:i + 1], g[i:i + 1],
                                    beta[i:i + 1], initial_state=s0, output_final_state=True,
                                    num_householder=n_h)
            _close(o[i], op[0], 1e-12, f"outputs request {i}")
            _close(states[i, -1], fp[0], 1e-12, f"last state request {i}")
            for t in range(q.shape[1]):
                _, ft = oracle.prefill(q[i:i + 1, :t + 1], k[i:i + 1, :t + 1],
                                       v[i:i + 1, :t + 1], g[i:i + 1, :t + 1],
                                       beta[i:i + 1, :t + 1], initial_state=s0,
                                       output_final_state=True, num_householder=n_h)
                _close(states[i, t], ft[0], 1e-12, f"state after token {t} request {i}")
            if r >= 0:
                _close(cache[r], fp[0], 1e-12, f"slot {r}")
        untouched = [s for s in range(cache.shape[0]) if s not in idx[idx >= 0]]
        assert np.array_equal(cache[untouched], before[untouched])


def test_one_token_equals_decode():
    q, k, v, g, beta, cache = _inputs(33, T=1)
    c1, c2 = cache.copy(), cache.copy()
    idx = np.array([3, 1, -1, 6])
    o1, _ = oracle.decode_tokens(q, k, v, g, beta, c1, batch_indices=idx)
    o2 = oracle.decode(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], c2, batch_indices=idx)
    assert np.array_equal(o1[:, 0], o2) and np.array_equal(c1, c2)
