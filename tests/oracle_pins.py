"""Pins that tie the CPU oracle to facts fixed by the mathematics, not by itself.

Each pin takes the oracle's ctypes library handle (so the same battery can be
run against deliberately broken builds of the oracle, see test_oracle_mutants)
and raises AssertionError when the oracle disagrees with:
  * a hand-worked example (tests/golden/worked_example_k2v2.json),
  * closed forms of special cases (beta = 0, one token, K = V = 1),
  * exact identities of the Householder step (unit keys, orthonormal keys),
  * linearity, scale, grouping, packing, slot and continuity invariants,
  * the independent chunked evaluation (oracle/chunked.py) at many chunk sizes.
Everything here uses K = V so that a broken oracle build cannot index out of
bounds.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

import oracle
from oracle.chunked import chunked_prefill

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _unit(rng, shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _problem(seed, B=1, T=12, Hk=1, Hv=1, D=6, n_h=1, decay=0.3, h0=True):
    """Random fp64 inputs (batched layout)."""
    r = _rng(seed)
    q = _unit(r, (B, T, Hk, D))
    k = _unit(r, (B, T, n_h, Hk, D))
    v = r.standard_normal((B, T, n_h, Hv, D))
    g = -decay * r.uniform(0.0, 1.0, (B, T, Hv))
    beta = r.uniform(0.05, 0.95, (B, T, n_h, Hv))
    s0 = 0.5 * r.standard_normal((B, Hv, D, D)) if h0 else None
    return q, k, v, g, beta, s0


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = np.max(np.abs(a - b) / np.maximum(1.0, np.abs(b))) if a.size else 0.0
    assert err <= tol, f"{what}: max err {err:.3e} > {tol:.1e}"


# --------------------------------------------------------------------------------------

def pin_worked_example(lib):
    with open(os.path.join(GOLDEN, "worked_example_k2v2.json")) as f:
        ex = json.load(f)
    inp, exp_ = ex["inputs"], ex["expected"]

    def arr(x):
        return np.array([[float(Fraction(c)) for c in row] for row in x])

    q, k, v = arr(inp["q"]), arr(inp["k"]), arr(inp["v"])
    beta = np.array([float(Fraction(b)) for b in inp["beta"]])
    g = np.log(np.array([float(Fraction(a)) for a in inp["alpha"]]))
    scale = float(Fraction(inp["scale"]))
    o, fs = oracle.prefill(q[None, :, None], k[None, :, None], v[None, :, None],
                           g[None, :, None], beta[None, :, None], scale=scale,
                           output_final_state=True, lib=lib)
    _close(o[0, :, 0], arr(exp_["o"]), 1e-15, "worked example o")
    _close(fs[0, 0], arr(exp_["final_state"]), 1e-15, "worked example final state")
    _, fs1 = oracle.prefill(q[None, :1, None], k[None, :1, None], v[None, :1, None],
                            g[None, :1, None], beta[None, :1, None], scale=scale,
                            output_final_state=True, lib=lib)
    _close(fs1[0, 0], arr(exp_["state_after_t1"]), 1e-15, "worked example state t=1")


def pin_beta_zero_g_zero_is_identity(lib):
    q, k, v, g, beta, s0 = _problem(1, T=9, D=5)
    o, fs = oracle.prefill(q, k, v, 0 * g, 0 * beta, scale=0.7, initial_state=s0,
                           output_final_state=True, lib=lib)
    assert np.array_equal(fs, s0), "beta = 0, g = 0 must leave the state bit-identical"
    # o_t = scale * S_0 q_t with S_0 = H0^T
    _close(o[0, :, 0], 0.7 * q[0, :, 0] @ s0[0, 0], 1e-13, "beta=0 g=0 output")


def pin_beta_zero_closed_form(lib):
    q, k, v, g, beta, s0 = _problem(2, T=11, D=5, decay=2.0)
    o, fs = oracle.prefill(q, k, v, g, 0 * beta, scale=1.3, initial_state=s0,
                           output_final_state=True, lib=lib)
    G = np.cumsum(g[0, :, 0])
    _close(fs[0, 0], np.exp(G[-1]) * s0[0, 0], 1e-13, "beta=0 final state")
    want = 1.3 * np.exp(G)[:, None] * (q[0, :, 0] @ s0[0, 0])
    _close(o[0, :, 0], want, 1e-13, "beta=0 outputs")


def pin_single_token_closed_form(lib):
    q, k, v, g, beta, _ = _problem(3, T=1, D=7)
    o, fs = oracle.prefill(q, k, v, g, beta, scale=0.9, output_final_state=True, lib=lib)
    kk, vv, qq, b = k[0, 0, 0, 0], v[0, 0, 0, 0], q[0, 0, 0], beta[0, 0, 0, 0]
    _close(o[0, 0, 0], 0.9 * b * (kk @ qq) * vv, 1e-14, "one token output")
    _close(fs[0, 0], b * np.outer(kk, vv), 1e-14, "one token state")


def pin_scalar_recurrence(lib):
    """K = V = 1: s_t = a_t s_{t-1} + b_t, a_t = e^{g_t}(1 - beta k^2), b_t = beta v k."""
    r = _rng(4)
    T = 15
    q = r.standard_normal((1, T, 1, 1))
    k = r.uniform(-1.2, 1.2, (1, T, 1, 1))
    v = r.standard_normal((1, T, 1, 1))
    g = -r.uniform(0, 1, (1, T, 1))
    beta = r.uniform(0, 1, (1, T, 1))
    s0 = np.array([[[[0.37]]]])
    o, fs = oracle.prefill(q, k, v, g, beta, scale=1.0, initial_state=s0,
                           output_final_state=True, lib=lib)
    a = np.exp(g[0, :, 0]) * (1.0 - beta[0, :, 0] * k[0, :, 0, 0] ** 2)
    b = beta[0, :, 0] * v[0, :, 0, 0] * k[0, :, 0, 0]
    for t in range(T):
        # closed form: s_t = (prod_{u<=t} a_u) s_0 + sum_{i<=t} (prod_{i<u<=t} a_u) b_i
        s_t = np.prod(a[: t + 1]) * 0.37 + sum(np.prod(a[i + 1: t + 1]) * b[i]
                                               for i in range(t + 1))
        _close(o[0, t, 0, 0], s_t * q[0, t, 0, 0], 1e-13, f"scalar output t={t}")
    _close(fs[0, 0, 0, 0], s_t, 1e-13, "scalar final state")


def pin_unit_key_projection(lib):
    """For |k| = 1: S_t k = e^g (1 - beta) S_{t-1} k + beta v, S_t x = e^g S_{t-1} x (x ⟂ k)."""
    q, k, v, g, beta, s0 = _problem(5, T=6, D=6)
    S_prev = s0[0, 0].T.copy()       # V x K
    h = s0
    for t in range(6):
        _, h = oracle.prefill(q[:, t:t + 1], k[:, t:t + 1], v[:, t:t + 1], g[:, t:t + 1],
                              beta[:, t:t + 1], initial_state=h, output_final_state=True,
                              lib=lib)
        S = h[0, 0].T
        kt, vt = k[0, t, 0, 0], v[0, t, 0, 0]
        a, b = np.exp(g[0, t, 0]), beta[0, t, 0, 0]
        _close(S @ kt, a * (1 - b) * (S_prev @ kt) + b * vt, 1e-13, "unit key direction")
        x = _rng(50 + t).standard_normal(6)
        x -= (x @ kt) * kt
        _close(S @ x, a * (S_prev @ x), 1e-13, "orthogonal direction")
        S_prev = S.copy()


def pin_orthonormal_retrieval(lib):
    """Orthonormal keys, beta = 1, g = 0, zero start: every stored value comes back."""
    r = _rng(6)
    D = 8
    Qm, _ = np.linalg.qr(r.standard_normal((D, D)))
    keys = Qm.T                                   # rows orthonormal
    vals = r.standard_normal((D, D))
    k = keys[None, :, None, :]
    v = vals[None, :, None, :]
    o, fs = oracle.prefill(k.copy(), k, v, np.zeros((1, D, 1)), np.ones((1, D, 1)),
                           scale=2.0, output_final_state=True, lib=lib)
    S = fs[0, 0].T
    _close(keys @ S.T, vals, 1e-13, "retrieval S k_j = v_j")
    _close(o[0, :, 0], 2.0 * vals, 1e-13, "query k_t right after writing it returns v_t")


def pin_linearity(lib):
    q, k, v, g, beta, s0 = _problem(7, T=10, D=5)
    _, _, v2, _, _, s02 = _problem(8, T=10, D=5)
    o1, f1 = oracle.prefill(q, k, v, g, beta, initial_state=s0, output_final_state=True, lib=lib)
    o2, f2 = oracle.prefill(q, k, v2, g, beta, initial_state=s02, output_final_state=True,
                            lib=lib)
    o3, f3 = oracle.prefill(q, k, v - 2.5 * v2, g, beta, initial_state=s0 - 2.5 * s02,
                            output_final_state=True, lib=lib)
    _close(o3, o1 - 2.5 * o2, 1e-12, "linear in (v, H0): outputs")
    _close(f3, f1 - 2.5 * f2, 1e-12, "linear in (v, H0): state")


def pin_scale(lib):
    q, k, v, g, beta, s0 = _problem(9, T=7, D=16)
    o1, _ = oracle.prefill(q, k, v, g, beta, scale=1.0, initial_state=s0, lib=lib)
    o2, _ = oracle.prefill(q, k, v, g, beta, scale=-0.3, initial_state=s0, lib=lib)
    od, _ = oracle.prefill(q, k, v, g, beta, initial_state=s0, lib=lib)
    _close(o2, -0.3 * o1, 1e-13, "output proportional to scale")
    _close(od, 0.25 * o1, 1e-13, "default scale 1/sqrt(16)")


def pin_l2norm_flag(lib):
    """With the flag on, rescaling q and k rows by positive factors changes nothing."""
    q, k, v, g, beta, s0 = _problem(10, T=8, D=6)
    r = _rng(11)
    cq = r.uniform(2, 5, q.shape[:-1] + (1,))
    ck = r.uniform(2, 5, k.shape[:-1] + (1,))
    o1, f1 = oracle.prefill(q, k, v, g, beta, initial_state=s0, output_final_state=True,
                            use_qk_l2norm=True, lib=lib)
    o2, f2 = oracle.prefill(q * cq, k * ck, v, g, beta, initial_state=s0,
                            output_final_state=True, use_qk_l2norm=True, lib=lib)
    _close(o2, o1, 1e-5, "l2norm flag output")
    _close(f2, f1, 1e-5, "l2norm flag state")
    o3, _ = oracle.prefill(q * cq, k * ck, v, g, beta, initial_state=s0, lib=lib)
    assert np.max(np.abs(o3 - o1)) > 1e-2, "without the flag, rescaled rows must matter"


def pin_l2norm_epsilon(lib):
    """Where the norm's epsilon sits.  A row x = a e_0 with a^2 = 1e-6 normalises to
    e_0 a / sqrt(a^2 + 1e-6) = e_0 / sqrt(2) when the epsilon is added under the
    square root; with it outside (a / (|a| + 1e-6)) or left out the component is
    ~0.999 or 1.  One token from a zero state then gives the closed form
    o = scale beta (k^ . q^) v = scale beta v / 2 and H = beta k^ v^T."""
    D = 4
    a = 1e-3
    q = np.zeros((1, 1, 1, D))
    k = np.zeros((1, 1, 1, 1, D))
    q[..., 0] = a
    k[..., 0] = -a                      # sign kept: k^ = -e_0 / sqrt(2)
    v = np.array([1.0, -2.0, 0.5, 3.0]).reshape(1, 1, 1, 1, D)
    g = np.array([-0.7]).reshape(1, 1, 1)
    beta = np.array([0.6]).reshape(1, 1, 1, 1)
    scale = 0.25
    o, fs = oracle.prefill(q, k, v, g, beta, scale=scale, output_final_state=True,
                           use_qk_l2norm=True, lib=lib)
    _close(o[0, 0, 0], scale * 0.6 * (-0.5) * v[0, 0, 0, 0], 1e-12, "l2norm epsilon output")
    h = np.zeros((D, D))
    h[0] = 0.6 * (-1.0 / np.sqrt(2.0)) * v[0, 0, 0, 0]
    _close(fs[0, 0], h, 1e-12, "l2norm epsilon state")


def pin_grouped_heads(lib):
    """Hk = 2, Hv = 4: value head h reads q/k head h // 2 (contiguous groups)."""
    q, k, v, g, beta, s0 = _problem(12, T=9, Hk=2, Hv=4, D=5)
    o, f = oracle.prefill(q, k, v, g, beta, initial_state=s0, output_final_state=True, lib=lib)
    rep = [0, 0, 1, 1]
    o2, f2 = oracle.prefill(q[:, :, rep], k[:, :, :, rep], v, g, beta, initial_state=s0,
                            output_final_state=True, lib=lib)
    _close(o, o2, 0, "grouped heads outputs")
    _close(f, f2, 0, "grouped heads state")


def pin_packed_equals_separate(lib):
    q, k, v, g, beta, _ = _problem(13, T=23, Hk=2, Hv=2, D=4)
    cu = np.array([0, 5, 5, 17, 23])
    s0 = 0.5 * _rng(14).standard_normal((4, 2, 4, 4))
    o, f = oracle.prefill(q, k, v, g, beta, cu_seqlens=cu, initial_state=s0,
                          output_final_state=True, lib=lib)
    for n in range(4):
        a, b = cu[n], cu[n + 1]
        on, fn = oracle.prefill(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b],
                                initial_state=s0[n:n + 1], output_final_state=True, lib=lib)
        _close(o[:, a:b], on, 0, f"packed seq {n} output")
        _close(f[n:n + 1], fn, 0, f"packed seq {n} state")
    # a batch of B sequences is the packed layout with uniform boundaries
    qb, kb, vb, gb, bb, sb = _problem(15, B=3, T=6, D=4)
    ob, fb = oracle.prefill(qb, kb, vb, gb, bb, initial_state=sb, output_final_state=True,
                            lib=lib)
    flat = [x.reshape((1, -1) + x.shape[2:]) for x in (qb, kb, vb, gb, bb)]
    of, ff = oracle.prefill(*flat, cu_seqlens=np.arange(4) * 6, initial_state=sb,
                            output_final_state=True, lib=lib)
    _close(of.reshape(ob.shape), ob, 0, "batched == uniform cu_seqlens")
    _close(ff, fb, 0, "batched == uniform cu_seqlens (state)")


def pin_chunked_matches_naive(lib):
    """The chunked evaluation equals the per-token recurrence for any chunk size."""
    q, k, v, g, beta, s0 = _problem(16, T=203, D=8, decay=0.05)
    o, f = oracle.prefill(q, k, v, g, beta, initial_state=s0, output_final_state=True, lib=lib)
    for C in (1, 7, 16, 64, 128, 256):
        oc, fc = chunked_prefill(q, k, v, g, beta, chunk_rows=C, initial_state=s0)
        _close(oc, o, 1e-11, f"chunked C={C} outputs")
        _close(fc, f, 1e-11, f"chunked C={C} state")
    # with two Householder sub-steps per token; chunks may split a token's sub-steps
    q, k, v, g, beta, s0 = _problem(17, T=61, D=8, n_h=2, decay=0.05)
    o, f = oracle.prefill(q, k, v, g, beta, initial_state=s0, output_final_state=True,
                          num_householder=2, lib=lib)
    for C in (1, 3, 16, 64):
        oc, fc = chunked_prefill(q, k, v, g, beta, chunk_rows=C, initial_state=s0,
                                 num_householder=2)
        _close(oc, o, 1e-11, f"chunked GDP C={C} outputs")
        _close(fc, f, 1e-11, f"chunked GDP C={C} state")


def pin_product_variant(lib):
    """Gated delta product == gated delta rule on interleaved rows (decay on sub-step 0)."""
    q, k, v, g, beta, s0 = _problem(18, T=10, D=5, n_h=2)
    o, f = oracle.prefill(q, k, v, g, beta, initial_state=s0, output_final_state=True,
                          num_householder=2, lib=lib)
    # rows r = 2t + j; the output of token t is read on row 2t + 1
    T = 10
    kr = k.reshape(1, 2 * T, 1, 5)
    vr = v.reshape(1, 2 * T, 1, 5)
    br = beta.reshape(1, 2 * T, 1)
    gr = np.zeros((1, 2 * T, 1))
    gr[:, 0::2] = g
    qr = np.repeat(q, 2, axis=1)
    orr, fr = oracle.prefill(qr, kr, vr, gr, br, initial_state=s0, output_final_state=True,
                             lib=lib)
    _close(o, orr[:, 1::2], 1e-13, "GDP == interleaved GDN outputs")
    _close(f, fr, 1e-13, "GDP == interleaved GDN state")
    # a second sub-step with beta = 0 is the plain rule on sub-step 0
    b0 = beta.copy()
    b0[:, :, 1] = 0
    o2, f2 = oracle.prefill(q, k, v, g, b0, initial_state=s0, output_final_state=True,
                            num_householder=2, lib=lib)
    o1, f1 = oracle.prefill(q, k[:, :, :1], v[:, :, :1], g, beta[:, :, :1], initial_state=s0,
                            output_final_state=True, lib=lib)
    _close(o2, o1, 1e-13, "GDP with beta_2 = 0 outputs")
    _close(f2, f1, 1e-13, "GDP with beta_2 = 0 state")


def pin_continuity(lib):
    """prefill(L) then decode steps == prefill(L + m); a split prefill == unsplit."""
    q, k, v, g, beta, s0 = _problem(19, B=1, T=20, Hk=2, Hv=4, D=6)
    o, f = oracle.prefill(q, k, v, g, beta, initial_state=s0, output_final_state=True, lib=lib)
    L = 13
    _, fa = oracle.prefill(q[:, :L], k[:, :L], v[:, :L], g[:, :L], beta[:, :L],
                           initial_state=s0, output_final_state=True, lib=lib)
    ob, fb = oracle.prefill(q[:, L:], k[:, L:], v[:, L:], g[:, L:], beta[:, L:],
                            initial_state=fa, output_final_state=True, lib=lib)
    _close(ob, o[:, L:], 1e-13, "split prefill outputs")
    _close(fb, f, 1e-13, "split prefill state")
    cache = fa.copy()
    for t in range(L, 20):
        od = oracle.decode(q[0, t:t + 1], k[0, t:t + 1, 0], v[0, t:t + 1, 0], g[0, t:t + 1],
                           beta[0, t:t + 1, 0], cache, lib=lib)
        _close(od[0], o[0, t], 1e-13, f"decode step t={t}")
    _close(cache, f, 1e-13, "decode steps == prefill state")


def pin_prefill_slots(lib):
    """Slot cache: read slot max(idx, 0), write only idx >= 0, other slots untouched."""
    q, k, v, g, beta, _ = _problem(20, T=14, Hk=1, Hv=2, D=4)
    # sequence 1 is zero-length padding, sequence 3 is padding with tokens
    cu = np.array([0, 4, 4, 9, 14])
    cache = _rng(21).standard_normal((5, 2, 4, 4))
    before = cache.copy()
    idx = np.array([3, -1, 1, -1])
    o, _ = oracle.prefill(q, k, v, g, beta, cu_seqlens=cu, initial_state=cache,
                          state_indices=idx, final_state_out=cache, lib=lib)
    assert np.array_equal(cache[[0, 2, 4]], before[[0, 2, 4]]), "untouched slots changed"
    a, b = cu[3], cu[4]
    op, _ = oracle.prefill(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b],
                           initial_state=before[0:1], lib=lib)
    _close(o[:, a:b], op, 0, "padding sequence reads slot 0")
    for n, s in ((0, 3), (2, 1)):
        a, b = cu[n], cu[n + 1]
        on, fn = oracle.prefill(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b],
                                initial_state=before[s:s + 1], output_final_state=True,
                                lib=lib)
        _close(o[:, a:b], on, 0, f"slot seq {n} output")
        _close(cache[s:s + 1], fn, 0, f"slot seq {n} state")


def pin_decode_slots(lib):
    """Decode: -1 reads slot 0 (clamped) and writes nothing; others update in place."""
    r = _rng(22)
    n, Hk, Hv, D = 5, 1, 2, 4
    q = _unit(r, (n, Hk, D))
    k = _unit(r, (n, Hk, D))
    v = r.standard_normal((n, Hv, D))
    g = -r.uniform(0, 1, (n, Hv))
    beta = r.uniform(0, 1, (n, Hv))
    cache = r.standard_normal((7, Hv, D, D))
    before = cache.copy()
    idx = np.array([4, -1, 2, 6, -1])
    out = oracle.decode(q, k, v, g, beta, cache, batch_indices=idx, lib=lib)
    assert np.array_equal(cache[[0, 1, 3, 5]], before[[0, 1, 3, 5]]), "untouched slots changed"
    for i in range(n):
        s = max(idx[i], 0)
        one = before[s:s + 1].copy()
        oi = oracle.decode(q[i:i + 1], k[i:i + 1], v[i:i + 1], g[i:i + 1], beta[i:i + 1], one,
                           lib=lib)
        _close(out[i], oi[0], 0, f"decode row {i} output")
        if idx[i] >= 0:
            _close(cache[idx[i]], one[0], 0, f"decode row {i} state")
    # the single step is the prefill of one token from that state
    o1, f1 = oracle.prefill(q[None, :1], k[None, :1], v[None, :1], g[None, :1], beta[None, :1],
                            initial_state=before[4:5], output_final_state=True, lib=lib)
    _close(out[0], o1[0, 0], 1e-14, "decode == one-token prefill (output)")
    _close(cache[4], f1[0], 1e-14, "decode == one-token prefill (state)")


ALL_PINS = [
    pin_worked_example,
    pin_beta_zero_g_zero_is_identity,
    pin_beta_zero_closed_form,
    pin_single_token_closed_form,
    pin_scalar_recurrence,
    pin_unit_key_projection,
    pin_orthonormal_retrieval,
    pin_linearity,
    pin_scale,
    pin_l2norm_flag,
    pin_l2norm_epsilon,
    pin_grouped_heads,
    pin_packed_equals_separate,
    pin_chunked_matches_naive,
    pin_product_variant,
    pin_continuity,
    pin_prefill_slots,
    pin_decode_slots,
]
