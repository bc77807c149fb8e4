"""The backward oracle (oracle/backward.py) against facts that do not come from itself.

* its forward pass equals the pinned C oracle (so it differentiates the definition);
* its gradients equal central finite differences of the C oracle's forward;
* closed forms: one token from a zero state; beta = 0 (pure decay of H0);
* the chunked form equals it at many chunk sizes, packed and grouped;
* planted mistakes in the chunked form are each caught by the chunked check.
"""
import types

import numpy as np
import pytest

import oracle
from oracle import backward as OB

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def _unit(r, shape):
    x = r.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _problem(seed, B=1, T=9, Hk=1, Hv=2, K=4, V=3, decay=0.4, h0=True):
    r = np.random.default_rng(seed)
    q = _unit(r, (B, T, Hk, K))
    k = _unit(r, (B, T, Hk, K))
    v = r.standard_normal((B, T, Hv, V))
    g = -decay * r.uniform(0.0, 1.0, (B, T, Hv))
    beta = r.uniform(0.05, 0.95, (B, T, Hv))
    s0 = 0.5 * r.standard_normal((B, Hv, K, V)) if h0 else None
    do = r.standard_normal((B, T, Hv, V))
    dht = r.standard_normal((B, Hv, K, V))
    return q, k, v, g, beta, s0, do, dht


def _maxdiff(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return float(np.max(np.abs(a - b) / np.maximum(1.0, np.abs(b)))) if a.size else 0.0


def test_forward_equals_c_oracle():
    q, k, v, g, beta, s0, do, dht = _problem(1, B=2, T=11, Hk=2, Hv=4, K=5, V=5)
    res = OB.prefill_backward(q, k, v, g, beta, do, dht, initial_state=s0, scale=0.7,
                              return_forward=True)
    o, fs = oracle.prefill(q, k, v, g, beta, initial_state=s0, scale=0.7,
                           output_final_state=True)
    assert _maxdiff(res["o"], o) < 1e-13
    assert _maxdiff(res["final_state"], fs) < 1e-13


def _loss_c(q, k, v, g, beta, s0, do, dht, scale):
    """<o, do> + <H_T, dht> evaluated with the C oracle (an independent forward)."""
    o, fs = oracle.prefill(q, k, v, g, beta, initial_state=s0, scale=scale,
                           output_final_state=True)
    return float(np.sum(o * do) + np.sum(fs * dht))


@pytest.mark.parametrize("seed", [2, 3])
def test_gradients_equal_finite_differences(seed):
    q, k, v, g, beta, s0, do, dht = _problem(seed, T=6, Hk=1, Hv=2, K=3, V=3)
    scale = 0.8
    res = OB.prefill_backward(q, k, v, g, beta, do, dht, initial_state=s0, scale=scale)
    args = {"q": q, "k": k, "v": v, "g": g, "beta": beta, "s0": s0}
    grad_name = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "s0": "dh0"}
    eps = 1e-6
    for name, x in args.items():
        fd = np.zeros_like(x)
        for i in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[i] += eps
            xm[i] -= eps
            ap, am = dict(args, **{name: xp}), dict(args, **{name: xm})
            fd[i] = (_loss_c(**ap, do=do, dht=dht, scale=scale)
                     - _loss_c(**am, do=do, dht=dht, scale=scale)) / (2 * eps)
        err = _maxdiff(res[grad_name[name]], fd)
        assert err < 1e-7, (name, err)


def test_single_token_closed_form():
    # one token from a zero state: o = scale beta (k.q) v, H = beta k v^T
    r = np.random.default_rng(4)
    K = V = 5
    q, k = _unit(r, (1, 1, 1, K)), _unit(r, (1, 1, 1, K))
    v, do = r.standard_normal((1, 1, 1, V)), r.standard_normal((1, 1, 1, V))
    dht = r.standard_normal((1, 1, K, V))
    g, beta, scale = np.array([[[-0.3]]]), np.array([[[0.6]]]), 0.9
    res = OB.prefill_backward(q, k, v, g, beta, do, dht, scale=scale)
    qq, kk, vv, dd, D = q[0, 0, 0], k[0, 0, 0], v[0, 0, 0], do[0, 0, 0], dht[0, 0]
    b, c = 0.6, kk @ qq
    assert _maxdiff(res["dv"][0, 0, 0], scale * b * c * dd + b * D.T @ kk) < 1e-14
    assert _maxdiff(res["dq"][0, 0, 0], scale * b * (dd @ vv) * kk) < 1e-14
    assert _maxdiff(res["dk"][0, 0, 0], scale * b * (dd @ vv) * qq + b * D @ vv) < 1e-14
    assert _maxdiff(res["dbeta"][0, 0, 0], scale * c * (dd @ vv) + kk @ D @ vv) < 1e-14
    assert abs(res["dg"][0, 0, 0]) < 1e-15      # a zero state does not see the decay


def test_beta_zero_closed_form():
    # beta = 0: H_t = e^{G_t} H0 and o_t = scale e^{G_t} H0^T q_t
    q, k, v, g, beta, s0, do, dht = _problem(5, T=7, Hk=1, Hv=1, K=4, V=4)
    beta = np.zeros_like(beta)
    scale = 0.6
    res = OB.prefill_backward(q, k, v, g, beta, do, dht, initial_state=s0, scale=scale)
    G = np.cumsum(g[0, :, 0])
    H0 = s0[0, 0]
    assert np.max(np.abs(res["dv"])) == 0.0 and np.max(np.abs(res["dk"])) < 1e-15
    dq = scale * np.exp(G)[:, None] * (do[0, :, 0] @ H0.T)
    assert _maxdiff(res["dq"][0, :, 0], dq) < 1e-14
    dh0 = scale * np.einsum("t,tk,tv->kv", np.exp(G), q[0, :, 0], do[0, :, 0]) \
        + np.exp(G[-1]) * dht[0, 0]
    assert _maxdiff(res["dh0"][0, 0], dh0) < 1e-14
    per_t = scale * np.exp(G) * np.einsum("tk,kv,tv->t", q[0, :, 0], H0, do[0, :, 0])
    per_t[-1] += np.exp(G[-1]) * np.sum(dht[0, 0] * H0)
    assert _maxdiff(res["dg"][0, :, 0], np.cumsum(per_t[::-1])[::-1]) < 1e-13


@pytest.mark.parametrize("C", [1, 5, 16, 64])
def test_chunked_equals_autograd_packed_grouped(C):
    r = np.random.default_rng(6)
    lens = [0, 23, 70, 1]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, beta, _, do, _ = _problem(7, B=1, T=int(cu[-1]), Hk=2, Hv=4, K=5, V=4)
    s0 = 0.5 * r.standard_normal((len(lens), 4, 5, 4))
    dht = r.standard_normal((len(lens), 4, 5, 4))
    a = OB.prefill_backward(q, k, v, g, beta, do, dht, cu_seqlens=cu, initial_state=s0)
    c = OB.chunked_backward(q, k, v, g, beta, do, dht, chunk_size=C, cu_seqlens=cu,
                            initial_state=s0)
    for n in NAMES:
        assert _maxdiff(c[n], a[n]) < 1e-12, n


def test_packed_equals_separate_and_groups_sum():
    q, k, v, g, beta, s0, do, dht = _problem(8, B=2, T=8, Hk=1, Hv=2, K=3, V=3)
    batched = OB.prefill_backward(q, k, v, g, beta, do, dht, initial_state=s0)
    cu = np.array([0, 8, 16])
    packed = OB.prefill_backward(*(x.reshape((1, 16) + x.shape[2:]) for x in (q, k, v, g, beta)),
                                 do.reshape(1, 16, 2, 3), dht, cu_seqlens=cu, initial_state=s0)
    for n in NAMES:
        assert _maxdiff(packed[n].reshape(batched[n].shape), batched[n]) < 1e-14, n
    # a shared q/k head gets the sum of the gradients of its repeated copies
    rep = OB.prefill_backward(np.repeat(q, 2, axis=2), np.repeat(k, 2, axis=2), v, g, beta, do,
                              dht, initial_state=s0)
    assert _maxdiff(batched["dq"][:, :, 0], rep["dq"].sum(axis=2)) < 1e-14
    assert _maxdiff(batched["dk"][:, :, 0], rep["dk"].sum(axis=2)) < 1e-14


# Planted mistakes in the chunked form: each must break its agreement with autograd.
CHUNK_MUTANTS = {
    "dR_not_transposed": ("dR = Tm.T @ dD", "dR = Tm @ dD"),
    "no_state_path_in_dD": ("dD = P.T @ dOc + Kt @ dHn", "dD = P.T @ dOc"),
    "dA_sign": ("dA = -np.where(strict, dR @ D.T, 0.0)", "dA = np.where(strict, dR @ D.T, 0.0)"),
    "no_w_term": ("dG[-1] += np.exp(G[-1]) * np.sum(dHn * H0) + w.sum()",
                  "dG[-1] += np.exp(G[-1]) * np.sum(dHn * H0)"),
    "forward_cumsum_dg": ("dg = np.cumsum(dG[::-1])[::-1]", "dg = np.cumsum(dG)"),
    "no_decay_on_dH0": ("dH0 = np.exp(G[-1]) * dHn", "dH0 = dHn"),
}


@pytest.mark.parametrize("name", sorted(CHUNK_MUTANTS))
def test_chunked_check_rejects_mutant(name):
    import inspect
    src = inspect.getsource(OB)
    old, new = CHUNK_MUTANTS[name]
    assert src.count(old) == 1, name
    mod = types.ModuleType("backward_mutant")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new), "backward_mutant", "exec"), mod.__dict__)
    q, k, v, g, beta, s0, do, dht = _problem(9, T=20, Hk=1, Hv=1, K=4, V=4)
    a = OB.prefill_backward(q, k, v, g, beta, do, dht, initial_state=s0)
    c = mod.chunked_backward(q, k, v, g, beta, do, dht, chunk_size=8, initial_state=s0)
    assert max(_maxdiff(c[n], a[n]) for n in NAMES) > 1e-6, name


def test_torch_gates_equal_gate_oracle():
    import torch
    r = np.random.default_rng(20)
    alpha = r.standard_normal((50, 3)) * 30
    b = r.standard_normal((50, 3)) * 30
    A_log, dt_bias = np.log(r.uniform(1, 16, 3)), r.standard_normal(3)
    g, beta = OB.gates_torch(*(torch.tensor(x) for x in (alpha, b, A_log, dt_bias)))
    g0, b0 = oracle.gates(alpha, b, A_log, dt_bias)
    assert _maxdiff(g.numpy(), g0) < 1e-14 and _maxdiff(beta.numpy(), b0) < 1e-15


def _raw_problem(seed):
    q, k, v, g, beta, s0, do, dht = _problem(seed, T=6, Hk=1, Hv=2, K=3, V=3)
    r = np.random.default_rng(seed + 100)
    q, k = 2.5 * q + 0.3 * r.standard_normal(q.shape), 0.7 * k + 0.2 * r.standard_normal(k.shape)
    alpha, b = r.standard_normal(g.shape), r.standard_normal(beta.shape)
    A_log, dt_bias = np.log(r.uniform(1, 4, 2)), np.log(np.expm1(r.uniform(0.01, 0.1, 2)))
    return q, k, v, alpha, b, s0, do, dht, A_log, dt_bias


def test_l2norm_and_raw_gate_gradients_equal_finite_differences():
    q, k, v, alpha, b, s0, do, dht, A_log, dt_bias = _raw_problem(21)
    scale = 0.8
    res = OB.prefill_backward(q, k, v, alpha, b, do, dht, initial_state=s0, scale=scale,
                              use_qk_l2norm=True, A_log=A_log, dt_bias=dt_bias)
    args = {"q": q, "k": k, "v": v, "alpha": alpha, "b": b, "A_log": A_log, "dt_bias": dt_bias}
    name = {"q": "dq", "k": "dk", "v": "dv", "alpha": "dg", "b": "dbeta", "A_log": "dA_log",
            "dt_bias": "ddt_bias"}

    def loss(a):
        gg, bb = oracle.gates(a["alpha"], a["b"], a["A_log"], a["dt_bias"])
        o, fs = oracle.prefill(a["q"], a["k"], a["v"], gg, bb, initial_state=s0, scale=scale,
                               output_final_state=True, use_qk_l2norm=True)
        return float(np.sum(o * do) + np.sum(fs * dht))

    eps = 1e-6
    for nm, x in args.items():
        fd = np.zeros_like(x)
        for i in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[i] += eps
            xm[i] -= eps
            fd[i] = (loss(dict(args, **{nm: xp})) - loss(dict(args, **{nm: xm}))) / (2 * eps)
        err = _maxdiff(res[name[nm]], fd)
        assert err < 1e-6, (nm, err)


def test_l2norm_gradient_is_orthogonal_to_the_input():
    # the loss sees q only through q / |q| (up to the 1e-6 inside the root), so the
    # gradient has no component along q
    q, k, v, alpha, b, s0, do, dht, A_log, dt_bias = _raw_problem(22)
    res = OB.prefill_backward(q, k, v, alpha, b, do, dht, initial_state=s0, use_qk_l2norm=True)
    for x, dx in ((q, res["dq"]), (k, res["dk"])):
        dots = np.sum(x * dx, axis=-1)
        assert np.max(np.abs(dots)) < 1e-5 * np.max(np.abs(dx)), np.max(np.abs(dots))


def _gdp_problem(seed, B=1, T=5, Hk=1, Hv=2, K=3, V=3, n_h=2):
    r = np.random.default_rng(seed)
    q = _unit(r, (B, T, Hk, K))
    k = _unit(r, (B, T, n_h, Hk, K))
    v = r.standard_normal((B, T, n_h, Hv, V))
    g = -0.4 * r.uniform(0.0, 1.0, (B, T, Hv))
    beta = r.uniform(0.05, 0.95, (B, T, n_h, Hv))
    s0 = 0.5 * r.standard_normal((B, Hv, K, V))
    do = r.standard_normal((B, T, Hv, V))
    dht = r.standard_normal((B, Hv, K, V))
    return q, k, v, g, beta, s0, do, dht


def test_gdp_forward_equals_c_oracle():
    q, k, v, g, beta, s0, do, dht = _gdp_problem(30, B=2, T=7, Hk=1, Hv=2, K=4, V=4)
    res = OB.prefill_backward(q, k, v, g, beta, do, dht, initial_state=s0, return_forward=True)
    o, fs = oracle.prefill(q, k, v, g, beta, initial_state=s0, output_final_state=True,
                           num_householder=2)
    assert _maxdiff(res["o"], o) < 1e-13 and _maxdiff(res["final_state"], fs) < 1e-13


def test_gdp_gradients_equal_finite_differences():
    q, k, v, g, beta, s0, do, dht = _gdp_problem(31)
    res = OB.prefill_backward(q, k, v, g, beta, do, dht, initial_state=s0)
    args = {"q": q, "k": k, "v": v, "g": g, "beta": beta, "s0": s0}
    name = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "s0": "dh0"}

    def loss(a):
        o, fs = oracle.prefill(a["q"], a["k"], a["v"], a["g"], a["beta"], initial_state=a["s0"],
                               output_final_state=True, num_householder=2)
        return float(np.sum(o * do) + np.sum(fs * dht))

    eps = 1e-6
    for nm, x in args.items():
        fd = np.zeros_like(x)
        for i in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[i] += eps
            xm[i] -= eps
            fd[i] = (loss(dict(args, **{nm: xp})) - loss(dict(args, **{nm: xm}))) / (2 * eps)
        assert _maxdiff(res[name[nm]], fd) < 1e-7, nm


def test_gdp_gradients_equal_gdn_on_interleaved_rows():
    # the product is the delta rule on rows t*n_h + j with the decay on each token's
    # first row and the query (and dO) on its last row; the gradients map row by row
    q, k, v, g, beta, s0, do, dht = _gdp_problem(32, T=6, Hk=1, Hv=2, K=4, V=4)
    gdp = OB.prefill_backward(q, k, v, g, beta, do, dht, initial_state=s0)
    B, T, n_h = q.shape[0], q.shape[1], 2
    R = T * n_h
    qr = np.zeros((B, R) + q.shape[2:])
    qr[:, n_h - 1::n_h] = q
    dor = np.zeros((B, R) + do.shape[2:])
    dor[:, n_h - 1::n_h] = do
    gr = np.zeros((B, R, g.shape[-1]))
    gr[:, 0::n_h] = g
    gdn = OB.prefill_backward(qr, k.reshape((B, R) + k.shape[3:]), v.reshape((B, R) + v.shape[3:]),
                              gr, beta.reshape(B, R, -1), dor, dht, initial_state=s0)
    assert _maxdiff(gdp["dq"], gdn["dq"][:, n_h - 1::n_h]) < 1e-13
    assert _maxdiff(gdp["dg"], gdn["dg"][:, 0::n_h]) < 1e-13
    for nm in ("dk", "dv", "dbeta"):
        assert _maxdiff(gdp[nm], gdn[nm].reshape(gdp[nm].shape)) < 1e-13, nm
    assert _maxdiff(gdp["dh0"], gdn["dh0"]) < 1e-13
