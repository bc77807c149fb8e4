"""The oracle's gate function (oracle/gating.py) against facts fixed by the
mathematics: closed forms, a library routine for softplus and for the logistic
function, exact identities, and the per-head broadcast; then the same pins
against planted mistakes, so that the battery is not vacuous."""
from __future__ import annotations

import math

import numpy as np
import pytest
import scipy.special

import oracle
from oracle import gating as G


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = float(np.max(np.abs(a - b) / np.maximum(1.0, np.abs(b)))) if a.size else 0.0
    assert err <= tol, f"{what}: max err {err:.3e} > {tol:.1e}"


def pin_closed_forms(fn):
    # softplus(0) = ln 2, A = exp(0) = 1, sigmoid(0) = 1/2
    g, b = fn(np.zeros((1, 1)), np.zeros((1, 1)), np.zeros(1), np.zeros(1))
    _close(g, [[-math.log(2.0)]], 1e-15, "g at alpha = dt_bias = A_log = 0")
    _close(b, [[0.5]], 1e-15, "beta at b = 0")
    # A_log = ln 3 triples the decay; sigmoid(ln 3) = 3/4; softplus(ln 3) = ln 4
    g, b = fn(np.full((1, 1), math.log(3.0)), np.full((1, 1), math.log(3.0)),
              np.full(1, math.log(3.0)), np.zeros(1))
    _close(g, [[-3.0 * math.log(4.0)]], 1e-15, "g at alpha = ln 3, A = 3")
    _close(b, [[0.75]], 1e-15, "beta at b = ln 3")
    # dt_bias adds to alpha before the softplus
    g1, _ = fn(np.full((1, 1), 0.25), np.zeros((1, 1)), np.zeros(1), np.full(1, 0.5))
    g2, _ = fn(np.full((1, 1), 0.75), np.zeros((1, 1)), np.zeros(1), np.zeros(1))
    _close(g1, g2, 1e-15, "dt_bias shifts alpha")


def pin_library_routines(fn):
    x = np.concatenate([np.linspace(-745.0, 709.0, 4001),
                        [-1e-12, 0.0, 1e-12, 30.0, 37.0, 750.0, 1e3, 1e4]])
    g, b = fn(x[None], x[None], np.zeros(x.size), np.zeros(x.size))
    _close(-g[0], np.logaddexp(0.0, x), 4e-16, "softplus vs numpy.logaddexp")
    _close(b[0], scipy.special.expit(x), 4e-16, "sigmoid vs scipy.special.expit")


def pin_identities(fn):
    rng = np.random.default_rng(7)
    x = rng.normal(0.0, 6.0, 2000)
    z = np.zeros(x.size)
    gp, bp = fn(x[None], x[None], z, z)
    gm, bm = fn(-x[None], -x[None], z, z)
    _close(-gp - (-gm), x[None], 2e-15, "softplus(x) - softplus(-x) = x")
    _close(bp + bm, np.ones((1, x.size)), 5e-16, "sigmoid(x) + sigmoid(-x) = 1")
    # softplus' = sigmoid (central difference)
    h = 1e-5
    ga, _ = fn((x + h)[None], x[None], z, z)
    gb, _ = fn((x - h)[None], x[None], z, z)
    _close((gb - ga) / (2 * h), bp, 1e-9, "softplus' = sigmoid")
    assert np.all(gp < 0) and np.all((bp > 0) & (bp < 1)), "ranges"


def pin_per_head_broadcast(fn):
    rng = np.random.default_rng(8)
    T, n_h, H = 5, 2, 3
    alpha = rng.standard_normal((T, H))
    b = rng.standard_normal((T, n_h, H))
    A_log = np.log(rng.uniform(1.0, 16.0, H))
    dt = np.log(np.expm1(rng.uniform(0.001, 0.1, H)))
    g, beta = fn(alpha, b, A_log, dt)
    for h in range(H):
        for t in range(T):
            gs, _ = fn(alpha[t:t + 1, h:h + 1], b[t:t + 1, 0, h:h + 1], A_log[h:h + 1], dt[h:h + 1])
            _close(g[t, h], gs[0, 0], 0, f"g head {h}")
            for s in range(n_h):
                _, bs = fn(alpha[t:t + 1, h:h + 1], b[t:t + 1, s, h:h + 1], A_log[h:h + 1],
                           dt[h:h + 1])
                _close(beta[t, s, h], bs[0, 0], 0, f"beta head {h}")


PINS = [pin_closed_forms, pin_library_routines, pin_identities, pin_per_head_broadcast]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_gate_pin(pin):
    pin(oracle.gates)


# plausible mistakes in a gate function; each must fail at least one pin
def _m_sign(a, b, A, d):
    g, be = G.gates(a, b, A, d)
    return -g, be


def _m_A_not_exp(a, b, A, d):
    return -np.asarray(A, dtype=np.float64) * G.softplus(np.asarray(a) + d), G.sigmoid(b)


def _m_log1p_x(a, b, A, d):
    x = np.asarray(a, dtype=np.float64) + d
    with np.errstate(invalid="ignore", divide="ignore"):
        return -np.exp(A) * np.log1p(np.abs(x)), G.sigmoid(b)


def _m_no_softplus(a, b, A, d):
    return -np.exp(A) * (np.asarray(a, dtype=np.float64) + d), G.sigmoid(b)


def _m_sigmoid_neg(a, b, A, d):
    g, _ = G.gates(a, b, A, d)
    return g, G.sigmoid(-np.asarray(b, dtype=np.float64))


def _m_dt_subtracted(a, b, A, d):
    return G.gates(a, b, A, -np.asarray(d, dtype=np.float64))


def _m_heads_reversed(a, b, A, d):
    return G.gates(a, b, np.asarray(A)[::-1], np.asarray(d)[::-1])


def _m_naive_softplus(a, b, A, d):
    x = np.asarray(a, dtype=np.float64) + d
    with np.errstate(over="ignore"):
        return -np.exp(A) * np.log(1.0 + np.exp(x)), G.sigmoid(b)


MUTANTS = [_m_sign, _m_A_not_exp, _m_log1p_x, _m_no_softplus, _m_sigmoid_neg, _m_dt_subtracted,
           _m_heads_reversed, _m_naive_softplus]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_gate_pins_reject_mutant(mutant):
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mutant)
        except (AssertionError, FloatingPointError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"mutant {mutant.__name__} passed every gate pin"
