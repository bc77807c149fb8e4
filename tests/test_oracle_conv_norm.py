"""The oracle's causal conv and gated RMS norm (oracle/conv_norm.py) against
facts fixed by the mathematics — shift and identity kernels, linearity, the
packing and chunking invariants, the logistic function of scipy, exact
normalisation identities — and the same pins against planted mistakes."""
from __future__ import annotations

import math

import numpy as np
import pytest
import scipy.special

from oracle import conv_norm as CN


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = float(np.max(np.abs(a - b) / np.maximum(1.0, np.abs(b)))) if a.size else 0.0
    assert err <= tol, f"{what}: {err:.3e} > {tol:.1e}"


def _data(seed, T=23, C=8, W=4, S=5):
    r = np.random.default_rng(seed)
    return (r.standard_normal((T, C)), r.standard_normal((C, W)), r.standard_normal(C),
            r.standard_normal((S, C, W - 1)))


# ---- conv pins (take the module-like namespace `m` so mutants can stand in) --------

def pin_conv_identity_and_shift(m):
    x, _, _, st = _data(1)
    C, W = x.shape[1], 4
    eye = np.zeros((C, W)); eye[:, W - 1] = 1.0
    y, _ = m.causal_conv1d(x, eye, None, conv_state=st, state_indices=[2], activation=None)
    _close(y, x, 0, "last tap = identity")
    shift = np.zeros((C, W)); shift[:, 0] = 1.0
    y, s1 = m.causal_conv1d(x, shift, None, conv_state=st, state_indices=[2], activation=None)
    _close(y[W - 1:], x[:-(W - 1)], 0, "first tap = shift by W-1")
    _close(y[:W - 1], st[2].T[:W - 1], 0, "shift reads the state before the start")
    _close(s1[2], x[-(W - 1):].T, 0, "new state = last W-1 inputs")


def pin_conv_silu_library(m):
    x, w, b, _ = _data(2)
    y0, _ = m.causal_conv1d(x, w, b, activation=None)
    y1, _ = m.causal_conv1d(x, w, b, activation="silu")
    _close(y1, y0 * scipy.special.expit(y0), 1e-15, "silu vs scipy.special.expit")


def pin_conv_linearity(m):
    r = np.random.default_rng(3)
    x1, w, _, _ = _data(4)
    x2 = r.standard_normal(x1.shape)
    y1, _ = m.causal_conv1d(x1, w, None, activation=None)
    y2, _ = m.causal_conv1d(x2, w, None, activation=None)
    y3, _ = m.causal_conv1d(2.0 * x1 - 3.0 * x2, w, None, activation=None)
    _close(y3, 2.0 * y1 - 3.0 * y2, 1e-13, "linear before the activation")


def pin_conv_packing_and_chunking(m):
    x, w, b, st = _data(5, T=30)
    cu = [0, 2, 2, 17, 30]
    idx = [3, -1, 0, 4]
    y, s = m.causal_conv1d(x, w, b, cu_seqlens=cu, conv_state=st, state_indices=idx)
    for n in range(4):
        row = max(idx[n], 0)
        yn, sn = m.causal_conv1d(x[cu[n]:cu[n + 1]], w, b, conv_state=st[row:row + 1],
                                 state_indices=[0])
        _close(y[cu[n]:cu[n + 1]], yn, 0, f"packed sequence {n}")
        if idx[n] >= 0:
            _close(s[idx[n]], sn[0], 0, f"state of sequence {n}")
    untouched = [1, 2]
    _close(s[untouched], st[untouched], 0, "rows nobody writes")
    # chunked: the second half continues from the first half's state (incl. a 2-token chunk)
    for cut in (2, 11):
        ya, sa = m.causal_conv1d(x[:cut], w, b, conv_state=st[:1], state_indices=[0])
        yb, sb = m.causal_conv1d(x[cut:], w, b, conv_state=sa, state_indices=[0])
        yf, sf = m.causal_conv1d(x, w, b, conv_state=st[:1], state_indices=[0])
        _close(np.concatenate([ya, yb]), yf, 1e-15, f"chunked at {cut}")
        _close(sb, sf, 0, f"state chunked at {cut}")


def pin_conv_decode_is_prefill(m):
    x, w, b, st = _data(6, T=6)
    xs = x[None]                                     # one request, 6 tokens
    y, s, wins = m.causal_conv1d_update(xs, st, w, b, batch_indices=[4])
    yp, sp = m.causal_conv1d(x, w, b, conv_state=st, state_indices=[4])
    _close(y[0], yp, 1e-15, "decode tokens = prefill")
    _close(s[4], sp[4], 0, "decode state = prefill state")
    for t in range(6):
        _, st_t = m.causal_conv1d(x[:t + 1], w, b, conv_state=st, state_indices=[4])
        _close(wins[0, t], st_t[4], 0, f"window after token {t}")


CONV_PINS = [pin_conv_identity_and_shift, pin_conv_silu_library, pin_conv_linearity,
             pin_conv_packing_and_chunking, pin_conv_decode_is_prefill]


# ---- norm pins ----------------------------------------------------------------------

def pin_norm_constant_group(m):
    a, eps = 0.3, 1e-5
    x = np.full((1, 2, 64), a)
    z = np.full((1, 2, 64), 40.0)                      # silu(40) = 40 to double precision
    w = np.linspace(0.5, 1.5, 128)
    y = m.gated_rmsnorm(x, z, w, eps=eps, norm_before_gate=True)
    _close(y.reshape(-1), a / math.sqrt(a * a + eps) * w * 40.0, 1e-14, "constant, gate after")
    y = m.gated_rmsnorm(x, z, w, eps=eps, norm_before_gate=False)
    u = a * 40.0
    _close(y.reshape(-1), u / math.sqrt(u * u + eps) * w, 1e-14, "constant, gate before")


def pin_norm_unit_rms(m):
    r = np.random.default_rng(7)
    x = r.standard_normal((5, 3, 128)) * r.uniform(0.1, 10, (5, 3, 1))
    z = r.standard_normal((5, 3, 128))
    ones = np.ones(3 * 128)
    y = m.gated_rmsnorm(x, z, ones, eps=0.0, norm_before_gate=False)
    _close(np.sqrt(np.mean(y * y, axis=-1)), np.ones((5, 3)), 1e-13, "unit RMS, gate before")
    y = m.gated_rmsnorm(x, z, ones, eps=0.0, norm_before_gate=True)
    g = z * scipy.special.expit(z)
    _close(np.sqrt(np.mean((y / g) ** 2, axis=-1)), np.ones((5, 3)), 1e-10, "unit RMS, gate after")
    # scale invariance (eps = 0) and the weight applied per channel of each head
    y2 = m.gated_rmsnorm(7.0 * x, z, ones, eps=0.0, norm_before_gate=True)
    _close(y2, y, 1e-13, "scale invariance")
    wv = r.uniform(0.5, 2.0, 3 * 128)
    y3 = m.gated_rmsnorm(x, z, wv, eps=0.0, norm_before_gate=True)
    _close(y3, y * wv.reshape(3, 128), 1e-13, "per-channel weight")


def pin_norm_gate_zero(m):
    r = np.random.default_rng(8)
    x = r.standard_normal((2, 2, 64))
    z = np.zeros((2, 2, 64))                           # silu(0) = 0
    for nbg in (False, True):
        y = m.gated_rmsnorm(x, z, np.ones(128), eps=1e-5, norm_before_gate=nbg)
        _close(y, np.zeros_like(y), 0, f"zero gate ({nbg})")


NORM_PINS = [pin_norm_constant_group, pin_norm_unit_rms, pin_norm_gate_zero]


@pytest.mark.parametrize("pin", CONV_PINS + NORM_PINS, ids=lambda p: p.__name__)
def test_conv_norm_pin(pin):
    pin(CN)


# ---- planted mistakes ---------------------------------------------------------------

class _Mutant:
    def __init__(self, **over):
        self.causal_conv1d = CN.causal_conv1d
        self.causal_conv1d_update = CN.causal_conv1d_update
        self.gated_rmsnorm = CN.gated_rmsnorm
        self.__dict__.update(over)


def _conv_reversed_taps(x, w, b=None, **kw):
    return CN.causal_conv1d(x, np.asarray(w)[:, ::-1], b, **kw)


def _conv_no_state(x, w, b=None, **kw):
    kw = dict(kw)
    kw.pop("conv_state", None)
    y, _ = CN.causal_conv1d(x, w, b, **kw)
    return y, None if "state_indices" not in kw else np.zeros((8, x.shape[1], w.shape[1] - 1))


def _conv_sigmoid(x, w, b=None, activation="silu", **kw):
    y, s = CN.causal_conv1d(x, w, b, activation=None, **kw)
    return (scipy.special.expit(y) if activation == "silu" else y), s


def _norm_sum(x, z, w, eps=1e-5, norm_before_gate=False):
    x = np.asarray(x); z = np.asarray(z)
    u = x if norm_before_gate else x * CN.silu(z)
    y = u / np.sqrt(np.sum(u * u, axis=-1, keepdims=True) + eps) * np.asarray(w).reshape(x.shape[1:])
    return y * CN.silu(z) if norm_before_gate else y


def _norm_gate_swapped(x, z, w, eps=1e-5, norm_before_gate=False):
    return CN.gated_rmsnorm(x, z, w, eps=eps, norm_before_gate=not norm_before_gate)


def _norm_eps_outside(x, z, w, eps=1e-5, norm_before_gate=False):
    x = np.asarray(x); z = np.asarray(z)
    u = x if norm_before_gate else x * CN.silu(z)
    y = u / (np.sqrt(np.mean(u * u, axis=-1, keepdims=True)) + eps) * np.asarray(w).reshape(x.shape[1:])
    return y * CN.silu(z) if norm_before_gate else y


MUTANTS = {
    "conv_reversed_taps": _Mutant(causal_conv1d=_conv_reversed_taps),
    "conv_no_state": _Mutant(causal_conv1d=_conv_no_state),
    "conv_sigmoid_not_silu": _Mutant(causal_conv1d=_conv_sigmoid),
    "norm_sum_not_mean": _Mutant(gated_rmsnorm=_norm_sum),
    "norm_gate_swapped": _Mutant(gated_rmsnorm=_norm_gate_swapped),
    "norm_eps_outside_sqrt": _Mutant(gated_rmsnorm=_norm_eps_outside),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_conv_norm_pins_reject_mutant(name):
    failed = []
    for pin in CONV_PINS + NORM_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(MUTANTS[name])
        except (AssertionError, ValueError, TypeError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
