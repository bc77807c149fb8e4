"""Short causal conv and gated RMS norm, fp64 — TEST INFRASTRUCTURE ONLY (oracle).

The steps around the recurrence in a GatedDeltaNet / GatedDeltaProductMixer layer
(Megatron Core API pages "core.ssm.gated_delta_net.gdn" and
"core.ssm.gated_delta_product"):

* causal_conv1d / causal_conv1d_update — the depthwise causal convolution of
  width W (d_conv) over each sequence's tokens, channel by channel:
      y[t][c] = act(bias[c] + sum_j weight[c][j] * x[t - (W-1) + j][c]),
  the inputs before a sequence's start taken from its conv state (the W-1
  previous inputs, oldest first; conv_initial_states for chunked prefill, the
  cached window for decode), act = SiLU(u) = u / (1 + exp(-u)) or the identity.
  The sequence leaves its last W-1 inputs as the new state.
* gated_rmsnorm — RMSNormGated over groups of G elements (one head):
      norm_before_gate = False:  u = x * silu(z),  y = u / sqrt(mean(u^2) + eps) * w
      norm_before_gate = True:   y = x / sqrt(mean(x^2) + eps) * w * silu(z).
The pages name these steps (d_conv, conv_initial_states, _decode_conv,
ExtendedRMSNorm = RMSNormGated, norm_before_gate) without formulas; the forms
above are the standard definitions of those named operations.
"""
from __future__ import annotations

import numpy as np


def silu(u):
    u = np.asarray(u, dtype=np.float64)
    with np.errstate(over="ignore"):
        return u / (1.0 + np.exp(-u))


def _conv_sequence(x, state, weight, bias, act):
    """x [L, C]; state [C, W-1] -> (y [L, C], new state [C, W-1])."""
    W = weight.shape[1]
    ext = np.concatenate([state.T, x], axis=0)          # [W-1+L, C], oldest first
    L = x.shape[0]
    y = np.zeros((L, x.shape[1]))
    for t in range(L):
        window = ext[t:t + W]                            # inputs x[t-(W-1)] .. x[t]
        u = bias + np.sum(weight.T * window, axis=0)
        y[t] = silu(u) if act else u
    return y, ext[ext.shape[0] - (W - 1):].T.copy()


def causal_conv1d(x, weight, bias=None, *, cu_seqlens=None, conv_state=None,
                  state_indices=None, activation="silu"):
    """x [tokens, C]; weight [C, W]; returns (y [tokens, C], updated conv_state copy)."""
    x = np.asarray(x, dtype=np.float64)
    weight = np.asarray(weight, dtype=np.float64)
    C, W = weight.shape
    bias = np.zeros(C) if bias is None else np.asarray(bias, dtype=np.float64)
    cu = [0, x.shape[0]] if cu_seqlens is None else [int(c) for c in cu_seqlens]
    state = None if conv_state is None else np.array(conv_state, dtype=np.float64)
    new_state = None if state is None else state.copy()
    y = np.zeros_like(x)
    act = activation == "silu"
    for n in range(len(cu) - 1):
        t0, t1 = cu[n], cu[n + 1]
        row = n if state_indices is None else int(state_indices[n])
        s0 = np.zeros((C, W - 1)) if state is None else state[max(row, 0)]
        y[t0:t1], s1 = _conv_sequence(x[t0:t1], s0, weight, bias, act)
        if new_state is not None and row >= 0:
            new_state[row] = s1
    return y, new_state


def causal_conv1d_update(x, conv_state, weight, bias=None, *, batch_indices=None,
                         activation="silu"):
    """x [n, T, C]; conv_state [slots, C, W-1]; returns (y [n, T, C], updated state
    copy, windows [n, T, C, W-1] after each token).  Padding (-1) reads row 0 and
    writes nothing."""
    x = np.asarray(x, dtype=np.float64)
    weight = np.asarray(weight, dtype=np.float64)
    C, W = weight.shape
    bias = np.zeros(C) if bias is None else np.asarray(bias, dtype=np.float64)
    state = np.array(conv_state, dtype=np.float64)
    new_state = state.copy()
    n, T = x.shape[:2]
    idx = np.arange(n) if batch_indices is None else np.asarray(batch_indices)
    y = np.zeros_like(x)
    wins = np.zeros((n, T, C, W - 1))
    for i in range(n):
        s = state[max(int(idx[i]), 0)]
        for t in range(T):
            y[i, t:t + 1], s = _conv_sequence(x[i, t:t + 1], s, weight, bias,
                                              activation == "silu")
            wins[i, t] = s
        if idx[i] >= 0:
            new_state[int(idx[i])] = s
    return y, new_state, wins


def gated_rmsnorm(x, z, weight, *, eps=1e-5, norm_before_gate=False):
    """x, z [tokens, heads, G]; weight [heads * G]."""
    x = np.asarray(x, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64).reshape(x.shape[1:])
    u = x if norm_before_gate else x * silu(z)
    y = u / np.sqrt(np.mean(u * u, axis=-1, keepdims=True) + eps) * w
    return y * silu(z) if norm_before_gate else y
