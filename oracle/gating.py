"""Gates from raw projections, fp64 — TEST INFRASTRUCTURE ONLY (part of the oracle).

GatedDeltaNet._compute_gates (Megatron Core API page
"core.ssm.gated_delta_net.gdn") computes the per-head log-decay g and the write
strength beta from the per-token projections (the "alpha" and "beta" outputs of
the fused input projection) and the per-head parameters A_log and dt_bias; with
the kernel-fused inputs of _prepare_inference_inputs the kernel does it.  The
pages name the parameters but print no formula.  Reading: the softplus time-step
parametrisation the names denote (A = exp(A_log) > 0 as in A_init_range, a
time step softplus(alpha + dt_bias) with dt_bias the inverse softplus of a step
in [dt_min, dt_max] as on page "core.ssm.gated_delta_product"):

    g_t    = -exp(A_log[h]) * softplus(alpha_t + dt_bias[h]),
    beta_t = sigmoid(b_t) = 1 / (1 + exp(-b_t)),
    softplus(x) = log(1 + exp(x)).

Written from these definitions in float64; softplus is split at 0 so that exp
never overflows: for x > 0, log(1 + e^x) = x + log(1 + e^-x).
"""
from __future__ import annotations

import numpy as np


def softplus(x):
    x = np.asarray(x, dtype=np.float64)
    neg = np.minimum(x, 0.0)                 # exp of a non-positive number only
    pos = np.maximum(x, 0.0)
    return pos + np.log1p(np.exp(neg - pos))


def sigmoid(b):
    b = np.asarray(b, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-b))


def gates(alpha, b, A_log, dt_bias):
    """(g, beta) in float64.  ``A_log`` and ``dt_bias`` hold one value per value
    head and broadcast along the last (head) axis of ``alpha`` and ``b``."""
    alpha = np.asarray(alpha, dtype=np.float64)
    A_log = np.asarray(A_log, dtype=np.float64)
    dt_bias = np.asarray(dt_bias, dtype=np.float64)
    g = -np.exp(A_log) * softplus(alpha + dt_bias)
    return g, sigmoid(b)
