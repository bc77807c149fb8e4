"""Seeded synthetic workloads for the gated delta rule.

Inputs only: this module draws random tensors with the shapes and value
distributions of the workloads the library is measured on, and holds none of the
recurrence's arithmetic.  Both the GPU path and the CPU oracle consume what it
makes, so it imports neither.

Value recipe (all draws from numpy's PCG64, one generator per workload, seed
given per workload, draw order fixed as written below):
  * q, k, v ~ N(0, 1) drawn in float32; q and k are divided by their L2 norm per
    (token, head) row in float32 before the cast to the input dtype;
  * beta = sigmoid(N(0, 1));
  * g = -A_h * softplus(x + dt_bias_h) with A_h ~ U(1, 16) per head,
    x ~ N(0, 1) per (token, head) and dt_bias_h = log(expm1(dt_h)),
    dt_h ~ U(0.001, 0.1) per head (the gate parametrisation of
    GatedDeltaNet._compute_gates / GatedDeltaProductMixer._compute_gating and the
    A_init_range / dt_min / dt_max defaults on the Megatron Core API pages
    "core.ssm.gated_delta_net.gdn" and "core.ssm.gated_delta_product");
    decay variants "slow" (g ~ -U(0, 0.05)) and "zero" (g = 0) exist so that
    state carried across chunks is not forgotten within one chunk;
  * states ~ N(0, 0.1) in float32 where a workload asks for a random state;
  * raw gate inputs (:func:`with_raw_gates`, for kernels that form the gates):
    alpha, b ~ N(0, 1) per (token, [sub-step,] head) in place of g and beta,
    A_log_h = log(A_h) with A_h ~ U(1, 16) and dt_bias_h = log(expm1(dt_h)) with
    dt_h ~ U(0.001, 0.1) (the inverse softplus of the time step), so that the
    gates they define follow the distribution above.
bf16 tensors are rounded from float32 with round-to-nearest-even and stored as
uint16 bit patterns; :func:`as_f64` gives the exact values both sides compute on.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


# ---- bf16 storage --------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def store(x32: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values -> storage array for ``dtype`` (float32, or uint16 bf16 bits)."""
    if dtype == F32:
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == BF16:
        return f32_to_bf16_bits(x32)
    raise ValueError(dtype)


def as_f64(a: np.ndarray, dtype: Optional[str] = None) -> np.ndarray:
    """Exact float64 values of a storage array (uint16 arrays are bf16 bits)."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def round_bf16_f32(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to bf16 and kept as float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


# ---- draws -------------------------------------------------------------------------

def _unit_rows(rng, shape):
    x = rng.standard_normal(shape, dtype=np.float32)
    x /= np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return x


def _gates(rng, T, H, decay, batch=1):
    """g [batch, T, H] (float32) for the chosen decay variant."""
    if decay == "config":
        A = rng.uniform(1.0, 16.0, size=H)
        dt = rng.uniform(0.001, 0.1, size=H)
        dt_bias = np.log(np.expm1(dt))
        x = rng.standard_normal((batch, T, H))
        g = -A * np.logaddexp(0.0, x + dt_bias)
    elif decay == "slow":
        g = -rng.uniform(0.0, 0.05, size=(batch, T, H))
    elif decay == "zero":
        g = np.zeros((batch, T, H))
    else:
        raise ValueError(decay)
    return g.astype(np.float32)


def _beta(rng, shape):
    return (1.0 / (1.0 + np.exp(-rng.standard_normal(shape)))).astype(np.float32)


# ---- workload containers ------------------------------------------------------------

@dataclass
class PrefillWorkload:
    name: str
    dtype: str                      # storage dtype of q, k, v
    q: np.ndarray                   # [B,T,Hk,K]
    k: np.ndarray                   # [B,T,Hk,K] or [B,T,n_h,Hk,K]
    v: np.ndarray                   # [B,T,Hv,V] or [B,T,n_h,Hv,V]
    g: np.ndarray                   # [B,T,Hv] float32
    beta: np.ndarray                # [B,T,Hv] or [B,T,n_h,Hv] float32
    chunk_size: int
    num_householder: int = 1
    cu_seqlens: Optional[np.ndarray] = None      # int32 [N+1]
    initial_state: Optional[np.ndarray] = None   # float32 [N or slots, Hv, K, V]
    state_indices: Optional[np.ndarray] = None   # int32 [N]
    output_final_state: bool = True
    meta: dict = field(default_factory=dict)
    A_log: Optional[np.ndarray] = None           # float32 [Hv]: g, beta are raw projections
    dt_bias: Optional[np.ndarray] = None         # float32 [Hv]

    @property
    def shape(self):
        B, T, Hk, K = self.q.shape
        return B, T, Hk, self.v.shape[-2], K, self.v.shape[-1]

    @property
    def num_seqs(self):
        return self.q.shape[0] if self.cu_seqlens is None else len(self.cu_seqlens) - 1

    @property
    def tokens(self):
        return self.q.shape[0] * self.q.shape[1]


@dataclass
class DecodeWorkload:
    name: str
    dtype: str
    q: np.ndarray                   # [n,Hk,K]
    k: np.ndarray                   # [n,Hk,K]
    v: np.ndarray                   # [n,Hv,V]
    g: np.ndarray                   # [n,Hv] float32
    beta: np.ndarray                # [n,Hv] float32
    cache: np.ndarray               # [slots,Hv,K,V] float32
    batch_indices: Optional[np.ndarray]  # int32 [n] (-1 = padding)
    meta: dict = field(default_factory=dict)
    A_log: Optional[np.ndarray] = None           # float32 [Hv]: g, beta are raw projections
    dt_bias: Optional[np.ndarray] = None         # float32 [Hv]


def with_raw_gates(wl, seed):
    """A copy of a prefill or decode workload whose g and beta are replaced by raw
    gate projections (alpha, b) and per-head A_log, dt_bias (see the recipe above)."""
    from dataclasses import replace
    rng = np.random.default_rng([seed, 0x6A7E])
    Hv = wl.g.shape[-1]
    A_log = np.log(rng.uniform(1.0, 16.0, size=Hv)).astype(np.float32)
    dt_bias = np.log(np.expm1(rng.uniform(0.001, 0.1, size=Hv))).astype(np.float32)
    alpha = rng.standard_normal(wl.g.shape, dtype=np.float32)
    b = rng.standard_normal(wl.beta.shape, dtype=np.float32)
    return replace(wl, name=wl.name + "_rawgates", g=alpha, beta=b, A_log=A_log,
                   dt_bias=dt_bias)


# ---- the measured workloads ---------------------------------------------------------

def prefill_dense(name, seed, B, T, Hk, Hv, K, V, dtype, chunk_size, *, decay="config",
                  initial_state="zeros", num_householder=1):
    """Batched prefill: B sequences of T tokens (GDN, or GDP with n_h sub-steps)."""
    rng = np.random.default_rng(seed)
    n_h = num_householder
    kshape = (B, T, Hk, K) if n_h == 1 else (B, T, n_h, Hk, K)
    vshape = (B, T, Hv, V) if n_h == 1 else (B, T, n_h, Hv, V)
    bshape = (B, T, Hv) if n_h == 1 else (B, T, n_h, Hv)
    q = store(_unit_rows(rng, (B, T, Hk, K)), dtype)
    k = store(_unit_rows(rng, kshape), dtype)
    v = store(rng.standard_normal(vshape, dtype=np.float32), dtype)
    beta = _beta(rng, bshape)
    g = _gates(rng, T, Hv, decay, batch=B)
    if initial_state == "zeros":
        h0 = None
    elif initial_state == "random":
        h0 = (0.1 * rng.standard_normal((B, Hv, K, V), dtype=np.float32)).astype(np.float32)
    else:
        raise ValueError(initial_state)
    return PrefillWorkload(name, dtype, q, k, v, g, beta, chunk_size, n_h,
                           initial_state=h0, meta={"seed": seed, "decay": decay})


def prefill_packed(name, seed, lengths, Hk, Hv, K, V, dtype, chunk_size, *, decay="config",
                   num_slots=None, slot_init="zeros"):
    """Packed varlen prefill (B = 1) writing each sequence's state to its own slot.

    Slots: a cache of ``num_slots`` (default 2N); sequence n uses slot perm[n] of a
    random N-subset; those slots start at zero (fresh requests) or random, the
    others hold random sentinel values that must come back unchanged.
    """
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, dtype=np.int64)
    N = len(lengths)
    cu = np.zeros(N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    q = store(_unit_rows(rng, (1, T, Hk, K)), dtype)
    k = store(_unit_rows(rng, (1, T, Hk, K)), dtype)
    v = store(rng.standard_normal((1, T, Hv, V), dtype=np.float32), dtype)
    beta = _beta(rng, (1, T, Hv))
    g = _gates(rng, T, Hv, decay)
    S = int(num_slots if num_slots is not None else 2 * N)
    slots = rng.permutation(S)[:N].astype(np.int32)
    cache = rng.standard_normal((S, Hv, K, V), dtype=np.float32)
    if slot_init == "zeros":
        cache[slots] = 0.0
    elif slot_init == "random":
        cache[slots] *= np.float32(0.1)
    else:
        raise ValueError(slot_init)
    return PrefillWorkload(name, dtype, q, k, v, g, beta, chunk_size, 1, cu_seqlens=cu,
                           initial_state=cache, state_indices=slots,
                           meta={"seed": seed, "decay": decay, "lengths": lengths.tolist(),
                                 "num_slots": S})


def varlen_lengths(seed, num_seqs=8, max_len=8192):
    """Sequence lengths ~ U{1..max_len} (inclusive) for the packed workload."""
    rng = np.random.default_rng([seed, 0x5E9])
    return rng.integers(1, max_len + 1, size=num_seqs)


def config0(decay="config"):
    """fp32, B=1, T=256, H=2, K=V=64, chunk 64, zero initial state."""
    return prefill_dense("gdn_f32_B1_T256_H2_D64", 0, 1, 256, 2, 2, 64, 64, F32, 64, decay=decay)


def config1(decay="config", T=4096, B=4):
    """bf16, B=4, T=4096, H=16, K=V=128, chunk 64, random initial state."""
    return prefill_dense(f"gdn_bf16_B{B}_T{T}_H16_D128", 1, B, T, 16, 16, 128, 128, BF16, 64,
                         decay=decay, initial_state="random")


def config2(decay="config", num_seqs=8, max_len=8192, lengths=None):
    """Packed varlen bf16: 8 sequences of U{1..8192} tokens, 16 q/k heads, 32 v heads."""
    if lengths is None:
        lengths = varlen_lengths(2, num_seqs, max_len)
    return prefill_packed(f"gdn_varlen_bf16_N{len(lengths)}_Hk16_Hv32_D128", 2, lengths, 16, 32,
                          128, 128, BF16, 64, decay=decay, num_slots=2 * len(lengths))


def config4(decay="config", T=65536, H=32):
    """GDP with 2 Householder sub-steps, bf16, B=1, T=65536, H=32, chunk 128 tokens."""
    return prefill_dense(f"gdp2_bf16_B1_T{T}_H{H}_D128", 4, 1, T, H, H, 128, 128, BF16, 128,
                         decay=decay, initial_state="random", num_householder=2)


def long_packed(T=65536):
    """One long request packed alone (cu_seqlens) over a 4-slot cache: T tokens,
    16 q/k heads, 32 v heads, K = V = 128, bf16, chunk 64."""
    return prefill_packed(f"gdn_packed_bf16_N1_T{T}_Hk16_Hv32_D128", 5, [T], 16, 32, 128, 128,
                          BF16, 64, num_slots=4, slot_init="random")


def config3(n=128, num_slots=256, Hk=16, Hv=32, K=128, V=128, num_padding=16, seed=3):
    """Decode: one bf16 token per request over a [256,32,128,128] fp32 slot cache.

    g and beta are rounded to bf16 values and stored as float32, so reading them as
    either dtype gives the same numbers.  ``batch_indices``: an ordered random
    subset of the slots for the real requests, -1 at ``num_padding`` random rows.
    """
    rng = np.random.default_rng(seed)
    q = store(_unit_rows(rng, (n, Hk, K)), BF16)
    k = store(_unit_rows(rng, (n, Hk, K)), BF16)
    v = store(rng.standard_normal((n, Hv, V), dtype=np.float32), BF16)
    g = round_bf16_f32(_gates(rng, n, Hv, "config")[0])
    beta = round_bf16_f32(_beta(rng, (n, Hv)))
    cache = np.empty((num_slots, Hv, K, V), dtype=np.float32)
    chunk = 16
    for s0 in range(0, num_slots, chunk):     # bounded temporaries for the 512 MiB cache
        s1 = min(s0 + chunk, num_slots)
        cache[s0:s1] = rng.standard_normal((s1 - s0, Hv, K, V), dtype=np.float32)
        cache[s0:s1] *= np.float32(0.1)
    real = rng.permutation(num_slots)[: n - num_padding].astype(np.int32)
    pad_rows = np.sort(rng.permutation(n)[:num_padding])
    idx = np.full(n, -1, dtype=np.int32)
    idx[np.setdiff1d(np.arange(n), pad_rows)] = real
    return DecodeWorkload(f"decode_bf16_n{n}_slots{num_slots}_Hk{Hk}_Hv{Hv}_D{K}", BF16, q, k,
                          v, g, beta, cache, idx, meta={"seed": seed, "padding_rows":
                                                        pad_rows.tolist()})


@dataclass
class BackwardWorkload:
    """Inputs of a backward call: the forward's inputs (dense initial states) plus
    the upstream gradients of the outputs and of the final state."""
    fwd: PrefillWorkload
    do: np.ndarray                  # [B,T,Hv,V] storage dtype, ~ N(0,1)
    dht: Optional[np.ndarray]       # [N,Hv,K,V] float32 ~ N(0,1), or None


def backward_workload(name, seed, *, Hk, Hv, D, dtype, B=1, T=None, lengths=None,
                      decay="config", initial_state=True, final_grad=True, num_householder=1):
    """Backward inputs: batched (B, T) or packed (``lengths``, B = 1), q/k/v/g/beta as
    in the forward recipe (k, v, beta per Householder sub-step when
    ``num_householder`` > 1), initial states ~ N(0, 0.1), dO and dH_T ~ N(0, 1)."""
    rng = np.random.default_rng([seed, 0xBAC])
    if lengths is not None:
        lengths = np.asarray(lengths, dtype=np.int64)
        N = len(lengths)
        cu = np.zeros(N + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
        B, T = 1, int(cu[-1])
    else:
        N, cu = B, None
    n_h = int(num_householder)
    sub = () if n_h == 1 else (n_h,)
    q = store(_unit_rows(rng, (B, T, Hk, D)), dtype)
    k = store(_unit_rows(rng, (B, T) + sub + (Hk, D)), dtype)
    v = store(rng.standard_normal((B, T) + sub + (Hv, D), dtype=np.float32), dtype)
    beta = _beta(rng, (B, T) + sub + (Hv,))
    g = _gates(rng, T, Hv, decay, batch=B)
    h0 = (0.1 * rng.standard_normal((N, Hv, D, D), dtype=np.float32)).astype(np.float32) \
        if initial_state else None
    fwd = PrefillWorkload(name, dtype, q, k, v, g, beta, 64 // n_h, n_h, cu_seqlens=cu,
                          initial_state=h0, meta={"seed": seed, "decay": decay})
    do = store(rng.standard_normal((B, T, Hv, D), dtype=np.float32), dtype)
    dht = rng.standard_normal((N, Hv, D, D), dtype=np.float32) if final_grad else None
    return BackwardWorkload(fwd, do, dht)
