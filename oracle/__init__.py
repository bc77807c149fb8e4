"""CPU oracle for the gated delta rule — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never imports, links or
calls it, and the two share no code.

Two independent CPU evaluations of the recurrence, both in fp64:

* :func:`prefill` / :func:`decode` — the definition, one token at a time, in
  plain C (``gdr_oracle.c``), OpenMP across independent (sequence, value head)
  pairs.  This is the oracle the GPU path is compared with.
* :func:`oracle.chunked.chunked_prefill` — the chunked (WY / UT transform)
  evaluation written with NumPy, used to check that chunking leaves the result
  unchanged for any chunk size.
* :func:`gates` (``oracle/gating.py``) — the gates g and beta from the raw
  per-token projections and the per-head parameters A_log and dt_bias.
* ``oracle/conv_norm.py`` — the short causal conv (prefill and cached decode)
  and the gated RMS norm around the recurrence.

The recurrence is the gated delta rule named on the Megatron Core API page
"core.ssm.gated_delta_net.gdn" (function torch_chunk_gated_delta_rule) and, with
several Householder sub-steps per token, the gated delta product of the page
"core.ssm.gated_delta_product" (class GatedDeltaProductMixer).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

from .gating import gates  # noqa: F401  (re-exported)
from . import conv_norm  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgdr_oracle.so")
_lock = threading.Lock()
_lib = None

_i64p = ctypes.POINTER(ctypes.c_int64)
_f64p = ctypes.POINTER(ctypes.c_double)


def build(out_path: str = _LIB_PATH, src: str = _SRC, extra_flags=()) -> str:
    """Compile the oracle with gcc (IEEE fp64: no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", "-Wall", "-Werror",
           "-I", _HERE, *extra_flags, src, "-o", out_path + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out_path + ".tmp", out_path)
    return out_path


def _bind(lib):
    lib.gdr_oracle_threads.argtypes = [ctypes.c_int]
    lib.gdr_oracle_threads.restype = ctypes.c_int
    lib.gdr_oracle_prefill.argtypes = [
        ctypes.c_int64, _i64p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int64, _f64p, _f64p, _f64p, _f64p, _f64p, ctypes.c_double, ctypes.c_int,
        _f64p, _i64p, _f64p, _f64p, ctypes.c_int]
    lib.gdr_oracle_prefill.restype = ctypes.c_int
    lib.gdr_oracle_decode.argtypes = [
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int64, _f64p, _f64p, _f64p, _f64p, _f64p, ctypes.c_double, ctypes.c_int,
        _f64p, ctypes.c_int64, _i64p, _f64p, ctypes.c_int]
    lib.gdr_oracle_decode.restype = ctypes.c_int
    return lib


def load_library(path: str | None = None):
    """Load (building first if absent) the oracle shared library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH) or (
                    os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
                build()
            _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _f64(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a, typ=_f64p):
    return None if a is None else a.ctypes.data_as(typ)


def threads_used(threads: int = 0) -> int:
    return int(load_library().gdr_oracle_threads(int(threads)))


def prefill(q, k, v, g, beta, *, scale=None, cu_seqlens=None, initial_state=None,
            state_indices=None, output_final_state=False, use_qk_l2norm=False,
            num_householder=1, final_state_out=None, threads=0, lib=None):
    """fp64 per-token recurrence over packed or batched sequences.

    Shapes (batched layout, B sequences of T tokens; with ``cu_seqlens`` B = 1):
      q [B,T,Hk,K]; k [B,T,Hk,K] or [B,T,n_h,Hk,K]; v [B,T,Hv,V] or [B,T,n_h,Hv,V];
      g [B,T,Hv]; beta [B,T,Hv] or [B,T,n_h,Hv].
    ``initial_state`` [N,Hv,K,V] (or a slot cache when ``state_indices`` is given).
    ``final_state_out``: array written in place (slot cache semantics); otherwise
    a fresh [N,Hv,K,V] array is returned when ``output_final_state``.
    Returns (o [B,T,Hv,V], final_state or None), fp64.
    """
    lib = lib or load_library()
    q = _f64(q)
    B, T, Hk, K = q.shape
    n_h = int(num_householder)
    k = _f64(k).reshape(B, T, n_h, Hk, K)
    Hv = v.shape[-2]
    V = v.shape[-1]
    v = _f64(v).reshape(B, T, n_h, Hv, V)
    g = _f64(g).reshape(B, T, Hv)
    beta = _f64(beta).reshape(B, T, n_h, Hv)
    if cu_seqlens is None:
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        assert B == 1, "packed sequences use batch size 1"
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    if scale is None:
        scale = 1.0 / np.sqrt(K)
    h0 = _f64(initial_state)
    idx = None if state_indices is None else np.ascontiguousarray(state_indices, dtype=np.int64)
    if final_state_out is not None:
        assert final_state_out.dtype == np.float64 and final_state_out.flags.c_contiguous
        fs = final_state_out
    elif output_final_state:
        fs = np.zeros((N, Hv, K, V), dtype=np.float64)
    else:
        fs = None
    out = np.zeros((B, T, Hv, V), dtype=np.float64)
    rc = lib.gdr_oracle_prefill(
        N, _ptr(cu, _i64p), Hk, Hv, K, V, n_h, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
        float(scale), int(bool(use_qk_l2norm)), _ptr(h0), _ptr(idx, _i64p), _ptr(fs), _ptr(out),
        int(threads))
    if rc != 0:
        raise RuntimeError(f"gdr_oracle_prefill failed with code {rc}")
    return out, fs


def decode(q, k, v, g, beta, cache, *, batch_indices=None, scale=None, use_qk_l2norm=False,
           num_householder=1, threads=0, lib=None):
    """One token per request; ``cache`` [slots,Hv,K,V] fp64 is updated in place.

    q [n,Hk,K]; k [n,Hk,K] or [n,n_h,Hk,K]; v [n,Hv,V] or [n,n_h,Hv,V];
    g [n,Hv]; beta [n,Hv] or [n,n_h,Hv].  Returns o [n,Hv,V] fp64.
    """
    lib = lib or load_library()
    q = _f64(q)
    n, Hk, K = q.shape
    n_h = int(num_householder)
    Hv, V = v.shape[-2], v.shape[-1]
    k = _f64(k).reshape(n, n_h, Hk, K)
    v = _f64(v).reshape(n, n_h, Hv, V)
    g = _f64(g).reshape(n, Hv)
    beta = _f64(beta).reshape(n, n_h, Hv)
    assert cache.dtype == np.float64 and cache.flags.c_contiguous
    slots = cache.shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(K)
    idx = None if batch_indices is None else np.ascontiguousarray(batch_indices, dtype=np.int64)
    out = np.zeros((n, Hv, V), dtype=np.float64)
    rc = lib.gdr_oracle_decode(
        n, Hk, Hv, K, V, n_h, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale),
        int(bool(use_qk_l2norm)), _ptr(cache), slots, _ptr(idx, _i64p), _ptr(out), int(threads))
    if rc != 0:
        raise RuntimeError(f"gdr_oracle_decode failed with code {rc}")
    return out


def decode_tokens(q, k, v, g, beta, cache, *, batch_indices=None, scale=None,
                  use_qk_l2norm=False, num_householder=1, threads=0, lib=None):
    """Several decode tokens per request (token axis 1, ssm_decode's [n, seq_len, ...]
    form on page "core.ssm.gated_delta_product"): the single-token step of
    :func:`decode` applied token after token to a private copy of each request's
    slot state; the slot in ``cache`` (fp64, in place) is written at the end unless
    the request is padding (index -1, whose copy starts from slot 0).

    Returns (o [n,T,Hv,V], states [n,T,Hv,K,V]: the state after each token).
    """
    n, T = q.shape[0], q.shape[1]
    idx = np.arange(n) if batch_indices is None else np.asarray(batch_indices)
    work = np.ascontiguousarray(np.stack([cache[max(int(r), 0)] for r in idx]))
    outs, states = [], []
    for t in range(T):
        outs.append(decode(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], work, scale=scale,
                           use_qk_l2norm=use_qk_l2norm, num_householder=num_householder,
                           threads=threads, lib=lib))
        states.append(work.copy())
    for i, r in enumerate(idx):
        if r >= 0:
            cache[int(r)] = work[i]
    return np.stack(outs, axis=1), np.stack(states, axis=1)
