"""MI355X (gfx950) gated delta rule: chunked prefill and slot-indexed decode.

Python face of libgdr.so (C ABI in include/gdr.h).  These functions only
marshal arguments: torch tensors provide device memory and the current HIP
stream, and every step of the computation runs in the library's kernels.

    o, final_state = chunk_gated_delta_rule(q, k, v, g, beta, scale=None,
        chunk_size=64, initial_state=None, output_final_state=False,
        use_qk_l2norm_in_kernel=False, cu_seqlens=None, **kwargs)
    o = ssm_decode(q, k, v, g, beta, ssm_state, batch_indices=None, ...)

The signature of chunk_gated_delta_rule follows torch_chunk_gated_delta_rule on
the Megatron Core API page "core.ssm.gated_delta_net.gdn" (extra keyword
arguments are accepted and ignored there too); ssm_decode follows ssm_decode on
the pages "core.ssm.gated_delta_net.gdn" / "core.ssm.gated_delta_product".

Both take the gates either formed (g, beta) or, with ``A_log`` and ``dt_bias``
([Hv] float32) given, as the raw per-token projections (g holds alpha, beta holds
the logits b); the kernels then form g = -exp(A_log) softplus(alpha + dt_bias)
and beta = sigmoid(b) themselves (GatedDeltaNet._compute_gates, page
"core.ssm.gated_delta_net.gdn").
"""
from __future__ import annotations

import math

from . import _lib

__all__ = ["chunk_gated_delta_rule", "chunk_gated_delta_rule_noalloc",
           "chunk_gated_delta_rule_backward", "ssm_decode",
           "causal_conv1d", "causal_conv1d_update", "gated_rmsnorm", "library", "abi_version"]


def library():
    """The loaded libgdr.so (raises if it has not been built)."""
    return _lib.load()


def abi_version() -> int:
    return int(library().gdr_abi_version())


def _torch():
    import torch
    return torch


def _dtype_code(dt):
    torch = _torch()
    if dt == torch.float32:
        return _lib.GDR_DTYPE_F32
    if dt == torch.bfloat16:
        return _lib.GDR_DTYPE_BF16
    raise ValueError(f"unsupported dtype {dt} (float32 or bfloat16)")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check(t, name, dtype=None, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() not in (ndim if isinstance(ndim, tuple) else (ndim,)):
        raise ValueError(f"{name} has {t.dim()} dims")


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes_stream(s)


def ctypes_stream(s):
    return s.cuda_stream if hasattr(s, "cuda_stream") else int(s)


def _raise(code, what):
    if code != _lib.GDR_OK:
        raise RuntimeError(f"{what} failed: {_lib.status_string(code)}")


def _gate_params(A_log, dt_bias, Hv, torch):
    """gate_mode and the [Hv] parameter tensors (both or neither must be given)."""
    if A_log is None and dt_bias is None:
        return 0, None, None
    if A_log is None or dt_bias is None:
        raise ValueError("A_log and dt_bias go together (raw gate projections)")
    for name, t in (("A_log", A_log), ("dt_bias", dt_bias)):
        _check(t, name, dtype=torch.float32, ndim=1)
        if t.numel() != Hv:
            raise ValueError(f"{name} needs one entry per value head ({Hv})")
    return 1, A_log, dt_bias


def prefill_args(q, k, v, g, beta, *, scale=None, chunk_size=64, initial_state=None,
                 final_state=None, use_qk_l2norm_in_kernel=False, cu_seqlens=None,
                 state_indices=None, out=None, A_log=None, dt_bias=None,
                 boundary_states=None, boundary_interval=0):
    """Fill a gdr_prefill_args struct from tensors (no checks beyond shapes)."""
    B, T, Hk, K = q.shape
    n_h = k.shape[2] if k.dim() == 5 else 1
    Hv, V = v.shape[-2], v.shape[-1]
    a = _lib.PrefillArgs()
    a.batch, a.seqlen = B, T
    a.num_seqs = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
    a.num_qk_heads, a.num_v_heads, a.head_k, a.head_v = Hk, Hv, K, V
    a.num_householder = n_h
    a.chunk_size = int(chunk_size)
    a.qkv_dtype = _dtype_code(q.dtype)
    a.out_dtype = _dtype_code(out.dtype)
    a.use_qk_l2norm = int(bool(use_qk_l2norm_in_kernel))
    a.scale = float("nan") if scale is None else float(scale)
    a.num_slots = initial_state.shape[0] if (state_indices is not None and
                                             initial_state is not None) else (
        final_state.shape[0] if (state_indices is not None and final_state is not None) else 0)
    a.q, a.k, a.v, a.g, a.beta = _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta)
    a.cu_seqlens = _ptr(cu_seqlens)
    a.state_indices = _ptr(state_indices)
    a.initial_state = _ptr(initial_state)
    a.final_state = _ptr(final_state)
    a.out = _ptr(out)
    a.workspace = None
    a.workspace_bytes = 0
    a.gate_mode = 0 if A_log is None else 1
    a.A_log, a.dt_bias = _ptr(A_log), _ptr(dt_bias)
    a.boundary_states = _ptr(boundary_states)
    a.boundary_interval = int(boundary_interval or 0)
    return a


def boundary_count(lengths, interval):
    """Entries a prefill writes to ``boundary_states``: sum of floor(L_n / interval)."""
    return int(sum(int(L) // int(interval) for L in lengths))


def chunk_gated_delta_rule(q, k, v, g, beta, scale=None, chunk_size=64, initial_state=None,
                           output_final_state=False, use_qk_l2norm_in_kernel=False,
                           cu_seqlens=None, *, state_indices=None, out_dtype=None, out=None,
                           final_state=None, stream=None, A_log=None, dt_bias=None,
                           boundary_states=None, boundary_interval=None, workspace=None,
                           segments=True, **kwargs):
    """Chunked prefill of the gated delta rule (packed or batched sequences).

    q [B,T,Hk,K]; k [B,T,Hk,K] or [B,T,n_h,Hk,K]; v [B,T,Hv,V] or [B,T,n_h,Hv,V]
    (float32 or bfloat16, one dtype); g [B,T,Hv] and beta [B,T,Hv] /
    [B,T,n_h,Hv] float32; cu_seqlens int32 [N+1] (B must be 1).
    initial_state float32 [N,Hv,K,V]; with ``state_indices`` (int32 [N]) it is a
    slot cache [slots,Hv,K,V], read at max(idx, 0) and written back in place at
    idx >= 0 (or into ``final_state`` if given).
    With ``A_log`` and ``dt_bias`` ([Hv] float32), g and beta are the raw gate
    projections alpha and b, and the kernel forms the gates.
    ``boundary_states`` float32 [E,Hv,K,V] with ``boundary_interval`` (tokens, a
    multiple of 64) receives each sequence's state after every whole multiple of
    the interval, sequences in order (E = boundary_count(lengths, interval)).
    Long sequences (batched rows, or packed sequences without boundary states)
    that leave compute units idle run in segments (three passes of the chunked
    kernel and a state combine) when a workspace of gdr_prefill_workspace_bytes is
    given.  When ``workspace`` is None that workspace is ALLOCATED here with
    torch.empty (a device allocation per call) unless ``segments`` is False (then
    the single pass runs); callers that cannot allocate pass their own
    ``workspace`` or use chunk_gated_delta_rule_noalloc.
    Returns (o [B,T,Hv,V], final_state or None).
    """
    torch = _torch()
    lib = library()
    _check(q, "q", ndim=4)
    _check(k, "k", dtype=q.dtype, ndim=(4, 5))
    _check(v, "v", dtype=q.dtype, ndim=(4, 5))
    _check(g, "g", dtype=torch.float32, ndim=3)
    _check(beta, "beta", dtype=torch.float32, ndim=(3, 4))
    B, T, Hk, K = q.shape
    n_h = k.shape[2] if k.dim() == 5 else 1
    Hv, V = v.shape[-2], v.shape[-1]
    _gate_params(A_log, dt_bias, Hv, torch)
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", dtype=torch.int32, ndim=1)
    N = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
    if state_indices is not None:
        _check(state_indices, "state_indices", dtype=torch.int32, ndim=1)
        if state_indices.numel() != N:
            raise ValueError("state_indices needs one entry per sequence")
        if initial_state is None and final_state is None:
            raise ValueError("state_indices needs the slot cache as initial_state")
        if final_state is None:
            final_state = initial_state
    elif output_final_state and final_state is None:
        final_state = torch.empty((N, Hv, K, V), dtype=torch.float32, device=q.device)
    for name, st in (("initial_state", initial_state), ("final_state", final_state),
                     ("boundary_states", boundary_states)):
        if st is not None:
            _check(st, name, dtype=torch.float32, ndim=4)
    if (boundary_states is None) != (boundary_interval is None):
        raise ValueError("boundary_states and boundary_interval go together")
    if out is None:
        od = v.dtype if out_dtype is None else out_dtype
        out = torch.empty((B, T, Hv, V), dtype=od, device=q.device)
    else:
        _check(out, "out", ndim=4)
    a = prefill_args(q, k, v, g, beta, scale=scale, chunk_size=chunk_size,
                     initial_state=initial_state, final_state=final_state,
                     use_qk_l2norm_in_kernel=use_qk_l2norm_in_kernel, cu_seqlens=cu_seqlens,
                     state_indices=state_indices, out=out, A_log=A_log, dt_bias=dt_bias,
                     boundary_states=boundary_states, boundary_interval=boundary_interval)
    # long sequences may run in segments, with a workspace (single pass without)
    need = int(lib.gdr_prefill_workspace_bytes(a))
    if workspace is None and need > 0 and segments:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _check(workspace, "workspace", dtype=torch.uint8, ndim=1)
        a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel()
    _raise(lib.gdr_chunk_gated_delta_rule(a, _stream(stream)), "gdr_chunk_gated_delta_rule")
    ret_state = final_state if (output_final_state or state_indices is not None) else None
    return out, ret_state


def chunk_gated_delta_rule_noalloc(q, k, v, g, beta, *, out, scale=None, chunk_size=64,
                                   initial_state=None, final_state=None,
                                   use_qk_l2norm_in_kernel=False, cu_seqlens=None,
                                   state_indices=None, A_log=None, dt_bias=None,
                                   boundary_states=None, boundary_interval=None, stream=None):
    """chunk_gated_delta_rule for callers that cannot allocate: the caller passes
    ``out`` (and ``final_state`` when one is wanted; with ``state_indices`` the slot
    cache is updated in place), nothing is allocated here or in the library, and
    long batched rows take the segment path on the library's per-GPU scratch
    (gdr_chunk_gated_delta_rule_noalloc).  Calls on one GPU share that scratch:
    keep them on one stream.  Returns ``out``."""
    torch = _torch()
    lib = library()
    _check(q, "q", ndim=4)
    _check(k, "k", dtype=q.dtype, ndim=(4, 5))
    _check(v, "v", dtype=q.dtype, ndim=(4, 5))
    _check(g, "g", dtype=torch.float32, ndim=3)
    _check(beta, "beta", dtype=torch.float32, ndim=(3, 4))
    _check(out, "out", ndim=4)
    _gate_params(A_log, dt_bias, v.shape[-2], torch)
    for name, t in (("cu_seqlens", cu_seqlens), ("state_indices", state_indices)):
        if t is not None:
            _check(t, name, dtype=torch.int32, ndim=1)
    if state_indices is not None and final_state is None:
        final_state = initial_state
    for name, st in (("initial_state", initial_state), ("final_state", final_state),
                     ("boundary_states", boundary_states)):
        if st is not None:
            _check(st, name, dtype=torch.float32, ndim=4)
    if (boundary_states is None) != (boundary_interval is None):
        raise ValueError("boundary_states and boundary_interval go together")
    a = prefill_args(q, k, v, g, beta, scale=scale, chunk_size=chunk_size,
                     initial_state=initial_state, final_state=final_state,
                     use_qk_l2norm_in_kernel=use_qk_l2norm_in_kernel, cu_seqlens=cu_seqlens,
                     state_indices=state_indices, out=out, A_log=A_log, dt_bias=dt_bias,
                     boundary_states=boundary_states, boundary_interval=boundary_interval)
    _raise(lib.gdr_chunk_gated_delta_rule_noalloc(a, _stream(stream)),
           "gdr_chunk_gated_delta_rule_noalloc")
    return out


def decode_args(q, k, v, g, beta, ssm_state, *, batch_indices=None, scale=None,
                use_qk_l2norm_in_kernel=False, out=None, A_log=None, dt_bias=None,
                intermediate_ssm_state=None):
    multi = q.dim() == 4                     # [n, T, Hk, K]: several tokens per request
    n, Hk, K = q.shape[0], q.shape[-2], q.shape[-1]
    T = q.shape[1] if multi else 1
    n_h = k.shape[-3] if k.dim() == (5 if multi else 4) else 1
    Hv, V = v.shape[-2], v.shape[-1]
    a = _lib.DecodeArgs()
    a.batch, a.num_qk_heads, a.num_v_heads, a.head_k, a.head_v = n, Hk, Hv, K, V
    a.num_householder = n_h
    a.num_slots = ssm_state.shape[0]
    a.qkv_dtype = _dtype_code(q.dtype)
    a.out_dtype = _dtype_code(out.dtype)
    a.use_qk_l2norm = int(bool(use_qk_l2norm_in_kernel))
    a.scale = float("nan") if scale is None else float(scale)
    a.q, a.k, a.v, a.g, a.beta = _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta)
    a.state = _ptr(ssm_state)
    a.batch_indices = _ptr(batch_indices)
    a.out = _ptr(out)
    a.gate_mode = 0 if A_log is None else 1
    a.A_log, a.dt_bias = _ptr(A_log), _ptr(dt_bias)
    a.num_tokens = T
    a.intermediate_state = _ptr(intermediate_ssm_state)
    return a


def ssm_decode(q, k, v, g, beta, ssm_state, batch_indices=None, scale=None,
               use_qk_l2norm_in_kernel=False, *, out_dtype=None, out=None, stream=None,
               A_log=None, dt_bias=None, intermediate_ssm_state=None):
    """One decode token per request, updating ``ssm_state`` [slots,Hv,K,V] in place.

    q [n,Hk,K]; k [n,Hk,K] or [n,n_h,Hk,K]; v [n,Hv,V] or [n,n_h,Hv,V];
    g [n,Hv]; beta [n,Hv] or [n,n_h,Hv] (float32); batch_indices int32 [n]
    (-1: padding, reads slot 0, writes nothing) or None (request i <-> slot i).
    With ``A_log`` and ``dt_bias`` ([Hv] float32), g and beta are the raw gate
    projections alpha and b, and the kernel forms the gates.
    Several tokens per request: every tensor gains a token axis after the request
    axis (q [n,T,Hk,K], k [n,T,(n_h,)Hk,K], v [n,T,(n_h,)Hv,V], g [n,T,Hv], beta
    [n,T,(n_h,)Hv]); the state advances token by token and ``intermediate_ssm_state``
    (float32 [n,T,Hv,K,V]) receives the state after each token.  Returns o
    [n,Hv,V] ([n,T,Hv,V] for several tokens).
    """
    torch = _torch()
    lib = library()
    _check(q, "q", ndim=(3, 4))
    t = 1 if q.dim() == 4 else 0            # extra token axis
    _check(k, "k", dtype=q.dtype, ndim=(3 + t, 4 + t))
    _check(v, "v", dtype=q.dtype, ndim=(3 + t, 4 + t))
    _check(g, "g", dtype=torch.float32, ndim=2 + t)
    _check(beta, "beta", dtype=torch.float32, ndim=(2 + t, 3 + t))
    _check(ssm_state, "ssm_state", dtype=torch.float32, ndim=4)
    if batch_indices is not None:
        _check(batch_indices, "batch_indices", dtype=torch.int32, ndim=1)
    n = q.shape[0]
    Hv, V = v.shape[-2], v.shape[-1]
    _gate_params(A_log, dt_bias, Hv, torch)
    lead = (n, q.shape[1]) if t else (n,)
    if intermediate_ssm_state is not None:
        _check(intermediate_ssm_state, "intermediate_ssm_state", dtype=torch.float32, ndim=5)
        if tuple(intermediate_ssm_state.shape) != (n, lead[-1] if t else 1, Hv,
                                                   ssm_state.shape[2], V):
            raise ValueError("intermediate_ssm_state must be [n, T, Hv, K, V]")
    if out is None:
        od = v.dtype if out_dtype is None else out_dtype
        out = torch.empty(lead + (Hv, V), dtype=od, device=q.device)
    else:
        _check(out, "out", ndim=3 + t)
    a = decode_args(q, k, v, g, beta, ssm_state, batch_indices=batch_indices, scale=scale,
                    use_qk_l2norm_in_kernel=use_qk_l2norm_in_kernel, out=out, A_log=A_log,
                    dt_bias=dt_bias, intermediate_ssm_state=intermediate_ssm_state)
    _raise(lib.gdr_ssm_decode(a, _stream(stream)), "gdr_ssm_decode")
    return out


def default_scale(head_k: int) -> float:
    return 1.0 / math.sqrt(head_k)


# ---- the steps around the recurrence: short causal conv, gated RMS norm -----------------

def conv_prefill_args(x, weight, bias, cu_seqlens, *, conv_state=None, state_indices=None,
                      activation="silu", out=None):
    a = _lib.ConvPrefillArgs()
    a.tokens, a.channels = x.shape[0], x.shape[1]
    a.num_seqs = cu_seqlens.numel() - 1
    a.width = weight.shape[1]
    a.dtype = _dtype_code(x.dtype)
    a.activation = {"silu": 1, None: 0, "none": 0}[activation]
    a.num_slots = conv_state.shape[0] if (conv_state is not None and
                                          state_indices is not None) else 0
    a.x, a.weight, a.bias = _ptr(x), _ptr(weight), _ptr(bias)
    a.cu_seqlens, a.state_indices = _ptr(cu_seqlens), _ptr(state_indices)
    a.conv_state, a.out = _ptr(conv_state), _ptr(out)
    return a


def causal_conv1d(x, weight, bias=None, *, cu_seqlens=None, conv_state=None,
                  state_indices=None, activation="silu", out=None, stream=None):
    """Depthwise causal conv over packed sequences: x [tokens, C] (float32 or
    bfloat16), weight float32 [C, W], bias float32 [C] or None, cu_seqlens int32
    [N+1] (None: one sequence).  conv_state float32 [rows, C, W-1] (rows addressed
    by state_indices, -1 = padding) supplies the inputs before each sequence and
    receives its last W-1 inputs, in place.  Returns y [tokens, C]."""
    torch = _torch()
    lib = library()
    _check(x, "x", ndim=2)
    _check(weight, "weight", dtype=torch.float32, ndim=2)
    if bias is not None:
        _check(bias, "bias", dtype=torch.float32, ndim=1)
    if cu_seqlens is None:
        cu_seqlens = torch.tensor([0, x.shape[0]], dtype=torch.int32, device=x.device)
    _check(cu_seqlens, "cu_seqlens", dtype=torch.int32, ndim=1)
    if conv_state is not None:
        _check(conv_state, "conv_state", dtype=torch.float32, ndim=3)
    if state_indices is not None:
        _check(state_indices, "state_indices", dtype=torch.int32, ndim=1)
    if out is None:
        out = torch.empty_like(x)
    a = conv_prefill_args(x, weight, bias, cu_seqlens, conv_state=conv_state,
                          state_indices=state_indices, activation=activation, out=out)
    _raise(lib.gdr_causal_conv1d_prefill(a, _stream(stream)), "gdr_causal_conv1d_prefill")
    return out


def conv_decode_args(x, weight, bias, conv_state, *, batch_indices=None, activation="silu",
                     intermediate_state=None, out=None):
    a = _lib.ConvDecodeArgs()
    a.batch = x.shape[0]
    a.num_tokens = x.shape[1] if x.dim() == 3 else 1
    a.channels = x.shape[-1]
    a.width = weight.shape[1]
    a.dtype = _dtype_code(x.dtype)
    a.activation = {"silu": 1, None: 0, "none": 0}[activation]
    a.num_slots = conv_state.shape[0]
    a.x, a.weight, a.bias = _ptr(x), _ptr(weight), _ptr(bias)
    a.batch_indices, a.conv_state = _ptr(batch_indices), _ptr(conv_state)
    a.intermediate_state, a.out = _ptr(intermediate_state), _ptr(out)
    return a


def causal_conv1d_update(x, conv_state, weight, bias=None, *, batch_indices=None,
                         activation="silu", intermediate_state=None, out=None, stream=None):
    """The cached conv step: x [n, C] or [n, T, C]; conv_state float32 [slots, C, W-1]
    updated in place at batch_indices (None: request i <-> row i; -1: padding
    reads row 0, writes nothing); intermediate_state float32 [n, T, C, W-1] or
    None receives the window after each token.  Returns y shaped like x."""
    torch = _torch()
    lib = library()
    _check(x, "x", ndim=(2, 3))
    _check(conv_state, "conv_state", dtype=torch.float32, ndim=3)
    _check(weight, "weight", dtype=torch.float32, ndim=2)
    if bias is not None:
        _check(bias, "bias", dtype=torch.float32, ndim=1)
    if batch_indices is not None:
        _check(batch_indices, "batch_indices", dtype=torch.int32, ndim=1)
    if intermediate_state is not None:
        _check(intermediate_state, "intermediate_state", dtype=torch.float32, ndim=4)
    if out is None:
        out = torch.empty_like(x)
    a = conv_decode_args(x, weight, bias, conv_state, batch_indices=batch_indices,
                         activation=activation, intermediate_state=intermediate_state, out=out)
    _raise(lib.gdr_causal_conv1d_decode(a, _stream(stream)), "gdr_causal_conv1d_decode")
    return out


def gated_rmsnorm(x, z, weight, *, eps=1e-5, norm_before_gate=False, out=None, stream=None):
    """Gated RMS norm per (token, head) group: x, z [tokens, heads, group] (one
    dtype); weight float32 [heads * group].  norm_before_gate False: norm(x *
    silu(z)) * w; True: norm(x) * w * silu(z).  Returns y like x."""
    torch = _torch()
    lib = library()
    _check(x, "x", ndim=3)
    _check(z, "z", dtype=x.dtype, ndim=3)
    _check(weight, "weight", dtype=torch.float32, ndim=1)
    if tuple(z.shape) != tuple(x.shape) or weight.numel() != x.shape[1] * x.shape[2]:
        raise ValueError("z must match x and weight must have heads * group entries")
    if out is None:
        out = torch.empty_like(x)
    a = _lib.GatedRMSNormArgs()
    a.tokens, a.heads, a.group = x.shape
    a.dtype = _dtype_code(x.dtype)
    a.norm_before_gate = int(bool(norm_before_gate))
    a.eps = float(eps)
    a.x, a.z, a.weight, a.out = _ptr(x), _ptr(z), _ptr(weight), _ptr(out)
    _raise(lib.gdr_gated_rmsnorm(a, _stream(stream)), "gdr_gated_rmsnorm")
    return out


def backward_args(q, k, v, g, beta, do, *, dq, dk, dv, dg, dbeta, dh0=None, dht=None,
                  scale=None, initial_state=None, cu_seqlens=None, workspace=None,
                  use_qk_l2norm_in_kernel=False, A_log=None, dt_bias=None, dA_log=None,
                  ddt_bias=None):
    """Fill a gdr_backward_args struct from tensors (no checks beyond shapes)."""
    B, T, Hk, K = q.shape
    Hv, V = v.shape[-2], v.shape[-1]
    a = _lib.BackwardArgs()
    a.batch, a.seqlen = B, T
    a.num_seqs = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
    a.num_qk_heads, a.num_v_heads, a.head_k, a.head_v = Hk, Hv, K, V
    a.qkv_dtype = _dtype_code(q.dtype)
    a.scale = float("nan") if scale is None else float(scale)
    a.q, a.k, a.v, a.g, a.beta = _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta)
    a.cu_seqlens = _ptr(cu_seqlens)
    a.initial_state = _ptr(initial_state)
    a.d_out = _ptr(do)
    a.d_final_state = _ptr(dht)
    a.dq, a.dk, a.dv, a.dg, a.dbeta = _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta)
    a.d_initial_state = _ptr(dh0)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel()
    a.use_qk_l2norm = int(bool(use_qk_l2norm_in_kernel))
    a.gate_mode = 0 if A_log is None else 1
    a.A_log, a.dt_bias = _ptr(A_log), _ptr(dt_bias)
    a.dA_log, a.ddt_bias = _ptr(dA_log), _ptr(ddt_bias)
    a.num_householder = k.shape[2] if k.dim() == 5 else 1
    return a


def chunk_gated_delta_rule_backward(q, k, v, g, beta, do, dht=None, scale=None,
                                    initial_state=None, cu_seqlens=None, *, workspace=None,
                                    stream=None, use_qk_l2norm_in_kernel=False, A_log=None,
                                    dt_bias=None):
    """Gradients of the chunked prefill (gated delta rule, or the gated delta
    product when k, v are [B,T,n_h,H,D] and beta [B,T,n_h,Hv], n_h = 2).

    With ``use_qk_l2norm_in_kernel`` the forward normalised q and k, and dq, dk are
    the gradients of the raw q, k.  With ``A_log`` and ``dt_bias`` ([Hv] float32), g
    and beta are the raw gate projections; dg and dbeta are then their gradients
    and the result gains dA_log, ddt_bias ([Hv]).

    q, k [B,T,Hk,D]; v, do [B,T,Hv,D] (float32 or bfloat16, one dtype); g, beta
    [B,T,Hv] float32; dht (gradient of the final state) and initial_state float32
    [N,Hv,D,D] or None; cu_seqlens int32 [N+1] (B must be 1).
    Returns (dq, dk, dv, dg, dbeta, dh0), float32, shaped like q, k, v, g, beta and
    the initial state ([N,Hv,D,D]) (plus dA_log, ddt_bias with raw gates).  ``workspace``: a uint8 GPU tensor of at least
    the library's gdr_backward_workspace_bytes (allocated here when None).
    """
    torch = _torch()
    lib = library()
    _check(q, "q", ndim=4)
    _check(k, "k", dtype=q.dtype, ndim=(4, 5))
    _check(v, "v", dtype=q.dtype, ndim=(4, 5))
    _check(do, "do", dtype=q.dtype, ndim=4)
    _check(g, "g", dtype=torch.float32, ndim=3)
    _check(beta, "beta", dtype=torch.float32, ndim=(3, 4))
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", dtype=torch.int32, ndim=1)
    for name, st in (("initial_state", initial_state), ("dht", dht)):
        if st is not None:
            _check(st, name, dtype=torch.float32, ndim=4)
    B, T, Hk, K = q.shape
    Hv, V = v.shape[-2], v.shape[-1]
    N = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
    dev = q.device
    f32 = torch.float32
    dq = torch.empty((B, T, Hk, K), dtype=f32, device=dev)
    dk = torch.empty(k.shape, dtype=f32, device=dev)
    dv = torch.empty(v.shape, dtype=f32, device=dev)
    dg = torch.empty((B, T, Hv), dtype=f32, device=dev)
    dbeta = torch.empty(beta.shape, dtype=f32, device=dev)
    dh0 = torch.empty((N, Hv, K, V), dtype=f32, device=dev)
    gate_mode, A_log, dt_bias = _gate_params(A_log, dt_bias, Hv, torch)
    dA_log = torch.empty((Hv,), dtype=f32, device=dev) if gate_mode else None
    ddt_bias = torch.empty((Hv,), dtype=f32, device=dev) if gate_mode else None
    a = backward_args(q, k, v, g, beta, do, dq=dq, dk=dk, dv=dv, dg=dg, dbeta=dbeta, dh0=dh0,
                      dht=dht, scale=scale, initial_state=initial_state, cu_seqlens=cu_seqlens,
                      use_qk_l2norm_in_kernel=use_qk_l2norm_in_kernel, A_log=A_log,
                      dt_bias=dt_bias, dA_log=dA_log, ddt_bias=ddt_bias)
    need = int(lib.gdr_backward_workspace_bytes(a))
    if workspace is None:
        # 256-byte alignment: the caching allocator hands out 512-byte aligned blocks
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _check(workspace, "workspace", dtype=torch.uint8, ndim=1)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = workspace.numel()
    _raise(lib.gdr_chunk_gated_delta_rule_backward(a, _stream(stream)),
           "gdr_chunk_gated_delta_rule_backward")
    if gate_mode:
        return dq, dk, dv, dg, dbeta, dh0, dA_log, ddt_bias
    return dq, dk, dv, dg, dbeta, dh0


def backward_workspace_bytes(q, v, *, num_seqs=None, num_qk_heads=None, num_householder=1):
    """gdr_backward_workspace_bytes for these shapes (host-only)."""
    B, T, Hk, K = q.shape
    a = _lib.BackwardArgs()
    a.num_householder = int(num_householder)
    a.batch, a.seqlen = B, T
    a.num_seqs = B if num_seqs is None else int(num_seqs)
    a.num_qk_heads = Hk if num_qk_heads is None else int(num_qk_heads)
    a.num_v_heads, a.head_k, a.head_v = v.shape[-2], K, v.shape[-1]
    a.qkv_dtype = _dtype_code(q.dtype)
    return int(library().gdr_backward_workspace_bytes(a))
