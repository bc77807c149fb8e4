"""ctypes view of the C ABI in include/gdr.h (libgdr.so, built in-tree for gfx950).

There is no fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdr.so")

GDR_OK = 0
GDR_ERR_INVALID_ARG = 1
GDR_ERR_UNSUPPORTED = 2
GDR_ERR_WORKSPACE = 3
GDR_ERR_HIP = 4
GDR_DTYPE_F32 = 0
GDR_DTYPE_BF16 = 1
ABI_VERSION = 4   # GDR_ABI_VERSION the structures below are laid out for

# Every symbol include/gdr.h declares.
EXPORTS = (
    "gdr_abi_version",
    "gdr_status_string",
    "gdr_validate_prefill",
    "gdr_validate_decode",
    "gdr_prefill_workspace_bytes",
    "gdr_chunk_gated_delta_rule",
    "gdr_chunk_gated_delta_rule_noalloc",
    "gdr_ssm_decode",
    "gdr_validate_conv_prefill",
    "gdr_validate_conv_decode",
    "gdr_validate_gated_rmsnorm",
    "gdr_causal_conv1d_prefill",
    "gdr_causal_conv1d_decode",
    "gdr_gated_rmsnorm",
    "gdr_validate_backward",
    "gdr_backward_workspace_bytes",
    "gdr_chunk_gated_delta_rule_backward",
)


class PrefillArgs(ctypes.Structure):
    """gdr_prefill_args (field order and types as in include/gdr.h)."""
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("seqlen", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32),
        ("num_qk_heads", ctypes.c_int32),
        ("num_v_heads", ctypes.c_int32),
        ("head_k", ctypes.c_int32),
        ("head_v", ctypes.c_int32),
        ("num_householder", ctypes.c_int32),
        ("chunk_size", ctypes.c_int32),
        ("qkv_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("use_qk_l2norm", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("num_slots", ctypes.c_int32),
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("g", ctypes.c_void_p),
        ("beta", ctypes.c_void_p),
        ("cu_seqlens", ctypes.c_void_p),
        ("state_indices", ctypes.c_void_p),
        ("initial_state", ctypes.c_void_p),
        ("final_state", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("gate_mode", ctypes.c_int32),
        ("A_log", ctypes.c_void_p),
        ("dt_bias", ctypes.c_void_p),
        ("boundary_states", ctypes.c_void_p),
        ("boundary_interval", ctypes.c_int32),
    ]


class DecodeArgs(ctypes.Structure):
    """gdr_decode_args (field order and types as in include/gdr.h)."""
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_qk_heads", ctypes.c_int32),
        ("num_v_heads", ctypes.c_int32),
        ("head_k", ctypes.c_int32),
        ("head_v", ctypes.c_int32),
        ("num_householder", ctypes.c_int32),
        ("num_slots", ctypes.c_int32),
        ("qkv_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("use_qk_l2norm", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("g", ctypes.c_void_p),
        ("beta", ctypes.c_void_p),
        ("state", ctypes.c_void_p),
        ("batch_indices", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("gate_mode", ctypes.c_int32),
        ("A_log", ctypes.c_void_p),
        ("dt_bias", ctypes.c_void_p),
        ("num_tokens", ctypes.c_int32),
        ("intermediate_state", ctypes.c_void_p),
    ]


class ConvPrefillArgs(ctypes.Structure):
    """gdr_conv_prefill_args."""
    _fields_ = [
        ("tokens", ctypes.c_int32), ("num_seqs", ctypes.c_int32), ("channels", ctypes.c_int32),
        ("width", ctypes.c_int32), ("dtype", ctypes.c_int32), ("activation", ctypes.c_int32),
        ("num_slots", ctypes.c_int32), ("x", ctypes.c_void_p), ("weight", ctypes.c_void_p),
        ("bias", ctypes.c_void_p), ("cu_seqlens", ctypes.c_void_p),
        ("state_indices", ctypes.c_void_p), ("conv_state", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
    ]


class ConvDecodeArgs(ctypes.Structure):
    """gdr_conv_decode_args."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_tokens", ctypes.c_int32), ("channels", ctypes.c_int32),
        ("width", ctypes.c_int32), ("dtype", ctypes.c_int32), ("activation", ctypes.c_int32),
        ("num_slots", ctypes.c_int32), ("x", ctypes.c_void_p), ("weight", ctypes.c_void_p),
        ("bias", ctypes.c_void_p), ("batch_indices", ctypes.c_void_p),
        ("conv_state", ctypes.c_void_p), ("intermediate_state", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
    ]


class GatedRMSNormArgs(ctypes.Structure):
    """gdr_gated_rmsnorm_args."""
    _fields_ = [
        ("tokens", ctypes.c_int32), ("heads", ctypes.c_int32), ("group", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("norm_before_gate", ctypes.c_int32), ("eps", ctypes.c_float),
        ("x", ctypes.c_void_p), ("z", ctypes.c_void_p), ("weight", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
    ]


class BackwardArgs(ctypes.Structure):
    """gdr_backward_args."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
        ("num_qk_heads", ctypes.c_int32), ("num_v_heads", ctypes.c_int32),
        ("head_k", ctypes.c_int32), ("head_v", ctypes.c_int32), ("qkv_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("g", ctypes.c_void_p), ("beta", ctypes.c_void_p), ("cu_seqlens", ctypes.c_void_p),
        ("initial_state", ctypes.c_void_p), ("d_out", ctypes.c_void_p),
        ("d_final_state", ctypes.c_void_p),
        ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
        ("dg", ctypes.c_void_p), ("dbeta", ctypes.c_void_p), ("d_initial_state", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("use_qk_l2norm", ctypes.c_int32), ("gate_mode", ctypes.c_int32),
        ("A_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p),
        ("dA_log", ctypes.c_void_p), ("ddt_bias", ctypes.c_void_p),
        ("num_householder", ctypes.c_int32),
    ]


_lock = threading.Lock()
_lib = None


def load(path: str = LIB_PATH):
    """Load libgdr.so; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None and path == LIB_PATH:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with __graft_entry__.build() "
                "(or python gated_delta_rule_71_amd/build.py); there is no fallback path")
        lib = ctypes.CDLL(path)
        lib.gdr_abi_version.argtypes = []
        lib.gdr_abi_version.restype = ctypes.c_int
        lib.gdr_status_string.argtypes = [ctypes.c_int]
        lib.gdr_status_string.restype = ctypes.c_char_p
        lib.gdr_validate_prefill.argtypes = [ctypes.POINTER(PrefillArgs)]
        lib.gdr_validate_prefill.restype = ctypes.c_int
        lib.gdr_validate_decode.argtypes = [ctypes.POINTER(DecodeArgs)]
        lib.gdr_validate_decode.restype = ctypes.c_int
        lib.gdr_prefill_workspace_bytes.argtypes = [ctypes.POINTER(PrefillArgs)]
        lib.gdr_prefill_workspace_bytes.restype = ctypes.c_size_t
        lib.gdr_chunk_gated_delta_rule.argtypes = [ctypes.POINTER(PrefillArgs), ctypes.c_void_p]
        lib.gdr_chunk_gated_delta_rule.restype = ctypes.c_int
        lib.gdr_chunk_gated_delta_rule_noalloc.argtypes = [ctypes.POINTER(PrefillArgs),
                                                           ctypes.c_void_p]
        lib.gdr_chunk_gated_delta_rule_noalloc.restype = ctypes.c_int
        lib.gdr_ssm_decode.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.c_void_p]
        lib.gdr_ssm_decode.restype = ctypes.c_int
        for name, typ in (("conv_prefill", ConvPrefillArgs), ("conv_decode", ConvDecodeArgs),
                          ("gated_rmsnorm", GatedRMSNormArgs)):
            v = getattr(lib, f"gdr_validate_{name}")
            v.argtypes = [ctypes.POINTER(typ)]
            v.restype = ctypes.c_int
        for name, typ in (("causal_conv1d_prefill", ConvPrefillArgs),
                          ("causal_conv1d_decode", ConvDecodeArgs),
                          ("gated_rmsnorm", GatedRMSNormArgs)):
            f = getattr(lib, f"gdr_{name}")
            f.argtypes = [ctypes.POINTER(typ), ctypes.c_void_p]
            f.restype = ctypes.c_int
        lib.gdr_validate_backward.argtypes = [ctypes.POINTER(BackwardArgs)]
        lib.gdr_validate_backward.restype = ctypes.c_int
        lib.gdr_backward_workspace_bytes.argtypes = [ctypes.POINTER(BackwardArgs)]
        lib.gdr_backward_workspace_bytes.restype = ctypes.c_size_t
        lib.gdr_chunk_gated_delta_rule_backward.argtypes = [ctypes.POINTER(BackwardArgs),
                                                            ctypes.c_void_p]
        lib.gdr_chunk_gated_delta_rule_backward.restype = ctypes.c_int
        if lib.gdr_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{path} has ABI version {lib.gdr_abi_version()}, the bindings "
                               f"expect {ABI_VERSION}: rebuild it")
        if path == LIB_PATH:
            _lib = lib
        return lib


def status_string(code: int) -> str:
    return load().gdr_status_string(int(code)).decode()
