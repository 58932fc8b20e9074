"""ctypes view of libsa.so; mirrors include/sa.h field for field.

Argument marshalling only: every step of the computation runs in the HIP
library.  There is no fallback: if libsa.so is missing, loading raises.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsa.so")

SA_OK, SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED, SA_ERR_DEVICE = 0, 1, 2, 3
SA_DTYPE_BF16, SA_DTYPE_F32 = 0, 1
SA_MODE_BLOCKS, SA_MODE_GATHER, SA_MODE_STRIDED = 0, 1, 2
ABI_VERSION = 2

EXPORTED = ("sa_build_block_mask", "sa_attn_workspace_bytes", "sa_attn_strided_plan", "sa_attn_fwd", "sa_indexer_scores", "sa_topk",
            "sa_indexer_topk_workspace", "sa_indexer_topk", "sa_indexer_topk_noalloc", "sa_merge_partial",
            "sa_select_blocks_workspace", "sa_select_blocks", "sa_attn_bwd_workspace", "sa_attn_bwd",
            "sa_last_error", "sa_abi_version")

_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_P = ctypes.c_void_p


class SaPattern(ctypes.Structure):
    _fields_ = [
        ("causal", _I64),
        ("q_offset", _I64),
        ("window_left", _I64),
        ("window_right", _I64),
        ("sinks", _I64),
        ("stride", _I64),
        ("stride_phase", _I64),
        ("global_tokens", _I64),
        ("unit", _I64),
        ("unit_window", _I64),
        ("rand_units", _P),
        ("n_rand", _I64),
        ("rand_rows", _I64),
    ]


class SaAttnArgs(ctypes.Structure):
    _fields_ = [
        ("q", _P),
        ("k", _P),
        ("v", _P),
        ("o", _P),
        ("lse", _P),
        ("batch", _I64),
        ("heads", _I64),
        ("n_q", _I64),
        ("n_kv", _I64),
        ("head_dim", _I64),
        ("o_dtype", _I64),
        ("q_strides", _I64 * 3),
        ("k_strides", _I64 * 3),
        ("v_strides", _I64 * 3),
        ("o_strides", _I64 * 3),
        ("softmax_scale", ctypes.c_double),
        ("mode", _I64),
        ("block_q", _I64),
        ("block_kv", _I64),
        ("kv_count", _P),
        ("kv_index", _P),
        ("kv_partial", _P),
        ("pattern", SaPattern),
        ("gather_idx", _P),
        ("topk", _I64),
        ("gather_bh_stride", _I64),
        ("workspace", _P),
        ("workspace_bytes", _I64),
        ("per_head_lists", _I64),
    ]


class SaSelectArgs(ctypes.Structure):
    _fields_ = [
        ("q", _P),
        ("k", _P),
        ("batch", _I64),
        ("heads", _I64),
        ("n_q", _I64),
        ("n_kv", _I64),
        ("head_dim", _I64),
        ("q_strides", _I64 * 3),
        ("k_strides", _I64 * 3),
        ("q_offset", _I64),
        ("block_q", _I64),
        ("block_kv", _I64),
        ("n_select", _I64),
        ("kv_count", _P),
        ("kv_index", _P),
        ("kv_partial", _P),
        ("live_pairs", _P),
        ("workspace", _P),
        ("workspace_bytes", _I64),
    ]


class SaAttnBwdArgs(ctypes.Structure):
    _fields_ = [
        ("q", _P),
        ("k", _P),
        ("v", _P),
        ("o", _P),
        ("lse", _P),
        ("dout", _P),
        ("dq", _P),
        ("dk", _P),
        ("dv", _P),
        ("batch", _I64),
        ("heads", _I64),
        ("n_q", _I64),
        ("n_kv", _I64),
        ("head_dim", _I64),
        ("softmax_scale", ctypes.c_double),
        ("block_q", _I64),
        ("block_kv", _I64),
        ("kv_count", _P),
        ("kv_index", _P),
        ("kv_partial", _P),
        ("per_head_lists", _I64),
        ("pattern", SaPattern),
        ("workspace", _P),
        ("workspace_bytes", _I64),
    ]


class SaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libsa status {status}: {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} not found: build it with `python -m block_sparse_attention_sa_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.sa_build_block_mask.argtypes = [ctypes.POINTER(SaPattern), _I64, _I64, _I32, _I32, _P, _P,
                                          _P, _P, _P]
        L.sa_build_block_mask.restype = ctypes.c_int
        L.sa_attn_workspace_bytes.argtypes = [ctypes.POINTER(SaAttnArgs)]
        L.sa_attn_workspace_bytes.restype = ctypes.c_size_t
        L.sa_attn_strided_plan.argtypes = [ctypes.POINTER(SaAttnArgs), _P]
        L.sa_attn_strided_plan.restype = ctypes.c_int
        L.sa_attn_fwd.argtypes = [ctypes.POINTER(SaAttnArgs), _P]
        L.sa_attn_fwd.restype = ctypes.c_int
        L.sa_indexer_scores.argtypes = [_P, _P, _I64, _I64, _I32, _I64, _P, _P]
        L.sa_indexer_scores.restype = ctypes.c_int
        L.sa_topk.argtypes = [_P, _I64, _I64, _I64, _I32, _P, _P]
        L.sa_topk.restype = ctypes.c_int
        L.sa_indexer_topk_workspace.argtypes = [_I64, _I64, _I32]
        L.sa_indexer_topk_workspace.restype = ctypes.c_size_t
        L.sa_indexer_topk.argtypes = [_P, _P, _I64, _I64, _I32, _I64, _I32, _P, _P, _P, ctypes.c_size_t, _P]
        L.sa_indexer_topk.restype = ctypes.c_int
        L.sa_indexer_topk_noalloc.argtypes = [_P, _P, _I64, _I64, _I32, _I64, _I32, _P, _P]
        L.sa_indexer_topk_noalloc.restype = ctypes.c_int
        L.sa_select_blocks_workspace.argtypes = [ctypes.POINTER(SaSelectArgs)]
        L.sa_select_blocks_workspace.restype = ctypes.c_size_t
        L.sa_select_blocks.argtypes = [ctypes.POINTER(SaSelectArgs), _P]
        L.sa_select_blocks.restype = ctypes.c_int
        L.sa_attn_bwd_workspace.argtypes = [ctypes.POINTER(SaAttnBwdArgs)]
        L.sa_attn_bwd_workspace.restype = ctypes.c_size_t
        L.sa_attn_bwd.argtypes = [ctypes.POINTER(SaAttnBwdArgs), _P]
        L.sa_attn_bwd.restype = ctypes.c_int
        L.sa_merge_partial.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _I32, ctypes.POINTER(_I64),
                                       ctypes.POINTER(_I64), _I32, _I64, _I64, _P]
        L.sa_merge_partial.restype = ctypes.c_int
        L.sa_last_error.argtypes = []
        L.sa_last_error.restype = ctypes.c_char_p
        L.sa_abi_version.argtypes = []
        L.sa_abi_version.restype = ctypes.c_int32
        if L.sa_abi_version() != ABI_VERSION:
            raise RuntimeError("libsa ABI version mismatch")
        _lib = L
    return _lib


def check(status: int) -> None:
    if status != SA_OK:
        msg = lib().sa_last_error().decode(errors="replace")
        raise SaError(status, msg)
