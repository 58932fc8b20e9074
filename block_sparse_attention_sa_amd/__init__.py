"""Block-sparse attention forward for MI355X (gfx950).

Python binding of libsa.so (C ABI in include/sa.h).  PyTorch supplies device
memory and streams; every step of the computation runs in the HIP kernels of
the library.  The functions mirror the library's entry points:

* :func:`build_block_mask`  -> ``sa_build_block_mask``
* :func:`attn_fwd`          -> ``sa_attn_fwd`` (block lists or gather lists)
* :func:`indexer_scores`, :func:`topk`, :func:`indexer_topk`
                            -> ``sa_indexer_scores``, ``sa_topk``, ``sa_indexer_topk``

There is no CPU fallback: without the built library (or without a GPU) the
calls raise.
"""

from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional

import numpy as np

from . import _lib
from ._lib import SaError  # noqa: F401

__all__ = ["BlockLists", "build_block_mask", "select_blocks", "attn_fwd", "attn_bwd", "attn_workspace_bytes", "attn_fwd_strided",
           "attn_workspace_bytes_strided", "strided_plan", "merge_partial", "indexer_scores", "topk", "indexer_topk",
           "indexer_topk_workspace_bytes", "indexer_topk_noalloc", "describe", "SaError"]


def _torch():
    import torch
    return torch


def _stream_ptr(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _get(pattern, key, default):
    if isinstance(pattern, dict):
        return pattern.get(key, default)
    return getattr(pattern, key, default)


@dataclasses.dataclass
class DevicePattern:
    """A pattern with its random table resident on the device."""

    struct: _lib.SaPattern
    table: Optional[object]  # torch tensor kept alive


def device_pattern(pattern, device) -> DevicePattern:
    torch = _torch()
    table = _get(pattern, "rand_table", None)
    t = None
    if table is not None:
        arr = np.ascontiguousarray(table, dtype=np.int32)
        t = torch.from_numpy(arr).to(device)
    s = _lib.SaPattern(
        causal=int(_get(pattern, "causal", 0)),
        q_offset=int(_get(pattern, "q_offset", 0)),
        window_left=int(_get(pattern, "window_left", -1)),
        window_right=int(_get(pattern, "window_right", 0)),
        sinks=int(_get(pattern, "sinks", 0)),
        stride=int(_get(pattern, "stride", 0)),
        stride_phase=int(_get(pattern, "stride_phase", 0)),
        global_tokens=int(_get(pattern, "global_tokens", 0)),
        unit=int(_get(pattern, "unit", 0)),
        unit_window=int(_get(pattern, "unit_window", -1)),
        rand_units=t.data_ptr() if t is not None else None,
        n_rand=int(t.shape[1]) if t is not None else 0,
        rand_rows=int(t.shape[0]) if t is not None else 0,
    )
    return DevicePattern(s, t)


@dataclasses.dataclass
class BlockLists:
    """Output of :func:`build_block_mask` (device tensors)."""

    kv_count: object    # int32 [nqb] (per_head: [B*H, nqb])
    kv_index: object    # int32 [nqb, nkb] (per_head: [B*H, nqb, nkb])
    kv_partial: object  # uint8 like kv_index
    live_pairs: object  # int64 [1]
    n_q: int
    n_kv: int
    block_q: int
    block_kv: int
    pattern: DevicePattern
    per_head: bool = False


def build_block_mask(pattern, n_q: int, n_kv: int, block_q: int, block_kv: int,
                     device="cuda", out: Optional[BlockLists] = None) -> BlockLists:
    """Per-query-block live key-block lists of ``pattern`` (``sa_build_block_mask``)."""
    torch = _torch()
    device = torch.device(device)
    nqb, nkb = -(-n_q // block_q), -(-n_kv // block_kv)
    if out is None:
        dp = device_pattern(pattern, device)
        out = BlockLists(
            kv_count=torch.empty(nqb, dtype=torch.int32, device=device),
            kv_index=torch.empty((nqb, nkb), dtype=torch.int32, device=device),
            kv_partial=torch.empty((nqb, nkb), dtype=torch.uint8, device=device),
            live_pairs=torch.empty(1, dtype=torch.int64, device=device),
            n_q=n_q, n_kv=n_kv, block_q=block_q, block_kv=block_kv, pattern=dp)
    _lib.check(_lib.lib().sa_build_block_mask(
        ctypes.byref(out.pattern.struct), n_q, n_kv, block_q, block_kv,
        out.kv_count.data_ptr(), out.kv_index.data_ptr(), out.kv_partial.data_ptr(),
        out.live_pairs.data_ptr(), _stream_ptr(device)))
    return out


def select_blocks(q, k, block_q: int, block_kv: int, n_select: int, q_offset: int = 0, workspace=None,
                  out: Optional[BlockLists] = None) -> BlockLists:
    """Content-selected key blocks per (b, h, query block) (``sa_select_blocks``): the
    block's own key blocks plus the ``n_select`` causally reachable ones whose mean key
    scores highest against the block's mean query.  q [B, H, n_q, d], k [B, H, n_kv, d]
    bfloat16.  The result drives :func:`attn_fwd` with a causal element mask."""
    torch = _torch()
    for t in (q, k):
        if t.dtype != torch.bfloat16 or not t.is_cuda or t.dim() != 4:
            raise ValueError("q and k must be 4-d bfloat16 CUDA tensors")
    B, H, n_q, d = q.shape
    n_kv = k.shape[2]
    nqb, nkb = -(-n_q // block_q), -(-n_kv // block_kv)
    dev = q.device
    if out is None:
        out = BlockLists(
            kv_count=torch.empty((B * H, nqb), dtype=torch.int32, device=dev),
            kv_index=torch.empty((B * H, nqb, nkb), dtype=torch.int32, device=dev),
            kv_partial=torch.empty((B * H, nqb, nkb), dtype=torch.uint8, device=dev),
            live_pairs=torch.empty(1, dtype=torch.int64, device=dev),
            n_q=n_q, n_kv=n_kv, block_q=block_q, block_kv=block_kv,
            pattern=device_pattern(dict(causal=1, q_offset=q_offset, window_left=n_kv + q_offset), dev),
            per_head=True)
    a = _lib.SaSelectArgs()
    a.q, a.k = q.data_ptr(), k.data_ptr()
    a.batch, a.heads, a.n_q, a.n_kv, a.head_dim = B, H, n_q, n_kv, d
    a.q_strides[:] = _strides3(q)
    a.k_strides[:] = _strides3(k)
    a.q_offset, a.block_q, a.block_kv, a.n_select = int(q_offset), block_q, block_kv, int(n_select)
    a.kv_count, a.kv_index = out.kv_count.data_ptr(), out.kv_index.data_ptr()
    a.kv_partial, a.live_pairs = out.kv_partial.data_ptr(), out.live_pairs.data_ptr()
    need = int(_lib.lib().sa_select_blocks_workspace(ctypes.byref(a)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
    _lib.check(_lib.lib().sa_select_blocks(ctypes.byref(a), _stream_ptr(dev)))
    return out


def _strides3(t) -> list:
    if t.numel() == 0:  # nothing is read or written: report the contiguous strides
        d = int(t.shape[-1])
        return [int(t.shape[1]) * int(t.shape[2]) * d, int(t.shape[2]) * d, d]
    s = t.stride()
    if s[-1] != 1:
        raise ValueError("the last dimension must be contiguous")
    return [int(s[0]), int(s[1]), int(s[2])]


def attn_fwd(q, k, v, blocks: Optional[BlockLists] = None, gather_idx=None, *,
             o_dtype=None, softmax_scale: Optional[float] = None, out=None, lse=None,
             want_lse: bool = True, workspace=None, split: bool = True):
    """Block-sparse (``blocks``) or per-query gather (``gather_idx``) attention forward.

    q [B, H, n_q, d], k/v [B, H, n_kv, d] bfloat16 on the GPU.  ``gather_idx``
    is int32 [n_q, topk] shared by every (b, h), or [B, H, n_q, topk].
    In gather mode over a long key range, and in block mode for the rows of
    global tokens that see every key, the library can take a split form that
    needs scratch (``attn_workspace_bytes``): pass a uint8 CUDA tensor as
    ``workspace``, or leave it None and one is allocated for the call;
    ``split=False`` forces the single-pass form.
    Returns (O [B, H, n_q, d] in ``o_dtype`` (default float32), LSE float32
    [B, H, n_q] or None).
    """
    torch = _torch()
    if (blocks is None) == (gather_idx is None):
        raise ValueError("pass exactly one of blocks / gather_idx")
    for t in (q, k, v):
        if t.dtype != torch.bfloat16 or not t.is_cuda or t.dim() != 4:
            raise ValueError("q, k, v must be 4-d bfloat16 CUDA tensors")
    B, H, n_q, d = q.shape
    n_kv = k.shape[2]
    if k.shape != (B, H, n_kv, d) or v.shape != (B, H, n_kv, d):
        raise ValueError("k/v shape mismatch")
    o_dtype = torch.float32 if o_dtype is None else o_dtype
    if out is None:
        out = torch.empty((B, H, n_q, d), dtype=o_dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H, n_q), dtype=torch.float32, device=q.device)
    if tuple(out.shape) != (B, H, n_q, d) or not out.is_cuda:
        raise ValueError("out must be a CUDA tensor of shape [B, H, n_q, d]")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_cuda or not lse.is_contiguous()
                            or lse.numel() != B * H * n_q):
        raise ValueError("lse must be a contiguous float32 CUDA tensor of B * H * n_q values")
    a = _lib.SaAttnArgs()
    a.q, a.k, a.v, a.o = q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr()
    a.lse = lse.data_ptr() if lse is not None else None
    a.batch, a.heads, a.n_q, a.n_kv, a.head_dim = B, H, n_q, n_kv, d
    a.o_dtype = _lib.SA_DTYPE_F32 if out.dtype == torch.float32 else _lib.SA_DTYPE_BF16
    if out.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("o_dtype must be float32 or bfloat16")
    a.q_strides[:] = _strides3(q)
    a.k_strides[:] = _strides3(k)
    a.v_strides[:] = _strides3(v)
    a.o_strides[:] = _strides3(out)
    a.softmax_scale = float(softmax_scale) if softmax_scale else 0.0
    keep = []
    if blocks is not None:
        if blocks.n_q != n_q or blocks.n_kv != n_kv:
            raise ValueError("block lists were built for another n_q / n_kv")
        a.mode = _lib.SA_MODE_BLOCKS
        a.block_q, a.block_kv = blocks.block_q, blocks.block_kv
        a.kv_count = blocks.kv_count.data_ptr()
        a.kv_index = blocks.kv_index.data_ptr()
        a.kv_partial = blocks.kv_partial.data_ptr()
        a.pattern = blocks.pattern.struct
        a.per_head_lists = 1 if blocks.per_head else 0
        if blocks.per_head and tuple(blocks.kv_count.shape) != (B * H, -(-n_q // blocks.block_q)):
            raise ValueError("per-head block lists were built for another batch * heads")
    else:
        g = gather_idx
        if g.dtype != torch.int32 or not g.is_cuda or not g.is_contiguous():
            raise ValueError("gather_idx must be a contiguous int32 CUDA tensor")
        a.mode = _lib.SA_MODE_GATHER
        a.gather_idx = g.data_ptr()
        a.topk = int(g.shape[-1])
        if g.dim() == 2:
            if g.shape[0] != n_q:
                raise ValueError("gather_idx rows must equal n_q")
            a.gather_bh_stride = 0
        elif g.dim() == 4 and tuple(g.shape[:3]) == (B, H, n_q):
            a.gather_bh_stride = n_q * a.topk
        else:
            raise ValueError("gather_idx must be [n_q, topk] or [B, H, n_q, topk]")
        keep.append(g)
    need = int(_lib.lib().sa_attn_workspace_bytes(ctypes.byref(a))) if split else 0
    if need > 0:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        if workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 CUDA tensor")
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel()
    _lib.check(_lib.lib().sa_attn_fwd(ctypes.byref(a), _stream_ptr(q.device)))
    return out, lse



def attn_bwd(q, k, v, o, lse, dout, blocks: BlockLists, *, softmax_scale: Optional[float] = None,
             dq=None, dk=None, dv=None, workspace=None):
    """Gradients (dQ, dK, dV) of the block-sparse attention (``sa_attn_bwd``) for the
    upstream gradient ``dout``.  q, k, v, dout bfloat16 contiguous [B, H, n, d]; o float32
    and lse float32 are the forward's outputs for the same ``blocks``.  Returns float32
    (dq [B, H, n_q, d], dk, dv [B, H, n_kv, d])."""
    torch = _torch()
    for t in (q, k, v, dout):
        if t.dtype != torch.bfloat16 or not t.is_cuda or t.dim() != 4 or not t.is_contiguous():
            raise ValueError("q, k, v, dout must be contiguous 4-d bfloat16 CUDA tensors")
    B, H, n_q, d = q.shape
    n_kv = k.shape[2]
    if tuple(dout.shape) != (B, H, n_q, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("shape mismatch")
    if o.dtype != torch.float32 or not o.is_contiguous() or tuple(o.shape) != (B, H, n_q, d):
        raise ValueError("o must be the forward's contiguous float32 output")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != B * H * n_q:
        raise ValueError("lse must be the forward's contiguous float32 logsumexp")
    if blocks.n_q != n_q or blocks.n_kv != n_kv:
        raise ValueError("block lists were built for another n_q / n_kv")
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty((B, H, n_q, d), **f32) if dq is None else dq
    dk = torch.empty((B, H, n_kv, d), **f32) if dk is None else dk
    dv = torch.empty((B, H, n_kv, d), **f32) if dv is None else dv
    a = _lib.SaAttnBwdArgs()
    a.q, a.k, a.v, a.o, a.lse, a.dout = (t.data_ptr() for t in (q, k, v, o, lse, dout))
    a.dq, a.dk, a.dv = dq.data_ptr(), dk.data_ptr(), dv.data_ptr()
    a.batch, a.heads, a.n_q, a.n_kv, a.head_dim = B, H, n_q, n_kv, d
    a.softmax_scale = float(softmax_scale) if softmax_scale else 0.0
    a.block_q, a.block_kv = blocks.block_q, blocks.block_kv
    a.kv_count, a.kv_index, a.kv_partial = (t.data_ptr() for t in (blocks.kv_count, blocks.kv_index,
                                                                    blocks.kv_partial))
    a.per_head_lists = 1 if blocks.per_head else 0
    a.pattern = blocks.pattern.struct
    need = int(_lib.lib().sa_attn_bwd_workspace(ctypes.byref(a)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
    _lib.check(_lib.lib().sa_attn_bwd(ctypes.byref(a), _stream_ptr(q.device)))
    return dq, dk, dv


def merge_partial(out, lse, o2, lse2, group: int = 1, q_first: int = 0, n2: Optional[int] = None):
    """Fold a second partial result (``o2``, ``lse2``) into (``out``, ``lse``) in place
    (``sa_merge_partial``): out/o2 float32 [B, H, n, d] views, lse float32 [B, H, n]
    contiguous; rows q = q_first + i*group + r (i < n2) take the second part, whose LSE
    sits at lse2[b, h, r, i]."""
    torch = _torch()
    for t in (out, lse, o2, lse2):
        if t.dtype != torch.float32 or not t.is_cuda:
            raise ValueError("merge_partial takes float32 CUDA tensors")
    if not lse.is_contiguous() or not lse2.is_contiguous():
        raise ValueError("lse and lse2 must be contiguous")
    B, H, n, d = out.shape
    if tuple(o2.shape) != (B, H, n, d) or tuple(lse.shape) != (B, H, n):
        raise ValueError("shape mismatch")
    if n2 is None:
        n2 = -(-(n - q_first) // group)
    if lse2.numel() != B * H * group * n2:
        raise ValueError("lse2 must hold batch * heads * group * n2 values")
    os3 = (ctypes.c_int64 * 3)(*_strides3(out))
    o2s = (ctypes.c_int64 * 3)(*_strides3(o2))
    _lib.check(_lib.lib().sa_merge_partial(out.data_ptr(), lse.data_ptr(), o2.data_ptr(), lse2.data_ptr(),
                                           B, H, n, d, os3, o2s, group, q_first, n2, _stream_ptr(out.device)))


def _strided_args(q, k, v, pattern, out, lse, softmax_scale):
    a = _lib.SaAttnArgs()
    B, H, n, d = q.shape
    a.q, a.k, a.v, a.o = q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr()
    a.lse = lse.data_ptr()
    a.batch, a.heads, a.n_q, a.n_kv, a.head_dim = B, H, n, n, d
    a.o_dtype = _lib.SA_DTYPE_F32
    a.q_strides[:] = _strides3(q)
    a.k_strides[:] = _strides3(k)
    a.v_strides[:] = _strides3(v)
    a.o_strides[:] = _strides3(out)
    a.softmax_scale = float(softmax_scale) if softmax_scale else 0.0
    a.mode = _lib.SA_MODE_STRIDED
    a.pattern = _template_struct(pattern)
    return a


def strided_plan(pattern, batch: int, heads: int, n: int, head_dim: int, device="cuda"):
    """The workspace of ``attn_fwd_strided`` with the block lists of its parts built in it
    (``sa_attn_strided_plan``); reusable by every call with the same pattern and length."""
    torch = _torch()
    need = attn_workspace_bytes_strided(pattern, batch, heads, n, head_dim)
    if need == 0:
        raise ValueError("not the strided template that splits into band + residue views")
    ws = torch.empty(need, dtype=torch.uint8, device=device)
    a = _lib.SaAttnArgs()
    a.batch, a.heads, a.n_q, a.n_kv, a.head_dim = batch, heads, n, n, head_dim
    a.mode = _lib.SA_MODE_STRIDED
    a.pattern = _template_struct(pattern)
    a.k_strides[:] = a.v_strides[:] = [heads * n * head_dim, n * head_dim, head_dim]
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    _lib.check(_lib.lib().sa_attn_strided_plan(ctypes.byref(a), _stream_ptr(torch.device(device))))
    return ws


def attn_fwd_strided(q, k, v, pattern, *, softmax_scale: Optional[float] = None, out=None, lse=None,
                     workspace=None):
    """The strided template as disjoint key sets per row (``sa_attn_fwd``, ``SA_MODE_STRIDED``):
    the local band through block lists, the strided keys as causal attention between
    strided views (one per head and key residue; residue 0's view also holds the last row),
    merged by log-sum-exp in the kernel epilogue.  q, k, v bfloat16 [B, H, n, d]; ``pattern`` must be the template (causal,
    window_left = stride - 1, stride_phase = stride - 1, no other term; n a multiple of the
    stride, at least three groups), else the library rejects it.  ``workspace`` is a plan
    from ``strided_plan`` (made for the call when None).  Returns (O float32 [B, H, n, d],
    LSE [B, H, n])."""
    torch = _torch()
    for t in (q, k, v):
        if t.dtype != torch.bfloat16 or not t.is_cuda or t.dim() != 4 or t.stride(-1) != 1:
            raise ValueError("q, k, v must be 4-d bfloat16 CUDA tensors with contiguous rows")
    B, H, n, d = q.shape
    if tuple(k.shape) != (B, H, n, d) or tuple(v.shape) != (B, H, n, d):
        raise ValueError("q, k and v must have the same shape [B, H, n, d]")
    out = torch.empty((B, H, n, d), dtype=torch.float32, device=q.device) if out is None else out
    lse = torch.empty((B, H, n), dtype=torch.float32, device=q.device) if lse is None else lse
    if out.dtype != torch.float32 or tuple(out.shape) != (B, H, n, d):
        raise ValueError("out must be float32 [B, H, n, d]")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != B * H * n:
        raise ValueError("lse must be a contiguous float32 tensor of B * H * n values")
    if workspace is None:
        workspace = strided_plan(pattern, B, H, n, d, q.device)
    if workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 CUDA tensor")
    a = _strided_args(q, k, v, pattern, out, lse, softmax_scale)
    a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
    _lib.check(_lib.lib().sa_attn_fwd(ctypes.byref(a), _stream_ptr(q.device)))
    return out, lse


def _template_struct(pattern):
    g = lambda key, dflt: int(_get(pattern, key, dflt) or 0)
    return _lib.SaPattern(causal=g("causal", 0), q_offset=g("q_offset", 0), window_left=g("window_left", -1),
                          window_right=g("window_right", 0), sinks=g("sinks", 0), stride=g("stride", 0),
                          stride_phase=g("stride_phase", 0), global_tokens=g("global_tokens", 0),
                          unit=g("unit", 0), unit_window=g("unit_window", -1), rand_units=None,
                          n_rand=g("n_rand", 0), rand_rows=0)


def attn_workspace_bytes_strided(pattern, batch: int, heads: int, n: int, head_dim: int) -> int:
    """Scratch bytes of ``attn_fwd_strided`` (0: ``pattern`` is not the strided template).
    Touches no device."""
    a = _lib.SaAttnArgs()
    a.batch, a.heads, a.n_q, a.n_kv, a.head_dim = batch, heads, n, n, head_dim
    a.mode = _lib.SA_MODE_STRIDED
    a.pattern = _template_struct(pattern)
    return int(_lib.lib().sa_attn_workspace_bytes(ctypes.byref(a)))


def attn_workspace_bytes_blocks(blocks: BlockLists, batch: int, heads: int, head_dim: int) -> int:
    """Scratch bytes of block mode's long-row split for these lists (0 if it has none):
    without causality the query blocks of global tokens list every key block, and with
    more than 8 key blocks they are walked in chunks by separate workgroups.  Touches
    no device."""
    a = _lib.SaAttnArgs()
    a.batch, a.heads, a.n_q, a.n_kv, a.head_dim = batch, heads, blocks.n_q, blocks.n_kv, head_dim
    a.mode = _lib.SA_MODE_BLOCKS
    a.block_q, a.block_kv = blocks.block_q, blocks.block_kv
    a.pattern = blocks.pattern.struct
    a.per_head_lists = 1 if blocks.per_head else 0
    return int(_lib.lib().sa_attn_workspace_bytes(ctypes.byref(a)))


def attn_workspace_bytes(batch: int, heads: int, n_q: int, n_kv: int, head_dim: int, topk: int,
                         per_head_lists: bool = False) -> int:
    """Scratch bytes of the split gather form for these sizes (0 if it has none)."""
    a = _lib.SaAttnArgs()
    a.batch, a.heads, a.n_q, a.n_kv, a.head_dim = batch, heads, n_q, n_kv, head_dim
    a.mode = _lib.SA_MODE_GATHER
    a.topk = topk
    a.gather_bh_stride = n_q * topk if per_head_lists else 0
    return int(_lib.lib().sa_attn_workspace_bytes(ctypes.byref(a)))


def indexer_scores(q_idx, k_idx, q_offset: int, scores=None):
    """float32 [n_q, n_kv] indexer scores (entries s > q_offset + r untouched)."""
    torch = _torch()
    n_q, d = q_idx.shape
    n_kv = k_idx.shape[0]
    _check_idx(q_idx, k_idx)
    if scores is None:
        scores = torch.empty((n_q, n_kv), dtype=torch.float32, device=q_idx.device)
    _lib.check(_lib.lib().sa_indexer_scores(q_idx.data_ptr(), k_idx.data_ptr(), n_q, n_kv, d,
                                            int(q_offset), scores.data_ptr(),
                                            _stream_ptr(q_idx.device)))
    return scores


def topk(scores, q_offset: int, k: int, out=None):
    """int32 [n_q, k]: per row the k best candidates (score desc, index asc), ascending."""
    torch = _torch()
    if scores.dtype != torch.float32 or not scores.is_contiguous():
        raise ValueError("scores must be contiguous float32")
    n_q, n_kv = scores.shape
    if out is None:
        out = torch.empty((n_q, k), dtype=torch.int32, device=scores.device)
    _lib.check(_lib.lib().sa_topk(scores.data_ptr(), n_q, n_kv, int(q_offset), int(k),
                                  out.data_ptr(), _stream_ptr(scores.device)))
    return out


def indexer_topk_workspace_bytes(n_q: int, n_kv: int, k: int) -> int:
    """Scratch bytes of the streaming indexer + top-k (``sa_indexer_topk_workspace``)."""
    return int(_lib.lib().sa_indexer_topk_workspace(n_q, n_kv, k))


def indexer_topk(q_idx, k_idx, q_offset: int, k: int, out=None, scores=None, keep_scores: bool = False,
                 workspace=None):
    """Indexer scores and the top-k in one call (``sa_indexer_topk``); returns (idx, scores).

    By default the call streams: no score matrix is written (``scores`` is None
    on return) and the scratch is ``workspace`` (a uint8 CUDA tensor of at
    least ``indexer_topk_workspace_bytes`` bytes, allocated for the call when
    None).  With ``keep_scores`` (or a ``scores`` tensor) the scores are
    written to float32 [n_q, n_kv] first and the selection reads them back.
    """
    torch = _torch()
    n_q, d = q_idx.shape
    n_kv = k_idx.shape[0]
    _check_idx(q_idx, k_idx)
    if out is None:
        out = torch.empty((n_q, k), dtype=torch.int32, device=q_idx.device)
    if (keep_scores or scores is not None) and scores is None:
        scores = torch.empty((n_q, n_kv), dtype=torch.float32, device=q_idx.device)
    ws_ptr, ws_bytes = None, 0
    if scores is None:
        need = indexer_topk_workspace_bytes(n_q, n_kv, k)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q_idx.device)
        if workspace is not None:
            if workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
                raise ValueError("workspace must be a contiguous uint8 CUDA tensor")
            ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    _lib.check(_lib.lib().sa_indexer_topk(q_idx.data_ptr(), k_idx.data_ptr(), n_q, n_kv, d,
                                          int(q_offset), int(k),
                                          scores.data_ptr() if scores is not None else None,
                                          out.data_ptr(), ws_ptr, ws_bytes, _stream_ptr(q_idx.device)))
    return out, scores


def indexer_topk_noalloc(q_idx, k_idx, q_offset: int, k: int, out=None):
    """The streaming indexer + top-k on the library's fixed per-device scratch
    (``sa_indexer_topk_noalloc``): the C call allocates nothing.  Calls that
    overlap on one device race on that scratch.  Returns idx int32 [n_q, k]."""
    torch = _torch()
    n_q, d = q_idx.shape
    n_kv = k_idx.shape[0]
    _check_idx(q_idx, k_idx)
    if out is None:
        out = torch.empty((n_q, k), dtype=torch.int32, device=q_idx.device)
    _lib.check(_lib.lib().sa_indexer_topk_noalloc(q_idx.data_ptr(), k_idx.data_ptr(), n_q, n_kv, d, int(q_offset),
                                                  int(k), out.data_ptr(), _stream_ptr(q_idx.device)))
    return out


def _check_idx(q_idx, k_idx):
    torch = _torch()
    for t in (q_idx, k_idx):
        if t.dtype != torch.bfloat16 or not t.is_cuda or t.dim() != 2 or not t.is_contiguous():
            raise ValueError("indexer inputs must be contiguous 2-d bfloat16 CUDA tensors")
    if q_idx.shape[1] != k_idx.shape[1]:
        raise ValueError("indexer dims differ")


def describe(blocks: BlockLists, max_rows: int = 16) -> str:
    """Sparsity summary and an ASCII map of the live blocks ('#' full, '+' partial)."""
    cnt = blocks.kv_count.cpu().numpy()
    idx = blocks.kv_index.cpu().numpy()
    par = blocks.kv_partial.cpu().numpy()
    nqb, nkb = idx.shape
    live = int(cnt.sum())
    n_part = int(sum(par[i, : cnt[i]].sum() for i in range(nqb)))
    lines = [f"blocks {nqb}x{nkb} of {blocks.block_q}x{blocks.block_kv}: live {live} "
             f"(full {live - n_part}, partial {n_part}), sparsity "
             f"{100.0 * (nqb * nkb - live) / max(1, nqb * nkb):.2f}%, "
             f"live pairs {int(blocks.live_pairs.cpu()[0])}"]
    step = max(1, nqb // max_rows)
    for i in range(0, nqb, step):
        row = ["."] * nkb
        for e in range(cnt[i]):
            row[idx[i, e]] = "+" if par[i, e] else "#"
        lines.append("".join(row[:: max(1, nkb // 64)]))
    return "\n".join(lines)
