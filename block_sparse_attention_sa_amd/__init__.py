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

__all__ = ["BlockLists", "build_block_mask", "attn_fwd", "attn_workspace_bytes", "indexer_scores", "topk", "indexer_topk",
           "describe", "SaError"]


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

    kv_count: object    # int32 [nqb]
    kv_index: object    # int32 [nqb, nkb]
    kv_partial: object  # uint8 [nqb, nkb]
    live_pairs: object  # int64 [1]
    n_q: int
    n_kv: int
    block_q: int
    block_kv: int
    pattern: DevicePattern


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
    In gather mode over a long key range the library can take a split form
    that needs scratch (``attn_workspace_bytes``): pass a uint8 CUDA tensor
    as ``workspace``, or leave it None and one is allocated for the call;
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


def strided_stride(pattern, n_q: int, n_kv: int) -> int:
    """The stride S when ``pattern`` is the strided template that ``attn_fwd_strided`` computes
    as disjoint parts (causal; local band q - kv <= S - 1; strided keys with
    (q - kv) % S == S - 1; no other term; q_offset 0; n_q == n_kv a multiple of S with at least
    three groups of S rows), else 0."""
    g = lambda key, dflt: int(_get(pattern, key, dflt) or 0)
    S = g("stride", 0)
    if S <= 0 or g("stride_phase", 0) != S - 1 or not g("causal", 0):
        return 0
    if g("window_left", -1) != S - 1 or g("window_right", 0) != 0:
        return 0
    if g("sinks", 0) or g("global_tokens", 0) or g("unit", 0) or g("n_rand", 0) or g("q_offset", 0):
        return 0
    if n_q != n_kv or n_q % S or n_q // S < 3:
        return 0
    return S


@dataclasses.dataclass
class StridedPlan:
    """Block lists of the parts of a strided pattern (``plan_strided``)."""

    stride: int
    n: int
    band: BlockLists
    strided: BlockLists
    last: BlockLists


def plan_strided(pattern, n: int, block: int = 64, device="cuda",
                 residue_block: Optional[int] = None) -> StridedPlan:
    """Block lists for ``attn_fwd_strided``: the local band on the natural layout
    (block x block tiles); plain causal lists shared by every (head, key residue) view;
    and one row against every key of its view for the last query row."""
    S = strided_stride(pattern, n, n)
    if not S:
        raise ValueError("not the strided template that splits into band + residue views")
    G = n // S
    band = build_block_mask(dict(causal=1, window_left=S - 1, window_right=0), n, n, block, block, device)
    bs = residue_block or 64  # 64-row tiles: twice the workgroups of 128-row ones, 3 % faster
    # a local term whose window covers every row (a pattern without any term allows no pair)
    strided = build_block_mask(dict(causal=1, window_left=G, window_right=0), G - 2, G - 2, bs, bs, device)
    last = build_block_mask(dict(causal=0, window_left=G, window_right=G), 1, G - 1, 64, bs, device)
    return StridedPlan(S, n, band, strided, last)


def attn_fwd_strided(q, k, v, plan: StridedPlan, *, softmax_scale: Optional[float] = None,
                     out=None, lse=None, o2=None, lse2=None, lse3=None):
    """The strided template as disjoint key sets per query row, merged by LSE.

    * band: kv in [q - (S - 1), q], through block lists on the natural layout;
    * strided: kv = q - (S - 1) - S*m for m >= 1, i.e. keys kv = j*S + rho of one residue
      rho for the rows q = (i + 2)*S + rho - 1, with j <= i: for every key residue a plain
      causal attention between strided views of the same tensors (row step S rows, residue
      step one row; queries from row 2S - 1 on), no copy.  The views are batched as
      [heads, S residues, n/S - 2 rows, d];
    * the one row those views leave out, q = n - 1 (residue 0, one group further), against
      its keys j*S, j <= n/S - 2;
    * ``sa_merge_partial`` folds the two strided parts into the band part.
    q, k, v bfloat16 [B, H, n, d].  Returns (O float32 [B, H, n, d], LSE [B, H, n]);
    ``o2`` (float32 like O), ``lse2`` (float32 [B, H, S, n/S - 2]) and ``lse3`` (float32
    [B, H, 1, 1]) are scratch, allocated when None.
    """
    torch = _torch()
    for t in (q, k, v):
        if t.dtype != torch.bfloat16 or not t.is_cuda or t.dim() != 4 or t.stride(-1) != 1:
            raise ValueError("q, k, v must be 4-d bfloat16 CUDA tensors with contiguous rows")
    B, H, n, d = q.shape
    if tuple(k.shape) != (B, H, n, d) or tuple(v.shape) != (B, H, n, d):
        raise ValueError("q, k and v must have the same shape [B, H, n, d]")
    if n != plan.n:
        raise ValueError("plan was built for another sequence length")
    S, G = plan.stride, n // plan.stride
    f32, dev = torch.float32, q.device
    out = torch.empty((B, H, n, d), dtype=f32, device=dev) if out is None else out
    lse = torch.empty((B, H, n), dtype=f32, device=dev) if lse is None else lse
    if out.dtype != f32:
        raise ValueError("the strided form writes a float32 O")
    o2 = torch.empty((B, H, n, d), dtype=f32, device=dev) if o2 is None else o2
    lse2 = torch.empty((B, H, S, G - 2), dtype=f32, device=dev) if lse2 is None else lse2
    lse3 = torch.empty((B, H, 1, 1), dtype=f32, device=dev) if lse3 is None else lse3
    if tuple(o2.shape) != (B, H, n, d) or o2.dtype != f32:
        raise ValueError("o2 must be float32 [B, H, n, d]")
    if tuple(lse2.shape) != (B, H, S, G - 2) or tuple(lse3.shape) != (B, H, 1, 1):
        raise ValueError("lse2 must be [B, H, S, n/S - 2] and lse3 [B, H, 1, 1]")
    attn_fwd(q, k, v, plan.band, softmax_scale=softmax_scale, out=out, lse=lse)
    for b in range(B):
        def view(t, res, rows, first):
            st = t.stride()
            return t.as_strided((H, res, rows, d), (st[1], st[2], S * st[2], 1),
                                t.storage_offset() + b * st[0] + first * st[2])
        attn_fwd(view(q, S, G - 2, 2 * S - 1), view(k, S, G - 2, 0), view(v, S, G - 2, 0), plan.strided,
                 softmax_scale=softmax_scale, out=view(o2, S, G - 2, 2 * S - 1), lse=lse2[b])
        attn_fwd(view(q, 1, 1, n - 1), view(k, 1, G - 1, 0), view(v, 1, G - 1, 0), plan.last,
                 softmax_scale=softmax_scale, out=view(o2, 1, 1, n - 1), lse=lse3[b])
    merge_partial(out, lse, o2, lse2, group=S, q_first=2 * S - 1, n2=G - 2)
    merge_partial(out, lse, o2, lse3, group=1, q_first=n - 1, n2=1)
    return out, lse

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


def indexer_topk(q_idx, k_idx, q_offset: int, k: int, scores=None, out=None):
    """Indexer scores into ``scores`` (workspace) then the top-k; returns (idx, scores)."""
    torch = _torch()
    n_q, d = q_idx.shape
    n_kv = k_idx.shape[0]
    _check_idx(q_idx, k_idx)
    if scores is None:
        scores = torch.empty((n_q, n_kv), dtype=torch.float32, device=q_idx.device)
    if out is None:
        out = torch.empty((n_q, k), dtype=torch.int32, device=q_idx.device)
    _lib.check(_lib.lib().sa_indexer_topk(q_idx.data_ptr(), k_idx.data_ptr(), n_q, n_kv, d,
                                          int(q_offset), int(k), scores.data_ptr(),
                                          out.data_ptr(), _stream_ptr(q_idx.device)))
    return out, scores


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
