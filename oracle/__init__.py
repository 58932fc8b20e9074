"""fp64 CPU oracle for block-sparse attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import this package.  The product path (the HIP
library and its Python binding) never imports, links or executes anything
here, and nothing here imports the product.

The numeric work lives in ``oracle.c`` (plain C, fp64, OpenMP over rows),
built with gcc into ``liboracle.so`` by :func:`build`.  ``brute.py`` is a
second, dense numpy implementation for tiny inputs.

Parity status of each function (pins live in ``tests/test_oracle_pins.py``):

* ``block_lists``       pinned: the glossary's printed sparsity (85.47 % at
  seq 8192, window 1024, 4 sinks, 128x128 blocks), closed-form block and pair
  counts, the area-attention pair count, dense numpy reshape-sum brute force.
* ``attn_rows``         pinned: dense masked attention brute force (numpy),
  torch's fp64 scaled_dot_product_attention with a boolean mask and with
  ``is_causal`` (O), torch.logsumexp of the masked scores (LSE), Q = 0 closed
  form, single-key closed form, weights sum to 1.
* ``attn_gather_rows``  pinned: equals ``attn_rows`` when the list is the
  allowed set; brute force on tiny inputs.
* ``indexer_scores``    pinned: exact rational arithmetic with per-step
  float32 rounding on tiny inputs; fp64 part against numpy fp64 dot.
* ``topk_rows``         pinned: brute-force Python sort on tiny rows, all-ties
  (zero queries) gives 0..k-1, k >= candidates gives every candidate; NaN
  order against Python's sort on an explicit key.
* ``select_blocks``     pinned: numpy brute force of the block means and
  scores (another summation order) with a sort; zero queries (all ties: the
  lowest reachable blocks); planted one-hot keys with a known ranking;
  n_select >= reachable blocks gives every causal block.
* ``attn_sel_rows``     pinned: dense masked attention brute force with the
  mask built from the lists (numpy); every causal block selected equals
  causal attention (torch fp64 SDPA).
* ``attn_bwd``          pinned: torch fp64 autograd of the dense masked
  attention (a library routine), central finite differences of the oracle's
  own forward on tiny inputs, dQ = 0 and dK = 0 for rows with one allowed key,
  dV columns summing to the columns of dO (each row's weights sum to 1).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.c")
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (fp64, OpenMP) into liboracle.so."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp"
        cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
               "-shared", "-std=c11", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _SO)
    return _SO


class OrcPattern(ctypes.Structure):
    _fields_ = [
        ("causal", ctypes.c_int64),
        ("q_offset", ctypes.c_int64),
        ("window_left", ctypes.c_int64),
        ("window_right", ctypes.c_int64),
        ("sinks", ctypes.c_int64),
        ("stride", ctypes.c_int64),
        ("stride_phase", ctypes.c_int64),
        ("global_tokens", ctypes.c_int64),
        ("unit", ctypes.c_int64),
        ("unit_window", ctypes.c_int64),
        ("rand_units", ctypes.POINTER(ctypes.c_int32)),
        ("n_rand", ctypes.c_int64),
        ("rand_rows", ctypes.c_int64),
    ]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        lib.orc_allowed.argtypes = [ctypes.POINTER(OrcPattern), _I64, _I64]
        lib.orc_allowed.restype = ctypes.c_int
        lib.orc_block_lists.argtypes = [ctypes.POINTER(OrcPattern), _I64, _I64, _I32, _I32,
                                        _P, _P, _P, _P, _P]
        lib.orc_block_lists.restype = None
        lib.orc_attn_rows.argtypes = [ctypes.POINTER(OrcPattern), _P, _P, _P, _I64, _I64, _I32,
                                      ctypes.c_double, _P, _I64, _P, _P, _P]
        lib.orc_attn_rows.restype = None
        lib.orc_attn_gather_rows.argtypes = [_P, _P, _P, _I64, _I64, _I32, ctypes.c_double, _P,
                                             _I32, _I64, _P, _I64, _P, _P]
        lib.orc_attn_gather_rows.restype = None
        lib.orc_indexer_scores.argtypes = [_P, _P, _I64, _I32, _I64, _P, _I64, _P, _P]
        lib.orc_indexer_scores.restype = None
        lib.orc_topk_rows.argtypes = [_P, _P, _I64, _I64, _I32, _P]
        lib.orc_topk_rows.restype = None
        lib.orc_select_blocks.argtypes = [_P, _P, _I64, _I64, _I64, _I32, _I64, _I32, _I32, _I32, _P, _P, _P, _P]
        lib.orc_select_blocks.restype = None
        lib.orc_attn_sel_rows.argtypes = [_P, _P, _P, _I64, _I64, _I32, ctypes.c_double, _I64, _I32, _I32, _P, _P,
                                          _P, _I64, _P, _P]
        lib.orc_attn_sel_rows.restype = None
        lib.orc_attn_bwd.argtypes = [ctypes.POINTER(OrcPattern), _P, _P, _P, _P, _I64, _I64, _I32, ctypes.c_double,
                                     _P, _I64, _P, _P, _P]
        lib.orc_attn_bwd.restype = None
        lib.orc_num_threads.argtypes = []
        lib.orc_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().orc_num_threads())


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


class _PatternHolder:
    """Keeps the random table alive while the C struct points at it."""

    def __init__(self, pattern):
        get = (lambda k, dflt=0: pattern.get(k, dflt)) if isinstance(pattern, dict) else \
            (lambda k, dflt=0: getattr(pattern, k, dflt))
        table = get("rand_table", None)
        self.table = None if table is None else np.ascontiguousarray(table, dtype=np.int32)
        self.s = OrcPattern(
            causal=int(get("causal", 0)), q_offset=int(get("q_offset", 0)),
            window_left=int(get("window_left", -1)), window_right=int(get("window_right", 0)),
            sinks=int(get("sinks", 0)), stride=int(get("stride", 0)),
            stride_phase=int(get("stride_phase", 0)), global_tokens=int(get("global_tokens", 0)),
            unit=int(get("unit", 0)), unit_window=int(get("unit_window", -1)),
            rand_units=(self.table.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
                        if self.table is not None else None),
            n_rand=int(self.table.shape[1]) if self.table is not None else 0,
            rand_rows=int(self.table.shape[0]) if self.table is not None else 0,
        )


def allowed(pattern, q: int, kv: int) -> bool:
    h = _PatternHolder(pattern)
    return bool(_load().orc_allowed(ctypes.byref(h.s), int(q), int(kv)))


def block_lists(pattern, n_q: int, n_kv: int, bq: int, bk: int, with_cells: bool = False):
    """Returns dict(kv_count, kv_index, kv_partial, live_pairs[, cell_counts])."""
    h = _PatternHolder(pattern)
    nqb, nkb = -(-n_q // bq), -(-n_kv // bk)
    kv_count = np.zeros(nqb, np.int32)
    kv_index = np.zeros((nqb, nkb), np.int32)
    kv_partial = np.zeros((nqb, nkb), np.uint8)
    live = np.zeros(1, np.int64)
    cells = np.zeros((nqb, nkb), np.int64) if with_cells else None
    _load().orc_block_lists(ctypes.byref(h.s), n_q, n_kv, bq, bk, _ptr(kv_count), _ptr(kv_index),
                            _ptr(kv_partial), _ptr(live), _ptr(cells) if with_cells else None)
    out = dict(kv_count=kv_count, kv_index=kv_index, kv_partial=kv_partial,
               live_pairs=int(live[0]))
    if with_cells:
        out["cell_counts"] = cells
    return out


def attn_rows(pattern, q: np.ndarray, k: np.ndarray, v: np.ndarray, rows=None,
              scale: float | None = None, return_counts: bool = False):
    """fp64 attention for rows of contiguous [B, H, N, d] bf16-bit tensors.

    ``rows`` holds flattened (b*H + h) * n_q + query_row indices (default: all).
    Returns (O [n_rows, d] fp64, LSE [n_rows] fp64[, allowed counts]).
    """
    h = _PatternHolder(pattern)
    q = np.ascontiguousarray(q, np.uint16)
    k = np.ascontiguousarray(k, np.uint16)
    v = np.ascontiguousarray(v, np.uint16)
    B, H, n_q, d = q.shape
    n_kv = k.shape[2]
    if rows is None:
        rows = np.arange(B * H * n_q, dtype=np.int64)
    rows = np.ascontiguousarray(rows, np.int64)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.zeros((rows.size, d), np.float64)
    lse = np.zeros(rows.size, np.float64)
    cnt = np.zeros(rows.size, np.int64)
    _load().orc_attn_rows(ctypes.byref(h.s), _ptr(q), _ptr(k), _ptr(v), n_q, n_kv, d,
                          float(scale), _ptr(rows), rows.size, _ptr(o), _ptr(lse), _ptr(cnt))
    return (o, lse, cnt) if return_counts else (o, lse)


def attn_gather_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, idx: np.ndarray, rows=None,
                     scale: float | None = None, idx_per_head: bool = False):
    """fp64 attention of each query row over its own key list ``idx``.

    ``idx``: int32 [n_q, topk] shared by all (b, h), or [B*H, n_q, topk] when
    ``idx_per_head``.  Entries < 0 are padding.
    """
    q = np.ascontiguousarray(q, np.uint16)
    k = np.ascontiguousarray(k, np.uint16)
    v = np.ascontiguousarray(v, np.uint16)
    idx = np.ascontiguousarray(idx, np.int32)
    B, H, n_q, d = q.shape
    n_kv = k.shape[2]
    topk = idx.shape[-1]
    bh_stride = n_q * topk if idx_per_head else 0
    if rows is None:
        rows = np.arange(B * H * n_q, dtype=np.int64)
    rows = np.ascontiguousarray(rows, np.int64)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.zeros((rows.size, d), np.float64)
    lse = np.zeros(rows.size, np.float64)
    _load().orc_attn_gather_rows(_ptr(q), _ptr(k), _ptr(v), n_q, n_kv, d, float(scale),
                                 _ptr(idx), topk, bh_stride, _ptr(rows), rows.size, _ptr(o),
                                 _ptr(lse))
    return o, lse


def indexer_scores(q_idx: np.ndarray, k_idx: np.ndarray, q_offset: int, rows=None,
                   with_exact: bool = False):
    """fp32 chained-FMA indexer scores [n_rows, n_kv] (-inf where s > t)."""
    q_idx = np.ascontiguousarray(q_idx, np.uint16)
    k_idx = np.ascontiguousarray(k_idx, np.uint16)
    n_q, d = q_idx.shape
    n_kv = k_idx.shape[0]
    if rows is None:
        rows = np.arange(n_q, dtype=np.int64)
    rows = np.ascontiguousarray(rows, np.int64)
    sigma = np.zeros((rows.size, n_kv), np.float32)
    exact = np.zeros((rows.size, n_kv), np.float64) if with_exact else None
    _load().orc_indexer_scores(_ptr(q_idx), _ptr(k_idx), n_kv, d, int(q_offset), _ptr(rows),
                               rows.size, _ptr(sigma), _ptr(exact) if with_exact else None)
    return (sigma, exact) if with_exact else sigma


def topk_rows(sigma: np.ndarray, n_cand, k: int) -> np.ndarray:
    """Top-k under (score desc, index asc) of each row's first n_cand entries; ascending."""
    sigma = np.ascontiguousarray(sigma, np.float32)
    n_rows, n_kv = sigma.shape
    n_cand = np.ascontiguousarray(np.broadcast_to(np.asarray(n_cand, np.int64), (n_rows,)))
    idx = np.zeros((n_rows, k), np.int32)
    _load().orc_topk_rows(_ptr(sigma), _ptr(n_cand), n_rows, n_kv, int(k), _ptr(idx))
    return idx


def select_blocks(q: np.ndarray, k: np.ndarray, q_offset: int, bq: int, bk: int, n_select: int):
    """Content-selected key blocks of q [B, H, n_q, d], k [B, H, n_kv, d] (bf16 bits).

    Returns dict(kv_count [B*H, nqb], kv_index [B*H, nqb, nkb], kv_partial, live_pairs)."""
    q = np.ascontiguousarray(q, np.uint16)
    k = np.ascontiguousarray(k, np.uint16)
    B, H, n_q, d = q.shape
    n_kv = k.shape[2]
    nqb, nkb = -(-n_q // bq), -(-n_kv // bk)
    kv_count = np.zeros((B * H, nqb), np.int32)
    kv_index = np.zeros((B * H, nqb, nkb), np.int32)
    kv_partial = np.zeros((B * H, nqb, nkb), np.uint8)
    live = np.zeros(1, np.int64)
    _load().orc_select_blocks(_ptr(q), _ptr(k), B * H, n_q, n_kv, d, int(q_offset), bq, bk, int(n_select),
                              _ptr(kv_count), _ptr(kv_index), _ptr(kv_partial), _ptr(live))
    return dict(kv_count=kv_count, kv_index=kv_index, kv_partial=kv_partial, live_pairs=int(live[0]))


def attn_sel_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_offset: int, bq: int, bk: int, kv_count,
                  kv_index, rows=None, scale: float | None = None):
    """fp64 attention of rows over their query block's selected key blocks, causal."""
    q = np.ascontiguousarray(q, np.uint16)
    k = np.ascontiguousarray(k, np.uint16)
    v = np.ascontiguousarray(v, np.uint16)
    kv_count = np.ascontiguousarray(kv_count, np.int32)
    kv_index = np.ascontiguousarray(kv_index, np.int32)
    B, H, n_q, d = q.shape
    n_kv = k.shape[2]
    if rows is None:
        rows = np.arange(B * H * n_q, dtype=np.int64)
    rows = np.ascontiguousarray(rows, np.int64)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.zeros((rows.size, d), np.float64)
    lse = np.zeros(rows.size, np.float64)
    _load().orc_attn_sel_rows(_ptr(q), _ptr(k), _ptr(v), n_q, n_kv, d, float(scale), int(q_offset), bq, bk,
                              _ptr(kv_count), _ptr(kv_index), _ptr(rows), rows.size, _ptr(o), _ptr(lse))
    return o, lse


def attn_bwd(pattern, q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray, heads=None,
             scale: float | None = None):
    """fp64 gradients (dQ, dK, dV) of the masked attention for the slices ``heads``
    (flattened b*H + h indices; default all) of [B, H, N, d] bf16-bit tensors and
    an upstream gradient ``dout`` (bf16 bits like q).  Shapes [n_heads, N, d]."""
    h = _PatternHolder(pattern)
    q = np.ascontiguousarray(q, np.uint16)
    k = np.ascontiguousarray(k, np.uint16)
    v = np.ascontiguousarray(v, np.uint16)
    dout = np.ascontiguousarray(dout, np.uint16)
    B, H, n_q, d = q.shape
    n_kv = k.shape[2]
    bh = np.arange(B * H, dtype=np.int64) if heads is None else np.ascontiguousarray(heads, np.int64)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    dq = np.zeros((bh.size, n_q, d), np.float64)
    dk = np.zeros((bh.size, n_kv, d), np.float64)
    dv = np.zeros((bh.size, n_kv, d), np.float64)
    _load().orc_attn_bwd(ctypes.byref(h.s), _ptr(q), _ptr(k), _ptr(v), _ptr(dout), n_q, n_kv, d, float(scale),
                         _ptr(bh), bh.size, _ptr(dq), _ptr(dk), _ptr(dv))
    return dq, dk, dv
