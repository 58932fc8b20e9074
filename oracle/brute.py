"""Dense numpy brute force for tiny inputs -- TEST INFRASTRUCTURE ONLY.

A second implementation, independent of ``oracle.c``, of what the pages define
directly: a dense boolean mask over the full score matrix, scores
q.k^T / sqrt(d) with disallowed pairs set to -inf, a row softmax and the
product with V (blog "Sparse transformers: how to cut the O(n^2) of
attention", section on how it looks in code); and the split of a mask into
fixed-size blocks whose share of empty blocks is the sparsity figure
("Sparse Attention" glossary, section on turning a pattern into savings).
Everything is materialised n x n, so only tiny sizes are practical.
"""

from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(
        np.float64)


def masked_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
                     scale: float | None = None):
    """q [n_q, d], k/v [n_kv, d] float64, mask [n_q, n_kv] bool (True = allowed).

    Returns (O [n_q, d], LSE [n_q]); a row with no allowed key gives O = 0 and
    LSE = -inf.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    scores = (q @ k.T) * scale
    scores = np.where(mask, scores, -np.inf)
    m = scores.max(axis=-1, keepdims=True)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(scores - m_safe)
    s = e.sum(axis=-1, keepdims=True)
    w = np.divide(e, s, out=np.zeros_like(e), where=s > 0)
    o = w @ v
    with np.errstate(divide="ignore"):
        lse = (m_safe + np.log(s))[:, 0]
    lse = np.where(empty[:, 0], -np.inf, lse)
    return o, lse


def block_counts(mask: np.ndarray, bq: int, bk: int):
    """Allowed-pair count and clipped size of every (query block, key block) cell."""
    n_q, n_kv = mask.shape
    nqb, nkb = -(-n_q // bq), -(-n_kv // bk)
    padded = np.zeros((nqb * bq, nkb * bk), bool)
    padded[:n_q, :n_kv] = mask
    counts = padded.reshape(nqb, bq, nkb, bk).sum(axis=(1, 3)).astype(np.int64)
    valid = np.zeros_like(padded)
    valid[:n_q, :n_kv] = True
    sizes = valid.reshape(nqb, bq, nkb, bk).sum(axis=(1, 3)).astype(np.int64)
    return counts, sizes


def block_lists(mask: np.ndarray, bq: int, bk: int):
    """kv_count, kv_index (ascending, -1 pad), kv_partial, live_pairs from a dense mask."""
    counts, sizes = block_counts(mask, bq, bk)
    nqb, nkb = counts.shape
    kv_count = np.zeros(nqb, np.int32)
    kv_index = np.full((nqb, nkb), -1, np.int32)
    kv_partial = np.zeros((nqb, nkb), np.uint8)
    for i in range(nqb):
        live = np.nonzero(counts[i] > 0)[0]
        kv_count[i] = live.size
        kv_index[i, : live.size] = live
        kv_partial[i, : live.size] = (counts[i, live] != sizes[i, live]).astype(np.uint8)
    return dict(kv_count=kv_count, kv_index=kv_index, kv_partial=kv_partial,
                live_pairs=int(counts.sum()))
