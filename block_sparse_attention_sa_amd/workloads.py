"""Seeded synthetic workloads: the five attention configurations and their inputs.

This module holds data only: shapes, pattern parameters and seeded random
tensors.  It contains none of the attention arithmetic, so both the HIP path
and the CPU oracle can take their inputs from it without sharing any of the
method's code.

Inputs follow the recipe used throughout the tests and the benchmark:

* every tensor is drawn from ``numpy.random.Generator(PCG64(seed))`` with
  ``seed = 20261203 + 100 * config_id + tensor_id`` (tensor ids: q=0, k=1,
  v=2, indexer queries=3, indexer keys=4, random-block table=5);
* floating tensors are standard normal float32 rounded to bfloat16 with
  round-to-nearest-even, returned as the raw ``uint16`` bit patterns so that
  every consumer sees identical bits;
* the BigBird-style random table draws, for every query block outside the
  global rows, ``n_rand`` distinct key blocks uniformly without replacement
  from the blocks that are neither in the query's sliding window nor global.

Pattern vocabulary (the fields of the pattern descriptor, in the pages'
terms: "Sparse Attention" glossary, section on common sparsity patterns, and
the sparse-transformer blog, section on the main sparsity templates):

``causal``        key position must not exceed query position
``window_left``   local band: ``q - kv <= window_left`` (negative: term off)
``window_right``  and ``kv - q <= window_right``
``sinks``         the first ``sinks`` keys are visible to every query
``stride``/``stride_phase``  strided keys: ``q >= kv`` and
                  ``(q - kv) % stride == stride_phase``
``global_tokens`` positions below it attend to and are attended by all
``unit``/``unit_window``  block-level band ``|q//unit - kv//unit| <= unit_window``
``n_rand``        random key units per query unit (table drawn here)
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

SEED_BASE = 20261203
TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "q_idx": 3, "k_idx": 4, "rand": 5}


def seed_for(config_id: int, tensor: str) -> int:
    return SEED_BASE + 100 * int(config_id) + TENSOR_IDS[tensor]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    out = (r & np.uint64(0xFFFF)).astype(np.uint16)
    # NaN stays NaN (never produced by the generators, kept for completeness)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def randn_bf16(shape, seed: int) -> np.ndarray:
    """Standard-normal bfloat16 bits of the given shape from one PCG64 stream."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return f32_to_bf16_bits(rng.standard_normal(size=shape, dtype=np.float32))


@dataclasses.dataclass
class Pattern:
    causal: int = 0
    q_offset: int = 0
    window_left: int = -1
    window_right: int = 0
    sinks: int = 0
    stride: int = 0
    stride_phase: int = 0
    global_tokens: int = 0
    unit: int = 0
    unit_window: int = -1
    n_rand: int = 0
    rand_table: Optional[np.ndarray] = None  # int32 [rows, n_rand], -1 = empty

    def as_dict(self) -> dict:
        d = dataclasses.asdict(self)
        d.pop("rand_table")
        return d


@dataclasses.dataclass
class AttnConfig:
    cid: int
    name: str
    B: int
    H: int
    N: int
    d: int
    block: int
    pattern: Pattern


def bigbird_random_table(n_units: int, n_rand: int, unit_window: int,
                         global_units: int, seed: int) -> np.ndarray:
    """Random key units per query unit, distinct, outside window and global units.

    Rows that belong to global query units get -1 (they already see every key).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    table = np.full((n_units, n_rand), -1, dtype=np.int32)
    allu = np.arange(n_units)
    for qu in range(global_units, n_units):
        excluded = (np.abs(allu - qu) <= unit_window) | (allu < global_units)
        cand = allu[~excluded]
        pick = rng.choice(cand, size=min(n_rand, cand.size), replace=False)
        table[qu, : pick.size] = pick
    return table


def attn_config(cid: int) -> AttnConfig:
    """Configurations 1-4 (block-list attention)."""
    if cid == 1:
        return AttnConfig(1, "tiny_window128_sinks4_n512", 1, 2, 512, 64, 64,
                          Pattern(causal=1, window_left=128, window_right=0, sinks=4))
    if cid == 2:
        return AttnConfig(2, "window1024_sinks4_n8192_h32_d128", 1, 32, 8192, 128, 128,
                          Pattern(causal=1, window_left=1024, window_right=0, sinks=4))
    if cid == 3:
        return AttnConfig(3, "strided128_n16384_h16_d64", 1, 16, 16384, 64, 128,
                          Pattern(causal=1, window_left=127, window_right=0,
                                  stride=128, stride_phase=127))
    if cid == 4:
        n_units = 16384 // 64
        table = bigbird_random_table(n_units, 3, 1, 2, seed_for(4, "rand"))
        return AttnConfig(4, "bigbird_n16384_b2_h12_d64", 2, 12, 16384, 64, 64,
                          Pattern(causal=0, global_tokens=128, unit=64, unit_window=1,
                                  n_rand=3, rand_table=table))
    raise ValueError(f"no block-list attention config {cid}")


def attn_inputs(cfg: AttnConfig, n: Optional[int] = None, heads: Optional[int] = None,
                batch: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Q, K, V bf16 bits, layout [B, H, N, d] contiguous.

    ``n``/``heads``/``batch`` shrink the shape for small test cases; the seeds
    stay those of the configuration.
    """
    B = cfg.B if batch is None else batch
    H = cfg.H if heads is None else heads
    N = cfg.N if n is None else n
    shape = (B, H, N, cfg.d)
    return {t: randn_bf16(shape, seed_for(cfg.cid, t)) for t in ("q", "k", "v")}


@dataclasses.dataclass
class TopkConfig:
    cid: int
    name: str
    H: int
    n_q: int
    n_kv: int
    d: int
    d_idx: int
    topk: int

    @property
    def q_offset(self) -> int:
        return self.n_kv - self.n_q


def topk_config(cid: int = 5) -> TopkConfig:
    if cid != 5:
        raise ValueError("only configuration 5 is a top-k gather workload")
    return TopkConfig(5, "dsa_topk2048_q1024_ctx65536_h16_d128", 16, 1024, 65536, 128, 64, 2048)


def topk_inputs(cfg: TopkConfig, n_q: Optional[int] = None, n_kv: Optional[int] = None,
                heads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Indexer queries/keys [n_q, d_idx] / [n_kv, d_idx] and Q [1,H,n_q,d], K/V [1,H,n_kv,d]."""
    nq = cfg.n_q if n_q is None else n_q
    nkv = cfg.n_kv if n_kv is None else n_kv
    H = cfg.H if heads is None else heads
    out = {
        "q_idx": randn_bf16((nq, cfg.d_idx), seed_for(cfg.cid, "q_idx")),
        "k_idx": randn_bf16((nkv, cfg.d_idx), seed_for(cfg.cid, "k_idx")),
        "q": randn_bf16((1, H, nq, cfg.d), seed_for(cfg.cid, "q")),
        "k": randn_bf16((1, H, nkv, cfg.d), seed_for(cfg.cid, "k")),
        "v": randn_bf16((1, H, nkv, cfg.d), seed_for(cfg.cid, "v")),
    }
    return out


@dataclasses.dataclass
class SelectConfig:
    """Content-selected key blocks (the glossary's Native Sparse Attention block
    selection): each (b, h, query block) keeps its own key block plus the
    ``n_select`` causally reachable key blocks of highest mean-query . mean-key."""
    cid: int
    name: str
    B: int
    H: int
    N: int
    d: int
    block: int
    n_select: int


def select_config(cid: int = 6) -> SelectConfig:
    if cid != 6:
        raise ValueError("only workload 6 is a content-selected block workload")
    return SelectConfig(6, "nsa_select8_n8192_h32_d128", 1, 32, 8192, 128, 128, 8)


def select_inputs(cfg: SelectConfig, n: Optional[int] = None, heads: Optional[int] = None,
                  batch: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Q, K, V bf16 bits [B, H, N, d] for the content-selected workload (seeds of
    workload ``cfg.cid``)."""
    B = cfg.B if batch is None else batch
    H = cfg.H if heads is None else heads
    N = cfg.N if n is None else n
    shape = (B, H, N, cfg.d)
    return {t: randn_bf16(shape, seed_for(cfg.cid, t)) for t in ("q", "k", "v")}
