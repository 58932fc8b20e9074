"""GPU block-list builder vs the oracle: bit-exact on every output."""

import numpy as np
import pytest

import oracle
import block_sparse_attention_sa_amd as sa
from block_sparse_attention_sa_amd import workloads as W
from tests.parity_util import random_pattern

pytestmark = pytest.mark.gpu


def _compare(got, want, ctx):
    cnt = got.kv_count.cpu().numpy()
    np.testing.assert_array_equal(cnt, want["kv_count"], err_msg=f"{ctx} kv_count")
    np.testing.assert_array_equal(got.kv_index.cpu().numpy(), want["kv_index"], err_msg=f"{ctx} kv_index")
    np.testing.assert_array_equal(got.kv_partial.cpu().numpy(), want["kv_partial"], err_msg=f"{ctx} kv_partial")
    assert int(got.live_pairs.cpu()[0]) == want["live_pairs"], ctx


@pytest.mark.parametrize("cid", [1, 2, 3, 4])
def test_configs_bit_exact(cid):
    cfg = W.attn_config(cid)
    print(f"builder config {cid} N={cfg.N} block={cfg.block}", flush=True)
    got = sa.build_block_mask(cfg.pattern, cfg.N, cfg.N, cfg.block, cfg.block)
    want = oracle.block_lists(cfg.pattern, cfg.N, cfg.N, cfg.block, cfg.block)
    _compare(got, want, f"config {cid}")
    expect_live = {1: 26, 2: 595, 3: 8256, 4: 2542}[cid]
    assert int(got.kv_count.sum()) == expect_live


@pytest.mark.parametrize("seed", range(24))
def test_random_patterns_ragged(seed):
    rng = np.random.default_rng(500 + seed)
    n_q, n_kv = int(rng.integers(1, 700)), int(rng.integers(1, 700))
    bq, bk = int(rng.choice([32, 64, 128, 96])), int(rng.choice([32, 64, 128, 160]))
    pat = random_pattern(rng, n_q, n_kv)
    print(f"builder seed {seed} n_q={n_q} n_kv={n_kv} bq={bq} bk={bk} {sorted(pat)}", flush=True)
    got = sa.build_block_mask(pat, n_q, n_kv, bq, bk)
    want = oracle.block_lists(pat, n_q, n_kv, bq, bk)
    _compare(got, want, f"seed {seed}")


def test_degenerate_sizes():
    pat = dict(causal=1, window_left=16, window_right=0)
    got = sa.build_block_mask(pat, 0, 100, 64, 64)
    assert int(got.live_pairs.cpu()[0]) == 0
    got = sa.build_block_mask(pat, 100, 0, 64, 64)
    assert int(got.live_pairs.cpu()[0]) == 0
    assert np.all(got.kv_count.cpu().numpy() == 0)
    # nothing allowed at all
    none = dict(causal=1, window_left=-1)
    got = sa.build_block_mask(none, 300, 300, 64, 64)
    assert int(got.kv_count.sum()) == 0 and int(got.live_pairs.cpu()[0]) == 0
    # everything allowed
    full = dict(global_tokens=1 << 30)
    got = sa.build_block_mask(full, 257, 129, 64, 64)
    want = oracle.block_lists(full, 257, 129, 64, 64)
    _compare(got, want, "dense")
    assert want["live_pairs"] == 257 * 129


def test_repeat_is_identical():
    cfg = W.attn_config(2)
    a = sa.build_block_mask(cfg.pattern, cfg.N, cfg.N, cfg.block, cfg.block)
    b = sa.build_block_mask(cfg.pattern, cfg.N, cfg.N, cfg.block, cfg.block)
    for f in ("kv_count", "kv_index", "kv_partial", "live_pairs"):
        assert bool((getattr(a, f) == getattr(b, f)).all())


@pytest.mark.parametrize("seed", range(4))
def test_long_rows(seed):
    """Rows of more than 512 key blocks: many count workgroups per query block, and
    a compaction in which each of the 256 threads owns several cells."""
    rng = np.random.default_rng(900 + seed)
    n_q, n_kv, bq, bk = int(rng.integers(40, 130)), int(rng.integers(16500, 21000)), 64, 32
    assert (n_kv + bk - 1) // bk > 512
    pat = random_pattern(rng, n_q, n_kv)
    print(f"builder long rows seed {seed} n_q={n_q} n_kv={n_kv} {sorted(pat)}", flush=True)
    got = sa.build_block_mask(pat, n_q, n_kv, bq, bk)
    want = oracle.block_lists(pat, n_q, n_kv, bq, bk)
    _compare(got, want, f"long rows seed {seed}")
