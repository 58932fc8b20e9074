"""sa_indexer_topk_noalloc (the streaming indexer + top-k on the library's fixed
per-device scratch) against sa_indexer_topk with a caller workspace: the same
indices, on two calls in a row, the second with a smaller input."""

import numpy as np
import pytest
import torch

import block_sparse_attention_sa_amd as sa
from block_sparse_attention_sa_amd import _lib
from block_sparse_attention_sa_amd import workloads as W
from tests.parity_util import to_dev_bf16

pytestmark = pytest.mark.gpu


def _rbf(rng, *shape):
    return W.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def test_noalloc_matches_workspace_form_twice_then_rejects_oversize():
    rng = np.random.default_rng(2024)
    cases = [(1024, 65536, 2048, 65536 - 1024), (37, 5000, 333, 4963)]   # largest fitting size, then smaller
    for n_q, n_kv, k, off in cases:
        qi, ki = to_dev_bf16(_rbf(rng, n_q, 64)), to_dev_bf16(_rbf(rng, n_kv, 64))
        print(f"noalloc n_q={n_q} n_kv={n_kv} k={k}", flush=True)
        assert sa.indexer_topk_workspace_bytes(n_q, n_kv, k) <= 64 << 20
        got = sa.indexer_topk_noalloc(qi, ki, off, k)
        want, _ = sa.indexer_topk(qi, ki, off, k)
        torch.cuda.synchronize()
        assert torch.equal(got, want)
    # above the fixed scratch: a clear error before any launch
    qi = torch.zeros((4096, 64), dtype=torch.bfloat16, device="cuda")
    ki = torch.zeros((65536, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(_lib.SaError) as e:
        assert sa.indexer_topk_workspace_bytes(4096, 65536, 2048) > 64 << 20
        sa.indexer_topk_noalloc(qi, ki, 0, 2048)
    assert e.value.status == _lib.SA_ERR_UNSUPPORTED and "scratch" in str(e.value)
