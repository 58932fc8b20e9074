"""The C ABI on a side stream and under HIP graph capture: same bits as eager
calls on the default stream."""

import numpy as np
import pytest
import torch

import block_sparse_attention_sa_amd as sa
from block_sparse_attention_sa_amd import workloads as W
from tests.parity_util import to_dev_bf16

pytestmark = pytest.mark.gpu


def _inputs(seed):
    rng = np.random.default_rng(seed)
    f = lambda *s: W.f32_to_bf16_bits(rng.standard_normal(s, dtype=np.float32))
    B, H, n, d = 1, 4, 1000, 128
    q, k, v = (to_dev_bf16(f(B, H, n, d)) for _ in range(3))
    qi, ki = to_dev_bf16(f(n, 64)), to_dev_bf16(f(n, 64))
    pat = dict(causal=1, window_left=300, window_right=0, sinks=4)
    return pat, n, q, k, v, qi, ki


def _path(pat, n, q, k, v, qi, ki):
    """One pass: block lists, block-sparse attention, indexer + top-k, gather attention."""
    bl = sa.build_block_mask(pat, n, n, 128, 128)
    o, lse = sa.attn_fwd(q, k, v, bl)
    idx, _ = sa.indexer_topk(qi, ki, 0, 64)
    og, lg = sa.attn_fwd(q, k, v, gather_idx=idx)
    return [bl.kv_count, bl.kv_index, bl.kv_partial, bl.live_pairs, o, lse, idx, og, lg]


def test_side_stream_bit_identical():
    args = _inputs(1)
    ref = [t.clone() for t in _path(*args)]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()  # default priority
    with torch.cuda.stream(side):
        got = _path(*args)
    side.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)


def test_graph_capture_replays_bit_identical():
    args = _inputs(2)
    ref = [t.clone() for t in _path(*args)]
    torch.cuda.synchronize()
    # warm-up on a side stream, then capture one pass
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _path(*args)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = _path(*args)
    for rep in range(3):
        # eager work between replays: clear the outputs, so each replay must
        # write them again
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"graph replay {rep}", flush=True)
        for a, b in zip(ref, outs):
            assert torch.equal(a, b), f"replay {rep}"
