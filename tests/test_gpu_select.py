"""Content-selected key blocks (sa_select_blocks) bit for bit against the oracle,
and attention over the per-(b, h) lists (sa_attn_fwd, per_head_lists) against the
oracle's attention over the same selection (O <= 1e-2, LSE <= 1e-3)."""

import numpy as np
import pytest
import torch

import oracle
import block_sparse_attention_sa_amd as sa
from block_sparse_attention_sa_amd import workloads as W
from tests.parity_util import check_o_lse, to_dev_bf16

pytestmark = pytest.mark.gpu


def _rand(rng, B, H, n_q, n_kv, d):
    f = lambda *s: W.f32_to_bf16_bits(rng.standard_normal(s, dtype=np.float32))
    return f(B, H, n_q, d), f(B, H, n_kv, d), f(B, H, n_kv, d)


def _compare_lists(got, want, ctx):
    np.testing.assert_array_equal(got.kv_count.cpu().numpy(), want["kv_count"], err_msg=ctx)
    np.testing.assert_array_equal(got.kv_index.cpu().numpy(), want["kv_index"], err_msg=ctx)
    np.testing.assert_array_equal(got.kv_partial.cpu().numpy(), want["kv_partial"], err_msg=ctx)
    assert int(got.live_pairs.cpu()[0]) == want["live_pairs"], ctx


CASES = [(2, 3, 300, 300, 0, 64, 64, 64, 2), (1, 2, 256, 1000, 744, 128, 128, 128, 3),
         (1, 2, 333, 777, 444, 64, 128, 128, 4), (2, 1, 130, 130, 0, 128, 64, 64, 50),
         (1, 4, 520, 520, 0, 64, 64, 128, 0)]


@pytest.mark.parametrize("B,H,n_q,n_kv,off,d,bq,bk,n_sel", CASES)
def test_select_and_attend_small(B, H, n_q, n_kv, off, d, bq, bk, n_sel):
    rng = np.random.default_rng(n_q + n_kv + d + bq + n_sel)
    q, k, v = _rand(rng, B, H, n_q, n_kv, d)
    print(f"select B={B} H={H} n_q={n_q} n_kv={n_kv} off={off} d={d} bq={bq} bk={bk} n_sel={n_sel}", flush=True)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    sel = sa.select_blocks(qd, kd, bq, bk, n_sel, q_offset=off)
    want = oracle.select_blocks(q, k, off, bq, bk, n_sel)
    _compare_lists(sel, want, "lists")
    for od in (torch.float32, torch.bfloat16):
        o, lse = sa.attn_fwd(qd, kd, vd, sel, o_dtype=od)
        o_ref, lse_ref = oracle.attn_sel_rows(q, k, v, off, bq, bk, want["kv_count"], want["kv_index"])
        check_o_lse(o.float().cpu().numpy().reshape(-1, d), lse.cpu().numpy().reshape(-1), o_ref, lse_ref,
                    bf16_out=od == torch.bfloat16, ctx=f"attention {od}")


def test_select_zero_queries_takes_lowest_blocks():
    rng = np.random.default_rng(31)
    n, bq, n_sel = 640, 64, 3
    _, k, _ = _rand(rng, 1, 2, n, n, 64)
    qd = torch.zeros((1, 2, n, 64), dtype=torch.bfloat16, device="cuda")
    sel = sa.select_blocks(qd, to_dev_bf16(k), bq, bq, n_sel)
    cnt, idx = sel.kv_count.cpu().numpy(), sel.kv_index.cpu().numpy()
    for bh in range(2):
        for i in range(n // bq):
            assert idx[bh, i, : cnt[bh, i]].tolist() == sorted(set(range(min(i, n_sel))) | {i})


def test_select_workload_all_rows():
    """Workload 6 at full size (B=1, H=32, N=8192, d=128, 128-token blocks, the own
    block plus 8 selected): lists bit for bit, every row's attention within tolerance,
    and the heads select different blocks."""
    cfg = W.select_config()
    inp = W.select_inputs(cfg)
    qd, kd, vd = (to_dev_bf16(inp[t]) for t in ("q", "k", "v"))
    print("select workload 6 full size", flush=True)
    sel = sa.select_blocks(qd, kd, cfg.block, cfg.block, cfg.n_select)
    o, lse = sa.attn_fwd(qd, kd, vd, sel)
    torch.cuda.synchronize()
    want = oracle.select_blocks(inp["q"], inp["k"], 0, cfg.block, cfg.block, cfg.n_select)
    _compare_lists(sel, want, "workload 6 lists")
    o_ref, lse_ref = oracle.attn_sel_rows(inp["q"], inp["k"], inp["v"], 0, cfg.block, cfg.block,
                                          want["kv_count"], want["kv_index"])
    check_o_lse(o.cpu().numpy().reshape(-1, cfg.d), lse.cpu().numpy().reshape(-1), o_ref, lse_ref, ctx="workload 6")
    idx = want["kv_index"]
    assert any(not np.array_equal(idx[0], idx[h]) for h in range(1, cfg.H))
