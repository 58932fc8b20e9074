"""GPU block-sparse attention vs the fp64 oracle (O <= 1e-2, LSE <= 1e-3)."""

import numpy as np
import pytest
import torch

import oracle
import block_sparse_attention_sa_amd as sa
from block_sparse_attention_sa_amd import workloads as W
from tests.parity_util import check_o_lse, full_config_reference, random_pattern, to_dev_bf16

pytestmark = pytest.mark.gpu


def _run(pat, q, k, v, bq, bk, o_dtype=torch.float32):
    n_q, n_kv = q.shape[2], k.shape[2]
    bl = sa.build_block_mask(pat, n_q, n_kv, bq, bk)
    return sa.attn_fwd(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), bl, o_dtype=o_dtype)


def _rand(rng, B, H, nq, nkv, d):
    f = lambda *s: W.f32_to_bf16_bits(rng.standard_normal(s, dtype=np.float32))
    return f(B, H, nq, d), f(B, H, nkv, d), f(B, H, nkv, d)


CASES = [(d, bq, bk, of) for d in (64, 128) for bq in (64, 128) for bk in (64, 128)
         for of in ("f32", "bf16")]


@pytest.mark.parametrize("d,bq,bk,of", CASES)
def test_small_ragged_window_sinks(d, bq, bk, of):
    rng = np.random.default_rng(d * 7 + bq + bk * 3 + (of == "bf16"))
    n_q, n_kv = 333, 301
    q, k, v = _rand(rng, 2, 2, n_q, n_kv, d)
    pat = dict(causal=1, window_left=90, window_right=0, sinks=3, q_offset=10)
    print(f"attn small d={d} bq={bq} bk={bk} o={of}", flush=True)
    od = torch.float32 if of == "f32" else torch.bfloat16
    o, lse = _run(pat, q, k, v, bq, bk, od)
    o_ref, lse_ref = oracle.attn_rows(pat, q, k, v)
    check_o_lse(o.float().cpu().numpy().reshape(-1, d), lse.cpu().numpy().reshape(-1), o_ref, lse_ref,
                bf16_out=(of == "bf16"), ctx=f"d={d} bq={bq} bk={bk} {of}")



@pytest.mark.parametrize("profile", ["rising", "falling", "spikes", "large_q"])
@pytest.mark.parametrize("d,bq,bk", [(128, 128, 128), (128, 64, 64), (64, 128, 64)])
def test_score_ranges_across_tiles(profile, d, bq, bk):
    """Score scales that change from key tile to key tile: the row's softmax
    reference (set on the first sub-tile it sees) must be raised and the
    accumulator rescaled whenever later keys dominate ("rising", "spikes",
    "large_q"), and keys far below it must still be summed correctly ("falling")."""
    rng = np.random.default_rng(1000 * ["rising", "falling", "spikes", "large_q"].index(profile) + d + bq + 3 * bk)
    n_q, n_kv = 333, 301
    f = lambda *s: rng.standard_normal(s, dtype=np.float32)
    q, k, v = f(1, 2, n_q, d), f(1, 2, n_kv, d), f(1, 2, n_kv, d)
    j = np.arange(n_kv, dtype=np.float32)
    if profile == "rising":
        k *= (0.2 + j / 12.0)[None, None, :, None]
    elif profile == "falling":
        k *= (0.2 + (n_kv - j) / 12.0)[None, None, :, None]
    elif profile == "spikes":
        k[:, :, ::37] *= 25.0
    else:
        q *= 30.0
    q, k, v = (W.f32_to_bf16_bits(x) for x in (q, k, v))
    pat = dict(causal=1, window_left=200, window_right=0, sinks=2, q_offset=20)
    print(f"attn score ranges {profile} d={d} bq={bq} bk={bk}", flush=True)
    o, lse = _run(pat, q, k, v, bq, bk)
    o_ref, lse_ref = oracle.attn_rows(pat, q, k, v)
    check_o_lse(o.cpu().numpy().reshape(-1, d), lse.cpu().numpy().reshape(-1), o_ref, lse_ref,
                ctx=f"{profile} d={d} bq={bq} bk={bk}")


SPLIT_CASES = [(2048, 2048, 64, 64, 64, "f32", 0, 130), (1500, 1777, 128, 64, 128, "bf16", 0, 200),
               (1333, 2200, 64, 128, 64, "f32", 40, 100), (2100, 2100, 128, 128, 128, "f32", 0, 300),
               (600, 560, 64, 64, 128, "f32", 0, 70), (700, 1100, 128, 128, 64, "bf16", 5, 150)]


def test_long_row_split_threshold():
    """Nine key blocks split (chunks of 8 and 1 list entries), eight do not."""
    pat = dict(causal=0, global_tokens=70, unit=64, unit_window=1)
    assert sa.attn_workspace_bytes_blocks(sa.build_block_mask(pat, 600, 560, 64, 64), 2, 2, 128) > 0
    assert sa.attn_workspace_bytes_blocks(sa.build_block_mask(pat, 600, 512, 64, 64), 2, 2, 128) == 0


@pytest.mark.parametrize("n_q,n_kv,bq,bk,d,of,q_off,g", SPLIT_CASES)
def test_long_row_split_global_tokens(n_q, n_kv, bq, bk, d, of, q_off, g):
    """Without causality the query blocks of global tokens list every key block; past 8
    key blocks they run as chunks of 8 list entries whose partial (O, LSE) are merged by
    log-sum-exp.  Every row against the oracle, with the split and without it."""
    rng = np.random.default_rng(n_q + n_kv + bq + bk + d + q_off + g)
    q, k, v = _rand(rng, 2, 2, n_q, n_kv, d)
    u = 64
    table = rng.integers(-1, -(-n_kv // u), size=(-(-(n_q + q_off) // u), 3)).astype(np.int32)
    pat = dict(causal=0, global_tokens=g, unit=u, unit_window=1, rand_table=table, q_offset=q_off)
    bl = sa.build_block_mask(pat, n_q, n_kv, bq, bk)
    assert sa.attn_workspace_bytes_blocks(bl, 2, 2, d) > 0
    qd, kd, vd = (to_dev_bf16(x) for x in (q, k, v))
    od = torch.float32 if of == "f32" else torch.bfloat16
    print(f"attn long-row split n_q={n_q} n_kv={n_kv} bq={bq} bk={bk} d={d} {of} q_off={q_off} g={g}", flush=True)
    o_ref, lse_ref = oracle.attn_rows(pat, q, k, v)
    for split in (True, False):
        o, lse = sa.attn_fwd(qd, kd, vd, bl, o_dtype=od, split=split)
        torch.cuda.synchronize()
        check_o_lse(o.float().cpu().numpy().reshape(-1, d), lse.cpu().numpy().reshape(-1), o_ref, lse_ref,
                    bf16_out=(of == "bf16"), ctx=f"split={split} n_q={n_q} bq={bq} bk={bk} {of}")


@pytest.mark.parametrize("seed", range(16))
def test_random_patterns(seed):
    rng = np.random.default_rng(900 + seed)
    d = int(rng.choice([64, 128]))
    bq, bk = int(rng.choice([64, 128])), int(rng.choice([64, 128]))
    n_q, n_kv = int(rng.integers(1, 400)), int(rng.integers(1, 400))
    pat = random_pattern(rng, n_q, n_kv)
    q, k, v = _rand(rng, 1, 2, n_q, n_kv, d)
    print(f"attn random seed={seed} d={d} bq={bq} bk={bk} n_q={n_q} n_kv={n_kv} {sorted(pat)}", flush=True)
    o, lse = _run(pat, q, k, v, bq, bk)
    o_ref, lse_ref = oracle.attn_rows(pat, q, k, v)
    check_o_lse(o.cpu().numpy().reshape(-1, d), lse.cpu().numpy().reshape(-1), o_ref, lse_ref,
                ctx=f"seed {seed}")


def test_config1_full():
    cfg = W.attn_config(1)
    inp = W.attn_inputs(cfg)
    o, lse = _run(cfg.pattern, inp["q"], inp["k"], inp["v"], cfg.block, cfg.block)
    o_ref, lse_ref = oracle.attn_rows(cfg.pattern, inp["q"], inp["k"], inp["v"])
    check_o_lse(o.cpu().numpy().reshape(-1, cfg.d), lse.cpu().numpy().reshape(-1), o_ref, lse_ref,
                ctx="config 1")


@pytest.mark.parametrize("cid", [2, 3, 4])
@pytest.mark.parametrize("of", ["f32", "bf16"])
def test_full_configs_all_rows(cid, of):
    """Full-size launch (the benchmark's configuration); every row of every
    (batch, head) against the oracle."""
    cfg, inp, o_ref, lse_ref = full_config_reference(cid)
    print(f"attn config {cid} o={of} B={cfg.B} H={cfg.H} N={cfg.N} d={cfg.d}", flush=True)
    od = torch.float32 if of == "f32" else torch.bfloat16
    o, lse = _run(cfg.pattern, inp["q"], inp["k"], inp["v"], cfg.block, cfg.block, od)
    torch.cuda.synchronize()
    check_o_lse(o.float().cpu().numpy().reshape(-1, cfg.d), lse.cpu().numpy().reshape(-1), o_ref, lse_ref,
                bf16_out=(of == "bf16"), ctx=f"config {cid} {of}")
    # no empty rows in these configurations
    assert np.isfinite(lse_ref).all()


def test_value_ones_give_ones_and_weights_sum():
    cfg = W.attn_config(2)
    inp = W.attn_inputs(cfg, heads=4)
    ones = np.full_like(inp["v"], W.f32_to_bf16_bits(np.ones(1, np.float32))[0])
    o, lse = _run(cfg.pattern, inp["q"], inp["k"], ones, cfg.block, cfg.block)
    assert float((o - 1.0).abs().max()) <= 1e-2


def test_zero_queries_closed_form():
    """Q = 0: LSE = ln(number of allowed keys), O = mean of the allowed V rows."""
    cfg = W.attn_config(1)
    inp = W.attn_inputs(cfg)
    q0 = np.zeros_like(inp["q"])
    o, lse = _run(cfg.pattern, q0, inp["k"], inp["v"], cfg.block, cfg.block)
    o_ref, lse_ref, cnt = oracle.attn_rows(cfg.pattern, q0, inp["k"], inp["v"], return_counts=True)
    np.testing.assert_allclose(lse.cpu().numpy().reshape(-1), np.log(cnt), atol=1e-3, rtol=0)
    check_o_lse(o.cpu().numpy().reshape(-1, cfg.d), lse.cpu().numpy().reshape(-1), o_ref, lse_ref)


def test_rows_without_allowed_keys():
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 1, 1, 200, 150, 64)
    pat = dict(causal=1, window_left=5, window_right=0, q_offset=0)
    # keys end at 150: rows q >= 156 see nothing
    o, lse = _run(pat, q, k, v, 64, 64)
    o_ref, lse_ref = oracle.attn_rows(pat, q, k, v)
    assert np.isneginf(lse_ref).sum() > 0
    check_o_lse(o.cpu().numpy().reshape(-1, 64), lse.cpu().numpy().reshape(-1), o_ref, lse_ref)


def test_n_kv_zero():
    rng = np.random.default_rng(4)
    q, k, v = _rand(rng, 1, 1, 70, 0, 64)
    o, lse = _run(dict(causal=1, window_left=5), q, k, v, 64, 64)
    assert torch.isneginf(lse).all() and (o == 0).all()


def test_run_to_run_bit_identical():
    cfg = W.attn_config(2)
    inp = W.attn_inputs(cfg, heads=4)
    q, k, v = (to_dev_bf16(inp[t]) for t in ("q", "k", "v"))
    bl = sa.build_block_mask(cfg.pattern, cfg.N, cfg.N, cfg.block, cfg.block)
    o1, l1 = sa.attn_fwd(q, k, v, bl)
    o2, l2 = sa.attn_fwd(q, k, v, bl)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_strided_layout_matches_contiguous():
    """[B, N, H, d] storage passed through strides gives the same result."""
    rng = np.random.default_rng(6)
    B, H, N, d = 1, 3, 256, 128
    q, k, v = _rand(rng, B, H, N, N, d)
    pat = dict(causal=1, window_left=60, window_right=0, sinks=2)
    o_ref, l_ref = _run(pat, q, k, v, 128, 64)
    qt, kt, vt = (to_dev_bf16(np.ascontiguousarray(x.transpose(0, 2, 1, 3))).permute(0, 2, 1, 3)
                  for x in (q, k, v))
    bl = sa.build_block_mask(pat, N, N, 128, 64)
    out = torch.empty((B, N, H, d), dtype=torch.float32, device="cuda").permute(0, 2, 1, 3)
    o, l = sa.attn_fwd(qt, kt, vt, bl, out=out)
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)


def test_dense_pattern_matches_causal_sdpa_fp32():
    """A window covering everything is plain causal attention (fp32 CPU reference)."""
    rng = np.random.default_rng(8)
    B, H, N, d = 1, 2, 384, 128
    q, k, v = _rand(rng, B, H, N, N, d)
    o, _ = _run(dict(causal=1, window_left=N), q, k, v, 128, 128)
    tq, tk, tv = (torch.from_numpy(W.bf16_bits_to_f32(x)) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    assert float((o.cpu() - ref).abs().max()) <= 1e-2


@pytest.mark.parametrize("d,bq,bk,n_kv", [(128, 128, 128, 301), (128, 64, 64, 301), (64, 128, 64, 301),
                                          (64, 64, 128, 320), (128, 128, 64, 384)])
def test_nan_rows_past_n_kv_and_invalid_list_entries(d, bq, bk, n_kv):
    """K and V are views into larger allocations whose rows past n_kv hold NaN
    (a preallocated cache with an unwritten tail), and query blocks list key
    blocks that do not exist (past the end and negative): nothing past n_kv may
    reach O or LSE.  Ragged n_kv takes the bounds-checked copy path, a multiple
    of 64 the fast one."""
    rng = np.random.default_rng(d + bq + bk + n_kv)
    B, H, n_q, pad = 1, 2, 333, 200
    q, k, v = _rand(rng, B, H, n_q, n_kv, d)
    nan = np.uint16(0x7FC0)
    kf = np.full((B, H, n_kv + pad, d), nan, np.uint16)
    vf = np.full((B, H, n_kv + pad, d), nan, np.uint16)
    kf[:, :, :n_kv], vf[:, :, :n_kv] = k, v
    kd, vd = to_dev_bf16(kf)[:, :, :n_kv], to_dev_bf16(vf)[:, :, :n_kv]
    pat = dict(causal=1, window_left=90, window_right=0, sinks=3, q_offset=10)
    bl = sa.build_block_mask(pat, n_q, n_kv, bq, bk)
    cnt, idx = bl.kv_count.cpu().numpy(), bl.kv_index.cpu().numpy()
    nkb = idx.shape[1]
    for i in range(cnt.size):  # append entries that are not key blocks where a row has room
        extra = [nkb + 3, -5, nkb][: nkb - cnt[i]]
        idx[i, cnt[i]: cnt[i] + len(extra)] = extra
        cnt[i] += len(extra)
    bl.kv_count.copy_(torch.from_numpy(cnt))
    bl.kv_index.copy_(torch.from_numpy(idx))
    print(f"attn NaN tail d={d} bq={bq} bk={bk} n_kv={n_kv}", flush=True)
    o, lse = sa.attn_fwd(to_dev_bf16(q), kd, vd, bl)
    o_ref, lse_ref = oracle.attn_rows(pat, q, k, v)
    check_o_lse(o.cpu().numpy().reshape(-1, d), lse.cpu().numpy().reshape(-1), o_ref, lse_ref,
                ctx=f"NaN tail d={d} bq={bq} bk={bk} n_kv={n_kv}")
