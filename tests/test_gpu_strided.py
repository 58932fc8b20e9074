"""The strided template computed as local band + residue views, merged by LSE in
the kernels' epilogues (sa_attn_fwd, SA_MODE_STRIDED), vs the fp64 oracle of the
whole pattern (O <= 1e-2, LSE <= 1e-3)."""

import numpy as np
import pytest
import torch

import oracle
import block_sparse_attention_sa_amd as sa
from block_sparse_attention_sa_amd import workloads as W
from tests.parity_util import check_o_lse, full_config_reference, to_dev_bf16

pytestmark = pytest.mark.gpu


def _rand(rng, B, H, n, d):
    f = lambda: W.f32_to_bf16_bits(rng.standard_normal((B, H, n, d), dtype=np.float32))
    return f(), f(), f()


def _pattern(S):
    return dict(causal=1, window_left=S - 1, window_right=0, stride=S, stride_phase=S - 1)


@pytest.mark.parametrize("B,H,S,G,d", [(1, 2, 128, 8, 64), (2, 2, 64, 10, 128), (1, 3, 32, 20, 64),
                                       (1, 1, 128, 3, 128)])
def test_strided_small_vs_oracle(B, H, S, G, d):
    rng = np.random.default_rng(7 * S + G + d + B)
    n = S * G
    q, k, v = _rand(rng, B, H, n, d)
    pat = _pattern(S)
    assert sa.attn_workspace_bytes_strided(pat, B, H, n, d) > 0
    print(f"strided small B={B} H={H} S={S} n={n} d={d}", flush=True)
    o, lse = sa.attn_fwd_strided(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), pat)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_rows(pat, q, k, v)
    check_o_lse(o.cpu().numpy().reshape(-1, d), lse.cpu().numpy().reshape(-1), o_ref, lse_ref,
                ctx=f"S={S} n={n} d={d}")


def test_strided_noncontiguous_layout():
    """[B, n, H, d] storage seen as [B, H, n, d]: the residue views follow the strides."""
    rng = np.random.default_rng(31)
    B, H, S, G, d = 1, 2, 64, 6, 64
    n = S * G
    q, k, v = _rand(rng, B, H, n, d)
    dev = [to_dev_bf16(np.ascontiguousarray(t.transpose(0, 2, 1, 3))).transpose(1, 2) for t in (q, k, v)]
    assert not dev[0].is_contiguous()
    print("strided non-contiguous layout", flush=True)
    o, lse = sa.attn_fwd_strided(*dev, _pattern(S))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_rows(_pattern(S), q, k, v)
    check_o_lse(o.cpu().numpy().reshape(-1, d), lse.cpu().numpy().reshape(-1), o_ref, lse_ref, ctx="bnhd")


def test_strided_full_size_all_rows():
    """The 16,384-token strided workload (stride 128, H = 16, d = 64): every row."""
    cfg, inp, o_ref, lse_ref = full_config_reference(3)
    pat = cfg.pattern.as_dict()
    q, k, v = (to_dev_bf16(inp[t]) for t in ("q", "k", "v"))
    print("strided full size", flush=True)
    o, lse = sa.attn_fwd_strided(q, k, v, pat)
    torch.cuda.synchronize()
    check_o_lse(o.cpu().numpy().reshape(-1, cfg.d), lse.cpu().numpy().reshape(-1), o_ref, lse_ref,
                ctx="config 3 strided form")


def test_strided_rejects_other_patterns_and_reuses_workspace():
    """Patterns that are not the template are rejected before any work; a workspace
    is reused by a second call on other inputs with the same shape."""
    rng = np.random.default_rng(9)
    B, H, S, G, d = 1, 2, 64, 5, 128
    n = S * G
    q, k, v = _rand(rng, B, H, n, d)
    with pytest.raises(ValueError):
        sa.attn_fwd_strided(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), dict(_pattern(S), sinks=2))
    ws = sa.strided_plan(_pattern(S), B, H, n, d)
    for seed in (1, 2):
        q, k, v = _rand(np.random.default_rng(seed), B, H, n, d)
        print(f"strided workspace reuse {seed}", flush=True)
        o, lse = sa.attn_fwd_strided(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), _pattern(S), workspace=ws)
        o_ref, lse_ref = oracle.attn_rows(_pattern(S), q, k, v)
        check_o_lse(o.cpu().numpy().reshape(-1, d), lse.cpu().numpy().reshape(-1), o_ref, lse_ref, ctx=f"reuse {seed}")


def test_merge_partial_closed_form():
    """sa_merge_partial against the log-sum-exp formula, with -inf on either side and a
    residue-ordered second LSE (rows q = q_first + i*S + r, i < n2)."""
    rng = np.random.default_rng(5)
    B, H, S, G, d = 2, 3, 16, 5, 128
    n, q_first, n2 = S * G, 2 * S - 1, G - 2
    o1 = rng.standard_normal((B, H, n, d)).astype(np.float32)
    o2 = rng.standard_normal((B, H, n, d)).astype(np.float32)
    l1 = (rng.standard_normal((B, H, n)) * 4).astype(np.float32)
    l2r = (rng.standard_normal((B, H, S, n2)) * 4).astype(np.float32)
    l1[0, 0, 40:44] = -np.inf
    l2r[0, 0, 3, :] = -np.inf
    l1[1, 2, 50] = -np.inf
    l2r[1, 2, (50 - q_first) % S, (50 - q_first) // S] = -np.inf   # both sides empty
    l2 = np.full((B, H, n), -np.inf, np.float64)
    has = np.zeros(n, bool)
    for q in range(q_first, n):
        r, i = (q - q_first) % S, (q - q_first) // S
        if i < n2:
            l2[:, :, q] = l2r[:, :, r, i]
            has[q] = True
    m = np.maximum(l1, l2)
    safe = np.where(np.isneginf(m), 0.0, m)
    w1 = np.where(np.isneginf(l1), 0.0, np.exp(l1 - safe))
    w2 = np.where(np.isneginf(l2), 0.0, np.exp(l2 - safe))
    tot = w1 + w2
    mix = (o1 * w1[..., None] + o2 * w2[..., None]) / np.where(tot > 0, tot, 1)[..., None]
    exp_o = np.where((tot > 0)[..., None] & has[None, None, :, None], mix, o1)
    exp_l = np.where((tot > 0) & has[None, None, :], safe + np.log(np.where(tot > 0, tot, 1)), l1)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    o, l = dev(o1), dev(l1)
    print("merge partial closed form", flush=True)
    sa.merge_partial(o, l, dev(o2), dev(l2r), group=S, q_first=q_first, n2=n2)
    torch.cuda.synchronize()
    np.testing.assert_allclose(o.cpu().numpy(), exp_o, rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(l.cpu().numpy(), exp_l, rtol=1e-5, atol=1e-5)
    assert np.array_equal(o.cpu().numpy()[:, :, ~has], o1[:, :, ~has])   # rows without a second part
