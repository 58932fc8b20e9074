"""Pins for the CPU oracle: facts fixed by the pages and by mathematics.

None of these compares the oracle with itself.  Each check uses something
independent: a number the pages print (fixtures under tests/golden/), a
closed form, a textbook/library routine (torch's fp64 scaled-dot-product
attention), exact rational arithmetic, or dense brute force written
separately (oracle/brute.py, numpy expressions of the pages' mask functions).
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from block_sparse_attention_sa_amd import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _bf16_f64(b):
    return brute.bf16_bits_to_f64(b)


# ----------------------------------------------------------------------------
# predicate and block lists
# ----------------------------------------------------------------------------

def _mask_local_plus_sinks(n, window, sinks):
    """The glossary's mask function, as a dense numpy expression."""
    q = np.arange(n)[:, None]
    kv = np.arange(n)[None, :]
    return (q >= kv) & (((q - kv) <= window) | (kv < sinks))


def test_glossary_sparsity_8192_window1024_sinks4():
    g = _gold("glossary_local_plus_sinks.json")
    pat = dict(causal=1, window_left=g["window"], window_right=0, sinks=g["sinks"])
    bl = oracle.block_lists(pat, g["seq_len"], g["seq_len"], g["block"], g["block"])
    nb = (g["seq_len"] // g["block"]) ** 2
    live = int(bl["kv_count"].sum())
    sparsity = 100.0 * (nb - live) / nb
    assert round(sparsity, 2) == g["printed_sparsity_percent"]
    # only one live count rounds to the printed figure
    ok = [n for n in range(nb + 1) if round(100.0 * (nb - n) / nb, 2) == g["printed_sparsity_percent"]]
    assert ok == [live] == [595]
    # printed shape: a diagonal band plus the left column
    nqb = g["seq_len"] // g["block"]
    for i in range(nqb):
        row = set(bl["kv_index"][i, : bl["kv_count"][i]].tolist())
        assert 0 in row
        assert i in row
        band = {j for j in row if j != 0}
        assert band == set(range(max(1, i - 8), i + 1))


def _window_sink_block_closed_form(N, Bb, W_, S):
    """Live / full blocks of causal window (inclusive) + S <= Bb sinks, N % Bb == 0."""
    nb = N // Bb
    mstar = (W_ + Bb - 1) // Bb
    live = sum(min(i, mstar) + 1 for i in range(nb)) + max(0, nb - 1 - mstar)
    mfull = (W_ - Bb + 1) // Bb
    full = sum(min(i, mfull) for i in range(nb))
    return live, full


def _window_sink_pairs_closed_form(N, W_, S):
    return W_ * (W_ + 1) // 2 + (N - W_) * (W_ + 1) + S * (S - 1) // 2 + S * (N - W_ - S)


@pytest.mark.parametrize("cid", [1, 2])
def test_window_sink_closed_forms(cid):
    cfg = W.attn_config(cid)
    p = cfg.pattern
    bl = oracle.block_lists(p, cfg.N, cfg.N, cfg.block, cfg.block)
    live, full = _window_sink_block_closed_form(cfg.N, cfg.block, p.window_left, p.sinks)
    assert int(bl["kv_count"].sum()) == live
    n_partial = int(sum(bl["kv_partial"][i, : bl["kv_count"][i]].sum() for i in range(len(bl["kv_count"]))))
    assert live - n_partial == full
    assert bl["live_pairs"] == _window_sink_pairs_closed_form(cfg.N, p.window_left, p.sinks)
    expect = {1: (26, 7, 59318), 2: (595, 420, 7900662)}[cid]
    assert (live, full, bl["live_pairs"]) == expect


def test_strided_config_closed_form():
    cfg = W.attn_config(3)
    bl = oracle.block_lists(cfg.pattern, cfg.N, cfg.N, cfg.block, cfg.block)
    nb = cfg.N // cfg.block
    assert int(bl["kv_count"].sum()) == nb * (nb + 1) // 2 == 8256
    assert int(bl["kv_partial"].sum()) == 8256  # every live block partial
    qs = np.arange(cfg.N)
    pairs = int(np.sum(np.minimum(qs, 127) + 1) + np.sum(np.maximum(0, (qs + 1) // 128 - 1)))
    assert bl["live_pairs"] == pairs == 3113279


def test_bigbird_config_seed_independent_counts():
    cfg = W.attn_config(4)
    for seed in (cfg_seed for cfg_seed in (W.seed_for(4, "rand"), 7, 123)):
        table = W.bigbird_random_table(256, 3, 1, 2, seed)
        pat = dict(cfg.pattern.as_dict(), rand_table=table)
        bl = oracle.block_lists(pat, cfg.N, cfg.N, cfg.block, cfg.block)
        assert int(bl["kv_count"].sum()) == 2542
        assert int(bl["kv_partial"].sum()) == 0
        assert bl["live_pairs"] == 2542 * 64 * 64
        # rows 0-1 global, the rest 7 (edges) or 8 blocks
        assert bl["kv_count"][0] == bl["kv_count"][1] == 256
        assert bl["kv_count"][2] == bl["kv_count"][255] == 7
        assert set(bl["kv_count"][3:255].tolist()) == {8}


def test_area_attention_pairs():
    g = _gold("pair_counts.json")["area_attention"]
    pat = dict(causal=0, unit=g["stripe_tokens"], unit_window=0)
    n = g["tokens"]
    bl = oracle.block_lists(pat, n, n, 64, 64)
    assert bl["live_pairs"] == int(round(g["fraction_scored"] * g["full_pairs_millions"] * 1e6))
    assert bl["live_pairs"] == g["stripes"] * g["stripe_tokens"] ** 2


def test_dense_pair_counts_from_blog():
    g = _gold("pair_counts.json")["dense_scores_per_head"]
    allpat = dict(causal=0, global_tokens=1 << 40)
    bl = oracle.block_lists(allpat, 1024, 1024, 128, 128)
    assert abs(bl["live_pairs"] - g["n_1024_approx"]) / g["n_1024_approx"] < 0.05
    bl = oracle.block_lists(allpat, 16384, 16384, 128, 128)
    assert bl["live_pairs"] // 1_000_000 == g["n_16384_millions"]


def _dense_mask(pat, n_q, n_kv):
    """Vectorised numpy restatement of every pattern term (independent of oracle.c)."""
    q = np.arange(n_q)[:, None] + pat.get("q_offset", 0)
    kv = np.arange(n_kv)[None, :]
    terms = np.zeros((n_q, n_kv), bool)
    wl = pat.get("window_left", -1)
    if wl >= 0:
        terms |= ((q - kv) <= wl) & ((kv - q) <= pat.get("window_right", 0))
    terms |= kv < pat.get("sinks", 0)
    st = pat.get("stride", 0)
    if st > 0:
        diff = q - kv
        terms |= (diff >= 0) & (np.mod(np.maximum(diff, 0), st) == pat.get("stride_phase", 0))
    g = pat.get("global_tokens", 0)
    terms |= (q < g) | (kv < g)
    u = pat.get("unit", 0)
    if u > 0:
        qu, ku = q // u, kv // u
        if pat.get("unit_window", -1) >= 0:
            terms |= np.abs(qu - ku) <= pat["unit_window"]
        tab = pat.get("rand_table")
        if tab is not None:
            for r in range(tab.shape[1]):
                col = np.full(qu.shape, -2)
                inside = qu < tab.shape[0]
                col = np.where(inside, tab[np.minimum(qu, tab.shape[0] - 1), r], -2)
                terms |= (col == ku)
    if pat.get("causal", 0):
        terms &= kv <= q
    return terms


def _random_pattern(rng, n_q, n_kv):
    pat = dict(causal=int(rng.integers(0, 2)), q_offset=int(rng.integers(0, 3)) * int(rng.integers(0, 40)))
    if rng.random() < 0.7:
        pat["window_left"] = int(rng.integers(0, 60))
        pat["window_right"] = int(rng.integers(0, 20))
    if rng.random() < 0.5:
        pat["sinks"] = int(rng.integers(1, 9))
    if rng.random() < 0.4:
        pat["stride"] = int(rng.integers(1, 40))
        pat["stride_phase"] = int(rng.integers(0, pat["stride"]))
    if rng.random() < 0.3:
        pat["global_tokens"] = int(rng.integers(1, 20))
    if rng.random() < 0.4:
        u = int(rng.integers(4, 40))
        pat["unit"] = u
        pat["unit_window"] = int(rng.integers(-1, 2))
        rows = -(-(n_q + pat["q_offset"]) // u)
        units = -(-n_kv // u)
        pat["rand_table"] = rng.integers(-1, units, size=(rows, 2)).astype(np.int32)
    return pat


@pytest.mark.parametrize("seed", range(12))
def test_block_lists_vs_dense_brute_force(seed):
    rng = np.random.default_rng(1000 + seed)
    n_q, n_kv = int(rng.integers(1, 200)), int(rng.integers(1, 200))
    bq, bk = int(rng.choice([16, 32, 64])), int(rng.choice([16, 32, 64]))
    pat = _random_pattern(rng, n_q, n_kv)
    got = oracle.block_lists(pat, n_q, n_kv, bq, bk)
    want = brute.block_lists(_dense_mask(pat, n_q, n_kv), bq, bk)
    for key in ("kv_count", "kv_index", "kv_partial"):
        np.testing.assert_array_equal(got[key], want[key], err_msg=key)
    assert got["live_pairs"] == want["live_pairs"]


def test_page_mask_function_matches_predicate():
    """The glossary's mask function and the blog's sliding-window mask, per pair."""
    n = 300
    pat = dict(causal=1, window_left=100, window_right=0, sinks=4)
    want = _mask_local_plus_sinks(n, 100, 4)
    assert np.array_equal(_dense_mask(pat, n, n), want)
    got = np.array([[oracle.allowed(pat, q, kv) for kv in range(n)] for q in range(0, n, 7)])
    assert np.array_equal(got, want[::7])
    # blog: causal j <= i and strict (i - j) < window
    win = 5
    i = np.arange(40)[:, None]
    j = np.arange(40)[None, :]
    blog = (j <= i) & ((i - j) < win)
    bpat = dict(causal=1, window_left=win - 1, window_right=0)
    got = np.array([[oracle.allowed(bpat, a, b) for b in range(40)] for a in range(40)])
    assert np.array_equal(got, blog)


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------

def _rand_qkv(rng, B, H, nq, nkv, d):
    f = lambda *s: W.f32_to_bf16_bits(rng.standard_normal(s, dtype=np.float32))
    return f(B, H, nq, d), f(B, H, nkv, d), f(B, H, nkv, d)


@pytest.mark.parametrize("seed", range(8))
def test_attention_vs_dense_masked_brute_force(seed):
    rng = np.random.default_rng(2000 + seed)
    nq, nkv, d = int(rng.integers(1, 90)), int(rng.integers(1, 90)), int(rng.choice([4, 16, 64]))
    pat = _random_pattern(rng, nq, nkv)
    q, k, v = _rand_qkv(rng, 1, 2, nq, nkv, d)
    o, lse = oracle.attn_rows(pat, q, k, v)
    mask = _dense_mask(pat, nq, nkv)
    for h in range(2):
        bo, blse = brute.masked_attention(_bf16_f64(q[0, h]), _bf16_f64(k[0, h]), _bf16_f64(v[0, h]), mask)
        np.testing.assert_allclose(o[h * nq:(h + 1) * nq], bo, rtol=0, atol=1e-12)
        np.testing.assert_array_equal(np.isinf(lse[h * nq:(h + 1) * nq]), np.isinf(blse))
        fin = np.isfinite(blse)
        np.testing.assert_allclose(lse[h * nq:(h + 1) * nq][fin], blse[fin], rtol=0, atol=1e-12)


def test_attention_vs_torch_sdpa_boolean_mask():
    cfg = W.attn_config(1)
    inp = W.attn_inputs(cfg)
    o, lse = oracle.attn_rows(cfg.pattern, inp["q"], inp["k"], inp["v"])
    mask = torch.from_numpy(_dense_mask(cfg.pattern.as_dict(), cfg.N, cfg.N))
    tq, tk, tv = (torch.from_numpy(_bf16_f64(inp[t])) for t in ("q", "k", "v"))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
    np.testing.assert_allclose(o.reshape(ref.shape), ref.numpy(), rtol=0, atol=1e-12)
    # LSE through torch's own reduction: logsumexp of the scaled scores, the
    # disallowed ones at -inf (every row of this pattern has an allowed key)
    sc = torch.matmul(tq, tk.transpose(-1, -2)) / np.sqrt(tq.shape[-1])
    ref_lse = torch.logsumexp(sc.masked_fill(~mask, float("-inf")), dim=-1)
    np.testing.assert_allclose(lse.reshape(ref_lse.shape), ref_lse.numpy(), rtol=0, atol=1e-12)


def test_dense_window_reduces_to_causal_attention():
    rng = np.random.default_rng(3)
    n, d = 200, 64
    q, k, v = _rand_qkv(rng, 1, 3, n, n, d)
    o, lse = oracle.attn_rows(dict(causal=1, window_left=n - 1, window_right=0), q, k, v)
    tq, tk, tv = (torch.from_numpy(_bf16_f64(x)) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    np.testing.assert_allclose(o.reshape(ref.shape), ref.numpy(), rtol=0, atol=1e-12)


def test_zero_queries_closed_form():
    """Q = 0: every allowed score is 0, so LSE = ln|A| and O = mean of V over A."""
    cfg = W.attn_config(1)
    inp = W.attn_inputs(cfg)
    q0 = np.zeros_like(inp["q"])
    o, lse, cnt = oracle.attn_rows(cfg.pattern, q0, inp["k"], inp["v"], return_counts=True)
    mask = _dense_mask(cfg.pattern.as_dict(), cfg.N, cfg.N)
    np.testing.assert_array_equal(cnt[: cfg.N], mask.sum(1))
    np.testing.assert_allclose(lse, np.log(cnt), rtol=0, atol=1e-12)
    vf = _bf16_f64(inp["v"])
    for h in range(cfg.H):
        mean = (mask.astype(np.float64) @ vf[0, h]) / mask.sum(1, keepdims=True)
        np.testing.assert_allclose(o[h * cfg.N:(h + 1) * cfg.N], mean, rtol=0, atol=1e-12)


def test_single_key_closed_form():
    """A row with exactly one allowed key returns that key's value row."""
    rng = np.random.default_rng(5)
    n, d = 50, 64
    q, k, v = _rand_qkv(rng, 1, 1, n, n, d)
    o, lse = oracle.attn_rows(dict(causal=1, window_left=0, window_right=0), q, k, v)
    np.testing.assert_array_equal(o, _bf16_f64(v[0, 0]))
    s = np.einsum("nd,nd->n", _bf16_f64(q[0, 0]), _bf16_f64(k[0, 0])) / math.sqrt(d)
    np.testing.assert_allclose(lse, s, rtol=0, atol=1e-12)


def test_weights_sum_to_one_and_empty_rows():
    cfg = W.attn_config(1)
    inp = W.attn_inputs(cfg, heads=1)
    o, lse = oracle.attn_rows(cfg.pattern, inp["q"], inp["k"], inp["v"])
    qf, kf = _bf16_f64(inp["q"][0, 0]), _bf16_f64(inp["k"][0, 0])
    s = qf @ kf.T / math.sqrt(cfg.d)
    mask = _dense_mask(cfg.pattern.as_dict(), cfg.N, cfg.N)
    tot = np.where(mask, np.exp(s - lse[:, None]), 0.0).sum(1)
    np.testing.assert_allclose(tot, 1.0, rtol=0, atol=1e-12)
    # a pattern that allows nothing: O = 0, LSE = -inf
    o, lse = oracle.attn_rows(dict(causal=1, window_left=-1), inp["q"][:, :, :5], inp["k"], inp["v"])
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_blog_toy_shape():
    g = _gold("blog_toy_shape.json")
    rng = np.random.default_rng(0)
    q, k, v = _rand_qkv(rng, 1, 1, g["n"], g["n"], g["d"])
    pat = dict(causal=1, window_left=g["window"] - 1, window_right=0)
    o, lse = oracle.attn_rows(pat, q, k, v)
    assert list(o.shape) == g["printed_output_shape"]
    i = np.arange(g["n"])[:, None]
    j = np.arange(g["n"])[None, :]
    mask = (j <= i) & ((i - j) < g["window"])
    bo, _ = brute.masked_attention(_bf16_f64(q[0, 0]), _bf16_f64(k[0, 0]), _bf16_f64(v[0, 0]), mask)
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12)


def test_sampled_rows_match_full_rows():
    cfg = W.attn_config(1)
    inp = W.attn_inputs(cfg)
    o, lse = oracle.attn_rows(cfg.pattern, inp["q"], inp["k"], inp["v"])
    rows = np.array([0, 3, 77, 511, 512, 1023])
    o2, lse2 = oracle.attn_rows(cfg.pattern, inp["q"], inp["k"], inp["v"], rows=rows)
    np.testing.assert_array_equal(o2, o[rows])
    np.testing.assert_array_equal(lse2, lse[rows])


# ----------------------------------------------------------------------------
# gather attention
# ----------------------------------------------------------------------------

def test_gather_equals_masked_when_list_is_allowed_set():
    cfg = W.attn_config(1)
    inp = W.attn_inputs(cfg)
    mask = _dense_mask(cfg.pattern.as_dict(), cfg.N, cfg.N)
    kmax = int(mask.sum(1).max())
    idx = np.full((cfg.N, kmax), -1, np.int32)
    for r in range(cfg.N):
        sel = np.nonzero(mask[r])[0]
        idx[r, : sel.size] = sel
    o, lse = oracle.attn_rows(cfg.pattern, inp["q"], inp["k"], inp["v"])
    og, lseg = oracle.attn_gather_rows(inp["q"], inp["k"], inp["v"], idx)
    np.testing.assert_allclose(og, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lseg, lse, rtol=0, atol=1e-12)


def test_gather_vs_brute_force_per_head_lists():
    rng = np.random.default_rng(9)
    nq, nkv, d, k = 20, 70, 16, 11
    q, kk, v = _rand_qkv(rng, 1, 2, nq, nkv, d)
    idx = np.stack([np.stack([np.sort(rng.choice(nkv, k, replace=False)) for _ in range(nq)])
                    for _ in range(2)]).astype(np.int32)
    idx[0, 3, 7:] = -1  # padding
    o, lse = oracle.attn_gather_rows(q, kk, v, idx, idx_per_head=True)
    for h in range(2):
        mask = np.zeros((nq, nkv), bool)
        for r in range(nq):
            sel = idx[h, r][idx[h, r] >= 0]
            mask[r, sel] = True
        bo, blse = brute.masked_attention(_bf16_f64(q[0, h]), _bf16_f64(kk[0, h]), _bf16_f64(v[0, h]), mask)
        np.testing.assert_allclose(o[h * nq:(h + 1) * nq], bo, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[h * nq:(h + 1) * nq], blse, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# indexer and top-k
# ----------------------------------------------------------------------------

def _round_f32(x: Fraction) -> Fraction:
    """Exact round-to-nearest-even of a rational to binary32."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 23)
    m = a / ulp
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def test_indexer_fp32_chain_exact_rational():
    rng = np.random.default_rng(11)
    nq, nkv, d, off = 6, 40, 64, 30
    qi = W.f32_to_bf16_bits(rng.standard_normal((nq, d), dtype=np.float32))
    ki = W.f32_to_bf16_bits(rng.standard_normal((nkv, d), dtype=np.float32))
    sig, ex = oracle.indexer_scores(qi, ki, off, with_exact=True)
    qf, kf = W.bf16_bits_to_f32(qi), W.bf16_bits_to_f32(ki)
    nonfused_differs = 0
    for r in range(nq):
        t = off + r
        for s in range(nkv):
            if s > t:
                assert np.isneginf(sig[r, s])
                continue
            acc = Fraction(0)
            for c in range(d):
                acc = _round_f32(Fraction(float(qf[r, c])) * Fraction(float(kf[s, c])) + acc)
            assert Fraction(float(sig[r, s])) == acc
            # fp64 value of the same dot product, via numpy's own dot
            assert abs(ex[r, s] - float(np.dot(qf[r].astype(np.float64), kf[s].astype(np.float64)))) < 1e-12
            # a pairwise numpy float32 sum generally lands elsewhere: the order is pinned
            nonfused_differs += float(np.sum(qf[r] * kf[s], dtype=np.float32)) != float(sig[r, s])
    assert nonfused_differs > 0


def _brute_topk(sig_row, n_cand, k):
    order = sorted(range(n_cand), key=lambda s: (-float(sig_row[s]), s))
    sel = sorted(order[:k])
    return sel + [-1] * (k - len(sel))


def test_topk_vs_python_sort_with_ties():
    rng = np.random.default_rng(12)
    n_rows, n_kv, k = 30, 300, 17
    sig = rng.integers(-5, 6, size=(n_rows, n_kv)).astype(np.float32)  # many ties
    sig[0, :50] = -0.0
    sig[0, 50:100] = 0.0
    n_cand = rng.integers(1, n_kv + 1, size=n_rows)
    got = oracle.topk_rows(sig, n_cand, k)
    for r in range(n_rows):
        assert got[r].tolist() == _brute_topk(sig[r], int(n_cand[r]), k)


def test_topk_nan_and_infinite_scores_python_sort():
    """NaN scores (either sign bit) rank above +inf and tie with each other; -0.0
    ties with +0.0.  Pinned against Python's sort on an explicit key."""
    rng = np.random.default_rng(16)
    n_rows, n_kv, k = 24, 200, 23
    sig = rng.integers(-3, 4, size=(n_rows, n_kv)).astype(np.float32)
    u = sig.view(np.uint32)
    for r in range(n_rows):
        pos = rng.choice(n_kv, size=int(rng.integers(0, 40)), replace=False)
        kinds = rng.integers(0, 6, size=pos.size)
        for p_, kd in zip(pos, kinds):
            u[r, p_] = [0x7FC00000, 0xFFC00000, 0x7F800001, 0x7F800000, 0xFF800000, 0x80000000][kd]
    sig[3, :] = np.nan                      # every candidate NaN
    sig[4, :150] = np.inf                   # more +inf than k, NaN after them
    sig[4, 190] = np.nan
    n_cand = rng.integers(1, n_kv + 1, size=n_rows)
    n_cand[3:5] = n_kv

    def key(row, s):
        x = float(row[s])
        return (0 if math.isnan(x) else 1, 0.0 if math.isnan(x) else -x, s)

    got = oracle.topk_rows(sig, n_cand, k)
    for r in range(n_rows):
        nc = int(n_cand[r])
        sel = sorted(sorted(range(nc), key=lambda s: key(sig[r], s))[:k])
        assert got[r].tolist() == sel + [-1] * (k - len(sel)), f"row {r}"
    assert got[3].tolist() == list(range(k))
    assert got[4].tolist() == sorted([190] + list(range(k - 1)))


def test_topk_zero_queries_all_ties():
    rng = np.random.default_rng(13)
    ki = W.f32_to_bf16_bits(rng.standard_normal((3000, 64), dtype=np.float32))
    qi = np.zeros((4, 64), np.uint16)
    off = 2996
    sig = oracle.indexer_scores(qi, ki, off)
    idx = oracle.topk_rows(sig, np.arange(4) + off + 1, 2048)
    for r in range(4):
        assert idx[r].tolist() == list(range(2048))


def test_topk_k_at_least_candidates():
    rng = np.random.default_rng(14)
    sig = rng.standard_normal((5, 100)).astype(np.float32)
    n_cand = np.array([1, 10, 50, 99, 100])
    idx = oracle.topk_rows(sig, n_cand, 120)
    for r in range(5):
        assert idx[r, : n_cand[r]].tolist() == list(range(n_cand[r]))
        assert np.all(idx[r, n_cand[r]:] == -1)


def test_topk_against_full_sort_on_indexer_scores():
    rng = np.random.default_rng(15)
    n_q, n_kv, off, k = 8, 5000, 4992, 2048
    qi = W.f32_to_bf16_bits(rng.standard_normal((n_q, 64), dtype=np.float32))
    ki = W.f32_to_bf16_bits(rng.standard_normal((n_kv, 64), dtype=np.float32))
    sig = oracle.indexer_scores(qi, ki, off)
    n_cand = np.arange(n_q) + off + 1
    got = oracle.topk_rows(sig, n_cand, k)
    for r in range(n_q):
        nc = int(n_cand[r])
        order = np.lexsort((np.arange(nc), -sig[r, :nc].astype(np.float64)))
        assert got[r].tolist() == sorted(order[:k].tolist())


# ----------------------------------------------------------------------------
# content-selected blocks (the glossary's NSA block selection)
# ----------------------------------------------------------------------------

def _numpy_selection(q, k, q_offset, bq, bk, n_sel):
    """Block means (rows past the end as zero), scores and the selection with
    numpy's own reductions; returns per (bh, i) the selected block set and the
    gap between the last chosen and the first rejected score."""
    B, H, n_q, d = q.shape
    n_kv = k.shape[2]
    nqb, nkb = -(-n_q // bq), -(-n_kv // bk)
    qf = np.zeros((B * H, nqb * bq, d))
    kf = np.zeros((B * H, nkb * bk, d))
    qf[:, :n_q] = _bf16_f64(q).reshape(B * H, n_q, d)
    kf[:, :n_kv] = _bf16_f64(k).reshape(B * H, n_kv, d)
    qm = qf.reshape(B * H, nqb, bq, d).mean(axis=2)
    km = kf.reshape(B * H, nkb, bk, d).mean(axis=2)
    scores = np.einsum("bid,bjd->bij", qm, km)
    out = {}
    for bh in range(B * H):
        for i in range(nqb):
            p0, p1 = q_offset + i * bq, q_offset + min((i + 1) * bq, n_q) - 1
            own = {j for j in range(nkb) if j * bk <= p1 and min((j + 1) * bk, n_kv) - 1 >= p0}
            cand = sorted((j for j in range(nkb) if j * bk <= p1 and j not in own),
                          key=lambda j: (-scores[bh, i, j], j))
            chosen = cand[:n_sel]
            gap = np.inf
            if len(cand) > n_sel and n_sel > 0:
                gap = scores[bh, i, cand[n_sel - 1]] - scores[bh, i, cand[n_sel]]
            out[(bh, i)] = (sorted(own | set(chosen)), gap)
    return out


def _lists_as_sets(sel):
    res = {}
    BH, nqb, _ = sel["kv_index"].shape
    for bh in range(BH):
        for i in range(nqb):
            res[(bh, i)] = sel["kv_index"][bh, i, : sel["kv_count"][bh, i]].tolist()
    return res


@pytest.mark.parametrize("n_q,n_kv,q_offset,bq,bk,n_sel", [(300, 300, 0, 64, 64, 2), (256, 512, 256, 128, 64, 3),
                                                           (200, 333, 133, 64, 128, 1), (130, 130, 0, 64, 64, 5)])
def test_select_blocks_vs_numpy_brute_force(n_q, n_kv, q_offset, bq, bk, n_sel):
    """The selection against numpy's means and scores (a different summation
    order; rows whose kept/rejected gap is within rounding are not compared)."""
    rng = np.random.default_rng(n_q + n_kv + bq + n_sel)
    f = lambda *s: W.f32_to_bf16_bits(rng.standard_normal(s, dtype=np.float32))
    q, k = f(1, 3, n_q, 32), f(1, 3, n_kv, 32)
    got = oracle.select_blocks(q, k, q_offset, bq, bk, n_sel)
    want = _numpy_selection(q, k, q_offset, bq, bk, n_sel)
    sets = _lists_as_sets(got)
    compared = 0
    for key, (blocks, gap) in want.items():
        if gap > 1e-9:
            assert sets[key] == blocks, key
            compared += 1
    assert compared >= len(want) - 1
    # partial flags and pair counts from the causal rule inside the chosen tiles
    lists = {}
    total = 0
    for (bh, i), blocks in sets.items():
        p0, p1 = q_offset + i * bq, q_offset + min((i + 1) * bq, n_q) - 1
        for e, j in enumerate(blocks):
            s0, s1 = j * bk, min((j + 1) * bk, n_kv)
            cnt = sum(max(0, min(s1, qp + 1) - s0) for qp in range(p0, p1 + 1))
            total += cnt
            assert got["kv_partial"][bh, i, e] == int(cnt != (p1 - p0 + 1) * (s1 - s0))
        assert np.all(got["kv_index"][bh, i, len(blocks):] == -1)
    assert got["live_pairs"] == total


def test_select_blocks_zero_queries_take_the_lowest_blocks():
    """Q = 0: every score is 0, so the ties go to the lowest reachable blocks."""
    rng = np.random.default_rng(21)
    n, bq, n_sel = 640, 64, 3
    k = W.f32_to_bf16_bits(rng.standard_normal((1, 2, n, 16), dtype=np.float32))
    q = np.zeros((1, 2, n, 16), np.uint16)
    got = _lists_as_sets(oracle.select_blocks(q, k, 0, bq, bq, n_sel))
    for (bh, i), blocks in got.items():
        assert blocks == sorted(set(range(min(i, n_sel))) | {i}), (bh, i)


def test_select_blocks_planted_ranking():
    """Keys of block j all equal v_j * e_0 and queries e_0: block j scores v_j,
    so the chosen blocks are the n_sel reachable ones of largest v_j."""
    n, bq, n_sel, d = 1024, 64, 4, 16
    nkb = n // bq
    vals = np.random.default_rng(22).permutation(nkb).astype(np.float32) + 1.0  # distinct, exact in bf16
    k = np.zeros((1, 1, n, d), np.uint16)
    k[0, 0, :, 0] = W.f32_to_bf16_bits(np.repeat(vals, bq))
    q = np.zeros((1, 1, n, d), np.uint16)
    q[0, 0, :, 0] = W.f32_to_bf16_bits(np.ones(1, np.float32))[0]
    got = _lists_as_sets(oracle.select_blocks(q, k, 0, bq, bq, n_sel))
    for i in range(nkb):
        best = sorted(range(i), key=lambda j: -vals[j])[:n_sel]
        assert got[(0, i)] == sorted(set(best) | {i}), i


def test_select_every_block_is_causal_attention():
    """n_select above the reachable blocks keeps every causal block: attention
    over the selection is causal attention (torch fp64 SDPA)."""
    rng = np.random.default_rng(23)
    n, d = 320, 64
    q, k, v = _rand_qkv(rng, 1, 2, n, n, d)
    sel = oracle.select_blocks(q, k, 0, 64, 64, 99)
    o, lse = oracle.attn_sel_rows(q, k, v, 0, 64, 64, sel["kv_count"], sel["kv_index"])
    tq, tk, tv = (torch.from_numpy(_bf16_f64(x)) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    np.testing.assert_allclose(o.reshape(ref.shape), ref.numpy(), rtol=0, atol=1e-12)
    assert sel["live_pairs"] == 2 * n * (n + 1) // 2


def test_attn_sel_rows_vs_dense_brute_force():
    """Attention over the selected blocks against the dense masked brute force
    with the mask built from the lists (causal inside the chosen tiles)."""
    rng = np.random.default_rng(24)
    n_q, n_kv, q_offset, bq, bk, d = 150, 230, 80, 64, 32, 16
    q, k, v = _rand_qkv(rng, 1, 2, n_q, n_kv, d)
    sel = oracle.select_blocks(q, k, q_offset, bq, bk, 2)
    o, lse = oracle.attn_sel_rows(q, k, v, q_offset, bq, bk, sel["kv_count"], sel["kv_index"])
    for h in range(2):
        mask = np.zeros((n_q, n_kv), bool)
        for r in range(n_q):
            i = r // bq
            for j in sel["kv_index"][h, i, : sel["kv_count"][h, i]]:
                cols = np.arange(j * bk, min((j + 1) * bk, n_kv))
                mask[r, cols[cols <= q_offset + r]] = True
        bo, blse = brute.masked_attention(_bf16_f64(q[0, h]), _bf16_f64(k[0, h]), _bf16_f64(v[0, h]), mask)
        np.testing.assert_allclose(o[h * n_q:(h + 1) * n_q], bo, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[h * n_q:(h + 1) * n_q], blse, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# backward (gradients of the masked attention)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_backward_vs_torch_autograd(seed):
    """dQ, dK, dV against torch fp64 autograd of the dense masked attention
    (loss = sum(O * dO)); rows with no allowed key included."""
    rng = np.random.default_rng(3000 + seed)
    nq, nkv, d = int(rng.integers(1, 70)), int(rng.integers(1, 70)), int(rng.choice([4, 16, 64]))
    pat = _random_pattern(rng, nq, nkv)
    q, k, v = _rand_qkv(rng, 1, 2, nq, nkv, d)
    g = W.f32_to_bf16_bits(rng.standard_normal((1, 2, nq, d), dtype=np.float32))
    dq, dk, dv = oracle.attn_bwd(pat, q, k, v, g)
    mask = torch.from_numpy(_dense_mask(pat, nq, nkv))
    tq, tk, tv = (torch.from_numpy(_bf16_f64(x)).requires_grad_(True) for x in (q, k, v))
    sc = torch.matmul(tq, tk.transpose(-1, -2)) / math.sqrt(d)
    sc = sc.masked_fill(~mask, float("-inf"))
    w = torch.softmax(sc, dim=-1).nan_to_num(0.0)   # rows without keys: weights 0
    o = torch.matmul(w, tv)
    (o * torch.from_numpy(_bf16_f64(g))).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy()[0], rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy()[0], rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy()[0], rtol=0, atol=1e-11)


def test_backward_finite_differences():
    """Central differences of the oracle's own forward: d(sum(O * dO)) / dx."""
    rng = np.random.default_rng(31)
    n, d = 12, 4
    pat = dict(causal=1, window_left=4, window_right=0, sinks=1)
    q, k, v = _rand_qkv(rng, 1, 1, n, n, d)
    g = W.f32_to_bf16_bits(rng.standard_normal((1, 1, n, d), dtype=np.float32))
    dq, dk, dv = oracle.attn_bwd(pat, q, k, v, g)
    gf = _bf16_f64(g)[0, 0]
    allowed = _dense_mask(pat, n, n)
    base = {t: _bf16_f64(x)[0, 0] for t, x in (("q", q), ("k", k), ("v", v))}

    def loss(qq, kk, vv):
        o, _ = brute.masked_attention(qq, kk, vv, allowed)
        return float((o * gf).sum())

    eps = 1e-6
    for name, grad in (("q", dq[0]), ("k", dk[0]), ("v", dv[0])):
        for (r, c) in ((0, 0), (5, 2), (11, 3), (7, 1)):
            plus = {t: x.copy() for t, x in base.items()}
            minus = {t: x.copy() for t, x in base.items()}
            plus[name][r, c] += eps
            minus[name][r, c] -= eps
            fd = (loss(plus["q"], plus["k"], plus["v"]) - loss(minus["q"], minus["k"], minus["v"])) / (2 * eps)
            assert abs(fd - grad[r, c]) < 1e-7, (name, r, c, fd, grad[r, c])


def test_backward_closed_forms():
    """A row that sees one key: its P is 1, so dS = 0 there (no dQ from it) and
    dV of that key gets the row's dO; with the diagonal-only pattern dQ = dK = 0
    and dV = dO.  Every column of dV sums to the column sums of dO (the weights
    of each row sum to 1)."""
    rng = np.random.default_rng(32)
    n, d = 40, 16
    q, k, v = _rand_qkv(rng, 1, 1, n, n, d)
    g = W.f32_to_bf16_bits(rng.standard_normal((1, 1, n, d), dtype=np.float32))
    dq, dk, dv = oracle.attn_bwd(dict(causal=1, window_left=0, window_right=0), q, k, v, g)
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_array_equal(dv[0], _bf16_f64(g)[0, 0])
    pat = dict(causal=1, window_left=9, window_right=0, sinks=2)
    dq, dk, dv = oracle.attn_bwd(pat, q, k, v, g)
    np.testing.assert_allclose(dv[0].sum(0), _bf16_f64(g)[0, 0].sum(0), rtol=0, atol=1e-10)
