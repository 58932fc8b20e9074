"""GPU indexer, top-k and gather attention vs the oracle.

Indexer scores and top-k indices are compared bit for bit (the indexer's
float32 chain has one fixed order on both sides).  Gather attention is
compared with the oracle evaluated on the GPU's own index lists, which
isolates the attention error from the selection.
"""

import numpy as np
import pytest
import torch

import oracle
import block_sparse_attention_sa_amd as sa
from block_sparse_attention_sa_amd import workloads as W
from tests.parity_util import check_o_lse, to_dev_bf16

pytestmark = pytest.mark.gpu


def _rbf(rng, *shape):
    return W.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


@pytest.mark.parametrize("n_q,n_kv,d,off", [(1, 1, 64, 0), (70, 300, 64, 230), (64, 1000, 32, 900),
                                            (130, 4100, 128, 3970), (5, 257, 8, 0), (33, 777, 256, 700),
                                            (17, 1300, 200, 1290), (200, 2050, 64, 1900), (3, 70, 24, 5)])
def test_indexer_bit_exact(n_q, n_kv, d, off):
    rng = np.random.default_rng(n_q + n_kv)
    qi, ki = _rbf(rng, n_q, d), _rbf(rng, n_kv, d)
    print(f"indexer n_q={n_q} n_kv={n_kv} d={d} off={off}", flush=True)
    got = torch.full((n_q, n_kv), float("nan"), device="cuda")
    sa.indexer_scores(to_dev_bf16(qi), to_dev_bf16(ki), off, scores=got)
    want = oracle.indexer_scores(qi, ki, off)
    g = got.cpu().numpy()
    for r in range(n_q):
        nc = min(off + r + 1, n_kv)
        assert np.array_equal(g[r, :nc].view(np.uint32), want[r, :nc].view(np.uint32)), f"row {r}"
        assert np.all(np.isnan(g[r, nc:])), "entries beyond the candidates must be untouched"


@pytest.mark.parametrize("n_q,n_kv,k,off", [(40, 5000, 2048, 4960), (16, 65536, 2048, 65520),
                                            (8, 3000, 4096, 2992), (12, 777, 100, 700), (4, 9, 3, 0),
                                            (300, 65536, 2048, 65236), (70, 40000, 1000, 39000),
                                            (33, 2100, 2048, 2060), (5, 65536, 4096, 0)])
def test_topk_bit_exact(n_q, n_kv, k, off):
    """Both forms of sa_indexer_topk (through the score matrix, and streaming)
    against the oracle's selection from its own scores."""
    rng = np.random.default_rng(k + n_kv)
    qi, ki = _rbf(rng, n_q, 64), _rbf(rng, n_kv, 64)
    print(f"topk n_q={n_q} n_kv={n_kv} k={k} off={off}", flush=True)
    n_cand = np.minimum(np.arange(n_q) + off + 1, n_kv)
    want = oracle.topk_rows(oracle.indexer_scores(qi, ki, off), n_cand, k)
    idx2, scores = sa.indexer_topk(to_dev_bf16(qi), to_dev_bf16(ki), off, k, keep_scores=True)
    idx1, none = sa.indexer_topk(to_dev_bf16(qi), to_dev_bf16(ki), off, k)
    assert none is None and scores is not None
    np.testing.assert_array_equal(idx2.cpu().numpy(), want)
    np.testing.assert_array_equal(idx1.cpu().numpy(), want)


def _one_hot_queries(n_q, d=64):
    q = np.zeros((n_q, d), np.uint16)
    q[:, 0] = W.f32_to_bf16_bits(np.ones(1, np.float32))[0]
    return q


@pytest.mark.parametrize("kind", ["sample_high", "sample_low", "all_equal", "few_distinct", "ascending"])
@pytest.mark.parametrize("n_kv,k", [(65536, 2048), (32768, 2048), (20000, 333)])
def test_streaming_topk_adversarial_orders(kind, n_kv, k):
    """One-hot indexer queries make every score equal a chosen key value, laid
    out so that the 1/32 sample misleads the threshold: sampled keys above all
    others (too few kept), below all others (every region overflows), all
    equal, few distinct values, or rising with the index.  The streaming form
    must fall back to the exact selection and still match the oracle."""
    rng = np.random.default_rng(n_kv + k + len(kind))
    n_q = 6
    p = np.arange(n_kv)
    sampled = (p % 2048) < 64
    if kind == "sample_high":
        v = np.where(sampled, 4.0 + rng.random(n_kv), rng.random(n_kv))
    elif kind == "sample_low":
        v = np.where(sampled, -4.0 - rng.random(n_kv), rng.random(n_kv))
    elif kind == "all_equal":
        v = np.full(n_kv, 0.75)
    elif kind == "few_distinct":
        v = rng.integers(-2, 3, size=n_kv).astype(np.float64)
    else:
        v = p / n_kv * 8.0
    ki = np.zeros((n_kv, 64), np.uint16)
    ki[:, 0] = W.f32_to_bf16_bits(v.astype(np.float32))
    ki[:, 1:] = _rbf(rng, n_kv, 63)        # never reaches the score: the query is zero there
    qi = _one_hot_queries(n_q)
    off = n_kv - n_q
    print(f"streaming top-k {kind} n_kv={n_kv} k={k}", flush=True)
    idx, _ = sa.indexer_topk(to_dev_bf16(qi), to_dev_bf16(ki), off, k)
    want = oracle.topk_rows(oracle.indexer_scores(qi, ki, off), np.arange(n_q) + off + 1, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), want)


@pytest.mark.parametrize("kind", ["nan_keys", "inf_keys", "huge", "tiny", "mixed_scale"])
def test_streaming_topk_special_values(kind):
    """The streaming form on indexer inputs whose scores are NaN or infinite, whose
    norms overflow float32 (the filter's bound is infinite), whose scores lie in the
    denormal range, or whose key norms differ by many octaves within a tile (the bound
    taken from the tile's largest norm is loose for the others): every row equals the
    oracle's selection (NaN above every number, ties to the lower index)."""
    rng = np.random.default_rng(len(kind) * 7 + 5)
    n_q, n_kv, k = 5, 20000, 1000
    qf = rng.standard_normal((n_q, 64)).astype(np.float32)
    kf = rng.standard_normal((n_kv, 64)).astype(np.float32)
    if kind == "nan_keys":
        kf[rng.integers(0, n_kv, 300), rng.integers(0, 64, 300)] = np.nan
    elif kind == "inf_keys":
        kf[rng.integers(0, n_kv, 300), rng.integers(0, 64, 300)] = np.inf
        kf[rng.integers(0, n_kv, 300), rng.integers(0, 64, 300)] = -np.inf
    elif kind == "huge":
        kf *= np.float32(2.0 ** 100)
        qf *= np.float32(2.0 ** 20)
    elif kind == "tiny":
        kf *= np.float32(2.0 ** -70)
        qf *= np.float32(2.0 ** -60)
    else:
        kf *= (np.float32(2.0) ** rng.integers(-30, 30, (n_kv, 1))).astype(np.float32)
    qi, ki = W.f32_to_bf16_bits(qf), W.f32_to_bf16_bits(kf)
    off = n_kv - n_q
    print(f"streaming top-k special values {kind}", flush=True)
    idx, _ = sa.indexer_topk(to_dev_bf16(qi), to_dev_bf16(ki), off, k)
    want = oracle.topk_rows(oracle.indexer_scores(qi, ki, off), np.arange(n_q) + off + 1, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), want)


@pytest.mark.parametrize("n_kv,k", [(65536, 2048), (20000, 1000)])
def test_streaming_topk_ties_at_kth(n_kv, k):
    """Exact ties straddling the k-th score on the streaming path itself: the key
    at rank k of each query row is copied to a few positions before and after it,
    so several candidates share the k-th score and only the lowest positions among
    them may be taken. Random keys otherwise, so the row is settled by the bracket
    and the tie rule of the select decides (not the direct fallback)."""
    rng = np.random.default_rng(n_kv + 3 * k)
    n_q = 4
    qf = rng.standard_normal((n_q, 64)).astype(np.float32)
    kf = rng.standard_normal((n_kv, 64)).astype(np.float32)
    qi, ki = W.f32_to_bf16_bits(qf), W.f32_to_bf16_bits(kf)
    off = n_kv - n_q
    base = oracle.indexer_scores(qi, ki, off)
    used = np.zeros(n_kv, bool)  # k-th keys and their copies stay as placed
    for row in range(n_q):
        order = np.argsort(-base[row, : off + row + 1], kind="stable")
        kth = int(order[k - 1])
        used[kth] = True
        free = np.setdiff1d(np.nonzero(~used[: off + 1])[0], order[:k + 64])
        dst = rng.choice(free, 5, replace=False)
        ki[dst] = ki[kth]
        used[dst] = True
    print(f"streaming top-k ties at k n_kv={n_kv} k={k}", flush=True)
    idx, _ = sa.indexer_topk(to_dev_bf16(qi), to_dev_bf16(ki), off, k)
    scores = oracle.indexer_scores(qi, ki, off)
    want = oracle.topk_rows(scores, np.arange(n_q) + off + 1, k)
    # the copies tie with the k-th score of their row (a later row's copies can
    # shift an earlier row's rank, so not necessarily in every row)
    tied = 0
    for row in range(n_q):
        kth_score = np.sort(scores[row, : off + row + 1])[::-1][k - 1]
        tied += int((scores[row, : off + row + 1] == kth_score).sum() >= 2)
    assert tied >= n_q - 1
    np.testing.assert_array_equal(idx.cpu().numpy(), want)


@pytest.mark.parametrize("scale", [0.88, 0.9])
def test_streaming_topk_rows_past_the_kept_cap(scale):
    """Rows that keep more candidates than the select holds at once: the sampled
    key rows (the first 64 of every 2,048) are scaled down, so the sample's upper
    quantile, and with it the threshold, sits lower and about 4,900 to 5,600
    candidates pass the filter, past the 5,120 the select loads. Such a row is
    trimmed to its largest kept scores before the selection; the result must
    still equal the oracle's top-k."""
    n_kv, k, n_q = 65536, 2048, 4
    rng = np.random.default_rng(7)
    qf = rng.standard_normal((n_q, 64)).astype(np.float32)
    kf = rng.standard_normal((n_kv, 64)).astype(np.float32)
    sampled = (np.arange(n_kv) % 2048) < 64
    kf[sampled] *= np.float32(scale)
    qi, ki = W.f32_to_bf16_bits(qf), W.f32_to_bf16_bits(kf)
    off = n_kv - n_q
    scores = oracle.indexer_scores(qi, ki, off)
    # the setup does what it says: rows past 5,120 kept at the sample threshold
    over = 0
    for row in range(n_q):
        nc = off + row + 1
        srow = scores[row, :nc]
        samp = srow[sampled[:nc]]
        rho = k * samp.size / nc
        lo = np.sort(samp)[::-1][int(np.ceil(rho + 6 * np.sqrt(rho) + 8)) - 1]
        over += int((srow >= lo).sum() > 5120)
    assert over >= 2
    print(f"streaming top-k past the kept cap, scale {scale}", flush=True)
    idx, _ = sa.indexer_topk(to_dev_bf16(qi), to_dev_bf16(ki), off, k)
    want = oracle.topk_rows(scores, np.arange(n_q) + off + 1, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), want)


def test_streaming_topk_reused_workspace_and_short_rows():
    """Rows from fewer candidates than k (padding) up to the whole key range in
    one call, and a workspace reused by a second, smaller call."""
    rng = np.random.default_rng(99)
    n_kv, k = 12000, 1500
    qi, ki = _rbf(rng, 400, 64), _rbf(rng, n_kv, 64)
    ws = torch.empty(sa.indexer_topk_workspace_bytes(400, n_kv, k), dtype=torch.uint8, device="cuda")
    for n_q, off in ((400, 0), (300, 11700), (37, 1400)):
        print(f"streaming top-k reuse n_q={n_q} off={off}", flush=True)
        got, _ = sa.indexer_topk(to_dev_bf16(qi[:n_q]), to_dev_bf16(ki), off, k, workspace=ws)
        n_cand = np.minimum(np.arange(n_q) + off + 1, n_kv)
        want = oracle.topk_rows(oracle.indexer_scores(qi[:n_q], ki, off), n_cand, k)
        np.testing.assert_array_equal(got.cpu().numpy(), want)


def test_topk_ties_signed_zero_and_padding():
    rng = np.random.default_rng(77)
    n_q, n_kv, k = 6, 6000, 2048
    s = rng.integers(-3, 4, size=(n_q, n_kv)).astype(np.float32)  # heavy ties
    s[1] = 0.0
    s[1, ::2] = -0.0
    s[2, :] = -1.0
    scores = torch.from_numpy(s).cuda()
    for off in (0, 1500, 5999):
        got = sa.topk(scores, off, k).cpu().numpy()
        want = oracle.topk_rows(s, np.minimum(np.arange(n_q) + off + 1, n_kv), k)
        np.testing.assert_array_equal(got, want, err_msg=f"offset {off}")
    # all-zero indexer queries: every score ties, lowest indices win
    ki = _rbf(rng, 4000, 64)
    idx, _ = sa.indexer_topk(torch.zeros((3, 64), dtype=torch.bfloat16, device="cuda"), to_dev_bf16(ki), 3997, 2048)
    assert np.array_equal(idx.cpu().numpy(), np.tile(np.arange(2048, dtype=np.int32), (3, 1)))


def _nan_scores(rng, n_q, n_kv, n_special):
    """Normal scores with NaNs of both signs (quiet and signalling bit patterns),
    +inf, -inf and signed zeros planted at random positions."""
    s = rng.standard_normal((n_q, n_kv)).astype(np.float32)
    u = s.view(np.uint32)
    for r in range(n_q):
        pos = rng.choice(n_kv, size=n_special, replace=False)
        u[r, pos] = rng.choice(np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFFBFFFFF, 0x7F800000,
                                         0xFF800000, 0x80000000, 0x00000000], np.uint32), size=n_special)
    return s


@pytest.mark.parametrize("n_kv,k,n_special", [(65536, 2048, 100), (65536, 2048, 5000), (9001, 333, 600),
                                              (4000, 2048, 3999), (777, 100, 7)])
def test_topk_nan_and_infinite_scores(n_kv, k, n_special):
    """A NaN score ranks above every number and NaNs tie (lowest index first);
    -inf ranks last; the selection matches the oracle's total order."""
    rng = np.random.default_rng(n_kv + k + n_special)
    n_q = 4
    s = _nan_scores(rng, n_q, n_kv, n_special)
    off = n_kv - 3
    print(f"topk NaN/inf n_kv={n_kv} k={k} specials={n_special}", flush=True)
    got = sa.topk(torch.from_numpy(s).cuda(), off, k).cpu().numpy()
    want = oracle.topk_rows(s, np.minimum(np.arange(n_q) + off + 1, n_kv), k)
    np.testing.assert_array_equal(got, want)


def _scores_of(kind, rng, n_q, n_kv):
    if kind == "normal":
        return (rng.standard_normal((n_q, n_kv)) * 8).astype(np.float32)
    if kind == "ascending":  # order carries all the structure
        return np.tile(np.arange(n_kv, dtype=np.float32), (n_q, 1)) + rng.random((n_q, 1), dtype=np.float32)
    if kind == "descending":
        return np.tile(-np.arange(n_kv, dtype=np.float32), (n_q, 1))
    if kind == "narrow":  # every score within a few ulps of 1.0
        return (1.0 + rng.integers(0, 64, size=(n_q, n_kv)) * np.float32(2.0 ** -23)).astype(np.float32)
    if kind == "ties":
        return rng.integers(-2, 3, size=(n_q, n_kv)).astype(np.float32)
    if kind == "equal":
        return np.full((n_q, n_kv), 0.5, np.float32)
    if kind == "wide":  # magnitudes over many octaves, both signs, signed zeros
        s = rng.standard_normal((n_q, n_kv)).astype(np.float32) * np.float32(2.0) ** rng.integers(-60, 60, (n_q, n_kv))
        s[:, ::97] = -0.0
        s[:, 1::89] = 0.0
        return s.astype(np.float32)
    if kind == "periodic":  # the best keys sit at one offset of every 1024
        s = rng.standard_normal((n_q, n_kv)).astype(np.float32)
        s[:, 5::1024] += 100.0
        s[:, 700::1024] += 50.0
        return s
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["normal", "ascending", "descending", "narrow", "ties", "equal", "wide",
                                  "periodic"])
@pytest.mark.parametrize("n_kv,k", [(65536, 2048), (65535, 4096), (65536, 1), (9001, 333), (8192, 2048)])
def test_topk_score_distributions(kind, n_kv, k):
    """Rows whose scores defeat a sampled threshold (ties, order, narrow range)
    must still give the exact selection; odd n_kv takes the unaligned loads."""
    rng = np.random.default_rng(n_kv + k)
    n_q = 3
    s = _scores_of(kind, rng, n_q, n_kv)
    off = n_kv - 2  # last row sees every key, the others one or two fewer
    print(f"topk {kind} n_kv={n_kv} k={k}", flush=True)
    got = sa.topk(torch.from_numpy(s).cuda(), off, k).cpu().numpy()
    want = oracle.topk_rows(s, np.minimum(np.arange(n_q) + off + 1, n_kv), k)
    np.testing.assert_array_equal(got, want)


_CFG5 = {}


def _config5_reference():
    """Configuration 5's inputs, the oracle's scores for every query row and its
    top-k selection, computed once per test process."""
    if not _CFG5:
        cfg = W.topk_config(5)
        inp = W.topk_inputs(cfg)
        want_s = oracle.indexer_scores(inp["q_idx"], inp["k_idx"], cfg.q_offset)
        want_idx = oracle.topk_rows(want_s, cfg.q_offset + np.arange(cfg.n_q) + 1, cfg.topk)
        _CFG5.update(cfg=cfg, inp=inp, scores=want_s, idx=want_idx)
    return _CFG5


def test_config5_indexer_topk_all_rows():
    """Configuration 5 at full size: the streaming selection and the two-step one
    (scores bit for bit too) on every query row."""
    ref = _config5_reference()
    cfg, inp = ref["cfg"], ref["inp"]
    qi, ki = to_dev_bf16(inp["q_idx"]), to_dev_bf16(inp["k_idx"])
    print("config 5 indexer+topk full size", flush=True)
    idx1, _ = sa.indexer_topk(qi, ki, cfg.q_offset, cfg.topk)
    idx2, scores = sa.indexer_topk(qi, ki, cfg.q_offset, cfg.topk, keep_scores=True)
    torch.cuda.synchronize()
    got_s = scores.cpu().numpy()
    for r in range(cfg.n_q):
        nc = cfg.q_offset + r + 1
        assert np.array_equal(got_s[r, :nc].view(np.uint32), ref["scores"][r, :nc].view(np.uint32)), f"row {r}"
    np.testing.assert_array_equal(idx2.cpu().numpy(), ref["idx"])
    np.testing.assert_array_equal(idx1.cpu().numpy(), ref["idx"])


# ---------------------------------------------------------------------------
# gather attention

@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("of", ["f32", "bf16"])
def test_gather_small_per_head_and_shared(d, of):
    rng = np.random.default_rng(d)
    B, H, n_q, n_kv, k = 1, 3, 50, 700, 96
    q, kk, v = _rbf(rng, B, H, n_q, d), _rbf(rng, B, H, n_kv, d), _rbf(rng, B, H, n_kv, d)
    od = torch.float32 if of == "f32" else torch.bfloat16
    shared = np.stack([np.sort(rng.choice(n_kv, k, replace=False)) for _ in range(n_q)]).astype(np.int32)
    shared[3, 50:] = -1          # padding
    shared[4, :] = -1            # no keys at all
    o, lse = sa.attn_fwd(to_dev_bf16(q), to_dev_bf16(kk), to_dev_bf16(v), gather_idx=torch.from_numpy(shared).cuda(),
                         o_dtype=od)
    o_ref, lse_ref = oracle.attn_gather_rows(q, kk, v, shared)
    check_o_lse(o.float().cpu().numpy().reshape(-1, d), lse.cpu().numpy().reshape(-1), o_ref, lse_ref,
                bf16_out=(of == "bf16"), ctx="shared")
    per = np.stack([np.stack([np.sort(rng.choice(n_kv, k, replace=False)) for _ in range(n_q)])
                    for _ in range(B * H)]).astype(np.int32)
    o, lse = sa.attn_fwd(to_dev_bf16(q), to_dev_bf16(kk), to_dev_bf16(v),
                         gather_idx=torch.from_numpy(per.reshape(B, H, n_q, k)).cuda(), o_dtype=od)
    o_ref, lse_ref = oracle.attn_gather_rows(q, kk, v, per, idx_per_head=True)
    check_o_lse(o.float().cpu().numpy().reshape(-1, d), lse.cpu().numpy().reshape(-1), o_ref, lse_ref,
                bf16_out=(of == "bf16"), ctx="per head")


def test_gather_of_whole_blocks_equals_block_mode():
    """Index lists that are unions of whole key blocks reproduce the block kernel."""
    cfg = W.attn_config(1)
    inp = W.attn_inputs(cfg)
    pat = dict(causal=0, unit=64, unit_window=0, global_tokens=64)  # every live tile full
    bl = sa.build_block_mask(pat, cfg.N, cfg.N, 64, 64)
    assert int(bl.kv_partial.sum()) == 0
    q, k, v = (to_dev_bf16(inp[t]) for t in ("q", "k", "v"))
    o_b, l_b = sa.attn_fwd(q, k, v, bl)
    cnt, idx = bl.kv_count.cpu().numpy(), bl.kv_index.cpu().numpy()
    lists = []
    for r in range(cfg.N):
        blocks = idx[r // 64, : cnt[r // 64]]
        lists.append(np.concatenate([np.arange(b * 64, b * 64 + 64) for b in blocks]))
    kmax = max(len(x) for x in lists)
    g = np.full((cfg.N, kmax), -1, np.int32)
    for r, x in enumerate(lists):
        g[r, : len(x)] = x
    o_g, l_g = sa.attn_fwd(q, k, v, gather_idx=torch.from_numpy(g).cuda())
    assert float((o_g - o_b).abs().max()) <= 2e-3
    assert float((l_g - l_b).abs().max()) <= 1e-4


def test_config5_gather_all_rows():
    """Gather attention of configuration 5 over the oracle's own selection, every
    (head, query) row."""
    ref = _config5_reference()
    cfg, inp = ref["cfg"], ref["inp"]
    print("config 5 gather attention full size", flush=True)
    q, k, v = (to_dev_bf16(inp[t]) for t in ("q", "k", "v"))
    o, lse = sa.attn_fwd(q, k, v, gather_idx=torch.from_numpy(ref["idx"]).cuda())
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_gather_rows(inp["q"], inp["k"], inp["v"], ref["idx"])
    check_o_lse(o.cpu().numpy().reshape(-1, cfg.d), lse.cpu().numpy().reshape(-1), o_ref, lse_ref,
                ctx="config 5")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("per_head", [False, True])
def test_gather_split_form(d, per_head):
    """Key ranges of 4 MB of K+V per head: n_kv spans several ranges, so the
    split form (partition, partial softmax per range, merge) runs; unsorted
    lists, duplicates, out-of-range entries, a list inside one range and an
    empty list are covered."""
    rng = np.random.default_rng(100 + d + per_head)
    B, H, n_q, k = 2, 2, 37, 300
    n_kv = (3 << 22) // (4 * d) + 123           # three full ranges and a ragged tail
    q, kk, v = _rbf(rng, B, H, n_q, d), _rbf(rng, B, H, n_kv, d), _rbf(rng, B, H, n_kv, d)
    nl = B * H if per_head else 1
    lists = rng.integers(0, n_kv, size=(nl, n_q, k)).astype(np.int32)  # unsorted, duplicates
    lists[:, 1, ::7] = -5                        # skipped entries
    lists[:, 2, ::5] = n_kv + 3
    lists[:, 3, :] = rng.integers(100, 200, size=k)   # all in the first range
    lists[:, 4, :] = -1                           # no key at all
    assert sa.attn_workspace_bytes(B, H, n_q, n_kv, d, k, per_head_lists=per_head) > 0
    gi = torch.from_numpy(lists.reshape(B, H, n_q, k) if per_head else lists[0]).cuda()
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(kk), to_dev_bf16(v)
    print(f"split gather d={d} per_head={per_head} n_kv={n_kv}", flush=True)
    o_s, l_s = sa.attn_fwd(qd, kd, vd, gather_idx=gi)
    o_1, l_1 = sa.attn_fwd(qd, kd, vd, gather_idx=gi, split=False)
    if per_head:
        o_ref, lse_ref = oracle.attn_gather_rows(q, kk, v, lists, idx_per_head=True)
    else:
        o_ref, lse_ref = oracle.attn_gather_rows(q, kk, v, lists[0])
    check_o_lse(o_s.cpu().numpy().reshape(-1, d), l_s.cpu().numpy().reshape(-1), o_ref, lse_ref, ctx="split")
    check_o_lse(o_1.cpu().numpy().reshape(-1, d), l_1.cpu().numpy().reshape(-1), o_ref, lse_ref, ctx="single")
    # repeated call: same bits (the partition keeps list order)
    o_s2, l_s2 = sa.attn_fwd(qd, kd, vd, gather_idx=gi)
    assert torch.equal(o_s, o_s2) and torch.equal(l_s, l_s2)



def test_gather_split_many_ranges():
    """More key ranges than the merge takes in one batch (41 ranges of 8,192
    keys at d = 128): rows whose maxima rise from batch to batch, a row with
    no key in the first batch, a row whose keys all sit in the last range and
    an empty row."""
    rng = np.random.default_rng(4242)
    B, H, n_q, k, d = 1, 2, 24, 400, 128
    n_kv = 40 * 8192 + 77
    q, kk, v = _rbf(rng, B, H, n_q, d), _rbf(rng, B, H, n_kv, d), _rbf(rng, B, H, n_kv, d)
    lists = rng.integers(0, n_kv, size=(n_q, k)).astype(np.int32)
    lists[1] = rng.integers(20 * 8192, n_kv, size=k)        # nothing in the first sixteen ranges
    lists[2] = rng.integers(40 * 8192, n_kv, size=k)        # the ragged last range only
    lists[3] = -1                                            # no key
    lists[4, : k // 2] = -1                                  # half padding
    assert sa.attn_workspace_bytes(B, H, n_q, n_kv, d, k) > 0
    gi = torch.from_numpy(lists).cuda()
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(kk), to_dev_bf16(v)
    print(f"split gather many ranges n_kv={n_kv}", flush=True)
    o_s, l_s = sa.attn_fwd(qd, kd, vd, gather_idx=gi)
    o_ref, lse_ref = oracle.attn_gather_rows(q, kk, v, lists)
    check_o_lse(o_s.cpu().numpy().reshape(-1, d), l_s.cpu().numpy().reshape(-1), o_ref, lse_ref, ctx="many ranges")

@pytest.mark.parametrize("split", [False, True])
def test_gather_list_lengths_at_batch_edges(split):
    """Lists whose valid keys end at, just before and just after each score
    batch (16 keys at d=128) and value batch (8 keys) edge and each 128-key
    block edge, so that every trimmed last block length is exercised; in the
    split form all keys of a list sit in one key range."""
    rng = np.random.default_rng(77 + split)
    d, B, H, k = 128, 1, 2, 300
    n_kv = (1 << 22) // (4 * d) + 5 if split else 4096   # two ranges (split) or one short row
    lengths = [1, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 130, 191, 192, 193, 255,
               256, 257, 300]
    n_q = len(lengths)
    q, kk, v = _rbf(rng, B, H, n_q, d), _rbf(rng, B, H, n_kv, d), _rbf(rng, B, H, n_kv, d)
    lists = np.full((n_q, k), -1, np.int32)
    for r, n in enumerate(lengths):
        lists[r, :n] = rng.integers(0, min(n_kv, 4000), size=n)  # first range only
    gi = torch.from_numpy(lists).cuda()
    if split:
        assert sa.attn_workspace_bytes(B, H, n_q, n_kv, d, k) > 0
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(kk), to_dev_bf16(v)
    print(f"gather list lengths split={split}", flush=True)
    o, l = sa.attn_fwd(qd, kd, vd, gather_idx=gi, split=split)
    o_ref, lse_ref = oracle.attn_gather_rows(q, kk, v, lists)
    check_o_lse(o.cpu().numpy().reshape(-1, d), l.cpu().numpy().reshape(-1), o_ref, lse_ref, ctx=f"split={split}")
