"""Shared helpers for the GPU parity tests (inputs, transfers, tolerances)."""

import numpy as np

from block_sparse_attention_sa_amd import workloads as W

# Tolerances stated for the hot path: O max abs 1e-2, LSE max abs 1e-3.
O_TOL = 1e-2
LSE_TOL = 1e-3


def to_dev_bf16(u16):
    import torch
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).cuda()


def bf16_half_ulp(x):
    """Half a bfloat16 ulp at |x| (the rounding error of storing x as bf16)."""
    ax = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 8)


def check_o_lse(o_gpu, lse_gpu, o_ref, lse_ref, bf16_out=False, ctx=""):
    """O within 1e-2 (+ half a bf16 ulp of the reference when O is stored as bf16),
    LSE within 1e-3; rows with no allowed key must give O = 0 and LSE = -inf."""
    o_gpu = np.asarray(o_gpu, np.float64)
    lse_gpu = np.asarray(lse_gpu, np.float64)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_gpu), empty), f"{ctx}: empty-row mismatch"
    assert np.all(o_gpu[empty] == 0), f"{ctx}: empty rows must give O = 0"
    tol = O_TOL + (bf16_half_ulp(o_ref) if bf16_out else 0.0)
    err = np.abs(o_gpu - o_ref)
    bad = err > tol
    assert not bad.any(), f"{ctx}: O max err {err.max():.3e} at {np.argwhere(bad)[:5].tolist()}"
    fin = ~empty
    if fin.any():
        lerr = np.abs(lse_gpu[fin] - lse_ref[fin]).max()
        assert lerr <= LSE_TOL, f"{ctx}: LSE max err {lerr:.3e}"
    return float(err.max()) if err.size else 0.0


def random_pattern(rng, n_q, n_kv, allow_offset=True):
    pat = dict(causal=int(rng.integers(0, 2)))
    if allow_offset and rng.random() < 0.3:
        pat["q_offset"] = int(rng.integers(0, 100))
    if rng.random() < 0.8:
        pat["window_left"] = int(rng.integers(0, 200))
        pat["window_right"] = int(rng.integers(0, 60))
    if rng.random() < 0.5:
        pat["sinks"] = int(rng.integers(1, 9))
    if rng.random() < 0.4:
        pat["stride"] = int(rng.integers(1, 130))
        pat["stride_phase"] = int(rng.integers(0, pat["stride"]))
    if rng.random() < 0.25:
        pat["global_tokens"] = int(rng.integers(1, 40))
    if rng.random() < 0.4:
        u = int(rng.integers(8, 100))
        pat["unit"] = u
        pat["unit_window"] = int(rng.integers(-1, 2))
        rows = -(-(n_q + pat.get("q_offset", 0)) // u)
        units = -(-n_kv // u)
        pat["rand_table"] = rng.integers(-1, units, size=(rows, 3)).astype(np.int32)
    return pat


_FULL_REF = {}


def full_config_reference(cid):
    """Inputs and the oracle's O and LSE over every row of attention configuration
    ``cid`` at its full size, computed once per test process."""
    if cid not in _FULL_REF:
        import oracle
        cfg = W.attn_config(cid)
        inp = W.attn_inputs(cfg)
        o_ref, lse_ref = oracle.attn_rows(cfg.pattern, inp["q"], inp["k"], inp["v"])
        _FULL_REF[cid] = (cfg, inp, o_ref, lse_ref)
    return _FULL_REF[cid]


__all__ = ["W"]
