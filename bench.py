#!/usr/bin/env python3
"""Benchmark of the block-sparse attention forward on one MI355X.

Workload (the glossary's worked pattern): B=1, H=32, N=8192, d=128, causal
sliding window 1024 (inclusive) + 4 sink tokens, 128x128 blocks; Q, K, V
bfloat16 ~ N(0, 1) from fixed seeds.  One step = one pass of the hot path:
the block-list builder followed by the fused block-sparse attention (element
masks on partial tiles only), inputs resident in HBM.

Metric: effective TFLOP/s over live pairs = 4 * d * live_pairs / step time
(2 products x 2 flop per multiply-add; the softmax is not counted).

Also reported on the same JSON line:
  roofline      the attention kernel's achieved TFLOP/s over live pairs per
                launch (HIP events on the launch stream) against the bf16
                dense MFMA peak, plus HBM traffic from committed rocprofv3
                counters when they belong to the current kernel source;
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the same
                workload on this machine's host cores;
  dsa_prefill   the content-selected path on its own workload (1,024
                queries at the end of a 65,536-token context, H=16, d=128,
                indexer d_I=64, top-2048): indexer, top-k and gather times.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_block_window1024_sinks4_n8192_traffic.json")
ATTN_SRC = os.path.join(ROOT, "block_sparse_attention_sa_amd", "csrc", "attn_block.hip")


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def src_hash(path=ATTN_SRC) -> str:
    """Hash of the kernel source with comments and blank space removed, so a
    comment edit does not orphan the committed counters."""
    import re
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    code = "\n".join(" ".join(line.split()) for line in text.splitlines() if line.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def _traffic():
    """HBM bytes per attention launch from committed counters, if they match this source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != src_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--o-dtype", choices=["f32", "bf16"], default="f32")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dsa", action="store_true")
    ap.add_argument("--no-strided", action="store_true")
    ap.add_argument("--no-select", action="store_true")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--no-other", action="store_true", help="skip the tiny and BigBird-style block workloads")
    ap.add_argument("--only", choices=["dsa", "strided", "select", "bwd", "window128", "bigbird", "dma_calib"],
                    help="time one secondary workload alone (for per-kernel profiles; prints only its object)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="the CPU oracle repeats whole passes over the workload until this much time has passed")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="run one plain device copy (negation) of this many MiB before the steps; "
                         "its HBM counters calibrate FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, "
                         "WRITE_SIZE) of a run with --copy-calib-mib into the committed traffic figure")
    ap.add_argument("--calib-mib", type=int, default=256, help="size used with --copy-calib-mib")
    ap.add_argument("--dma-calib-from", metavar="FETCH_CSV",
                    help="no GPU: FETCH_SIZE factor of the attention kernel's own loads, from a rocprofv3 "
                         "--pmc FETCH_SIZE counter_collection.csv of a run with --only dma_calib")
    ap.add_argument("--sustain-steps", type=int, default=300,
                    help="after the timed steps, run this many more steps untimed and then time 50 again "
                         "(the 'sustained' object: the shader clock settles after a few hundred steps of "
                         "sustained load); 0 skips it. value and roofline come from the timed steps only")
    args = ap.parse_args()
    if args.traffic_from:
        return _write_traffic(args.traffic_from[0], args.traffic_from[1], args.calib_mib)
    if args.dma_calib_from:
        return _dma_factor(args.dma_calib_from)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU; there is no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import block_sparse_attention_sa_amd as sa
    from block_sparse_attention_sa_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")

    def dev_bf16(u16):
        return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).to(dev)

    cfg = W.attn_config(2)
    _log(f"bench: generating inputs for {cfg.name}")
    inp = W.attn_inputs(cfg)
    q, k, v = (dev_bf16(inp[t]) for t in ("q", "k", "v"))
    o_dtype = torch.float32 if args.o_dtype == "f32" else torch.bfloat16
    out = torch.empty((cfg.B, cfg.H, cfg.N, cfg.d), dtype=o_dtype, device=dev)
    lse = torch.empty((cfg.B, cfg.H, cfg.N), dtype=torch.float32, device=dev)
    bl = sa.build_block_mask(cfg.pattern, cfg.N, cfg.N, cfg.block, cfg.block, device=dev)
    torch.cuda.synchronize()
    live_pairs_per_head = int(bl.live_pairs.cpu()[0])
    live_blocks = int(bl.kv_count.sum())
    n_partial = int(sum(int(bl.kv_partial[i, : int(bl.kv_count[i])].sum()) for i in range(bl.kv_count.numel())))
    assert live_blocks == 595 and live_pairs_per_head == 7900662, (live_blocks, live_pairs_per_head)
    live_pairs = live_pairs_per_head * cfg.B * cfg.H
    flops = 4.0 * cfg.d * live_pairs
    tile_flops = 4.0 * cfg.d * cfg.block * cfg.block * live_blocks * cfg.B * cfg.H

    if args.only:
        sections = {
            "dsa": lambda: _bench_dsa(sa, W, np, torch, dev, dev_bf16),
            "strided": lambda: _bench_strided(sa, W, np, torch, dev, dev_bf16),
            "select": lambda: _bench_select(sa, W, np, torch, dev, dev_bf16),
            "bwd": lambda: _bench_bwd(sa, np, torch, dev, cfg, q, k, v, bl, out, lse, live_pairs, live_blocks),
            "window128": lambda: _bench_blocks(sa, W, np, torch, dev, dev_bf16, 1),
            "bigbird": lambda: _bench_blocks(sa, W, np, torch, dev, dev_bf16, 4),
            "dma_calib": lambda: _dma_calib(sa, torch, dev, cfg, q, k, v, out, lse),
        }
        print(json.dumps({args.only: sections[args.only]()}), flush=True)
        return 0

    if args.copy_calib_mib > 0:
        n = args.copy_calib_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)  # reads and writes exactly n * 4 bytes
        torch.cuda.synchronize()
        del src, dst

    def step():
        sa.build_block_mask(cfg.pattern, cfg.N, cfg.N, cfg.block, cfg.block, device=dev, out=bl)
        sa.attn_fwd(q, k, v, bl, out=out, lse=lse)

    _log(f"bench: warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    _log(f"bench: timing {args.steps} steps")
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        ev[i][0].record(stream)
        sa.build_block_mask(cfg.pattern, cfg.N, cfg.N, cfg.block, cfg.block, device=dev, out=bl)
        ev[i][1].record(stream)
        sa.attn_fwd(q, k, v, bl, out=out, lse=lse)
        ev[i][2].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    builder_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    attn_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    value = flops / (ms_per_step * 1e-3) / 1e12
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    _log(f"bench: step {ms_per_step * 1e3:.1f} us (builder {builder_ms * 1e3:.1f} us, attention "
         f"{attn_ms * 1e3:.1f} us) -> {value:.1f} TFLOP/s over live pairs")

    # the attention kernel alone, median over at least 50 launches, warm (L2 and
    # MALL as the previous launch left them) and cold (a 1 GiB buffer written
    # between launches)
    reps = max(50, args.steps)
    warm, cold = [], []
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        sa.attn_fwd(q, k, v, bl, out=out, lse=lse)
        e1.record(stream)
        warm.append((e0, e1))
    for _ in range(reps):
        flush.fill_(1.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        sa.attn_fwd(q, k, v, bl, out=out, lse=lse)
        e1.record(stream)
        cold.append((e0, e1))
    torch.cuda.synchronize()
    del flush
    attn_med_ms = float(np.median([a.elapsed_time(b) for a, b in warm]))
    attn_cold_ms = float(np.median([a.elapsed_time(b) for a, b in cold]))

    # Sustained load: the GPU's clock dips a few milliseconds into a burst of
    # these steps and settles higher after a few hundred; a job that runs the
    # step continuously sees the settled rate.  Reported beside, not as, value.
    sustained = None
    if args.sustain_steps > 0:
        for _ in range(args.sustain_steps):
            step()
        sev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(50)]
        for e in sev:
            e[0].record(stream)
            sa.build_block_mask(cfg.pattern, cfg.N, cfg.N, cfg.block, cfg.block, device=dev, out=bl)
            e[1].record(stream)
            sa.attn_fwd(q, k, v, bl, out=out, lse=lse)
            e[2].record(stream)
        torch.cuda.synchronize()
        s_step = float(np.mean([e[0].elapsed_time(e[2]) for e in sev]))
        s_attn = float(np.mean([e[1].elapsed_time(e[2]) for e in sev]))
        s_med = float(np.median([e[1].elapsed_time(e[2]) for e in sev]))
        sustained = {
            "note": f"50 steps timed after {args.sustain_steps} more untimed steps of sustained load",
            "ms_per_step": round(s_step, 5),
            "tflops_over_live_pairs_per_step": round(flops / (s_step * 1e-3) / 1e12, 2),
            "attention_us_mean": round(s_attn * 1e3, 2),
            "attention_us_median": round(s_med * 1e3, 2),
            "attention_frac_of_peak": round(flops / (s_attn * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        }

    traffic = _traffic()
    result = {
        "metric": "effective TFLOP/s over live pairs (and % bf16 MFMA peak), 1x MI355X",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "causal sliding window 1024 + 4 sinks, B=1 H=32 N=8192 d=128, 128x128 blocks "
                        "(the glossary's worked pattern)",
            "batch": cfg.B, "heads": cfg.H, "seq_len": cfg.N, "head_dim": cfg.d,
            "block": cfg.block, "live_blocks_per_head": live_blocks, "partial_blocks_per_head": n_partial,
            "live_pairs": live_pairs, "o_dtype": args.o_dtype,
            "pct_bf16_peak_over_live_pairs": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
            "builder_us": round(builder_ms * 1e3, 2), "attention_us": round(attn_ms * 1e3, 2),
            "attention_tflops_over_live_tiles": round(tile_flops / (attn_ms * 1e-3) / 1e12, 2),
            "attention_us_median_warm": round(attn_med_ms * 1e3, 2),
            "attention_us_median_cold": round(attn_cold_ms * 1e3, 2),
            "attention_median_reps": reps,
            "attention_tflops_over_live_pairs_median_warm": round(flops / (attn_med_ms * 1e-3) / 1e12, 2),
            "attention_tflops_over_live_tiles_median_warm": round(tile_flops / (attn_med_ms * 1e-3) / 1e12, 2),
        },
        "roofline": {
            "kernel": "attn_block_kernel<128,128,128>",
            "bound": "mfma",
            "achieved": round(attn_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "algorithmic_flop_per_launch": flops,
        },
    }
    if sustained is not None:
        result["sustained"] = sustained

    if not args.no_dsa:
        result["dsa_prefill"] = _bench_dsa(sa, W, np, torch, dev, dev_bf16)

    if not args.no_strided:
        result["strided"] = _bench_strided(sa, W, np, torch, dev, dev_bf16)

    if not args.no_select:
        result["content_selected"] = _bench_select(sa, W, np, torch, dev, dev_bf16)

    if not args.no_bwd:
        result["backward"] = _bench_bwd(sa, np, torch, dev, cfg, q, k, v, bl, out, lse, live_pairs, live_blocks)

    if not args.no_other:
        result["window128_sinks4_n512"] = _bench_blocks(sa, W, np, torch, dev, dev_bf16, 1)
        result["bigbird_n16384"] = _bench_blocks(sa, W, np, torch, dev, dev_bf16, 4)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = _cpu_baseline(cfg, inp, args.cpu_seconds, np)

    print(json.dumps(result), flush=True)
    return 0


def _sustained_us(fn, np, torch, settle=300, reps=50):
    """Median of reps launches of fn (HIP events on the current stream) after settle
    untimed ones: the rate once the GPU's clock has settled under sustained load."""
    for _ in range(settle):
        fn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3


def _bench_strided(sa, W, np, torch, dev, dev_bf16, reps=10):
    """The strided workload both ways: block lists of the whole pattern (every causal tile is
    live, since the strided term touches each one), and the local band plus residue views."""
    cfg = W.attn_config(3)
    print("bench: generating the strided workload's inputs", file=sys.stderr, flush=True)
    inp = W.attn_inputs(cfg)
    q, k, v = (dev_bf16(inp[t]) for t in ("q", "k", "v"))
    pat = cfg.pattern.as_dict()
    stream = torch.cuda.current_stream(dev)
    bl = sa.build_block_mask(pat, cfg.N, cfg.N, cfg.block, cfg.block, device=dev)
    shape = (cfg.B, cfg.H, cfg.N, cfg.d)
    o = torch.empty(shape, dtype=torch.float32, device=dev)
    lse = torch.empty(shape[:3], dtype=torch.float32, device=dev)
    ws = sa.strided_plan(pat, cfg.B, cfg.H, cfg.N, cfg.d, dev)
    ways = {
        "blocks": lambda: sa.attn_fwd(q, k, v, bl, out=o, lse=lse),
        "split": lambda: sa.attn_fwd_strided(q, k, v, pat, out=o, lse=lse, workspace=ws),
    }
    t = {}
    for name, fn in ways.items():
        fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in ev:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        t[name] = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e-3
    pairs = int(bl.live_pairs.item()) * cfg.B * cfg.H
    flop = 4.0 * cfg.d * pairs
    split_sus = _sustained_us(ways["split"], np, torch)
    return {
        "workload": "causal strided, stride 128 + local band of 128, B=1 H=16 N=16384 d=64",
        "live_pairs": pairs,
        "blocks_us": round(t["blocks"] * 1e6, 1),
        "blocks_tflops_over_live_pairs": round(flop / t["blocks"] / 1e12, 2),
        "split_us": round(t["split"] * 1e6, 1),
        "split_tflops_over_live_pairs": round(flop / t["split"] / 1e12, 2),
        "split_us_median_sustained": round(split_sus, 1),
        "split_note": "one sa_attn_fwd call (SA_MODE_STRIDED) on a plan built once by sa_attn_strided_plan: "
                      "64x64 band tiles, then causal 64-row tiles per (head, key residue) view (residue 0's "
                      "view also holds the last row), merged by log-sum-exp in the kernel epilogue",
    }

def _bench_bwd(sa, np, torch, dev, cfg, q, k, v, bl, out, lse, live_pairs, live_blocks, reps=20):
    """The backward at the headline workload: dQ, dK, dV from the forward's O and LSE.
    Algorithmic work: 5 products per live pair (S, dP, dV, dQ, dK), 10 * d flop."""
    gen = torch.Generator(device=dev).manual_seed(20261203)
    g = torch.randn(q.shape, device=dev, generator=gen).to(torch.bfloat16)
    sa.attn_fwd(q, k, v, bl, out=out, lse=lse)
    dq, dk, dv = sa.attn_bwd(q, k, v, out, lse, g, bl)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        sa.attn_bwd(q, k, v, out, lse, g, bl, dq=dq, dk=dk, dv=dv)
        e1.record(stream)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    t = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e-3
    flop = 10.0 * cfg.d * live_pairs
    tile_flop = 10.0 * cfg.d * cfg.block * cfg.block * live_blocks * cfg.B * cfg.H
    return {
        "workload": "backward (dQ, dK, dV) of the headline workload, from its O and LSE",
        "us_median": round(t * 1e6, 1),
        "tflops_over_live_pairs": round(flop / t / 1e12, 2),
        "tflops_over_live_tiles": round(tile_flop / t / 1e12, 2),
        "pct_bf16_peak_over_live_pairs": round(100.0 * flop / t / 1e12 / PEAK_BF16_TFLOPS, 2),
        "flop_note": "10 * head_dim per live pair (S, dP, dV, dQ, dK products)",
    }


def _bench_blocks(sa, W, np, torch, dev, dev_bf16, cid, reps=50):
    """Block-list attention on another block workload (builder + attention timed apart)."""
    cfg = W.attn_config(cid)
    _log(f"bench: generating inputs for {cfg.name}")
    inp = W.attn_inputs(cfg)
    q, k, v = (dev_bf16(inp[t]) for t in ("q", "k", "v"))
    bl = sa.build_block_mask(cfg.pattern, cfg.N, cfg.N, cfg.block, cfg.block, device=dev)
    o = torch.empty((cfg.B, cfg.H, cfg.N, cfg.d), dtype=torch.float32, device=dev)
    lse = torch.empty((cfg.B, cfg.H, cfg.N), dtype=torch.float32, device=dev)
    sa.attn_fwd(q, k, v, bl, out=o, lse=lse)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = []
    for _ in range(reps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        sa.build_block_mask(cfg.pattern, cfg.N, cfg.N, cfg.block, cfg.block, device=dev, out=bl)
        e[1].record(stream)
        sa.attn_fwd(q, k, v, bl, out=o, lse=lse)
        e[2].record(stream)
        ev.append(e)
    torch.cuda.synchronize()
    tb = float(np.median([e[0].elapsed_time(e[1]) for e in ev])) * 1e-3
    ta = float(np.median([e[1].elapsed_time(e[2]) for e in ev])) * 1e-3
    ta_sus = _sustained_us(lambda: sa.attn_fwd(q, k, v, bl, out=o, lse=lse), np, torch)
    pairs = int(bl.live_pairs.item()) * cfg.B * cfg.H
    tiles = int(bl.kv_count.sum().item()) * cfg.B * cfg.H
    return {
        "workload": f"{cfg.name}: B={cfg.B} H={cfg.H} N={cfg.N} d={cfg.d}, {cfg.block}x{cfg.block} blocks",
        "live_pairs": pairs,
        "builder_us_median": round(tb * 1e6, 2),
        "attention_us_median": round(ta * 1e6, 2),
        "attention_tflops_over_live_pairs": round(4.0 * cfg.d * pairs / ta / 1e12, 2),
        "attention_tflops_over_live_tiles": round(4.0 * cfg.d * cfg.block * cfg.block * tiles / ta / 1e12, 2),
        "attention_us_median_sustained": round(ta_sus, 2),
        "sustained_note": "median of 50 launches after 300 untimed ones (settled clock)",
    }


def _bench_select(sa, W, np, torch, dev, dev_bf16, reps=20):
    """Content-selected key blocks (workload 6): the selection (block means, scores,
    top-n per query block and head) and the block kernel over the per-head lists."""
    cfg = W.select_config()
    _log("bench: generating the content-selected workload's inputs")
    inp = W.select_inputs(cfg)
    q, k, v = (dev_bf16(inp[t]) for t in ("q", "k", "v"))
    sel = sa.select_blocks(q, k, cfg.block, cfg.block, cfg.n_select)
    o = torch.empty((cfg.B, cfg.H, cfg.N, cfg.d), dtype=torch.float32, device=dev)
    lse = torch.empty((cfg.B, cfg.H, cfg.N), dtype=torch.float32, device=dev)
    ws = torch.empty(1 << 22, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    steps = [("select", lambda: sa.select_blocks(q, k, cfg.block, cfg.block, cfg.n_select, workspace=ws, out=sel)),
             ("attention", lambda: sa.attn_fwd(q, k, v, sel, out=o, lse=lse))]
    for _, fn in steps:
        fn()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    for e in ev:
        for j, (_, fn) in enumerate(steps):
            e[j].record(stream)
            fn()
        e[-1].record(stream)
    torch.cuda.synchronize()
    t = {name: float(np.median([e[j].elapsed_time(e[j + 1]) for e in ev])) * 1e-3 for j, (name, _) in enumerate(steps)}
    pairs = int(sel.live_pairs.item())
    tiles = int(sel.kv_count.sum().item())
    flop = 4.0 * cfg.d * pairs
    return {
        "workload": "content-selected key blocks (own block + top-8 by mean-query . mean-key per query block and "
                    "head), causal, B=1 H=32 N=8192 d=128, 128x128 blocks",
        "live_pairs": pairs, "tiles": tiles,
        "select_us": round(t["select"] * 1e6, 1),
        "attention_us": round(t["attention"] * 1e6, 1),
        "attention_tflops_over_live_pairs": round(flop / t["attention"] / 1e12, 2),
        "attention_tflops_over_live_tiles": round(4.0 * cfg.d * cfg.block * cfg.block * tiles / t["attention"] / 1e12, 2),
        "total_tflops_over_live_pairs": round(flop / (t["select"] + t["attention"]) / 1e12, 2),
    }


def _bench_dsa(sa, W, np, torch, dev, dev_bf16, reps=10):
    """The content-selected workload: the streaming indexer + top-k (no score
    matrix), the two-step form through the 268 MB score matrix (indexer, then
    top-k, timed apart), and the gather attention over the selection."""
    tc = W.topk_config(5)
    _log("bench: generating configuration-5 inputs (64K context)")
    ti = W.topk_inputs(tc)
    qi, ki = dev_bf16(ti["q_idx"]), dev_bf16(ti["k_idx"])
    q, k, v = (dev_bf16(ti[t]) for t in ("q", "k", "v"))
    scores = torch.empty((tc.n_q, tc.n_kv), dtype=torch.float32, device=dev)
    idx = torch.empty((tc.n_q, tc.topk), dtype=torch.int32, device=dev)
    ws = torch.empty(sa.indexer_topk_workspace_bytes(tc.n_q, tc.n_kv, tc.topk), dtype=torch.uint8, device=dev)
    o = torch.empty((1, tc.H, tc.n_q, tc.d), dtype=torch.float32, device=dev)
    lse = torch.empty((1, tc.H, tc.n_q), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    steps = [
        ("stream", lambda: sa.indexer_topk(qi, ki, tc.q_offset, tc.topk, out=idx, workspace=ws)),
        ("indexer", lambda: sa.indexer_scores(qi, ki, tc.q_offset, scores=scores)),
        ("topk", lambda: sa.topk(scores, tc.q_offset, tc.topk, out=idx)),
        ("gather", lambda: sa.attn_fwd(q, k, v, gather_idx=idx, out=o, lse=lse)),
    ]
    for _, fn in steps:
        fn()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(steps) + 1)] for _ in range(reps)]
    for e in ev:
        for j, (_, fn) in enumerate(steps):
            e[j].record(stream)
            fn()
        e[-1].record(stream)
    torch.cuda.synchronize()
    t = {name: float(np.median([e[j].elapsed_time(e[j + 1]) for e in ev])) * 1e-3
         for j, (name, _) in enumerate(steps)}
    cand = sum(min(tc.q_offset + r + 1, tc.n_kv) for r in range(tc.n_q))
    idx_bytes = 2 * (tc.n_q + tc.n_kv) * tc.d_idx + 4 * cand
    topk_bytes = 4 * cand + 4 * tc.n_q * tc.topk
    pairs = tc.H * tc.n_q * tc.topk
    gather_bytes = pairs * tc.d * 2 * 2 + tc.H * tc.n_q * tc.d * (2 + 4)
    return {
        "workload": "1024 queries at the end of a 65536-token causal context, H=16 d=128, indexer d_I=64, top-2048",
        "indexer_topk_stream_us": round(t["stream"] * 1e6, 1),
        "indexer_topk_stream_tflops_fp32": round(2.0 * tc.d_idx * cand / t["stream"] / 1e12, 2),
        "indexer_topk_stream_workspace_bytes": int(ws.numel()),
        "indexer_us": round(t["indexer"] * 1e6, 1),
        "indexer_gbs": round(idx_bytes / t["indexer"] / 1e9, 1),
        "indexer_tflops_fp32": round(2.0 * tc.d_idx * cand / t["indexer"] / 1e12, 2),
        "topk_us": round(t["topk"] * 1e6, 1),
        "topk_gbs": round(topk_bytes / t["topk"] / 1e9, 1),
        "gather_us": round(t["gather"] * 1e6, 1),
        "gather_gbs": round(gather_bytes / t["gather"] / 1e9, 1),
        "gather_tflops_over_pairs": round(4.0 * tc.d * pairs / t["gather"] / 1e12, 2),
        "total_us": round((t["stream"] + t["gather"]) * 1e6, 1),
        "total_note": "streaming indexer + top-k, then gather attention",
        "hbm_peak_gbs": PEAK_HBM_GBS,
    }


def _cpu_baseline(cfg, inp, seconds, np):
    """The fp64 oracle on the whole workload (every row of every head), repeated
    until `seconds` have passed; rate over the live pairs it evaluated."""
    import oracle  # the CPU oracle is the baseline leg here, nothing else
    rows = np.arange(cfg.B * cfg.H * cfg.N, dtype=np.int64)
    _log(f"bench: cpu oracle on the whole workload ({rows.size} rows), >= {seconds:.0f} s")
    t0 = time.perf_counter()
    oracle.block_lists(cfg.pattern, cfg.N, cfg.N, cfg.block, cfg.block)
    t1 = time.perf_counter()
    passes, pairs = 0, 0
    while True:
        _, _, cnt = oracle.attn_rows(cfg.pattern, inp["q"], inp["k"], inp["v"], rows=rows, return_counts=True)
        passes += 1
        pairs += int(cnt.sum())
        if time.perf_counter() - t1 >= seconds:
            break
    t2 = time.perf_counter()
    value = 4.0 * cfg.d * pairs / (t2 - t1) / 1e12
    return {
        "value": round(value, 6),
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "affinity_cpus": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"fp64 oracle attention, {passes} pass(es) over the whole workload ({cfg.H} heads x "
                  f"{cfg.N} rows, {pairs // passes} live pairs per pass) in {t2 - t1:.2f} s; its block "
                  f"lists for the whole matrix took {t1 - t0:.2f} s",
    }


def _counter_means(path, counter):
    """Per-kernel mean of one counter over the dispatches in a rocprofv3 counter_collection.csv."""
    import csv
    sums, counts = {}, {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            k = r["Kernel_Name"]
            sums[k] = sums.get(k, 0.0) + float(r["Counter_Value"])
            counts[k] = counts.get(k, 0) + 1
    return {k: (sums[k] / counts[k], counts[k]) for k in sums}


DMA_CALIB_LAUNCHES = 5


def _dma_calib(sa, torch, dev, cfg, q, k, v, out, lse):
    """The headline kernel on a block-diagonal pattern at the headline shape: each
    query block lists only its own key block, so every K and V tile is copied into
    LDS (LDS-DMA) by exactly one workgroup and Q is read once.  A FETCH_SIZE pass
    over this run gives the counter's factor for the kernel's own loads."""
    pat = dict(causal=1, window_left=0, window_right=0)
    bl = sa.build_block_mask(pat, cfg.N, cfg.N, cfg.block, cfg.block, device=dev)
    torch.cuda.synchronize()
    assert int(bl.kv_count.max()) == 1 and int(bl.kv_count.min()) == 1
    for _ in range(DMA_CALIB_LAUNCHES):
        sa.attn_fwd(q, k, v, bl, out=out, lse=lse)
    torch.cuda.synchronize()
    tensor = cfg.B * cfg.H * cfg.N * cfg.d * 2
    return {"workload": "block-diagonal lists at B=1 H=32 N=8192 d=128, 128x128 blocks", "launches":
            DMA_CALIB_LAUNCHES, "q_bytes": tensor, "kv_bytes": 2 * tensor}


def _dma_factor(fetch_csv):
    """Bytes the block-diagonal launch must read (Q, K and V once each) per FETCH_SIZE
    KiB, for each of its dispatches."""
    import csv
    per = {}
    with open(fetch_csv) as f:
        for r in csv.DictReader(f):
            if "attn_block_kernel<128, 128, 128" in r["Kernel_Name"] and r["Counter_Name"] == "FETCH_SIZE":
                per[int(r["Dispatch_Id"])] = per.get(int(r["Dispatch_Id"]), 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit("no attention dispatches in " + fetch_csv)
    kib = [per[d] for d in sorted(per)]
    tensor = 1 * 32 * 8192 * 128 * 2
    need = 3 * tensor
    out = {"dispatches": len(kib), "fetch_kib_per_dispatch": [round(x, 1) for x in kib],
           "bytes_read_once": need, "factor_per_dispatch": [round(need / (x * 1024.0), 4) for x in kib]}
    print(json.dumps(out))
    return 0


def _write_traffic(fetch_csv, write_csv, calib_mib):
    """HBM bytes per attention launch: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch) of the attention kernel, each scaled by known bytes / counter
    reading of the calibration copy (a negation of calib_mib MiB)."""
    fetch = _counter_means(fetch_csv, "FETCH_SIZE")
    write = _counter_means(write_csv, "WRITE_SIZE")

    def pick(table, word):
        keys = [k for k in table if word in k]
        if len(keys) != 1:
            raise SystemExit(f"expected one kernel matching {word!r}, found {keys}")
        return table[keys[0]], keys[0]

    (f_attn, nf), name = pick(fetch, "attn_block_kernel<128, 128, 128")
    (w_attn, nw), _ = pick(write, "attn_block_kernel<128, 128, 128")
    (f_copy, _), copy_name = pick(fetch, "neg_kernel")
    (w_copy, _), _ = pick(write, "neg_kernel")
    known_kib = calib_mib * 1024.0
    f_fac, w_fac = known_kib / f_copy, known_kib / w_copy
    out = {
        "kernel": name,
        "kernel_source_sha256_16": src_hash(),
        "fetch_kib_per_dispatch": round(f_attn, 1),
        "write_kib_per_dispatch": round(w_attn, 1),
        "dispatches": [nf, nw],
        "calibration": {"kernel": copy_name[:80], "bytes_read_and_written": calib_mib << 20,
                        "fetch_kib": round(f_copy, 1), "write_kib": round(w_copy, 1),
                        "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4)},
        "hbm_bytes_per_launch": round((f_attn * f_fac + w_attn * w_fac) * 1024.0),
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
