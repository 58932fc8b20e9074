"""Host-side check of the swizzled LDS tile layout of the head_dim-128 backward
kernels (csrc/attn_bwd.hip: tswz, LaneOffs, row_op, trr_op), restated here from
the kernel's own definitions: the swizzle permutes each row's 16-byte chunks, the
per-lane byte offsets with the chunk entered as an XOR reach the intended
(row, chunk) of a 32-row tile and stay inside it, and both read kinds (16-byte row
reads per 16 lanes, 8-byte transposing reads per 32 lanes) hit 64 distinct 4-byte
banks.  The gradients themselves are checked against the oracle by the GPU tests."""

import pytest


def tswz(D, r):
    return ((r & 15) ^ ((r & 3) << 2)) if D == 128 else (((r >> 1) & 7) ^ (((r >> 1) & 1) << 2))


def lane_offsets(D, lane):
    rb = 2 * D
    l32, hh = lane & 31, lane >> 5
    rof = 4 * (lane >> 5) + ((lane & 15) >> 2)
    cof = 16 * ((lane >> 4) & 1) + 4 * (lane & 3)
    row_off = l32 * rb + ((hh ^ tswz(D, l32)) << 4)
    t0 = rof * rb + (((cof >> 3) ^ tswz(D, rof)) << 4) + 2 * (cof & 7)
    t1 = (rof + 8) * rb + (((cof >> 3) ^ tswz(D, rof + 8)) << 4) + 2 * (cof & 7)
    return rof, cof, row_off, t0, t1


def max_bank_load(offsets, size):
    load = {}
    for o in offsets:
        for w in range(size // 4):
            b = (o // 4 + w) % 64
            load[b] = load.get(b, 0) + 1
    return max(load.values())


@pytest.mark.parametrize("D", [128, 64])
def test_swizzled_tile_addressing(D):
    rb = 2 * D
    phys = {}
    for r in range(32):
        for ch in range(D // 8):
            off = r * rb + ((ch ^ tswz(D, r)) << 4)
            assert 0 <= off <= 32 * rb - 16 and off not in phys
            phys[off] = (r, ch)
    for lane in range(64):
        rof, cof, row_off, t0, t1 = lane_offsets(D, lane)
        for c in range(D // 16):
            assert phys[row_off ^ (c << 5)] == (lane & 31, 2 * c + (lane >> 5))
        for ks in range(2):
            for db in range(D // 32):
                col = 32 * db + cof
                for t, row in ((t0, 16 * ks + rof), (t1, 16 * ks + rof + 8)):
                    off = 16 * ks * rb + (t ^ (db << 6))
                    assert phys[off & ~15] == (row, col >> 3)
                    assert off & 15 == 2 * (col & 7) and off + 8 <= 32 * rb


@pytest.mark.parametrize("D", [128, 64])
def test_swizzled_reads_are_conflict_free(D):
    for c in range(D // 16):
        for g in range(4):
            offs = [lane_offsets(D, l)[2] ^ (c << 5) for l in range(16 * g, 16 * g + 16)]
            assert max_bank_load(offs, 16) == 1
    rb = 2 * D
    for ks in range(2):
        for db in range(D // 32):
            for g in range(2):
                for which in (3, 4):
                    offs = [16 * ks * rb + (lane_offsets(D, l)[which] ^ (db << 6)) for l in range(32 * g, 32 * g + 32)]
                    assert max_bank_load(offs, 8) == 1
