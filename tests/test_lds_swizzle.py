"""Bank-conflict model of the backward kernels' LDS tile layout (CPU only).

The backward kernels keep Q, dO, K and V tiles in LDS row-major with 16-byte
chunks XOR-swizzled by row, and read them two ways: as 16-byte row pieces
(16 lanes take 16 consecutive rows at one logical chunk) and through the
transposing 8-byte reads (32 lanes take 4 consecutive rows x 4 consecutive
chunks, and the same 8 rows further on).  With the LDS modelled as 64 banks of
4 bytes, serving 16 lanes per pass for 16-byte reads and 32 for 8-byte reads,
the swizzle used there must give every pass distinct banks for both patterns;
the forward's K-tile swizzle (row & 15 at d = 128) does not for the second.
The swizzle and the read offsets are restated here from the kernel's
description; the GPU counters (SQ_LDS_BANK_CONFLICT) are what confirmed it.
"""
import pytest


def bswz(d, r):
    return (((r & 3) << 2) | ((r >> 2) & 3)) if d == 128 else ((((r >> 1) & 1) << 2) | ((r >> 2) & 3))


def kswz(d, r):
    return (r & 15) if d == 128 else ((r >> 1) & 7)


def worst_ways(addrs, nbytes, per_pass):
    worst = 1
    for p0 in range(0, len(addrs), per_pass):
        banks = {}
        for a in addrs[p0:p0 + per_pass]:
            for w in range(nbytes // 4):
                banks.setdefault((a // 4 + w) % 64, set()).add(a // 4 + w)
        worst = max(worst, max(len(s) for s in banks.values()))
    return worst


def row_read_ways(d, sw):
    rb = d * 2
    return max(worst_ways([(r0 + (l & 31)) * rb + (((2 * kb + (l >> 5)) ^ sw(d, r0 + (l & 31))) * 16)
                           for l in range(64)], 16, 16)
               for kb in range(d // 16) for r0 in (0, 32, 64, 96))


def tr_read_ways(d, sw):
    rb = d * 2
    worst = 1
    for db in range(d // 32):
        for r0 in range(0, 64, 16):
            for extra in (0, 8):
                addrs = []
                for l in range(64):
                    q, hf = l & 15, l >> 5
                    row = 4 * hf + (q >> 2) + extra + r0
                    col = 16 * ((l >> 4) & 1) + 4 * (q & 3) + 32 * db
                    addrs.append(row * rb + (((col >> 3) ^ sw(d, row)) * 16) + (col & 7) * 2)
                worst = max(worst, worst_ways(addrs, 8, 32))
    return worst


@pytest.mark.parametrize("d", [64, 128])
def test_backward_swizzle_is_conflict_free_both_ways(d):
    assert row_read_ways(d, bswz) == 1
    assert tr_read_ways(d, bswz) == 1
    # the second read of a transposing pair sits 8 rows on: its swizzle is the
    # first one's with bit 1 flipped (what the kernel's offsets assume)
    assert {bswz(d, r) ^ bswz(d, r + 8) for r in range(128) if r & 8 == 0} == {2}
    # every row's swizzle is a permutation of its chunks
    for r in range(64):
        assert sorted(c ^ bswz(d, r) for c in range(d // 8)) == list(range(d // 8))


@pytest.mark.parametrize("d,ways", [(64, 2), (128, 4)])
def test_k_style_swizzle_conflicts_on_transposing_reads(d, ways):
    assert row_read_ways(d, kswz) == 1
    assert tr_read_ways(d, kswz) == ways
