"""Pins of the oracle's repacked weight layout.

The Vulkore page's repack test (section 4 of its quant_test.cpp, "repacked
fast path") asks two things of a load-time repack: that the values rebuilt
from the repacked bytes equal the native dequantization bit for bit, and that
a row count which is not a multiple of the interleave group (it uses 130
rows) is padded correctly.  Both are pinned here, plus:

* the section tables are a permutation of each row's k-block (every byte
  exactly once), so the repack is lossless for any bytes;
* hand-derived positions: for each kind, a few bytes of a record whose source
  row and offset were worked out by hand from the kind's block layout and the
  lane that decodes them; a swapped j and G, a wrong block stride or a wrong
  section order moves them;
* padding rows are zero and the size is the native size rounded up to whole
  tiles.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from oracle import repack as rp

KINDS = ["Q4_0", "Q5_0", "Q8_0", "IQ4_NL", "MXFP4", "IQ4_XS", "Q4_K", "Q6_K"]


@pytest.mark.parametrize("kind", KINDS)
def test_sections_are_a_permutation_of_the_kblock(kind):
    B = rp.kblock_bytes(kind)
    row, off = rp.record_source(kind)
    assert row.size == 16 * B
    flat = np.sort(row * B + off)
    assert np.array_equal(flat, np.arange(16 * B))


@pytest.mark.parametrize("kind", KINDS)
def test_reconstruct_equals_dequant_bit_exactly_on_130_rows(kind):
    N, K = 130, 1024
    W = wl.random_weights(kind, N, K, wl.rng("repack_pin", kind))
    P = rp.repack(kind, W, N, K)
    assert P.size == rp.packed_bytes(kind, N, K) == 9 * 16 * (K // 256) * rp.kblock_bytes(kind)
    back = rp.reconstruct(kind, P, N, K)
    assert np.array_equal(back, W.reshape(N, -1))
    want = oracle.dequant(kind, W).reshape(N, K)
    got = rp.reconstruct_values(kind, P, N, K)
    assert np.array_equal(got.view(np.uint64), want.view(np.uint64))


@pytest.mark.parametrize("kind", KINDS)
def test_padding_rows_are_zero(kind):
    N, K = 18, 512
    W = wl.random_weights(kind, N, K, wl.rng("repack_pad", kind))
    P = rp.repack(kind, W, N, K)
    # Tile 1 holds rows 16, 17 and fourteen zero rows: every record byte
    # taken from its rows 2 .. 15 (rows 18 .. 31) is zero.
    B = rp.kblock_bytes(kind)
    row, off = rp.record_source(kind)
    rec = P.reshape(2, 2, 16 * B)[1]  # [k-block][record byte] of tile 1
    assert np.all(rec[:, row >= 2] == 0)
    assert np.any(rec[:, row < 2] != 0)


# (kind, record byte, source row j, offset in the row's k-block), worked out
# by hand.  Lane sections are 1024 bytes of 16-byte slots, slot 16 G + j.
HAND = [
    # Q4_0: slot (G=2, j=5) of lane section 1, byte 6 = block 4 + 6 // 4 = 5,
    # code byte 4 G + 6 % 4 = 10: offset 18 * 5 + 2 + 10.
    ("Q4_0", 1024 + 16 * (16 * 2 + 5) + 6, 5, 18 * 5 + 2 + 10),
    # Q4_0: the scale section starts at 2048; row 3's byte 5 = block 2's d, high byte.
    ("Q4_0", 2048 + 16 * 3 + 5, 3, 18 * 2 + 1),
    # MXFP4: slot (G=3, j=0) of lane section 0, byte 15 = block 3, code byte 15.
    ("MXFP4", 16 * (16 * 3) + 15, 0, 17 * 3 + 1 + 15),
    # MXFP4: row section of eight E8M0 bytes: row 9, byte 7 = block 7's exponent.
    ("MXFP4", 2048 + 8 * 9 + 7, 9, 17 * 7),
    # Q5_0: the qh section (32 bytes per row) follows the codes; row 1, byte 13
    # = block 3's qh byte 1.  Then the d section at 2048 + 512.
    ("Q5_0", 2048 + 32 * 1 + 13, 1, 22 * 3 + 2 + 1),
    ("Q5_0", 2048 + 512 + 16 * 15 + 14, 15, 22 * 7),
    ("Q5_0", 16 * (16 * 1 + 2) + 4, 2, 22 * 1 + 6 + 4),
    # Q8_0: four lane sections; section 3, slot (G=1, j=7), byte 9 = block 7,
    # code byte 8 + 1: offset 34 * 7 + 2 + 9.
    ("Q8_0", 3 * 1024 + 16 * (16 + 7) + 9, 7, 34 * 7 + 2 + 9),
    ("Q8_0", 4096 + 16 * 4 + 0, 4, 0),
    # IQ4_XS: section 1, slot (G=0, j=11), byte 5 = group 5, code byte 1.
    ("IQ4_XS", 1024 + 16 * 11 + 5, 11, 8 + 16 * 5 + 1),
    ("IQ4_XS", 2048 + 8 * 2 + 3, 2, 3),
    # Q4_K: slot (G=3, j=14) of section 1, byte 0 = code byte 32 * 3 + 16.
    ("Q4_K", 1024 + 16 * (48 + 14), 14, 16 + 96 + 16),
    ("Q4_K", 2048 + 16 * 6 + 4, 6, 4),
    # Q6_K: G = 3 is half 1, byte lane 1: its qh bytes (section 2) start at
    # 128 + 32 + 16; its second low-nibble run (section 1) at 64 + 32 + 16.
    ("Q6_K", 2 * 1024 + 16 * (48 + 2) + 3, 2, 128 + 32 + 16 + 3),
    ("Q6_K", 1024 + 16 * (48 + 2), 2, 64 + 32 + 16),
    ("Q6_K", 16 * (16 + 8) + 15, 8, 16 + 15),
    ("Q6_K", 3072 + 16 * 10 + 9, 10, 192 + 9),
    ("Q6_K", 3072 + 256 + 2 * 13 + 1, 13, 209),
]


@pytest.mark.parametrize("kind,at,j,off", HAND)
def test_hand_derived_positions(kind, at, j, off):
    N, K = 32, 512
    B = rp.kblock_bytes(kind)
    for seed in ("a", "b", "c"):
        W = wl.random_weights(kind, N, K, wl.rng("repack_hand", kind + seed)).reshape(N, -1)
        P = rp.repack(kind, W, N, K)
        # Tile 1, k-block 1.
        rec = P[(1 * 2 + 1) * 16 * B:][:16 * B]
        assert rec[at] == W[16 + j, B + off]
