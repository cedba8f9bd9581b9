"""The load-time repacked weight layout, defined on the CPU.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU baseline leg of ``bench.py`` may use it.  It shares no code with the HIP
library and never calls it.

The Vulkore page (``examples/llm/quant_test.cpp``, section 4, "repacked fast
path") repacks GGUF weights once at load time so that its matvec reads aligned
planes, and requires that the values reconstructed from the repacked bytes
equal the native dequantization bit for bit.  The layout here is this
library's own (a reading of that passage for 64-wide wavefronts, not the
page's plane format), and its definition is this module:

* Rows are taken in groups of 16 (a "tile"); a last, partial group is padded
  with zero rows.  K is taken in k-blocks of 256 elements, so one row's
  k-block is ``B`` consecutive bytes of its GGUF row (B = 144 for Q4_0,
  Q4_K and IQ4_NL's eight blocks, 136 for MXFP4 and IQ4_XS, 176 for Q5_0
  and Q5_K, 272 for Q8_0, 210 for Q6_K, 84 for Q2_K, 110 for Q3_K).
* Tile t, k-block b becomes one record of 16 B bytes at offset
  ``(t * n_kblocks + b) * 16 * B``: the same bytes, permuted, so the repacked
  tensor is exactly as large as the native one plus the padding rows.
* A record is a run of sections.  A *lane section* is 1024 bytes: 64 slots of
  16 bytes, slot ``16 G + j`` holding bytes of row j chosen by G (0..3).  A
  *row section* of width w is 16 slots of w bytes, slot j holding bytes of
  row j.  The tables below give, for byte i of a slot, its offset inside the
  row's k-block.

Every byte of every row's k-block appears exactly once in its record, so the
repack is lossless; ``reconstruct`` inverts it.
"""
from __future__ import annotations

import numpy as np

from . import dequant

# K elements per k-block, rows per tile.
KB_ELEMS = 256
TILE_ROWS = 16

_GEOMETRY = {  # kind: (block bytes, block elements), the GGUF block sizes
    "Q4_0": (18, 32), "Q5_0": (22, 32), "Q8_0": (34, 32), "IQ4_NL": (18, 32),
    "MXFP4": (17, 32), "IQ4_XS": (136, 256), "Q4_K": (144, 256), "Q6_K": (210, 256),
    "Q2_K": (84, 256), "Q3_K": (110, 256), "Q5_K": (176, 256),
}
_IDS = {2: "Q4_0", 6: "Q5_0", 8: "Q8_0", 20: "IQ4_NL", 39: "MXFP4", 23: "IQ4_XS", 12: "Q4_K", 14: "Q6_K",
        10: "Q2_K", 11: "Q3_K", 13: "Q5_K"}

KINDS = tuple(_GEOMETRY)


def _name(kind) -> str:
    if isinstance(kind, str):
        if kind not in _GEOMETRY:
            raise KeyError(f"{kind} has no repacked layout")
        return kind
    return _IDS[int(kind)]


def kblock_bytes(kind) -> int:
    """Bytes of one row's 256-element k-block."""
    bb, be = _GEOMETRY[_name(kind)]
    return bb * (KB_ELEMS // be)


# ---------------------------------------------------------------------------
# Section tables.  lane(c, G, i): byte i of lane section c's slot for group G.
# row(c, i): byte i of row section c's slot.  Offsets are inside one row's
# k-block; for the 32-element kinds block s of the k-block starts at s * bytes.
# ---------------------------------------------------------------------------
def _nibble_codes(block_bytes, code_at):
    """Two lane sections of 4-bit codes: slot (c, G) holds, for blocks
    s = 4c .. 4c+3 in turn, the four code bytes 4G .. 4G+3 of block s (their
    low nibbles are elements 4G.., their high nibbles 16 + 4G..)."""
    def lane(c, G, i):
        s = 4 * c + i // 4
        return block_bytes * s + code_at + 4 * G + i % 4
    return 2, lane


def _layout(kind):
    """(number of lane sections, lane(c, G, i), [(width, row(i)), ...])."""
    k = _name(kind)
    if k in ("Q4_0", "IQ4_NL"):
        n, lane = _nibble_codes(18, 2)
        return n, lane, [(16, lambda i: 18 * (i // 2) + i % 2)]       # the eight f16 scales d
    if k == "MXFP4":
        n, lane = _nibble_codes(17, 1)
        return n, lane, [(8, lambda i: 17 * i)]                        # the eight E8M0 bytes
    if k == "Q5_0":
        n, lane = _nibble_codes(22, 6)
        return n, lane, [(32, lambda i: 22 * (i // 4) + 2 + i % 4),    # the eight 32-bit qh words
                         (16, lambda i: 22 * (i // 2) + i % 2)]        # the eight f16 scales d
    if k == "Q8_0":
        def lane(c, G, i):  # blocks 2c, 2c+1: code bytes 8G .. 8G+7 of each
            s = 2 * c + i // 8
            return 34 * s + 2 + 8 * G + i % 8
        return 4, lane, [(16, lambda i: 34 * (i // 2) + i % 2)]
    if k == "IQ4_XS":
        def lane(c, G, i):  # groups 4c .. 4c+3: code bytes 4G .. 4G+3 of each group
            s = 4 * c + i // 4
            return 8 + 16 * s + 4 * G + i % 4
        return 2, lane, [(8, lambda i: i)]                             # d, scales_h, scales_l
    if k == "Q4_K":
        def lane(c, G, i):  # code bytes 32G + 16c .. +15 (sub-blocks 2G, 2G+1)
            return 16 + 32 * G + 16 * c + i
        return 2, lane, [(16, lambda i: i)]                            # d, dmin, 12 scale bytes
    if k == "Q6_K":
        def lane(c, G, i):  # half h = G // 2, byte lane a = G % 2
            h, a = G // 2, G % 2
            return (64 * h + 16 * a + i, 64 * h + 32 + 16 * a + i, 128 + 32 * h + 16 * a + i)[c]
        return 3, lane, [(16, lambda i: 192 + i),                      # the sixteen int8 scales
                         (2, lambda i: 208 + i)]                       # f16 d
    if k == "Q5_K":
        def lane(c, G, i):  # code bytes 32G + 16c .. +15 (sub-blocks 2G, 2G+1), after the 16-byte header and qh
            return 48 + 32 * G + 16 * c + i
        return 2, lane, [(32, lambda i: 16 + i),                       # qh[32]: every row's fifth bits
                         (16, lambda i: i)]                            # d, dmin, 12 scale bytes
    if k == "Q2_K":
        def lane(c, G, i):  # G = 2n + a: code bytes 32n + 16a .. +15
            return 16 + 16 * G + i
        return 1, lane, [(16, lambda i: i),                            # scales[16] (scale, min nibbles)
                         (4, lambda i: 80 + i)]                        # f16 d, dmin
    if k == "Q3_K":
        def lane(c, G, i):  # G = 2n + a: code bytes 32n + 16a .. +15
            return 32 + 16 * G + i
        return 1, lane, [(32, lambda i: i),                            # hmask[32]
                         (8, lambda i: 96 + i),                        # scale bytes 0..7 (low four bits)
                         (4, lambda i: 104 + i),                       # scale bytes 8..11 (top two bits)
                         (2, lambda i: 108 + i)]                       # f16 d
    raise KeyError(k)


def record_source(kind) -> tuple[np.ndarray, np.ndarray]:
    """(row, offset) of every byte of a record, in record order."""
    n_lane, lane, rows = _layout(kind)
    src_row, src_off = [], []
    for c in range(n_lane):
        for slot in range(64):
            G, j = slot // 16, slot % 16
            for i in range(16):
                src_row.append(j)
                src_off.append(lane(c, G, i))
    for width, row in rows:
        for j in range(TILE_ROWS):
            for i in range(width):
                src_row.append(j)
                src_off.append(row(i))
    return np.array(src_row, dtype=np.int64), np.array(src_off, dtype=np.int64)


def packed_bytes(kind, N: int, K: int) -> int:
    if K % KB_ELEMS:
        raise ValueError("K must be a multiple of 256")
    tiles = -(-N // TILE_ROWS)
    return tiles * TILE_ROWS * (K // KB_ELEMS) * kblock_bytes(kind)


def _as_tiles(kind, W, N: int, K: int) -> np.ndarray:
    """Native rows, padded with zero rows, as [tiles][16][k-blocks][B]."""
    B = kblock_bytes(kind)
    nkb = K // KB_ELEMS
    W = np.ascontiguousarray(W, dtype=np.uint8).reshape(N, nkb * B)
    tiles = -(-N // TILE_ROWS)
    padded = np.zeros((tiles * TILE_ROWS, nkb * B), dtype=np.uint8)
    padded[:N] = W
    return padded.reshape(tiles, TILE_ROWS, nkb, B)


def repack(kind, W, N: int, K: int) -> np.ndarray:
    """The repacked bytes of N native rows of K elements, as a flat uint8 array."""
    if K % KB_ELEMS:
        raise ValueError("K must be a multiple of 256")
    T = _as_tiles(kind, W, N, K)
    src_row, src_off = record_source(kind)
    # [tiles][k-blocks][record byte]
    rec = T[:, src_row, :, src_off]          # fancy indices first: [record byte][tiles][k-blocks]
    return np.ascontiguousarray(np.moveaxis(rec, 0, -1)).reshape(-1)


def reconstruct(kind, P, N: int, K: int) -> np.ndarray:
    """The native rows [N][row bytes] that the repacked bytes P hold."""
    B = kblock_bytes(kind)
    nkb = K // KB_ELEMS
    tiles = -(-N // TILE_ROWS)
    P = np.ascontiguousarray(P, dtype=np.uint8).reshape(tiles, nkb, TILE_ROWS * B)
    src_row, src_off = record_source(kind)
    T = np.zeros((tiles, TILE_ROWS, nkb, B), dtype=np.uint8)
    T[:, src_row, :, src_off] = np.moveaxis(P, -1, 0)
    return T.reshape(tiles * TILE_ROWS, nkb * B)[:N]


def reconstruct_values(kind, P, N: int, K: int) -> np.ndarray:
    """Exact (binary64) weights [N][K] held by the repacked bytes P."""
    return dequant(_name(kind), reconstruct(kind, P, N, K)).reshape(N, K)
