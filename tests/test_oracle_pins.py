"""Pins for the CPU oracle: checks against what the pages and mathematics fix,
independent of the oracle's own code.

* hand-decoded single blocks (tests/golden/hand_blocks.json), compared bit
  for bit (so -0.0 is distinct);
* an exhaustive binary16 sweep against numpy's float16 conversion;
* all 256 E8M0 bytes against ldexp(1, e - 127);
* Q4_0's -8 bias and Q5_0's fifth-bit splice;
* bit ownership: which elements each bit of a block moves;
* cross-format identities (Q5_K with no high bits is Q4_K, IQ4_XS with every
  group scale 33 is IQ4_NL, Q3_K with a full high mask is Q2_K without mins,
  Q2_K with pairwise-equal sub-block scales is Q4_K with two-bit codes, and
  Q3_K is Q6_K with codes 28..35 and scales -32..31: the two kinds the pages
  do not lay out are tied to two they do);
* the matmul against exact rational arithmetic, numpy's matmul, unit
  vectors, row selection and permutation;
* the routed-expert products against per-expert matmuls.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_blocks.json")
ALL_KINDS = list(wl.KINDS)


def _bits(a):
    return np.asarray(a, dtype=np.float64).view(np.uint64)


def _same_bits(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    both_nan = np.isnan(got) & np.isnan(want)
    return np.all(both_nan | (_bits(got) == _bits(want)))


def _golden_blocks():
    with open(GOLDEN) as f:
        return json.load(f)["blocks"]


@pytest.mark.parametrize("blk", _golden_blocks(), ids=lambda b: b["name"])
def test_hand_decoded_block(oracle_mod, blk):
    raw = np.full(blk["len"], blk["fill"], dtype=np.uint8)
    for off, val in blk["set"].items():
        raw[int(off)] = val
    _, be = wl.geometry(blk["kind"])
    want = np.full(be, np.nan)
    for start, end, val in blk["runs"]:
        want[start:end] = val
    for idx, val in blk["points"].items():
        want[int(idx)] = val
    assert not np.isnan(want).any(), "fixture leaves elements undefined"
    got = oracle_mod.dequant(blk["kind"], raw)
    bad = np.nonzero(_bits(got) != _bits(want))[0]
    assert bad.size == 0, f"{blk['name']}: elements {bad[:8]} got {got[bad[:8]]} want {want[bad[:8]]}"


def test_geometry_tables_agree(oracle_mod):
    for name, (_, bb, be) in wl.KINDS.items():
        assert oracle_mod.block_geometry(name) == (bb, be), name
    for absent in (3, 7, 9, 15, 16, 19, 21):  # Q4_1, Q5_1, Q8_1, Q8_K, IQ2_XXS, IQ1_S, IQ3_S
        with pytest.raises(KeyError):
            oracle_mod.block_geometry(absent)


def test_binary16_exhaustive(oracle_mod):
    """Every f16 pattern as the d of a Q8_0 block whose first code is 1."""
    pats = np.arange(65536, dtype=np.uint32)
    blocks = np.zeros((65536, 34), dtype=np.uint8)
    blocks[:, 0] = pats & 0xFF
    blocks[:, 1] = pats >> 8
    blocks[:, 2] = 1
    got = oracle_mod.dequant("Q8_0", blocks).reshape(65536, 32)[:, 0]
    want = pats.astype(np.uint16).view(np.float16).astype(np.float64)
    assert _same_bits(got, want)
    assert np.isnan(got).sum() == 2 * 1023  # every NaN pattern stays NaN
    assert _bits(got[0x8000]) == _bits(-0.0)


def test_e8m0_every_byte(oracle_mod):
    """Each MXFP4 scale byte e, with code 2 (E2M1 1.0) in element 0."""
    blocks = np.zeros((256, 17), dtype=np.uint8)
    blocks[:, 0] = np.arange(256)
    blocks[:, 1] = 2
    got = oracle_mod.dequant("MXFP4", blocks).reshape(256, 32)[:, 0]
    for e in range(255):
        assert got[e] == math.ldexp(1.0, e - 127), e
    assert got[127] == 1.0  # bias 127, not 128
    assert got[0] == 2.0 ** -127 and got[0] > 0
    assert math.isnan(got[255])  # reading: OCP MX reserves 0xFF for NaN


def test_q4_0_bias(oracle_mod):
    for byte, want in ((0x88, 0.0), (0x00, -8.0), (0xFF, 7.0)):
        blk = np.full(18, byte, dtype=np.uint8)
        blk[0], blk[1] = 0x00, 0x3C  # d = 1.0
        assert np.all(oracle_mod.dequant("Q4_0", blk) == want)


def test_q5_0_fifth_bit_splice(oracle_mod):
    for e in range(32):
        blk = np.zeros(22, dtype=np.uint8)
        blk[1] = 0x3C
        blk[2:6] = np.frombuffer(np.uint32(1 << e).tobytes(), dtype=np.uint8)
        got = oracle_mod.dequant("Q5_0", blk)
        want = np.full(32, -16.0)
        want[e] = 0.0
        assert np.array_equal(got, want), e
    g = wl.rng("pins", "q5_0")
    q4 = wl.random_weights("Q4_0", 64, 32, g).reshape(64, 18)
    for fill, shift in ((0x00, -8.0), (0xFF, 8.0)):
        q5 = np.zeros((64, 22), dtype=np.uint8)
        q5[:, 0:2] = q4[:, 0:2]
        q5[:, 2:6] = fill
        q5[:, 6:22] = q4[:, 2:18]
        d = q4[:, 0:2].copy().view(np.float16).astype(np.float64)
        want = oracle_mod.dequant("Q4_0", q4).reshape(64, 32) + shift * d
        assert np.array_equal(oracle_mod.dequant("Q5_0", q5).reshape(64, 32), want)


# Bit ownership: (bits per code, sub-block size, bits owned by each sub-block,
# bits shared by the whole block).
OWNERSHIP = {
    "Q8_0": (8, 32, 0, 16), "Q4_0": (4, 32, 0, 16), "Q5_0": (5, 32, 0, 16),
    "IQ4_NL": (4, 32, 0, 16), "MXFP4": (4, 32, 0, 8),
    "Q4_K": (4, 32, 12, 32), "Q5_K": (5, 32, 12, 32), "IQ4_XS": (4, 32, 6, 16),
    "Q6_K": (6, 16, 8, 16), "Q2_K": (2, 16, 8, 32), "Q3_K": (3, 16, 6, 16),
}


def _nondegenerate_block(oracle_mod, kind, g):
    """A config-distributed block in which flipping any single bit changes
    at least one element (no zero sub-block scale masks a code)."""
    bb, be = wl.geometry(kind)
    for _ in range(2000):
        blk = wl.random_weights(kind, 1, be, g).reshape(-1)
        base = oracle_mod.dequant(kind, blk)
        flips = np.repeat(blk[None, :], bb * 8, axis=0)
        for bit in range(bb * 8):
            flips[bit, bit // 8] ^= np.uint8(1 << (bit % 8))
        vals = oracle_mod.dequant(kind, flips).reshape(bb * 8, be)
        changed = ~((vals == base[None, :]) & (np.signbit(vals) == np.signbit(base)[None, :]))
        if changed.any(axis=1).all():
            return changed
    raise AssertionError(f"{kind}: no non-degenerate block found")


@pytest.mark.parametrize("kind", ALL_KINDS)
def test_bit_ownership(oracle_mod, kind):
    code_bits, sub, per_sub, whole = OWNERSHIP[kind]
    bb, be = wl.geometry(kind)
    changed = _nondegenerate_block(oracle_mod, kind, wl.rng("pins", f"own_{kind}"))
    sizes = changed.sum(axis=1)
    code = sizes == 1
    owner = np.argmax(changed, axis=1)
    per_elem = np.bincount(owner[code], minlength=be)
    assert np.all(per_elem == code_bits), f"code bits per element: {np.unique(per_elem)}"
    shared = np.nonzero(~code)[0]
    group_count = np.zeros(be // sub, dtype=int)
    whole_count = 0
    for bit in shared:
        idx = np.nonzero(changed[bit])[0]
        g0, g1 = idx.min() // sub, idx.max() // sub
        if g0 == g1 and per_sub:
            group_count[g0] += 1
        else:
            whole_count += 1
    assert np.all(group_count == per_sub), f"sub-block bits: {group_count}"
    assert whole_count == whole, f"block-wide bits: {whole_count}"
    assert code.sum() + group_count.sum() + whole_count == bb * 8


def test_q5_k_without_high_bits_is_q4_k(oracle_mod):
    q4 = wl.random_weights("Q4_K", 32, 256, wl.rng("pins", "q5k_q4k")).reshape(32, 144)
    q5 = np.zeros((32, 176), dtype=np.uint8)
    q5[:, 0:16] = q4[:, 0:16]
    q5[:, 48:176] = q4[:, 16:144]
    assert _same_bits(oracle_mod.dequant("Q5_K", q5), oracle_mod.dequant("Q4_K", q4))


def test_iq4_xs_with_unit_scales_is_iq4_nl(oracle_mod):
    g = wl.rng("pins", "iq4xs_nl")
    xs = wl.random_weights("IQ4_XS", 16, 256, g).reshape(16, 136)
    xs[:, 2], xs[:, 3] = 0xAA, 0xAA   # top bits 2 in every group
    xs[:, 4:8] = 0x11                 # low bits 1 in every group: ls = 33
    nl = np.zeros((16, 8, 18), dtype=np.uint8)
    nl[:, :, 0:2] = xs[:, None, 0:2]
    nl[:, :, 2:18] = xs[:, 8:136].reshape(16, 8, 16)
    assert _same_bits(oracle_mod.dequant("IQ4_XS", xs), oracle_mod.dequant("IQ4_NL", nl))


def test_q3_k_full_mask_is_q2_k_without_mins(oracle_mod):
    g = wl.rng("pins", "q3k_q2k")
    q2 = wl.random_weights("Q2_K", 16, 256, g).reshape(16, 84)
    t = g.integers(0, 16, size=(16, 16)).astype(np.uint8)   # sub-block scales 0..15
    q2[:, 0:16] = t                                          # mins 0
    s = t.astype(np.int64) + 32                              # Q3_K 6-bit scale = t + 32
    q3 = np.zeros((16, 110), dtype=np.uint8)
    q3[:, 0:32] = 0xFF
    q3[:, 32:96] = q2[:, 16:80]
    low = s & 15
    q3[:, 96:104] = (low[:, 0:8] | (low[:, 8:16] << 4)).astype(np.uint8)
    for m in range(4):
        hi = np.zeros(16, dtype=np.int64)
        for i in (m, m + 4, m + 8, m + 12):
            hi |= (s[:, i] >> 4) << (2 * (i // 4))
        q3[:, 104 + m] = hi.astype(np.uint8)
    q3[:, 108:110] = q2[:, 80:82]
    assert _same_bits(oracle_mod.dequant("Q3_K", q3), oracle_mod.dequant("Q2_K", q2))

def _f16_words(g, shape):
    """Finite, nonzero binary16 values (as uint16) of either sign."""
    v = (g.standard_normal(shape) * 0.5).astype(np.float16)
    v[v == 0] = np.float16(0.25)
    return v.view(np.uint16)


def test_q2_k_is_q4_k_with_two_bit_codes(oracle_mod):
    """Q2_K whose sub-blocks 2j and 2j+1 share scale a_j and min b_j (4 bits
    each) decodes to the same bits as Q4_K with sub-block j's scale a_j, min
    b_j, the same d and dmin, and codes 0..3 as its nibbles: d*a*q and dmin*b
    are exact in binary32 for both, so any placement slip in either layout
    shows.  Q4_K's layout is the one the pages print."""
    g = wl.rng("pins", "q2k_q4k")
    R = 24
    q = g.integers(0, 4, size=(R, 256))
    a = g.integers(0, 16, size=(R, 8))
    b = g.integers(0, 16, size=(R, 8))
    d, dmin = _f16_words(g, R), _f16_words(g, R)
    r = np.arange(256)
    q2 = np.zeros((R, 84), dtype=np.uint8)
    q2[:, 0:16] = (a | (b << 4))[:, np.arange(16) // 2]        # sc[i] = a | b << 4 of pair i / 2
    n, jj, l = r // 128, (r % 128) // 32, r % 32
    for row in range(R):
        np.bitwise_or.at(q2[row], 16 + 32 * n + l, (q[row] << (2 * jj)).astype(np.uint8))
    q2[:, 80:82] = d.view(np.uint8).reshape(R, 2)
    q2[:, 82:84] = dmin.view(np.uint8).reshape(R, 2)
    q4 = np.zeros((R, 144), dtype=np.uint8)
    q4[:, 0:2] = d.view(np.uint8).reshape(R, 2)
    q4[:, 2:4] = dmin.view(np.uint8).reshape(R, 2)
    q4[:, 4:8] = a[:, 0:4]                                     # 6-bit fields, high bits 0
    q4[:, 8:12] = b[:, 0:4]
    q4[:, 12:16] = a[:, 4:8] | (b[:, 4:8] << 4)
    pos = 16 + (r // 64) * 32 + r % 32
    hi = (r % 64) >= 32
    for row in range(R):
        np.bitwise_or.at(q4[row], pos, (q[row] << (4 * hi)).astype(np.uint8))
    assert _same_bits(oracle_mod.dequant("Q2_K", q2), oracle_mod.dequant("Q4_K", q4))


def test_q3_k_is_q6_k_with_three_bit_codes(oracle_mod):
    """Q3_K with two-bit codes q2, high-mask bits h and 6-bit scales s equals
    Q6_K with codes 32 + q2 - 4(1 - h) (28..35), int8 scales s - 32 and the
    same d: both are d * scale * code with exact binary32 products.  Q6_K's
    layout is the one the pages print."""
    g = wl.rng("pins", "q3k_q6k")
    R = 24
    q = g.integers(0, 4, size=(R, 256))
    h = g.integers(0, 2, size=(R, 256))
    sc = g.integers(0, 64, size=(R, 16))
    d = _f16_words(g, R)
    r = np.arange(256)
    n, jj, l = r // 128, (r % 128) // 32, r % 32
    q3 = np.zeros((R, 110), dtype=np.uint8)
    for row in range(R):
        np.bitwise_or.at(q3[row], l, (h[row] << (4 * n + jj)).astype(np.uint8))
        np.bitwise_or.at(q3[row], 32 + 32 * n + l, (q[row] << (2 * jj)).astype(np.uint8))
    low, high = sc & 15, sc >> 4
    q3[:, 96:104] = low[:, 0:8] | (low[:, 8:16] << 4)
    for m in range(4):
        q3[:, 104 + m] = sum(high[:, i] << (2 * (i // 4)) for i in (m, m + 4, m + 8, m + 12))
    q3[:, 108:110] = d.view(np.uint8).reshape(R, 2)
    code = 32 + q - 4 * (1 - h)
    hh, u = r // 128, r % 128
    l6, gq = u % 32, u // 32
    q6 = np.zeros((R, 210), dtype=np.uint8)
    for row in range(R):
        lo = (code[row] & 15) << (4 * (gq >= 2))
        np.bitwise_or.at(q6[row], 64 * hh + l6 + 32 * (gq & 1), lo.astype(np.uint8))
        np.bitwise_or.at(q6[row], 128 + 32 * hh + l6, ((code[row] >> 4) << (2 * gq)).astype(np.uint8))
    sub = 8 * hh + l6 // 16 + 2 * gq                           # the sub-block of element r
    assert np.array_equal(sub, r // 16)
    q6[:, 192:208] = (sc - 32).astype(np.int8).view(np.uint8)
    q6[:, 208:210] = d.view(np.uint8).reshape(R, 2)
    assert _same_bits(oracle_mod.dequant("Q3_K", q3), oracle_mod.dequant("Q6_K", q6))



@pytest.mark.parametrize("kind", ALL_KINDS)
def test_matmul_exact_brute_force(oracle_mod, kind):
    """N=3 rows of one block, M=2: the binary64 sum agrees with the exact
    rational sum to within K unit roundoffs of sum |w||x|."""
    bb, be = wl.geometry(kind)
    g = wl.rng("pins", f"bf_{kind}")
    W = wl.random_weights(kind, 3, be, g, scales="stress")
    X = wl.activations((2, be), np.float32, g)
    Y, B = oracle_mod.matmul(kind, W, be, X)
    Wd = oracle_mod.dequant(kind, W).reshape(3, be)
    for m in range(2):
        for n in range(3):
            exact = sum(Fraction(float(w)) * Fraction(float(x)) for w, x in zip(Wd[n], X[m]))
            mag = sum(abs(Fraction(float(w)) * Fraction(float(x))) for w, x in zip(Wd[n], X[m]))
            tol = be * 2.0 ** -52 * float(mag)
            assert abs(Fraction(Y[m, n]) - exact) <= Fraction(tol)
            assert abs(Fraction(B[m, n]) - mag) <= Fraction(tol)


@pytest.mark.parametrize("kind", ALL_KINDS)
def test_matmul_against_numpy_and_unit_vectors(oracle_mod, kind):
    bb, be = wl.geometry(kind)
    K, N, M = 2 * be if be == 256 else 8 * be, 37, 3
    g = wl.rng("pins", f"np_{kind}")
    W = wl.random_weights(kind, N, K, g)
    X = wl.activations((M, K), np.float16, g)
    Y, B = oracle_mod.matmul(kind, W, K, X)
    Wd = oracle_mod.dequant(kind, W).reshape(N, K)
    ref = X.astype(np.float64) @ Wd.T
    assert np.all(np.abs(Y - ref) <= 1e-12 * (np.abs(X.astype(np.float64)) @ np.abs(Wd).T) + 1e-300)
    assert np.allclose(B, np.abs(X.astype(np.float64)) @ np.abs(Wd).T, rtol=1e-12, atol=0)
    # unit vectors extract columns exactly
    for k in (0, 1, K // 2 + 3, K - 1):
        e = np.zeros((1, K), dtype=np.float32)
        e[0, k] = 1.0
        y, _ = oracle_mod.matmul(kind, W, K, e)
        assert np.array_equal(y[0], Wd[:, k])
    # row selection and row permutation
    rows = np.array([36, 0, 5, 5, 17])
    y_sel, _ = oracle_mod.matmul(kind, W, K, X, rows=rows)
    assert np.array_equal(y_sel, Y[:, rows])
    perm = np.array([2, 0, 1])
    y_perm, _ = oracle_mod.matmul(kind, W, K, X[perm])
    assert np.array_equal(y_perm, Y[perm])


def test_moe_matches_per_expert_matmul(oracle_mod):
    E, N, K, M, topk = 6, 9, 512, 5, 3
    g = wl.rng("pins", "moe")
    W = wl.random_weights("Q4_K", E * N, K, g)
    ids = wl.routing(M, E, topk, g)
    X = wl.activations((M, K), np.float16, g)
    H = wl.activations((M, topk, K), np.float16, g)
    Y, B = oracle_mod.moe("Q4_K", W, E, N, K, ids, X, x_per_slot=False)
    Yh, _ = oracle_mod.moe("Q4_K", W, E, N, K, ids, H, x_per_slot=True)
    rb = wl.row_bytes("Q4_K", K)
    Wr = W.reshape(E, N * rb)
    for t in range(M):
        for s in range(topk):
            e = ids[t, s]
            y, b = oracle_mod.matmul("Q4_K", Wr[e], K, X[t:t + 1])
            assert np.array_equal(Y[t, s], y[0]) and np.array_equal(B[t, s], b[0])
            y, _ = oracle_mod.matmul("Q4_K", Wr[e], K, H[t, s:s + 1])
            assert np.array_equal(Yh[t, s], y[0])
