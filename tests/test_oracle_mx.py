"""Pins of oracle/mx.py, the two-term MX FP8 activations of the scaled MXFP4
GEMM (CPU only).

* E4M3 decoding of all 256 codes and encoding of every tie, subnormal and
  boundary value against torch's float8_e4m3fn cast (a library routine);
* the block scale against a brute-force search over exponents;
* hand-worked blocks: a block of 1.0625s (the E4M3 tie 272 -> 256 and its
  residual), the 448 boundary, the mantissa boundary 0.875, an all-zero
  block, negative zero;
* the two-term error bound on random and wide-range blocks, and exactness
  for values E4M3 holds.
"""
import numpy as np
import pytest

from oracle import mx

torch = pytest.importorskip("torch")


def torch_e4m3(v):
    t = torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_decode_matches_the_library_on_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = mx.e4m3_decode(codes)
    nan = np.isnan(want)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(got[~nan], want[~nan])
    assert got[0x7E] == 448.0 and got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9 and got[0x38] == 1.0


def test_encode_matches_the_library_on_ties_subnormals_and_random_values():
    vals = mx.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))   # 0 .. 448
    mids = (vals[1:] + vals[:-1]) / 2                             # every tie (exact in f32)
    quarter = vals[:-1] + (vals[1:] - vals[:-1]) / 4
    g = np.random.default_rng(5)
    rnd = g.uniform(-448, 448, 20000)
    tiny = g.uniform(-2.0 ** -5, 2.0 ** -5, 5000)
    v = np.concatenate([vals, mids, quarter, -vals, -mids, rnd, tiny, [448.0, -448.0, 0.0, -0.0]]).astype(np.float32)
    assert np.array_equal(mx.e4m3_encode(v), torch_e4m3(v))
    # Round trip of every finite code.
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(mx.e4m3_encode(mx.e4m3_decode(codes)), codes)


def test_scale_is_the_smallest_power_of_two_that_fits():
    g = np.random.default_rng(7)
    amax = np.concatenate([g.lognormal(0, 8, 3000), [448.0, 448.0 * 2 ** -20, 1.75, 1.875, 0.875, 2.0 ** -126]])
    e = mx.scale_exponent(amax)
    for a, ei in zip(amax, e):
        cands = [k for k in range(-200, 200) if a / 2.0 ** k <= 448]
        assert ei == max(-127, min(127, cands[0])), a
    assert mx.scale_exponent(np.array([0.0]))[0] == -127


def test_block_of_1p0625():
    """amax 1.0625 -> 2^-8; 1.0625 * 256 = 272 is halfway between the E4M3
    values 256 and 288 and goes to 256 (even mantissa 0).  The residual
    0.0625 takes 2^-12 (0.0625 * 4096 = 256), code 256, so the two terms
    rebuild 1.0625 exactly."""
    X = np.full((1, 32), 1.0625, dtype=np.float32)
    hi, lo, s1, s2 = mx.quantize(X)
    assert s1[0, 0] == 127 - 8 and s2[0, 0] == 127 - 12
    assert np.all(hi == 0x78) and np.all(lo == 0x78)      # 0x78 = 2^8 * 1.0
    assert mx.e4m3_decode(0x78) == 256.0
    assert np.all(mx.rebuilt(X) == 1.0625)


def test_boundaries_448_and_0p875():
    X = np.zeros((3, 32), dtype=np.float32)
    X[0, 5] = 448.0                 # 448 / 2^0 fits: scale byte 127, code 0x7E
    X[1, 0] = 1.75                  # mantissa 0.875: 1.75 * 2^8 = 448 fits, scale 2^-8
    X[2, 31] = -1.875               # mantissa 0.9375: 2^-8 would give 480, so 2^-7: -240
    hi, lo, s1, s2 = mx.quantize(X)
    assert s1[0, 0] == 127 and hi[0, 5] == 0x7E
    assert s1[1, 0] == 127 - 8 and hi[1, 0] == 0x7E
    assert s1[2, 0] == 127 - 7 and hi[2, 31] == 0x80 | 0x77 and mx.e4m3_decode(0xF7) == -240.0
    assert np.all(lo == 0) and np.all(s2 == 0)            # exact: zero residual blocks
    assert np.array_equal(mx.rebuilt(X), X.astype(np.float64))


def test_zero_block_and_negative_zero():
    X = np.zeros((2, 64), dtype=np.float16)
    X[1, 3] = -0.0
    X[1, 40] = 3.0
    hi, lo, s1, s2 = mx.quantize(X)
    assert np.all(s1[0] == 0) and np.all(hi[0] == 0) and np.all(lo[0] == 0)
    assert hi[1, 3] == 0x80                                 # the sign of -0.0 is kept
    assert s1[1, 1] == 127 - 7 and hi[1, 40] == mx.e4m3_encode(np.float32(384.0))


@pytest.mark.parametrize("dist", ["normal", "wide", "sparse", "f16"])
def test_two_term_error_bound(dist):
    """|a - a'| <= 2^-8 |a| + 2^(e1 - 14) per element: the first term loses at
    most 2^-4 of |a| (or 2^(e1 - 10) in the subnormal range) and the second
    term 2^-4 of that."""
    g = np.random.default_rng({"normal": 1, "wide": 2, "sparse": 3, "f16": 4}[dist])
    if dist == "normal":
        X = g.standard_normal((64, 512)).astype(np.float32)
    elif dist == "wide":
        X = (g.standard_normal((64, 512)) * np.exp(g.uniform(-30, 30, (64, 512)))).astype(np.float32)
    elif dist == "sparse":
        X = np.where(g.random((64, 512)) < 0.9, 0, g.standard_normal((64, 512)) * 1e3).astype(np.float32)
    else:
        X = g.standard_normal((64, 512)).astype(np.float16)
    A = X.astype(np.float64)
    _, _, s1, _ = mx.quantize(X)
    e1 = np.repeat(s1.astype(np.int64) - 127, 32, axis=1)
    err = np.abs(A - mx.rebuilt(X))
    lim = 2.0 ** -8 * np.abs(A) + np.ldexp(1.0, e1 - 14)
    assert np.all(err <= lim)
    assert err.max() <= 2.0 ** -7 * np.abs(A).max()


def test_values_e4m3_holds_come_through_the_first_term():
    """Blocks of E4M3 values whose largest magnitude is 448, times a power of
    two per row: the block scale is that power, every element is exact in the
    first term and the residual block is zero."""
    g = np.random.default_rng(11)
    codes = g.integers(0, 0x7F, (16, 256)).astype(np.uint8)
    codes[:, ::32] = 0x7E                                   # 448 in every block
    sign = np.where(g.random((16, 256)) < 0.5, -1.0, 1.0)
    X = (mx.e4m3_decode(codes) * sign * 2.0 ** g.integers(-20, 20, (16, 1))).astype(np.float32)
    hi, lo, s1, s2 = mx.quantize(X)
    assert np.all(lo == 0) and np.all(s2 == 0)
    assert np.array_equal(mx.rebuilt(X), X.astype(np.float64))
