"""MX FP8 activations for the scaled FP8 x FP4 MXFP4 GEMM, on the CPU.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU baseline leg of ``bench.py`` may use it.  It shares no code with the HIP
library and never calls it.

The weight side is fixed by the pages: an MXFP4 block is one E8M0 scale byte
(2^(e - 127)) and 32 E2M1 codes (ferrox-cuda 0.20.0 codebook.rs, the MXFP4
row and ferrox_e8m0_to_f32), which gfx950's scaled matrix cores take as
they are.  The pages say nothing about the activation side of such a
product, and a single E4M3 rounding of each activation (relative error up to
2^-4) cannot hold the variant's bar of 2e-2 * sum|w||x| on every input (a
block of 1.0625s rounds each element 5.9 % low).  The plainest reading that
keeps the bar for every input is taken:

* OCP MX FP8 E4M3 elements: 1 sign, 4 exponent bits (bias 7), 3 mantissa
  bits, largest finite value 448, subnormals 2^-9 * m; rounding to nearest,
  ties to even mantissa, from the f32 value;
* a block scale is a power of two 2^e stored as the E8M0 byte e + 127: the
  smallest e with max|v| / 2^e <= 448 (so no element saturates), clamped to
  [-127, 127]; an all-zero block takes e = -127;
* each activation a of a 32-element block is split into two terms,
      a ~ 2^e1 * hi + 2^e2 * lo
  with hi = E4M3(a / 2^e1) on the block scale of a, and lo = E4M3(r / 2^e2)
  of the residual r = a - 2^e1 * hi on the block scale of the residuals.
  The matrix cores multiply both terms by the same weights.

The scaling by 2^-e and the residual are exact in f32 (a power of two times
an f32, and the difference of two numbers within a factor of two of each
other or of a number and zero), so the only roundings are the two E4M3
roundings: |a - (2^e1 hi + 2^e2 lo)| <= 2^-4 |r| + 2^(e2 - 10) with
|r| <= 2^-4 |a| + 2^(e1 - 10), i.e. about 2^-8 of |a|.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Values (binary64) of E4M3 codes; 0x7F and 0xFF are NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, (e - 7).astype(np.int64)))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e4m3_encode(v) -> np.ndarray:
    """E4M3 codes of f32 values v with |v| <= 448, nearest, ties to the even
    mantissa; the sign bit is v's (so -0.0 gives 0x80)."""
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    if np.any(np.abs(v) > E4M3_MAX) or np.any(np.isnan(v)):
        raise ValueError("E4M3 input outside [-448, 448]")
    sign = np.signbit(v).astype(np.int64) << 7
    a = np.abs(v)
    out = np.empty(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # Subnormals (and zero): m = RN(a / 2^-9) in 0..8; m = 8 is the code of
    # the smallest normal 2^-6, so the code is m itself.
    out[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)
    an = a[~sub]
    if an.size:
        _, x = np.frexp(an)            # an = f 2^x, f in [0.5, 1)
        E = x - 1                      # an in [2^E, 2^(E+1))
        m = np.rint((an / np.ldexp(1.0, E) - 1.0) * 8.0).astype(np.int64)   # 0..8, ties to even
        E = np.where(m == 8, E + 1, E)
        m = np.where(m == 8, 0, m)
        out[~sub] = ((E + 7) << 3) | m
    assert np.all((out & 0x7F) <= 0x7E)
    return (out | sign).astype(np.uint8)


def scale_exponent(amax) -> np.ndarray:
    """The smallest integer e with amax / 2^e <= 448, clamped to [-127, 127];
    -127 for amax = 0 (amax binary64, exact)."""
    amax = np.asarray(amax, dtype=np.float64)
    out = np.full(amax.shape, -127, dtype=np.int64)
    pos = amax > 0
    if np.any(pos):
        _, x = np.frexp(amax[pos])
        e = x - 10                      # a start below the answer
        for _ in range(4):              # step up while the condition fails
            bad = amax[pos] / np.ldexp(1.0, e) > E4M3_MAX
            e = np.where(bad, e + 1, e)
        assert np.all(amax[pos] / np.ldexp(1.0, e) <= E4M3_MAX)
        assert np.all(amax[pos] / np.ldexp(1.0, e - 1) > E4M3_MAX)
        out[pos] = e
    return np.clip(out, -127, 127)


def _f32_scale(a32, e) -> np.ndarray:
    """f32(a / 2^e), clamped to +-448 (the clamp matters only where the
    exponent was clamped)."""
    v = np.ldexp(a32.astype(np.float64), -e).astype(np.float32)
    return np.clip(v, -E4M3_MAX, E4M3_MAX)


def quantize(X):
    """The two-term MX FP8 form of activations X [M][K] (f32 or f16):
    (hi codes, lo codes) uint8 [M][K] in element order, and (e1 + 127,
    e2 + 127) E8M0 bytes uint8 [M][K/32]."""
    X = np.asarray(X)
    if X.dtype not in (np.float32, np.float16):
        raise TypeError("activations must be f32 or f16")
    X = np.atleast_2d(X).astype(np.float32)
    M, K = X.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    a = X.reshape(M, K // BLOCK, BLOCK)
    e1 = scale_exponent(np.max(np.abs(a.astype(np.float64)), axis=2))
    hi = e4m3_encode(_f32_scale(a, e1[:, :, None]))
    # Residual in f32 (exact, see the module docstring: checked here).
    back = np.ldexp(e4m3_decode(hi), e1[:, :, None]).astype(np.float32)
    r = (a - back).astype(np.float32)
    assert np.array_equal(r.astype(np.float64), a.astype(np.float64) - back.astype(np.float64)), "inexact residual"
    e2 = scale_exponent(np.max(np.abs(r.astype(np.float64)), axis=2))
    lo = e4m3_encode(_f32_scale(r, e2[:, :, None]))
    return (hi.reshape(M, K), lo.reshape(M, K), (e1 + 127).astype(np.uint8), (e2 + 127).astype(np.uint8))


def rebuilt(X) -> np.ndarray:
    """2^e1 hi + 2^e2 lo as binary64 [M][K] (exact)."""
    hi, lo, s1, s2 = quantize(X)
    M, K = hi.shape
    e1 = np.repeat(s1.astype(np.int64) - 127, BLOCK, axis=1)
    e2 = np.repeat(s2.astype(np.int64) - 127, BLOCK, axis=1)
    return np.ldexp(e4m3_decode(hi), e1) + np.ldexp(e4m3_decode(lo), e2)


def matmul_rebuilt(Wd, X):
    """(y, bound): the exact product of dequantized weights Wd [N][K]
    (binary64) with the rebuilt activations of X, and sum |w| |a'|."""
    A = rebuilt(X)
    Wd = np.asarray(Wd, dtype=np.float64)
    return A @ Wd.T, np.abs(A) @ np.abs(Wd).T
