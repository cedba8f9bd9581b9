"""Pins of the oracle's int8 activation quantization and product.

The reading (per 32-element block: d = amax / 127 in f32, q = x / d in f32
rounded to the nearest integer, ties to even) is tied to values fixed by it
and by arithmetic, not to the oracle's own code:

* blocks of integers whose largest magnitude is 127 quantize to themselves
  (d = 1), and power-of-two multiples of them to the same codes;
* exact halfway quotients round to even;
* an all-zero block gives d = 0 and zero codes;
* the element of largest magnitude always gets code +-127, and every
  rebuilt value lies within d/2 (1 + 2^-16) of x;
* the product against rebuilt activations, brute-forced from Q8_0 bytes by
  hand (f16 scale, int8 codes) with integer block sums, equals the oracle's;
* the quantization bound covers the distance between the two products.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from oracle import int8 as oi


def test_integer_blocks_with_max_127_are_exact():
    g = np.random.default_rng(3)
    k = g.integers(-127, 128, size=(3, 96)).astype(np.float32)
    k[:, 5] = 127.0
    k[:, 40] = -127.0
    k[:, 70] = 127.0
    q, d = oi.quantize(k)
    assert np.all(d == 1.0)
    assert np.array_equal(q.astype(np.float32), k)
    for scale in (2.0 ** -9, 2.0 ** 6):
        q2, d2 = oi.quantize((k * scale).astype(np.float32))
        assert np.all(d2 == np.float32(scale)) and np.array_equal(q2, q)
    q16, d16 = oi.quantize(k.astype(np.float16))
    assert np.array_equal(q16, q) and np.all(d16 == 1.0)


def test_halfway_quotients_round_to_even():
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = 127.0          # d = 1
    x[0, 1:7] = [2.5, 3.5, -2.5, -3.5, 0.5, -0.5]
    q, d = oi.quantize(x)
    assert d[0, 0] == 1.0
    assert list(q[0, :7]) == [127, 2, 4, -2, -4, 0, 0]


def test_zero_block():
    x = np.zeros((2, 64), dtype=np.float32)
    x[1, 32:] = 1.0
    q, d = oi.quantize(x)
    assert d[0, 0] == 0 and d[0, 1] == 0 and d[1, 0] == 0
    assert np.all(q[0] == 0) and np.all(q[1, :32] == 0)
    assert np.all(q[1, 32:] == 127)
    assert np.all(oi.rebuilt(x)[0] == 0)


def test_amax_maps_to_127_and_rebuilt_error_is_bounded():
    g = np.random.default_rng(4)
    X = (g.normal(size=(5, 4096)) * np.exp(g.normal(size=(5, 1)) * 3)).astype(np.float32)
    q, d = oi.quantize(X)
    qb = np.abs(q.reshape(5, -1, 32).astype(np.int32))
    assert np.all(qb.max(axis=2) == 127)
    err = np.abs(oi.rebuilt(X) - X.astype(np.float64))
    lim = np.repeat(d.astype(np.float64) / 2 * (1 + 2.0 ** -16), 32, axis=1)
    assert np.all(err <= lim)


def _f16(lo, hi):
    return float(np.frombuffer(bytes([lo, hi]), dtype=np.float16)[0])


def test_product_brute_forced_from_q8_0_bytes():
    """y[t][n] = sum_b d_w d_x sum_i code_i q_i, with d_w read from the block's
    first two bytes and the codes as signed bytes, by hand."""
    N, K, M = 3, 96, 2
    g = wl.rng("oracle_int8", "brute")
    W = wl.random_weights("Q8_0", N, K, g).reshape(N, -1)
    X = wl.activations((M, K), np.float32, g)
    q, d = oi.quantize(X)
    want = np.zeros((M, N))
    for t in range(M):
        for n in range(N):
            acc = 0.0
            for b in range(K // 32):
                blk = W[n, 34 * b:34 * b + 34]
                dw = _f16(int(blk[0]), int(blk[1]))
                codes = [int(np.int8(np.uint8(v))) for v in blk[2:]]
                isum = sum(c * int(q[t, 32 * b + i]) for i, c in enumerate(codes))
                acc += dw * float(d[t, b]) * isum
            want[t, n] = acc
    got, _ = oi.matmul_quantized("Q8_0", W, K, X)
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=0)


@pytest.mark.parametrize("kind", ["Q8_0", "Q4_0"])
def test_quantization_bound_covers_the_difference(kind):
    N, K, M = 40, 1024, 4
    g = wl.rng("oracle_int8", kind)
    W = wl.random_weights(kind, N, K, g)
    X = wl.activations((M, K), np.float32, g)
    yq, _ = oi.matmul_quantized(kind, W, K, X)
    y, B = oracle.matmul(kind, W, K, X)
    qb = oi.quantization_bound(kind, W, K, X)
    assert np.all(np.abs(yq - y) <= qb)
    # The bound is a real constraint, not a vacuous one: it is a small
    # fraction of sum |w||x| (about 1/254 of a block maximum per element).
    assert np.all(qb < 0.02 * B)
