"""GPU parity of the int8-activation GEMV (qmm_gemv_i8) against the oracle.

The activation quantization decides integers from f32 arithmetic; the kernel
and the oracle take those decisions in the same precision, so:

* the workspace's codes, scales and code sums equal the oracle's quantization
  bit for bit (codes compared after the documented lane-order permutation);
* y is held to f32 accumulation against the oracle's exact product with the
  rebuilt activations: |y - y_q| <= 2e-5 * sum |w| |d q| + 1e-6;
* and to the variant's own bar against the exact product with x itself:
  |y - y| <= quantization bound + 2e-5 * sum |w| |x| + 1e-6.
"""
import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gguf_block_quantized_kind_amd as qmm  # noqa: E402
from oracle import int8 as oi  # noqa: E402

from test_gpu_parity import SENTINEL, assert_within_bound, dev, filled, host, _sample_rows  # noqa: E402

KINDS = ["Q8_0", "Q4_0", "Q5_0", "IQ4_NL", "MXFP4"]
RTOL = 2e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qmm.load_library()


def lane_order(kind):
    """Element held at block position 8G + e (Q5_0, IQ4_NL and MXFP4 share
    Q4_0's nibble order)."""
    if kind == "Q8_0":
        return np.arange(32)
    return np.array([4 * G + e if e < 4 else 16 + 4 * G + e - 4 for G in range(4) for e in range(8)])


def run(kind, W, X, N, ws=None):
    M, K = X.shape
    Wd = W if torch.is_tensor(W) else dev(W)
    P = qmm.repack(kind, Wd, N, K)
    if ws is None:
        ws = torch.empty(qmm.qmm_gemv_i8_workspace_bytes(M, K), dtype=torch.uint8, device="cuda")
    y = filled((M, N))
    qmm.qmm_gemv_i8(kind, P, dev(X), y, M, N, K, ws)
    return host(y), ws


def read_workspace(ws, M, K):
    raw = host(ws)
    a256 = lambda v: (v + 255) // 256 * 256
    q = raw[:M * K].view(np.int8).reshape(M, K)
    d0 = a256(M * K)
    d = raw[d0:d0 + M * K // 8].view(np.float32).reshape(M, K // 32)
    s0 = d0 + a256(M * K // 8)
    s = raw[s0:s0 + M * K // 8].view(np.int32).reshape(M, K // 32)
    return q, d, s


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("xdt", ["f32", "f16"])
def test_quantized_activations_equal_the_oracle_bit_for_bit(kind, xdt):
    M, N, K = 5, 32, 1024
    g = wl.rng("gpu_i8_quant", f"{kind}_{xdt}")
    X = (g.normal(size=(M, K)) * np.exp(g.normal(size=(M, K // 32)) * 2).repeat(32, axis=1))
    X = X.astype(np.float16 if xdt == "f16" else np.float32)
    X[0, :32] = 0                              # an all-zero block
    X[1, :32] = 0
    X[1, 0] = 127                              # d = 1: exact halfway quotients
    X[1, 1:7] = [2.5, 3.5, -2.5, -3.5, 0.5, -0.5]
    W = wl.random_weights(kind, N, K, g)
    run(kind, W, X, N)
    _, ws = run(kind, W, X, N)
    q, d, s = read_workspace(ws, M, K)
    wq, wd = oi.quantize(X)
    perm = lane_order(kind)
    wq_lane = wq.reshape(M, K // 32, 32)[:, :, perm].reshape(M, K)
    assert np.array_equal(d.view(np.uint32), wd.view(np.uint32))
    assert np.array_equal(q, wq_lane)
    assert np.array_equal(s, wq.reshape(M, K // 32, 32).astype(np.int32).sum(axis=2))
    assert list(q[1, :1]) == [127] and d[1, 0] == 1.0


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("xdt", ["f32", "f16"])
def test_gemv_i8_parity(oracle_mod, kind, xdt):
    """N = 130 (a ragged tile), K = 1280 (five k-blocks over four waves),
    M = 1 .. 8."""
    N, K = 130, 1280
    g = wl.rng("gpu_i8", f"{kind}_{xdt}")
    W = wl.random_weights(kind, N, K, g)
    for M in (1, 2, 3, 7, 8):
        X = wl.activations((M, K), np.float16 if xdt == "f16" else np.float32, g)
        got, _ = run(kind, W, X, N)
        yq, Bq = oi.matmul_quantized(kind, W, K, X)
        assert_within_bound(got, yq, Bq, f"{kind} M={M} {xdt} vs rebuilt", rtol=RTOL)
        y, B = oracle_mod.matmul(kind, W, K, X)
        qb = oi.quantization_bound(kind, W, K, X)
        ratio = np.abs(got - y) / (qb + RTOL * B + 1e-6)
        assert ratio.max() <= 1.0, f"{kind} M={M}: {ratio.max()}"


@pytest.mark.parametrize("kind", KINDS)
def test_gemv_i8_integer_activations_are_exact(oracle_mod, kind):
    """Blocks of integers whose largest magnitude is 127 quantize to
    themselves, so the product is the exact one, up to f32 accumulation."""
    N, K, M = 48, 512, 4
    g = wl.rng("gpu_i8_int", kind)
    W = wl.random_weights(kind, N, K, g)
    X = g.integers(-127, 128, size=(M, K)).astype(np.float32)
    X[:, ::32] = 127
    got, _ = run(kind, W, X, N)
    y, B = oracle_mod.matmul(kind, W, K, X)
    assert_within_bound(got, y, B, kind, rtol=RTOL)


def test_gemv_i8_workspace_reuse_and_edges(oracle_mod):
    kind = "Q4_0"
    g = wl.rng("gpu_i8_edge", "x")
    N, K = 40, 768
    W = wl.random_weights(kind, N, K, g)
    X8 = wl.activations((8, K), np.float32, g)
    first, ws = run(kind, W, X8, N)
    one, _ = run(kind, W, X8[:1].copy(), N, ws)
    again, _ = run(kind, W, X8, N, ws)
    assert np.array_equal(first.view(np.uint32), again.view(np.uint32))
    assert np.array_equal(one[0].view(np.uint32), first[0].view(np.uint32))
    for N1, K1 in ((1, 256), (17, 256), (16, 2048)):
        W1 = wl.random_weights(kind, N1, K1, g)
        X1 = wl.activations((3, K1), np.float32, g)
        got, _ = run(kind, W1, X1, N1)
        yq, Bq = oi.matmul_quantized(kind, W1, K1, X1)
        assert_within_bound(got, yq, Bq, f"N={N1} K={K1}", rtol=RTOL)


@pytest.mark.parametrize("kind,M", [("Q4_0", 1), ("Q8_0", 8)])
def test_gemv_i8_full_size_sampled(oracle_mod, kind, M):
    """4096 x 4096 weights (the Q4_0 decode workload's shape)."""
    N = K = 4096
    g = wl.rng("gpu_i8_full", f"{kind}_{M}")
    W = wl.random_weights(kind, N, K, g)
    X = wl.activations((M, K), np.float32, g)
    got, _ = run(kind, W, X, N)
    assert not np.any(got == SENTINEL)
    rows = _sample_rows(N, g)
    yq, Bq = oi.matmul_quantized(kind, W, K, X, rows=rows)
    assert_within_bound(got[:, rows], yq, Bq, f"{kind} M={M}", rtol=RTOL)


def test_gemv_i8_largest_staged_shape(oracle_mod):
    """M * K at its limit (8 tokens x 32768: 64 KiB of staged scales and
    code sums per workgroup), on sampled rows."""
    kind, M, N, K = "Q8_0", 8, 48, 32768
    g = wl.rng("gpu_i8_max", "x")
    W = wl.random_weights(kind, N, K, g)
    X = wl.activations((M, K), np.float16, g)
    got, _ = run(kind, W, X, N)
    yq, Bq = oi.matmul_quantized(kind, W, K, X)
    assert_within_bound(got, yq, Bq, "M*K = 262144", rtol=RTOL)
