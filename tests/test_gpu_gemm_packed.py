"""GPU parity of the matmul over repacked weights (qmm_matmul_packed): the
prefill GEMM for M > 8, the packed GEMV below.

* random activations: |C - C_ref| <= 1e-3 * sum|w||a| + 1e-6 against the
  oracle's exact product over the NATIVE weights, for f16 and f32
  activations, token counts that span one to three 64-token tiles with a
  ragged tail, row counts that leave a partial 16-row tile and a partial
  128-row tile, and k-block counts that split unevenly over the four waves
  (5 k-blocks) or leave waves without work (1 k-block);
* one-hot rows: each output is the weight rounded once to f16, exactly (the
  f32 weight itself for IQ4_XS, whose group scales apply after the product);
* the same call twice gives the same bits (fixed summation order);
* the 512 x 4096 x 4096 prefill workload on sampled rows;
* grids whose 64 x 128 tiles would take more than one round of the compute
  units (64 x 192 tiles then): a ragged 200 x 9990 x 512 case on every row,
  twice for identical bits, and the 256 x 11008 x 4096 workload on sampled
  rows.
"""
import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gguf_block_quantized_kind_amd as qmm  # noqa: E402

from test_gpu_parity import SENTINEL, assert_within_bound, dev, filled, host, _sample_rows  # noqa: E402

KINDS = ["Q8_0", "Q4_0", "Q5_0", "IQ4_NL", "MXFP4", "IQ4_XS"]
# Kinds whose group scale multiplies each step's product in f32 (no weight
# rounding): a unit vector returns the f32 weight itself.
POST_SCALED = {"IQ4_XS"}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qmm.load_library()


def packed(kind, W, N, K):
    P = torch.full((qmm.qmm_packed_bytes(kind, N, K),), 0xA5, dtype=torch.uint8, device="cuda")
    qmm.qmm_repack(kind, dev(W), P, N, K)
    return P


def matmul(kind, P, X, N):
    M, K = X.shape
    C = filled((M, N))
    qmm.qmm_matmul_packed(kind, P, X if torch.is_tensor(X) else dev(X), C, M, N, K)
    return host(C)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("xdt", ["f16", "f32"])
@pytest.mark.parametrize("N,K", [(200, 1280), (300, 256), (16, 768)])
def test_matmul_packed_parity(oracle_mod, kind, xdt, N, K):
    g = wl.rng("gpu_gemm_packed", f"{kind}_{xdt}_{N}_{K}")
    W = wl.random_weights(kind, N, K, g)
    P = packed(kind, W, N, K)
    dt = np.float16 if xdt == "f16" else np.float32
    for M in (5, 9, 64, 130):
        X = wl.activations((M, K), dt, g)
        got = matmul(kind, P, X, N)
        Y, B = oracle_mod.matmul(kind, W, K, X)
        assert_within_bound(got, Y, B, f"{kind} M={M} N={N} K={K} {xdt}")


@pytest.mark.parametrize("kind", KINDS)
def test_matmul_packed_unit_vectors_return_f16_weights(oracle_mod, kind):
    N, K = 150, 1024
    # Stress scales, kept within the f16 range the GEMM's weights live in
    # (MXFP4: E8M0 exponents 100 .. 140, i.e. |w| <= 6 * 2^13).
    g = wl.rng("gpu_gemm_packed_unit", kind)
    W = (wl.random_weights(kind, N, K, g, e8m0_range=(100, 140)) if kind == "MXFP4"
         else wl.random_weights(kind, N, K, g, scales="stress"))
    want = oracle_mod.dequant(kind, W).reshape(N, K).astype(np.float32)
    if kind not in POST_SCALED:
        want = want.astype(np.float16).astype(np.float32)
    ks = [0, 1, 7, 8, 31, 32, 255, 256, 511, 600, K - 1] + list(range(100, 121))
    X = np.zeros((len(ks), K), dtype=np.float16)
    for i, k in enumerate(ks):
        X[i, k] = 1.0
    got = matmul(kind, packed(kind, W, N, K), X, N)
    for i, k in enumerate(ks):
        assert np.array_equal(got[i], want[:, k]), f"{kind} column {k}"


@pytest.mark.parametrize("kind", KINDS)
def test_matmul_packed_is_deterministic(kind):
    M, N, K = 200, 260, 2048
    g = wl.rng("gpu_gemm_packed_det", kind)
    P = packed(kind, wl.random_weights(kind, N, K, g), N, K)
    X = dev(wl.activations((M, K), np.float16, g))
    a, b = matmul(kind, P, X, N), matmul(kind, P, X, N)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("w", [w for w in wl.C3 if w.kind in KINDS], ids=lambda w: w.name)
def test_matmul_packed_full_size_sampled(oracle_mod, w):
    W = w.weights()
    P = packed(w.kind, W, w.N, w.K)
    X = w.x()
    got = matmul(w.kind, P, X, w.N)
    assert not np.any(got == SENTINEL)
    rows = _sample_rows(w.N, wl.rng(w.name, "sample_packed"))
    Y, B = oracle_mod.matmul(w.kind, W, w.K, X, rows=rows)
    assert_within_bound(got[:, rows], Y, B, w.name)


def _wide_grid(M, N):
    """True when the call takes the 64 x 192 tiles (the 64 x 128 grid would
    need more than one round of the compute units, the 64 x 192 grid one)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tm = (M + 63) // 64
    return tm * ((N + 127) // 128) > cus and tm * ((N + 191) // 192) <= cus


@pytest.mark.parametrize("kind", KINDS)
def test_matmul_packed_wide_grid_ragged(oracle_mod, kind):
    M, N, K = 200, 9990, 512
    assert _wide_grid(M, N)
    g = wl.rng("gpu_gemm_packed_wide", kind)
    W = wl.random_weights(kind, N, K, g)
    P = packed(kind, W, N, K)
    X = dev(wl.activations((M, K), np.float16, g))
    a, b = matmul(kind, P, X, N), matmul(kind, P, X, N)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    Y, B = oracle_mod.matmul(kind, W, K, host(X))
    assert_within_bound(a, Y, B, f"{kind} {M}x{N}x{K}")


@pytest.mark.parametrize("w", [w for w in wl.C4 if w.M > 8 and w.kind in KINDS], ids=lambda w: w.name)
def test_matmul_packed_wide_grid_workload_sampled(oracle_mod, w):
    assert _wide_grid(w.M, w.N)
    W = w.weights()
    P = packed(w.kind, W, w.N, w.K)
    X = w.x()
    got = matmul(w.kind, P, X, w.N)
    assert not np.any(got == SENTINEL)
    rows = _sample_rows(w.N, wl.rng(w.name, "sample_packed"))
    Y, B = oracle_mod.matmul(w.kind, W, w.K, X, rows=rows)
    assert_within_bound(got[:, rows], Y, B, w.name)
