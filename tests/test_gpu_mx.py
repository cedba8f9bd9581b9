"""GPU parity of the scaled FP8 x FP4 matrix-core GEMM for MXFP4 weights
(qmm_gemm_mx) against the oracle.

The variant rounds each activation once, to MX FP8 (a power-of-two scale per
32-element block, elements to E4M3), so it has a bar of its own:

* random normal activations: |C - C_ref| <= 2e-2 * sum|w||a| + 1e-6 against
  the oracle's exact binary64 product;
* activations that MX FP8 holds exactly (integers of magnitude <= 16, and
  one-hot rows): the f32-accumulation bar of the other paths,
  1e-3 * sum|w||a| + 1e-6, and for one-hot rows the f32 weight itself;
* K not a multiple of 128 takes the f16 GEMM, at that path's bar.
"""
import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gguf_block_quantized_kind_amd as qmm  # noqa: E402

from test_gpu_parity import SENTINEL, assert_within_bound, dev, filled, host, _sample_rows  # noqa: E402

KIND = "MXFP4"
MX_RTOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qmm.load_library()


def run(W, X, N, ws=None):
    M, K = X.shape
    C = filled((M, N))
    if ws is None:
        ws = torch.empty(qmm.qmm_gemm_mx_workspace_bytes(M, K), dtype=torch.uint8, device="cuda")
    qmm.qmm_gemm_mx(KIND, W if torch.is_tensor(W) else dev(W), dev(X), C, M, N, K, ws)
    return host(C)


@pytest.mark.parametrize("K", [1280, 2048])
@pytest.mark.parametrize("scales", ["config", "stress"])
@pytest.mark.parametrize("xdt", ["f16", "f32"])
def test_gemm_mx_unit_vectors_return_the_weights(oracle_mod, xdt, scales, K):
    """A one-hot row quantizes exactly (scale 2^-8, code 256), so each output
    is one weight times one, exactly.  K = 1280 is ten 128-k steps with rows
    of 680 bytes (the general path: two full turns of the unrolled loop and a
    ragged tail); K = 2048 has rows of 1088 bytes, a multiple of 16, and takes
    the aligned path for its first groups.  N = 300 leaves a partial 256-row
    tile."""
    N = 300
    W = wl.random_weights(KIND, N, K, wl.rng("gpu_mx_unit", f"{xdt}_{scales}"), scales=scales)
    want = oracle_mod.dequant(KIND, W).reshape(N, K).astype(np.float32)
    ks = [0, 1, 16, 17, 31, 127, 128, K // 3, K - 2, K - 1]
    X = np.zeros((len(ks), K), dtype=np.float16 if xdt == "f16" else np.float32)
    for i, k in enumerate(ks):
        X[i, k] = 1.0
    got = run(W, X, N)
    for i, k in enumerate(ks):
        assert np.array_equal(got[i], want[:, k]), f"column {k}: got {got[i][:4]} want {want[:4, k]}"


@pytest.mark.parametrize("xdt", ["f16", "f32"])
@pytest.mark.parametrize("K", [512, 1280, 2048, 2560])
def test_gemm_mx_exact_activations(oracle_mod, K, xdt):
    """Integers in [-16, 16] pass the MX FP8 quantization unchanged, so the
    result is the exact product up to f32 accumulation.  M spans one, two and
    three 64-token tiles (ragged), N two 256-row tiles (ragged).  K = 512 and
    1280 take the general path only; 2048 and 2560 (rows a multiple of 16
    bytes) run aligned groups, then the general path for the last steps."""
    N = 300
    g = wl.rng("gpu_mx_exact", f"{K}_{xdt}")
    W = wl.random_weights(KIND, N, K, g)
    Wd = dev(W)
    for M in (1, 64, 130):
        X = g.integers(-16, 17, size=(M, K)).astype(np.float16 if xdt == "f16" else np.float32)
        got = run(Wd, X, N)
        Y, B = oracle_mod.matmul(KIND, W, K, X)
        assert_within_bound(got, Y, B, f"M={M} K={K} {xdt}")


@pytest.mark.parametrize("xdt", ["f16", "f32"])
def test_gemm_mx_parity_random(oracle_mod, xdt):
    M, N, K = 130, 600, 1280
    g = wl.rng("gpu_mx_random", xdt)
    W = wl.random_weights(KIND, N, K, g)
    X = wl.activations((M, K), np.float16 if xdt == "f16" else np.float32, g)
    got = run(W, X, N)
    Y, B = oracle_mod.matmul(KIND, W, K, X)
    ratio = assert_within_bound(got, Y, B, f"M={M} {xdt}", rtol=MX_RTOL)
    print(f"worst error / bar: {ratio:.3g}")


def test_gemm_mx_workspace_reuse_and_determinism(oracle_mod):
    """One workspace for a 130-token call, then a 1-token call (its padding
    rows must be re-zeroed), then the 130-token call again, bit for bit."""
    N, K = 260, 512
    g = wl.rng("gpu_mx_reuse", "x")
    W = wl.random_weights(KIND, N, K, g)
    Wd = dev(W)
    ws = torch.empty(qmm.qmm_gemm_mx_workspace_bytes(130, K), dtype=torch.uint8, device="cuda")
    X = wl.activations((130, K), np.float16, g)
    first = run(Wd, X, N, ws)
    one = run(Wd, X[:1].copy(), N, ws)
    again = run(Wd, X, N, ws)
    assert np.array_equal(first.view(np.uint32), again.view(np.uint32))
    assert np.array_equal(one[0].view(np.uint32), first[0].view(np.uint32))
    Y, B = oracle_mod.matmul(KIND, W, K, X)
    assert_within_bound(first, Y, B, "M=130", rtol=MX_RTOL)


def test_gemm_mx_k_not_multiple_of_128_takes_the_f16_gemm(oracle_mod):
    M, N, K = 70, 130, 1312
    g = wl.rng("gpu_mx_fallback", "x")
    W = wl.random_weights(KIND, N, K, g)
    X = wl.activations((M, K), np.float16, g)
    got = run(W, X, N)
    Y, B = oracle_mod.matmul(KIND, W, K, X)
    assert_within_bound(got, Y, B, "K=1312")


def test_gemm_mx_full_size_sampled(oracle_mod):
    """The MXFP4 prefill workload (256 tokens, 11008 x 4096) on sampled rows."""
    w = next(x for x in wl.C4 if x.kind == KIND and x.M > 8)
    W = w.weights()
    X = w.x()
    got = run(W, X, w.N)
    assert not np.any(got == SENTINEL)
    rows = _sample_rows(w.N, wl.rng(w.name, "sample_mx"))
    Y, B = oracle_mod.matmul(KIND, W, w.K, X, rows=rows)
    ratio = assert_within_bound(got[:, rows], Y, B, w.name, rtol=MX_RTOL)
    print(f"worst error / bar: {ratio:.3g}")


def test_gemm_mx_large_grid(oracle_mod):
    """512 tokens x 7680 rows: 320 workgroups of 64 x 192, more than one per
    compute unit.  Small-integer activations pass the MX FP8 quantization
    exactly: the 1e-3 bar applies."""
    M, N, K = 512, 7680, 512
    g = wl.rng("gpu_mx_tall", "x")
    W = wl.random_weights(KIND, N, K, g)
    X = g.integers(-16, 17, size=(M, K)).astype(np.float16)
    got = run(W, X, N)
    rows = _sample_rows(N, g, n=120)
    Y, B = oracle_mod.matmul(KIND, W, K, X, rows=rows)
    assert not np.any(got == SENTINEL)
    assert_within_bound(got[:, rows], Y, B, "M=512 N=7680")


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (65, 17, 128), (3, 129, 384), (64, 193, 2048)])
def test_gemm_mx_edge_shapes(oracle_mod, M, N, K):
    """One 128-k step, a single weight row, ragged token and row tiles, and
    a K of whole aligned groups with fewer steps than the aligned path needs
    ahead: small-integer activations, so the 1e-3 bar applies."""
    g = wl.rng("gpu_mx_edge", f"{M}_{N}_{K}")
    W = wl.random_weights(KIND, N, K, g)
    X = g.integers(-16, 17, size=(M, K)).astype(np.float32)
    got = run(W, X, N)
    Y, B = oracle_mod.matmul(KIND, W, K, X)
    assert_within_bound(got, Y, B, f"M={M} N={N} K={K}")
