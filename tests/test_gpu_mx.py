"""GPU parity of the scaled FP8 x FP4 matrix-core GEMM for MXFP4 weights
(qmm_gemm_mx) against the oracle.

The variant splits each activation into two MX FP8 terms (oracle/mx.py:
a power-of-two scale per 32-element block, E4M3 elements, then the same for
the residual), so it has a bar of its own and a tighter one:

* the quantized workspace bit for bit against oracle/mx.py (codes in the
  MXFP4 nibble order, both scale planes, zero padding rows);
* random normal activations: |C - C_ref| <= 2e-2 * sum|w||a| + 1e-6 against
  the oracle's exact binary64 product, and the f32-accumulation bar
  1e-3 * sum|w||a'| + 1e-6 against the exact product of the weights with
  the rebuilt activations a' = 2^e1 hi + 2^e2 lo;
* a block of 1.0625s (which a single E4M3 term would round 5.9 % low) times
  weights of one sign;
* activations that MX FP8 holds exactly (integers of magnitude <= 16, and
  one-hot rows): the f32-accumulation bar of the other paths, and for
  one-hot rows the f32 weight itself;
* K not a multiple of 128 takes the f16 GEMM, at that path's bar.
"""
import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gguf_block_quantized_kind_amd as qmm  # noqa: E402

from test_gpu_parity import SENTINEL, assert_within_bound, dev, filled, host, _sample_rows  # noqa: E402
from oracle import mx  # noqa: E402

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


# Position p of a stored 32-element block holds element NIBBLE_ORDER[p].
NIBBLE_ORDER = np.array([(p >> 1) + (16 if p & 1 else 0) for p in range(32)])


def workspace_planes(ws, M, K):
    """(hi, lo, s1, s2) of the first M rows of a quantized workspace, codes
    put back in element order, and the padding rows' four planes."""
    Mp = (M + 63) // 64 * 64
    nb = K // 32
    b = ws.cpu().numpy()
    hi = b[:Mp * K].reshape(Mp, nb, 32)
    lo = b[Mp * K:2 * Mp * K].reshape(Mp, nb, 32)
    s1 = b[2 * Mp * K:2 * Mp * K + Mp * nb].reshape(Mp, nb)
    s2 = b[2 * Mp * K + Mp * nb:2 * Mp * K + 2 * Mp * nb].reshape(Mp, nb)
    inv = np.argsort(NIBBLE_ORDER)
    unperm = lambda c: c[:M][:, :, inv].reshape(M, K)  # noqa: E731
    pad = (hi[M:], lo[M:], s1[M:], s2[M:])
    return (unperm(hi), unperm(lo), s1[:M], s2[:M]), pad


@pytest.mark.parametrize("xdt", ["f16", "f32"])
@pytest.mark.parametrize("dist", ["normal", "wide", "sparse"])
def test_gemm_mx_workspace_matches_the_oracle_quantizer(xdt, dist):
    """The two-term MX FP8 codes and scale bytes bit for bit: normal
    activations, magnitudes spread over 2^+-12 (2^+-8 for f16), and blocks
    that are mostly zeros, -0.0 and exact E4M3 values.  M = 70 leaves 58
    padding rows, which must hold zero codes and scale byte 0."""
    M, N, K = 70, 64, 512
    g = wl.rng("gpu_mx_ws", f"{xdt}_{dist}")
    dt = np.float16 if xdt == "f16" else np.float32
    X = g.standard_normal((M, K))
    if dist == "wide":
        X = X * np.exp2(g.integers(-8 if xdt == "f16" else -12, 9 if xdt == "f16" else 13, (M, K // 32, 1))
                        ).repeat(32, axis=2).reshape(M, K)
    elif dist == "sparse":
        X = np.where(g.random((M, K)) < 0.7, 0.0, X)
        X[:, ::7] = -0.0
        X[:, 3::32] = 448.0 * 2.0 ** -6
    X = X.astype(dt)
    W = wl.random_weights(KIND, N, K, g)
    ws = torch.full((qmm.qmm_gemm_mx_workspace_bytes(M, K),), 0xA5, dtype=torch.uint8, device="cuda")
    run(W, X, N, ws)
    (hi, lo, s1, s2), pad = workspace_planes(ws, M, K)
    want = mx.quantize(X)
    for name, a, b in zip(("hi", "lo", "s1", "s2"), (hi, lo, s1, s2), want):
        bad = np.argwhere(a != b)
        assert bad.size == 0, f"{name}: {len(bad)} bytes differ, first at {bad[0]}: {a[tuple(bad[0])]:#x} vs {b[tuple(bad[0])]:#x}"
    for plane in pad:
        assert not np.any(plane)


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
    # Against the exact product with the rebuilt activations: f32 accumulation only.
    Wd = oracle_mod.dequant(KIND, W).reshape(N, K)
    Yr, Br = mx.matmul_rebuilt(Wd, X)
    assert_within_bound(got, Yr, Br, f"rebuilt M={M} {xdt}")


@pytest.mark.parametrize("xdt", ["f16", "f32"])
def test_gemm_mx_block_of_1p0625(oracle_mod, xdt):
    """Every activation 1.0625 and every weight code non-negative: one E4M3
    term would give 1.0 (the tie 272 -> 256), 5.9 % low on every output; the
    second term carries the 0.0625 and the product is exact up to f32
    accumulation."""
    M, N, K = 64, 128, 1024
    g = wl.rng("gpu_mx_1p0625", xdt)
    W = wl.random_weights(KIND, N, K, g).reshape(N, K // 32, 17).copy()
    W[:, :, 1:] &= 0x77                                     # codes 0..7: magnitudes >= 0
    W = W.reshape(-1)
    X = np.full((M, K), 1.0625, dtype=np.float16 if xdt == "f16" else np.float32)
    got = run(W, X, N)
    Y, B = oracle_mod.matmul(KIND, W, K, X)
    assert_within_bound(got, Y, B, f"1.0625 {xdt}")


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
