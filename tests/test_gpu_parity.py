"""GPU parity: the HIP path through the C ABI against the oracle, on the same
seeded inputs.

* dequant: bit for bit (NaN only against NaN, -0.0 only against -0.0);
* GEMV / GEMM / experts: |y - y_ref| <= 1e-3 * sum|w||x| + 1e-6 per element,
  with y_ref and the bound from the oracle in binary64;
* unit-vector activations: the GEMV returns the f32 weight itself, the GEMM
  its f16 rounding;
* outputs are prefilled with a sentinel that must be gone afterwards;
* full workload sizes are checked on sampled rows.
"""
import json
import os

import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gguf_block_quantized_kind_amd as qmm  # noqa: E402

ALL_KINDS = list(wl.KINDS)
SENTINEL = -1.0e30
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_blocks.json")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qmm.load_library()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def filled(shape):
    shape = (shape,) if isinstance(shape, int) else tuple(shape)
    return torch.full(shape, SENTINEL, dtype=torch.float32, device="cuda")


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_within_bound(y, y_ref, bound, what, rtol=1e-3, atol=1e-6):
    y = np.asarray(y, dtype=np.float64)
    assert not np.any(y == SENTINEL), f"{what}: outputs left untouched"
    assert np.all(np.isfinite(y)), f"{what}: non-finite outputs"
    err = np.abs(y - y_ref)
    lim = rtol * bound + atol
    ratio = err / lim
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert ratio.max() <= 1.0, (f"{what}: worst |err|/(rtol*bound+atol) = {ratio.max():.3g} at {worst}: "
                                f"got {y[worst]!r} want {y_ref[worst]!r} bound {bound[worst]!r}")
    return float(ratio.max())


def same_bits_f32(got, want64):
    got = np.asarray(got, dtype=np.float32)
    want = np.asarray(want64, dtype=np.float64).astype(np.float32)
    nan = np.isnan(want)
    ok = np.where(nan, np.isnan(got), got.view(np.uint32) == want.view(np.uint32))
    return ok


def small_K(kind):
    _, be = wl.geometry(kind)
    return 1280 if be == 256 else 1312   # 80 / 82 sub-blocks of 16: two passes of 64 lanes, ragged


# ---------------------------------------------------------------------------
# dequant
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("scales", ["config", "stress"])
@pytest.mark.parametrize("kind", ALL_KINDS)
def test_dequant_bit_exact(oracle_mod, kind, scales):
    bb, be = wl.geometry(kind)
    W = wl.random_weights(kind, 1, 1003 * be, wl.rng("gpu_dequant", f"{kind}_{scales}"), scales=scales)
    out = filled(1003 * be)
    qmm.qmm_dequant(kind, dev(W), out, 1003 * be)
    got = host(out)
    ok = same_bits_f32(got, oracle_mod.dequant(kind, W))
    bad = np.nonzero(~ok)[0]
    assert bad.size == 0, f"{kind}: {bad.size} mismatches, first at {bad[:5]}"


def test_dequant_hand_blocks():
    with open(GOLDEN) as f:
        blocks = json.load(f)["blocks"]
    for blk in blocks:
        raw = np.full(blk["len"], blk["fill"], dtype=np.uint8)
        for off, val in blk["set"].items():
            raw[int(off)] = val
        _, be = wl.geometry(blk["kind"])
        want = np.full(be, np.nan)
        for s, e, v in blk["runs"]:
            want[s:e] = v
        for i, v in blk["points"].items():
            want[int(i)] = v
        out = filled(be)
        qmm.qmm_dequant(blk["kind"], dev(raw), out, be)
        got = host(out)
        assert np.all(same_bits_f32(got, want)), blk["name"]


def test_dequant_f16_and_e8m0_sweeps():
    pats = np.arange(65536, dtype=np.uint32)
    q8 = np.zeros((65536, 34), dtype=np.uint8)
    q8[:, 0], q8[:, 1], q8[:, 2] = pats & 0xFF, pats >> 8, 1
    out = filled(65536 * 32)
    qmm.qmm_dequant("Q8_0", dev(q8), out, 65536 * 32)
    got = host(out).reshape(65536, 32)[:, 0]
    want = pats.astype(np.uint16).view(np.float16).astype(np.float32)
    assert np.all(np.where(np.isnan(want), np.isnan(got), got.view(np.uint32) == want.view(np.uint32)))
    mx = np.zeros((256, 17), dtype=np.uint8)
    mx[:, 0], mx[:, 1] = np.arange(256), 2
    out = filled(256 * 32)
    qmm.qmm_dequant("MXFP4", dev(mx), out, 256 * 32)
    got = host(out).reshape(256, 32)[:, 0]
    for e in range(255):
        assert got[e] == np.float32(np.ldexp(1.0, e - 127)), e
    assert np.isnan(got[255])


# ---------------------------------------------------------------------------
# GEMV
# ---------------------------------------------------------------------------
def gemv_Ks(kind):
    """K values that reach both GEMV paths: 1280 is a whole number of
    256-element k-blocks (the matrix-core path for every kind that has one);
    1312 is not, so the 32-element kinds take the f32 path there."""
    _, be = wl.geometry(kind)
    return (1280,) if be == 256 else (1280, 1312)


@pytest.mark.parametrize("xdt", ["f32", "f16"])
@pytest.mark.parametrize("kind", ALL_KINDS)
def test_gemv_parity(oracle_mod, kind, xdt):
    for K in gemv_Ks(kind):
        N = 130
        g = wl.rng("gpu_gemv", f"{kind}_{xdt}_{K}")
        W = wl.random_weights(kind, N, K, g)
        dt = np.float32 if xdt == "f32" else np.float16
        Wd = dev(W)
        for M in (1, 2, 3, 5, 8):
            X = wl.activations((M, K), dt, g)
            y = filled((M, N))
            qmm.qmm_gemv_ex(kind, Wd, dev(X), y, M, N, K)
            Y, B = oracle_mod.matmul(kind, W, K, X)
            assert_within_bound(host(y), Y, B, f"{kind} K={K} M={M} {xdt}")


@pytest.mark.parametrize("kind", ["Q2_K", "Q3_K", "Q4_K", "Q5_K", "Q6_K"])
def test_gemv_native_rows_more_tiles_than_units(oracle_mod, kind):
    """2 to 8 tokens over native rows at 4500 rows (282 tiles, the last one
    ragged): more tiles than compute units, so workgroups of one and two
    tiles and waves without a tile."""
    N, K = 4500, 768
    g = wl.rng("gpu_gemv_half_tiles", kind)
    W = wl.random_weights(kind, N, K, g)
    Wd = dev(W)
    for M, dt in ((2, np.float32), (5, np.float16), (8, np.float32)):
        X = wl.activations((M, K), dt, g)
        y = filled((M, N))
        qmm.qmm_gemv_ex(kind, Wd, dev(X), y, M, N, K)
        Y, B = oracle_mod.matmul(kind, W, K, X)
        assert_within_bound(host(y), Y, B, f"{kind} M={M} N={N} K={K}")


@pytest.mark.parametrize("kind,K", [(k, K) for k in ALL_KINDS for K in gemv_Ks(k)])
def test_gemv_unit_vectors_return_the_weights(oracle_mod, kind, K):
    N = 70
    W = wl.random_weights(kind, N, K, wl.rng("gpu_gemv_unit", kind), scales="stress")
    Wd = oracle_mod.dequant(kind, W).reshape(N, K).astype(np.float32)
    ks = [0, 1, 15, 16, 31, 32, K // 2 + 5, K - 1]
    X = np.zeros((len(ks), K), dtype=np.float32)
    for i, k in enumerate(ks):
        X[i, k] = 1.0
    y = filled((len(ks), N))
    qmm.qmm_gemv_ex(kind, dev(W), dev(X), y, len(ks), N, K)
    got = host(y)
    for i, k in enumerate(ks):
        assert np.array_equal(got[i], Wd[:, k]), f"{kind} column {k}"


def test_gemv_default_stream_entry_point(oracle_mod):
    N, K = 77, 4096
    g = wl.rng("gpu_gemv", "plain")
    W = wl.random_weights("Q4_0", N, K, g)
    x = wl.activations((K,), np.float32, g)
    y = filled((N,))
    qmm.qmm_gemv("Q4_0", dev(W), dev(x), y, N, K)
    Y, B = oracle_mod.matmul("Q4_0", W, K, x[None])
    assert_within_bound(host(y)[None], Y, B, "qmm_gemv")


# ---------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("xdt", ["f16", "f32"])
@pytest.mark.parametrize("kind", ALL_KINDS)
def test_gemm_parity(oracle_mod, kind, xdt):
    N, K = 200, small_K(kind)
    g = wl.rng("gpu_gemm", f"{kind}_{xdt}")
    W = wl.random_weights(kind, N, K, g)
    dt = np.float32 if xdt == "f32" else np.float16
    Wd = dev(W)
    for M in (1, 100, 130):
        X = wl.activations((M, K), dt, g)
        C = filled((M, N))
        qmm.qmm_gemm_ex(kind, Wd, dev(X), C, M, N, K)
        Y, B = oracle_mod.matmul(kind, W, K, X)
        assert_within_bound(host(C), Y, B, f"{kind} M={M} {xdt}")


@pytest.mark.parametrize("kind", ["Q8_0", "IQ4_NL", "MXFP4", "Q4_K"])
def test_gemm_large_grid_tiles(oracle_mod, kind):
    """A grid larger than one round of 128 x 64 tiles takes the eight-wave
    128 x 128 x 128 tiles; M, N and K are all ragged against them."""
    M, N = 300, 9000
    K = 1280 + (0 if wl.geometry(kind)[1] == 256 else 32)
    g = wl.rng("gpu_gemm_large", kind)
    W = wl.random_weights(kind, N, K, g)
    X = wl.activations((M, K), np.float16, g)
    C = filled((M, N))
    qmm.qmm_gemm_ex(kind, dev(W), dev(X), C, M, N, K)
    got = host(C)
    rows = _sample_rows(N, g, n=300)
    Y, B = oracle_mod.matmul(kind, W, K, X, rows=rows)
    assert not np.any(got == SENTINEL)
    assert_within_bound(got[:, rows], Y, B, f"{kind} M={M} N={N} K={K}")


@pytest.mark.parametrize("kind", ["Q8_0", "Q4_K"])
def test_gemm_large_grid_f32_activations(oracle_mod, kind):
    """f32 A on a grid past one round of 128 x 64 tiles: the large-tile
    shape with the activation split into two f16 planes."""
    M, N = 300, 9000
    K = 1280 if wl.geometry(kind)[1] == 256 else 1312
    g = wl.rng("gpu_gemm_large_f32", kind)
    W = wl.random_weights(kind, N, K, g)
    X = wl.activations((M, K), np.float32, g)
    C = filled((M, N))
    qmm.qmm_gemm_ex(kind, dev(W), dev(X), C, M, N, K)
    got = host(C)
    rows = _sample_rows(N, g, n=200)
    Y, B = oracle_mod.matmul(kind, W, K, X, rows=rows)
    assert not np.any(got == SENTINEL)
    assert_within_bound(got[:, rows], Y, B, f"{kind} f32 M={M} N={N} K={K}")


@pytest.mark.parametrize("kind", ALL_KINDS)
def test_gemm_unit_vectors_return_f16_weights(oracle_mod, kind):
    N, K = 130, small_K(kind)
    W = wl.random_weights(kind, N, K, wl.rng("gpu_gemm_unit", kind))
    want = oracle_mod.dequant(kind, W).reshape(N, K).astype(np.float32).astype(np.float16).astype(np.float32)
    ks = [0, 17, K // 3, K - 1]
    X = np.zeros((len(ks), K), dtype=np.float16)
    for i, k in enumerate(ks):
        X[i, k] = 1.0
    C = filled((len(ks), N))
    qmm.qmm_gemm_ex(kind, dev(W), dev(X), C, len(ks), N, K)
    got = host(C)
    for i, k in enumerate(ks):
        assert np.array_equal(got[i], want[:, k]), f"{kind} column {k}"


@pytest.mark.parametrize("kind", ALL_KINDS)
def test_matmul_edge_shapes(oracle_mod, kind):
    """Smallest shapes on every path: one block (and one 256-element
    k-block) of K, a single row and a ragged 17 rows, M from 1 to 65."""
    _, be = wl.geometry(kind)
    g = wl.rng("gpu_edge", kind)
    for K in sorted({be, 256}):
        for N in (1, 17):
            W = wl.random_weights(kind, N, K, g)
            Wd = dev(W)
            for M in (1, 8, 9, 65):
                X = wl.activations((M, K), np.float16, g)
                C = filled((M, N))
                qmm.qmm_matmul(kind, Wd, dev(X), C, M, N, K)
                Y, B = oracle_mod.matmul(kind, W, K, X)
                assert_within_bound(host(C), Y, B, f"{kind} K={K} N={N} M={M}")


def test_matmul_dispatch_and_determinism(oracle_mod):
    N, K = 300, 2048
    g = wl.rng("gpu_matmul", "dispatch")
    W = wl.random_weights("Q6_K", N, K, g)
    Wd = dev(W)
    for M in (8, 9):
        X = wl.activations((M, K), np.float16, g)
        Xd = dev(X)
        C1, C2 = filled((M, N)), filled((M, N))
        qmm.qmm_matmul("Q6_K", Wd, Xd, C1, M, N, K)
        qmm.qmm_matmul("Q6_K", Wd, Xd, C2, M, N, K)
        a, b = host(C1), host(C2)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "not run-to-run deterministic"
        Y, B = oracle_mod.matmul("Q6_K", W, K, X)
        assert_within_bound(a, Y, B, f"matmul M={M}")


# ---------------------------------------------------------------------------
# Routed experts
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("kind", ["Q4_K", "Q8_0", "MXFP4", "Q6_K", "IQ4_XS", "Q5_0", "Q5_K", "Q2_K", "Q3_K"])
def test_moe_parity(oracle_mod, kind):
    """The expert kernels on native rows: with whole 256-element k-blocks
    (K=1280) every kind takes a matrix-core form (M=40: items of 16 pairs;
    M=9: items of up to 8; M=2, 5: one pair per item -- the single-token and
    staged-activation kernels for the super-block kinds), and K=1312 (the
    32-element kinds only) the f32 one."""
    E, N, topk = 6, 130, 3
    for K in gemv_Ks(kind):
        for M in (5, 2, 9, 40):
            g = wl.rng("gpu_moe", f"{kind}_{K}_{M}")
            W = wl.random_weights(kind, E * N, K, g)
            ids = wl.routing(M, E, topk, g)
            ids[0] = [1, 2, 3]   # expert 1 is routed from two tokens
            ids[1] = [1, 4, 5]
            if M == 9:
                ids[:, 0] = 0    # expert 0 takes 9 pairs: two items of up to 8
            Wd, idd = dev(W), dev(ids)
            for per_slot, xdt in ((False, np.float16), (True, np.float32), (True, np.float16)):
                X = wl.activations((M, topk, K) if per_slot else (M, K), xdt, g)
                Y = filled((M, topk, N))
                nbytes = qmm.qmm_moe_workspace_bytes(E, M, topk)
                ws = torch.empty((nbytes + 3) // 4, dtype=torch.int32, device="cuda")
                qmm.qmm_moe(kind, Wd, E, idd, topk, dev(X), int(per_slot), Y, M, N, K, ws)
                Yr, Br = oracle_mod.moe(kind, W, E, N, K, ids, X, per_slot)
                assert_within_bound(host(Y), Yr, Br, f"{kind} K={K} M={M} moe per_slot={per_slot}")


# ---------------------------------------------------------------------------
# Full workload sizes, sampled rows
# ---------------------------------------------------------------------------
def _sample_rows(N, g, n=48):
    rows = np.unique(np.concatenate([[0, 1, N - 2, N - 1], g.choice(N, size=n, replace=False)]))
    return rows


@pytest.mark.parametrize("w", wl.C1 + wl.C2 + wl.C3 + wl.C4, ids=lambda w: w.name)
def test_workload_full_size_sampled(oracle_mod, w):
    W = w.weights()
    X = w.x()
    C = filled((w.M, w.N))
    qmm.qmm_matmul(w.kind, dev(W), dev(X), C, w.M, w.N, w.K)
    got = host(C)
    rows = _sample_rows(w.N, wl.rng(w.name, "sample"))
    Y, B = oracle_mod.matmul(w.kind, W, w.K, X, rows=rows)
    assert not np.any(got == SENTINEL)
    assert_within_bound(got[:, rows], Y, B, w.name)


@pytest.mark.parametrize("w", wl.C5, ids=lambda w: w.name)
def test_experts_full_size_sampled(oracle_mod, w):
    ids = w.ids()
    idd = dev(ids)
    for mat, N, K, X, per_slot in (("gu", w.N_gu, w.K_gu, w.x(), False), ("d", w.N_d, w.K_d, w.h(), True)):
        W = w.w_gu() if mat == "gu" else w.w_d()
        Y = filled((w.M, w.topk, N))
        nbytes = qmm.qmm_moe_workspace_bytes(w.E, w.M, w.topk)
        ws = torch.empty((nbytes + 3) // 4, dtype=torch.int32, device="cuda")
        qmm.qmm_moe(w.kind, dev(W), w.E, idd, w.topk, dev(X), int(per_slot), Y, w.M, N, K, ws)
        got = host(Y)
        assert not np.any(got == SENTINEL)
        rows = _sample_rows(N, wl.rng(w.name, f"sample_{mat}"), n=16)
        Yr, Br = oracle_mod.moe(w.kind, W, w.E, N, K, ids, X, per_slot, rows=rows)
        assert_within_bound(got[:, :, rows], Yr, Br, f"{w.name} {mat}")
