"""GPU parity of the load-time repack (qmm_repack) and the GEMV over it
(qmm_gemv_packed).

* the repacked bytes equal the oracle's repack byte for byte, on 130 rows
  (not a multiple of the 16-row tile, as the Vulkore page's repack test uses
  130 rows so that a padding mistake shows) and on one-row and one-tile
  shapes;
* the GEMV over the repacked bytes meets the GEMV bar against the oracle's
  product over the NATIVE weights: |y - y_ref| <= 1e-3 * sum|w||x| + 1e-6;
* one-hot activations return the f32 weights themselves (a zero weight
  may come back as +0);
* full workload sizes on sampled rows.
"""
import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gguf_block_quantized_kind_amd as qmm  # noqa: E402
from oracle import repack as rp  # noqa: E402

from test_gpu_parity import SENTINEL, assert_within_bound, dev, filled, host, _sample_rows  # noqa: E402

KINDS = list(rp.KINDS)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qmm.load_library()


def packed(kind, Wd, N, K):
    P = torch.full((qmm.qmm_packed_bytes(kind, N, K),), 0xA5, dtype=torch.uint8, device="cuda")
    qmm.qmm_repack(kind, Wd, P, N, K)
    return P


def gemv(kind, P, X, N):
    M, K = X.shape
    y = filled((M, N))
    qmm.qmm_gemv_packed(kind, P, dev(X), y, M, N, K)
    return host(y)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("N,K", [(130, 1024), (1, 256), (16, 512), (17, 768)])
def test_repack_matches_the_oracle_byte_for_byte(kind, N, K):
    W = wl.random_weights(kind, N, K, wl.rng("gpu_repack", f"{kind}_{N}_{K}"))
    got = host(packed(kind, dev(W), N, K))
    want = rp.repack(kind, W, N, K)
    assert got.shape == want.shape
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:4]}"


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("xdt", ["f32", "f16"])
def test_gemv_packed_parity(oracle_mod, kind, xdt):
    """N = 130 (eight full tiles and a ragged one), K = 1280 (five k-blocks:
    uneven between the waves that split K), M = 1 .. 8."""
    N, K = 130, 1280
    g = wl.rng("gpu_gemv_packed", f"{kind}_{xdt}")
    W = wl.random_weights(kind, N, K, g)
    P = packed(kind, dev(W), N, K)
    for M in (1, 2, 3, 5, 8):
        X = wl.activations((M, K), np.float16 if xdt == "f16" else np.float32, g)
        got = gemv(kind, P, X, N)
        Y, B = oracle_mod.matmul(kind, W, K, X)
        assert_within_bound(got, Y, B, f"{kind} M={M} {xdt}")


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("N,K", [(300, 2816), (40, 4096), (17, 512), (4500, 512)])
def test_gemv_packed_two_to_eight_tokens(oracle_mod, kind, N, K):
    """The 2-to-8-token kernel: K split over k-parts unevenly (11
    k-blocks: a k-part idles a round; 2 k-blocks), whole and remainder
    rounds of the weight pipeline, ragged tiles (N = 17, 300), and
    more tiles than compute units (N = 4500: workgroups of one and two
    tiles, waves without a tile)."""
    g = wl.rng("gpu_gemv_packed_xs", f"{kind}_{N}_{K}")
    W = wl.random_weights(kind, N, K, g)
    P = packed(kind, dev(W), N, K)
    for M, dt in ((2, np.float32), (4, np.float16), (6, np.float32), (8, np.float16), (8, np.float32)):
        X = wl.activations((M, K), dt, g)
        got = gemv(kind, P, X, N)
        Y, B = oracle_mod.matmul(kind, W, K, X)
        assert_within_bound(got, Y, B, f"{kind} M={M} N={N} K={K} {dt.__name__}")


@pytest.mark.parametrize("kind", KINDS)
def test_gemv_packed_unit_vectors_return_the_weights(oracle_mod, kind):
    N, K = 40, 512
    W = wl.random_weights(kind, N, K, wl.rng("gpu_packed_unit", kind))
    want = oracle_mod.dequant(kind, W).reshape(N, K).astype(np.float32)
    P = packed(kind, dev(W), N, K)
    for ks in ([0, 1, 31, 32, 255, 256, 300, 511], [17, 64, 100, 200, 257, 400, 480, 510]):
        X = np.zeros((len(ks), K), dtype=np.float32)
        for i, k in enumerate(ks):
            X[i, k] = 1.0
        got = gemv(kind, P, X, N)
        for i, k in enumerate(ks):
            # Equal values: a sum that starts from +0 returns MXFP4's -0.0 as +0.
            assert np.array_equal(got[i], want[:, k]), f"{kind} column {k}"


@pytest.mark.parametrize("kind", KINDS)
def test_gemv_packed_one_token_unit_vectors_return_the_weights(oracle_mod, kind):
    """One token (the kernel that scales sub-blocks after the products for
    Q4_K and Q6_K): x = e_k returns column k of the weights exactly, also
    with stress scales (signed f16 scales from about 2^-7 to 2^7)."""
    N, K = 40, 768
    for scales in (("config",) if kind == "MXFP4" else ("config", "stress")):
        W = wl.random_weights(kind, N, K, wl.rng("gpu_packed_unit1", f"{kind}_{scales}"), scales=scales)
        want = oracle_mod.dequant(kind, W).reshape(N, K).astype(np.float32)
        P = packed(kind, dev(W), N, K)
        for k in (0, 1, 15, 16, 31, 32, 63, 64, 127, 128, 200, 255, 256, 511, 600, 767):
            X = np.zeros((1, K), dtype=np.float32)
            X[0, k] = 1.0
            got = gemv(kind, P, X, N)
            assert np.array_equal(got[0], want[:, k]), f"{kind} {scales} column {k}"


@pytest.mark.parametrize("kind", ["Q4_K", "Q4_0", "MXFP4"])
def test_gemv_packed_single_row_and_single_kblock(oracle_mod, kind):
    for N, K in ((1, 256), (3, 256), (16, 256), (33, 256)):
        g = wl.rng("gpu_packed_edge", f"{kind}_{N}_{K}")
        W = wl.random_weights(kind, N, K, g)
        P = packed(kind, dev(W), N, K)
        X = wl.activations((4, K), np.float32, g)
        got = gemv(kind, P, X, N)
        Y, B = oracle_mod.matmul(kind, W, K, X)
        assert_within_bound(got, Y, B, f"{kind} N={N} K={K}")


@pytest.mark.parametrize("w", [w for w in wl.C1 + wl.C2 + wl.C4 if w.M <= 8], ids=lambda w: w.name)
def test_gemv_packed_full_size_sampled(oracle_mod, w):
    W = w.weights()
    X = w.x()
    P = packed(w.kind, dev(W), w.N, w.K)
    got = gemv(w.kind, P, X, w.N)
    assert not np.any(got == SENTINEL)
    rows = _sample_rows(w.N, wl.rng(w.name, "sample_packed"))
    Y, B = oracle_mod.matmul(w.kind, W, w.K, X, rows=rows)
    assert_within_bound(got[:, rows], Y, B, w.name)
    # The repacked bytes of sampled tiles against the oracle's repack of
    # those rows (tiles are independent).
    Bk = rp.kblock_bytes(w.kind)
    rec = 16 * Bk * (w.K // 256)
    Ph = host(P)
    Wr = W.reshape(w.N, -1)
    for t in (0, w.N // 32, (w.N - 1) // 16):
        rows_t = Wr[16 * t:16 * t + 16]
        want = rp.repack(w.kind, rows_t, rows_t.shape[0], w.K)
        assert np.array_equal(Ph[t * rec:(t + 1) * rec], want), f"tile {t}"


@pytest.mark.parametrize("kind", KINDS)
def test_moe_packed_parity(oracle_mod, kind):
    """Routed expert products over repacked experts (qmm_moe_packed), against
    the oracle's products over the native experts: N = 130 rows per expert
    (each expert's last tile padded), items of one pair (M = 2, 5), eight
    (M = 9) and sixteen (M = 40), an id outside [0, E) skipped."""
    E, N, topk, K = 6, 130, 3, 1280
    for M in (5, 2, 9, 40):
        g = wl.rng("gpu_moe_packed", f"{kind}_{M}")
        W = wl.random_weights(kind, E * N, K, g)
        ids = wl.routing(M, E, topk, g)
        ids[0] = [1, 2, 3]
        ids[1] = [1, 4, -1]   # skipped: its Y row keeps the sentinel
        if M == 9:
            ids[:, 0] = 0
        P = qmm.repack_experts(kind, dev(W), E, N, K)
        idd = dev(ids)
        for per_slot, xdt in ((False, np.float16), (True, np.float32)):
            X = wl.activations((M, topk, K) if per_slot else (M, K), xdt, g)
            Y = filled((M, topk, N))
            nbytes = qmm.qmm_moe_workspace_bytes(E, M, topk)
            ws = torch.empty((nbytes + 3) // 4, dtype=torch.int32, device="cuda")
            qmm.qmm_moe_packed(kind, P, E, idd, topk, dev(X), int(per_slot), Y, M, N, K, ws)
            got = host(Y)
            assert np.all(got[1, 2] == SENTINEL)
            got[1, 2] = 0.0
            ids_ok = ids.copy()
            ids_ok[1, 2] = 0      # the oracle takes only valid ids; that slot is compared as zero
            Yr, Br = oracle_mod.moe(kind, W, E, N, K, ids_ok, X, per_slot)
            Yr[1, 2] = 0.0
            Br[1, 2] = 0.0
            assert_within_bound(got, Yr, Br, f"{kind} M={M} per_slot={per_slot}")


@pytest.mark.parametrize("e", [x for x in wl.C5 if x.M in (1, 16, 256)], ids=lambda e: e.name)
def test_moe_packed_full_size_sampled(oracle_mod, e):
    """The expert workload's gate/up matrices, repacked, at 1, 16 and 256
    tokens (one pair per work item, and items of sixteen pairs), on sampled
    rows."""
    ids = e.ids()
    W = e.w_gu()
    X = e.x()
    P = qmm.repack_experts(e.kind, dev(W), e.E, e.N_gu, e.K_gu)
    Y = qmm.moe_packed(e.kind, P, e.E, dev(ids), dev(X), e.N_gu, e.K_gu, False)
    got = host(Y)
    rows = _sample_rows(e.N_gu, wl.rng(e.name, "sample_moe_packed"), n=24)
    Yr, Br = oracle_mod.moe(e.kind, W, e.E, e.N_gu, e.K_gu, ids, X, False, rows=rows)
    assert_within_bound(got[:, :, rows], Yr, Br, e.name)


@pytest.mark.parametrize("kind", ["MXFP4", "Q6_K", "Q5_0"])
def test_repack_reads_byte_aligned_weights(kind):
    """W may sit at any byte offset (17-, 22- and 210-byte blocks make odd
    offsets normal): the repack of W one byte into a buffer equals the
    oracle's repack."""
    N, K = 33, 512
    W = wl.random_weights(kind, N, K, wl.rng("gpu_repack_odd", kind)).reshape(-1)
    buf = torch.zeros(W.size + 1, dtype=torch.uint8, device="cuda")
    buf[1:] = dev(W)
    got = host(packed(kind, buf[1:], N, K))
    assert np.array_equal(got, rp.repack(kind, W, N, K))
