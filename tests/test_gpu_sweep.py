"""Seeded random-shape sweep of the GPU paths against the oracle, every
output compared (the bar of each test file: |y - y_ref| <= 1e-3 * sum|w||x|
+ 1e-6 for the products, the oracle's propagated tolerance for the expert
FFN):

* qmm_matmul over native rows and qmm_matmul_packed over repacked records:
  every kind, K in whole 256-element k-blocks up to 3072, 1 to 2499 rows,
  token counts from 1 to 200 (the decode GEMVs at 8 or fewer, the prefill
  GEMMs above), f16 and f32 activations; and 20 larger cases (up to 23999
  rows, K up to 8192, up to 600 tokens: grids of several rounds);
* qmm_moe / qmm_moe_packed: 1 to 39 experts, top-1 to top-8, 1 to 256
  tokens, shared or per-slot activations, sometimes a skipped slot;
* qmm_moe_ffn / qmm_moe_ffn_packed on the same routing (a token whose only
  slot is skipped must come back exactly zero).

The shapes come from one fixed seed, so the sweep is the same on every run.
"""
import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gguf_block_quantized_kind_amd as qmm  # noqa: E402
from oracle import repack as rp  # noqa: E402

from test_gpu_parity import SENTINEL, assert_within_bound, dev, filled, host  # noqa: E402

KINDS = ["Q4_0", "Q5_0", "Q8_0", "Q2_K", "Q3_K", "Q4_K", "Q5_K", "Q6_K", "IQ4_NL", "IQ4_XS", "MXFP4"]
PACKED = set(rp.KINDS)
PACKED_GEMM = {"Q8_0", "Q4_0", "Q5_0", "IQ4_NL", "MXFP4", "IQ4_XS"}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qmm.load_library()


def _matmul_cases(n):
    g = np.random.default_rng(20261203)
    for i in range(n):
        yield (i, KINDS[g.integers(len(KINDS))], int(g.choice([1, 2, 3, 4, 5, 7, 8, 9, 17, 64, 65, 130, 200])),
               int(g.integers(1, 2500)), 256 * int(g.integers(1, 13)), bool(g.integers(2)))


@pytest.mark.parametrize("chunk", range(4))
def test_sweep_matmul_native_and_packed(oracle_mod, chunk):
    for i, kind, M, N, K, f16 in list(_matmul_cases(240))[chunk::4]:
        r = wl.rng("gpu_sweep_matmul", str(i))
        W = wl.random_weights(kind, N, K, r)
        X = wl.activations((M, K), np.float16 if f16 else np.float32, r)
        Y, B = oracle_mod.matmul(kind, W, K, X)
        what = f"{kind} M={M} N={N} K={K} {'f16' if f16 else 'f32'}"
        Wd, Xd = dev(W), dev(X)
        C = filled((M, N))
        qmm.qmm_matmul(kind, Wd, Xd, C, M, N, K)
        assert_within_bound(host(C), Y, B, "native " + what)
        if kind in PACKED and (M <= 8 or kind in PACKED_GEMM):
            P = torch.full((qmm.qmm_packed_bytes(kind, N, K),), 0xA5, dtype=torch.uint8, device="cuda")
            qmm.qmm_repack(kind, Wd, P, N, K)
            C = filled((M, N))
            qmm.qmm_matmul_packed(kind, P, Xd, C, M, N, K)
            assert_within_bound(host(C), Y, B, "packed " + what)


def test_sweep_matmul_large_grids(oracle_mod):
    """Larger shapes, so that grids take several rounds of the compute
    units: up to 23999 rows, K up to 8192, up to 600 tokens."""
    g = np.random.default_rng(20261205)
    for i in range(20):
        kind = KINDS[g.integers(len(KINDS))]
        K, N = 256 * int(g.integers(1, 33)), int(g.integers(1, 24000))
        M, f16 = int(g.choice([1, 3, 8, 9, 100, 257, 600])), bool(g.integers(2))
        r = wl.rng("gpu_sweep_large", str(i))
        W = wl.random_weights(kind, N, K, r)
        X = wl.activations((M, K), np.float16 if f16 else np.float32, r)
        Y, B = oracle_mod.matmul(kind, W, K, X)
        what = f"{kind} M={M} N={N} K={K} {'f16' if f16 else 'f32'}"
        Wd, Xd = dev(W), dev(X)
        C = filled((M, N))
        qmm.qmm_matmul(kind, Wd, Xd, C, M, N, K)
        assert_within_bound(host(C), Y, B, "native " + what)
        if kind in PACKED and (M <= 8 or kind in PACKED_GEMM):
            P = torch.full((qmm.qmm_packed_bytes(kind, N, K),), 0xA5, dtype=torch.uint8, device="cuda")
            qmm.qmm_repack(kind, Wd, P, N, K)
            C = filled((M, N))
            qmm.qmm_matmul_packed(kind, P, Xd, C, M, N, K)
            assert_within_bound(host(C), Y, B, "packed " + what)


def _moe_cases(n):
    g = np.random.default_rng(20261204)
    for i in range(n):
        E = int(g.integers(1, 40))
        yield (i, KINDS[g.integers(len(KINDS))], E, int(g.integers(1, min(E, 8) + 1)),
               int(g.choice([1, 2, 3, 5, 8, 9, 16, 17, 40, 100, 256])), int(g.integers(1, 700)),
               256 * int(g.integers(1, 9)), bool(g.integers(2)), bool(g.integers(2)), bool(g.integers(2)))


@pytest.mark.parametrize("chunk", range(4))
def test_sweep_routed_experts_and_ffn(oracle_mod, chunk):
    for i, kind, E, topk, M, N, K, skip, per_slot, f16 in list(_moe_cases(80))[chunk::4]:
        r = wl.rng("gpu_sweep_moe", str(i))
        ids = wl.routing(M, E, topk, r)
        if skip and M > 2:
            ids[M // 2, 0] = -1
        inval = ids < 0
        valid_ids = np.where(inval, 0, ids).astype(np.int32)
        xdt = np.float16 if f16 else np.float32
        what = f"{kind} E={E} topk={topk} M={M} N={N} K={K} per_slot={per_slot}"
        # routed products
        W = wl.random_weights(kind, E * N, K, r)
        X = wl.activations((M, topk, K) if per_slot else (M, K), xdt, r)
        Yr, Br = oracle_mod.moe(kind, W, E, N, K, valid_ids, X, per_slot)
        Yr[inval] = 0.0
        Br[inval] = 0.0
        ws = torch.empty((qmm.qmm_moe_workspace_bytes(E, M, topk) + 3) // 4, dtype=torch.int32, device="cuda")
        Wd, idd, Xd = dev(W), dev(ids), dev(X)
        runs = [("moe", lambda Y: qmm.qmm_moe(kind, Wd, E, idd, topk, Xd, int(per_slot), Y, M, N, K, ws))]
        if kind in PACKED:
            P = qmm.repack_experts(kind, Wd, E, N, K)
            runs.append(("moe_packed",
                         lambda Y: qmm.qmm_moe_packed(kind, P, E, idd, topk, Xd, int(per_slot), Y, M, N, K, ws)))
        for name, run in runs:
            Y = filled((M, topk, N))
            run(Y)
            got = host(Y)
            assert np.all(got[inval] == SENTINEL), f"{name} {what}: a skipped slot was written"
            got[inval] = 0.0
            assert_within_bound(got, Yr, Br, f"{name} {what}")
        # expert FFN on the same routing
        N_ff, Kf = 256 * (1 + i % 3), 256 * (1 + (i // 3) % 4)
        W_gu = wl.random_weights(kind, E * 2 * N_ff, Kf, r)
        W_d = wl.random_weights(kind, E * Kf, N_ff, r)
        Xf = wl.activations((M, Kf), xdt, r)
        w = r.random((M, topk)).astype(np.float32)
        y, tol = oracle_mod.moe_ffn(kind, W_gu, W_d, E, N_ff, Kf, ids, w, Xf)
        wsf = torch.empty(max(qmm.qmm_moe_ffn_workspace_bytes(E, M, topk, N_ff, Kf), 1), dtype=torch.uint8,
                          device="cuda")
        gu, dn, wd, xf = dev(W_gu), dev(W_d), dev(w), dev(Xf)
        runs = [("ffn", lambda Y: qmm.qmm_moe_ffn(kind, gu, dn, E, idd, wd, topk, xf, Y, M, N_ff, Kf, wsf))]
        if kind in PACKED:
            Pg = qmm.repack_experts(kind, gu, E, 2 * N_ff, Kf)
            Pd = qmm.repack_experts(kind, dn, E, Kf, N_ff)
            runs.append(("ffn_packed",
                         lambda Y: qmm.qmm_moe_ffn_packed(kind, Pg, Pd, E, idd, wd, topk, xf, Y, M, N_ff, Kf, wsf)))
        for name, run in runs:
            Y = filled((M, Kf))
            run(Y)
            got = host(Y).astype(np.float64)
            err = np.abs(got - y)
            assert np.all(np.isfinite(got)) and np.all(err <= tol), (
                f"{name} {what} N_ff={N_ff}: worst {float(np.max(err - tol))} over the tolerance")
