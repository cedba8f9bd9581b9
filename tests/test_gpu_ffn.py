"""GPU parity of the routed expert FFN (qmm_moe_ffn) against the oracle's
binary64 composition, within the tolerance the oracle derives from the
per-matmul bar (1e-3 sum|w||x| + 1e-6 for each routed product, an f32
SiLU-product and an f32 combine).

Cases span the routed paths: 256-element kinds with N_ff and K whole
256-element k-blocks (matrix-core expert kernel, one-pair and grouped work
items by the pairs-per-expert rule), 32-element kinds with K not a multiple
of 256 (the f32 expert kernel), skipped slots (ids -1 and E), and the
128-expert, top-8 workload at full size on sampled output columns.
"""
import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gguf_block_quantized_kind_amd as qmm  # noqa: E402

from test_gpu_parity import SENTINEL, dev, host  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qmm.load_library()


def _weights(g, M, topk):
    w = g.uniform(0.05, 1.0, size=(M, topk))
    return (w / w.sum(axis=1, keepdims=True)).astype(np.float32)


def run_ffn(kind, W_gu, W_d, E, ids, w, X, N_ff):
    M, K = X.shape
    Y = torch.full((M, K), SENTINEL, dtype=torch.float32, device="cuda")
    ws = torch.empty(qmm.qmm_moe_ffn_workspace_bytes(E, M, ids.shape[1], N_ff, K), dtype=torch.uint8,
                     device="cuda")
    qmm.qmm_moe_ffn(kind, dev(W_gu), dev(W_d), E, dev(ids), dev(w), ids.shape[1], dev(X), Y, M, N_ff, K, ws)
    return host(Y)


def check(got, y, tol, what):
    assert not np.any(got == SENTINEL), f"{what}: outputs left untouched"
    err = np.abs(got.astype(np.float64) - y)
    # A row with no valid slot is exactly zero, with tolerance zero.
    ratio = np.divide(err, tol, out=np.where(err == 0, 0.0, np.inf), where=tol > 0)
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert ratio.max() <= 1.0, f"{what}: worst |err|/tol = {ratio.max():.3g} at {worst}: got {got[worst]} want {y[worst]}"
    return float(ratio.max())


@pytest.mark.parametrize("kind,N_ff,K", [("Q4_K", 256, 512), ("Q6_K", 512, 256), ("Q8_0", 96, 160),
                                         ("MXFP4", 256, 512), ("IQ4_XS", 256, 256)])
def test_ffn_parity(oracle_mod, kind, N_ff, K):
    E, topk = 6, 3
    g = wl.rng("gpu_ffn", f"{kind}_{N_ff}_{K}")
    W_gu = wl.random_weights(kind, E * 2 * N_ff, K, g)
    W_d = wl.random_weights(kind, E * K, N_ff, g)
    for M in (1, 5, 40):
        ids = wl.routing(M, E, topk, g)
        if M > 1:
            ids[1, 0] = -1      # skipped slots
            ids[M - 1, 2] = E
        w = _weights(g, M, topk)
        X = wl.activations((M, K), np.float16, g)
        got = run_ffn(kind, W_gu, W_d, E, ids, w, X, N_ff)
        y, tol = oracle_mod.moe_ffn(kind, W_gu, W_d, E, N_ff, K, ids, w, X)
        check(got, y, tol, f"{kind} M={M}")


@pytest.mark.parametrize("kind", ["Q4_K", "Q6_K", "Q5_K", "Q2_K", "Q3_K"])
@pytest.mark.parametrize("packed", [False, True])
def test_ffn_two_launches(oracle_mod, kind, packed):
    """The two-launch FFN (fewer than four pairs per expert, whole
    k-blocks), native and repacked: M = 1, 3, 5, 7 tokens with 16 experts,
    top 2 (experts with zero, one and several pairs), f16 and f32
    activations; skipped slots add nothing."""
    E, topk, N_ff, K = 16, 2, 512, 768
    g = wl.rng("gpu_ffn_two", f"{kind}_{packed}")
    W_gu = wl.random_weights(kind, E * 2 * N_ff, K, g)
    W_d = wl.random_weights(kind, E * K, N_ff, g)
    if packed:
        P_gu = qmm.repack_experts(kind, dev(W_gu), E, 2 * N_ff, K)
        P_d = qmm.repack_experts(kind, dev(W_d), E, K, N_ff)
    for M in (1, 3, 5, 7):
        ids = wl.routing(M, E, topk, g)
        if M > 2:
            ids[1, 1] = -1
        w = _weights(g, M, topk)
        X = wl.activations((M, K), np.float32 if M == 3 else np.float16, g)
        if packed:
            Y = torch.full((M, K), SENTINEL, dtype=torch.float32, device="cuda")
            ws = torch.empty(qmm.qmm_moe_ffn_workspace_bytes(E, M, topk, N_ff, K), dtype=torch.uint8, device="cuda")
            qmm.qmm_moe_ffn_packed(kind, P_gu, P_d, E, dev(ids), dev(w), topk, dev(X), Y, M, N_ff, K, ws)
            got = host(Y)
        else:
            got = run_ffn(kind, W_gu, W_d, E, ids, w, X, N_ff)
        y, tol = oracle_mod.moe_ffn(kind, W_gu, W_d, E, N_ff, K, ids, w, X)
        check(got, y, tol, f"{kind} packed={packed} M={M}")


def test_ffn_f32_activations(oracle_mod):
    kind, E, topk, N_ff, K, M = "Q4_K", 4, 2, 256, 256, 7
    g = wl.rng("gpu_ffn_f32", kind)
    W_gu = wl.random_weights(kind, E * 2 * N_ff, K, g)
    W_d = wl.random_weights(kind, E * K, N_ff, g)
    ids = wl.routing(M, E, topk, g)
    w = _weights(g, M, topk)
    X = wl.activations((M, K), np.float32, g)
    got = run_ffn(kind, W_gu, W_d, E, ids, w, X, N_ff)
    y, tol = oracle_mod.moe_ffn(kind, W_gu, W_d, E, N_ff, K, ids, w, X)
    check(got, y, tol, "f32 X")


@pytest.mark.parametrize("M", [1, 16])
def test_ffn_full_size_sampled(oracle_mod, M):
    """128 experts, top 8, gate/up [1536, 2048] and down [2048, 768] Q4_K,
    1 and 16 tokens; the oracle computes 64 sampled output columns."""
    e = next(x for x in wl.C5 if x.M == M)
    N_ff, K = e.N_gu // 2, e.K_gu
    ids = e.ids()
    W_gu, W_d = e.w_gu(), e.w_d()
    g = wl.rng(e.name, "ffn")
    w = _weights(g, e.M, e.topk)
    X = e.x()
    got = run_ffn(e.kind, W_gu, W_d, e.E, ids, w, X, N_ff)
    cols = np.unique(np.concatenate([[0, K - 1], g.choice(K, size=62, replace=False)]))
    y, tol = oracle_mod.moe_ffn(e.kind, W_gu, W_d, e.E, N_ff, K, ids, w, X, rows=cols)
    assert not np.any(got == SENTINEL)
    ratio = check(got[:, cols], y, tol, e.name)
    print(f"worst error / tolerance: {ratio:.3g}")


def test_ffn_all_slots_skipped_and_determinism(oracle_mod):
    """A token whose every slot is skipped gets a zero row; repeated calls on
    one workspace agree bit for bit (the combine sums slots in order)."""
    kind, E, topk, N_ff, K, M = "Q4_K", 5, 3, 256, 512, 6
    g = wl.rng("gpu_ffn_skip", kind)
    W_gu = wl.random_weights(kind, E * 2 * N_ff, K, g)
    W_d = wl.random_weights(kind, E * K, N_ff, g)
    ids = wl.routing(M, E, topk, g)
    ids[2, :] = [-1, E, -7]
    w = _weights(g, M, topk)
    X = wl.activations((M, K), np.float16, g)
    ws = torch.empty(qmm.qmm_moe_ffn_workspace_bytes(E, M, topk, N_ff, K), dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(2):
        Y = torch.full((M, K), SENTINEL, dtype=torch.float32, device="cuda")
        qmm.qmm_moe_ffn(kind, dev(W_gu), dev(W_d), E, dev(ids), dev(w), topk, dev(X), Y, M, N_ff, K, ws)
        outs.append(host(Y))
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    assert np.all(outs[0][2] == 0.0)
    y, tol = oracle_mod.moe_ffn(kind, W_gu, W_d, E, N_ff, K, ids, w, X)
    check(outs[0], y, tol, "skipped row")


def test_ffn_one_expert_top1(oracle_mod):
    """E = 1, top-1: every token takes the single expert with weight 1."""
    kind, N_ff, K, M = "Q8_0", 64, 96, 3
    g = wl.rng("gpu_ffn_e1", kind)
    W_gu = wl.random_weights(kind, 2 * N_ff, K, g)
    W_d = wl.random_weights(kind, K, N_ff, g)
    ids = np.zeros((M, 1), dtype=np.int32)
    w = np.ones((M, 1), dtype=np.float32)
    X = wl.activations((M, K), np.float16, g)
    got = run_ffn(kind, W_gu, W_d, 1, ids, w, X, N_ff)
    y, tol = oracle_mod.moe_ffn(kind, W_gu, W_d, 1, N_ff, K, ids, w, X)
    check(got, y, tol, "E=1 top-1")


@pytest.mark.parametrize("kind,N_ff,K", [("Q4_K", 256, 512), ("Q6_K", 512, 256), ("Q8_0", 256, 256),
                                         ("MXFP4", 256, 512), ("IQ4_XS", 256, 256)])
def test_ffn_packed_parity(oracle_mod, kind, N_ff, K):
    """The FFN over repacked experts (qmm_moe_ffn_packed) against the oracle
    over the native experts, one-pair and grouped items, a skipped slot."""
    E, topk = 6, 3
    g = wl.rng("gpu_ffn_packed", f"{kind}_{N_ff}_{K}")
    W_gu = wl.random_weights(kind, E * 2 * N_ff, K, g)
    W_d = wl.random_weights(kind, E * K, N_ff, g)
    P_gu = qmm.repack_experts(kind, dev(W_gu), E, 2 * N_ff, K)
    P_d = qmm.repack_experts(kind, dev(W_d), E, K, N_ff)
    for M in (1, 5, 40):
        ids = wl.routing(M, E, topk, g)
        if M > 1:
            ids[1, 2] = -1
        w = _weights(g, M, topk)
        X = wl.activations((M, K), np.float16, g)
        Y = torch.full((M, K), SENTINEL, dtype=torch.float32, device="cuda")
        ws = torch.empty(qmm.qmm_moe_ffn_workspace_bytes(E, M, topk, N_ff, K), dtype=torch.uint8, device="cuda")
        qmm.qmm_moe_ffn_packed(kind, P_gu, P_d, E, dev(ids), dev(w), topk, dev(X), Y, M, N_ff, K, ws)
        got = host(Y)
        y, tol = oracle_mod.moe_ffn(kind, W_gu, W_d, E, N_ff, K, ids, w, X)
        check(got, y, tol, f"{kind} M={M} packed")
