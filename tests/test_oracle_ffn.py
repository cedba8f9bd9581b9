"""Pins of the oracle's routed expert FFN (gate/up, SiLU(gate) * up, down,
weighted top-k combine) against closed forms.

The FFN is model semantics the pages do not spell out; these pins tie the
oracle's composition to mathematics rather than to itself:

* SiLU: silu(0) = 0, silu(x) - silu(-x) = x, silu(ln 3) = (3/4) ln 3, and its
  two asymptotes;
* the whole FFN on hand-built Q8_0 experts whose rows are constant: every
  gate output is c_e S_t, every up output v_e S_t (S_t = sum_k x[t][k]), every
  down output r_e N_ff silu(c_e S_t) v_e S_t, so y has a closed form that
  fails if gate and up are swapped, SiLU lands on the wrong half, a slot
  takes another slot's weight or expert, or a skipped id contributes;
* the tolerance is non-negative and grows with the combine weights.
"""
import math

import numpy as np
import pytest

import oracle


def test_silu_closed_forms():
    x = np.array([0.0, math.log(3.0), -math.log(3.0), 1e-300, 40.0, -40.0, 750.0, -750.0])
    s = oracle.silu(x)
    assert s[0] == 0.0
    assert s[1] == pytest.approx(0.75 * math.log(3.0), rel=1e-15)
    assert s[2] == pytest.approx(-0.25 * math.log(3.0), rel=1e-15)
    assert s[3] == pytest.approx(0.5e-300, rel=1e-15)
    assert s[4] == pytest.approx(40.0, rel=1e-15)
    assert s[5] == pytest.approx(-40.0 * math.exp(-40.0), rel=1e-12)
    assert s[6] == 750.0 and s[7] == pytest.approx(0.0, abs=1e-300)
    r = np.random.default_rng(1).normal(scale=5.0, size=1000)
    np.testing.assert_allclose(oracle.silu(r) - oracle.silu(-r), r, rtol=1e-14, atol=1e-14)


def _q8_0_rows(codes_per_row, K):
    """Q8_0 rows whose every element is the row's integer code (scale 1.0)."""
    rows = []
    for c in codes_per_row:
        blk = np.empty(34, dtype=np.uint8)
        blk[0], blk[1] = 0x00, 0x3C          # f16 1.0, little-endian
        blk[2:] = np.uint8(np.int8(c).view(np.uint8))
        rows.append(np.tile(blk, K // 32))
    return np.stack(rows)


def test_ffn_closed_form_on_constant_experts():
    E, N_ff, K, M, topk = 4, 64, 96, 3, 3
    c = [1, -2, 3, 1]    # gate codes per expert
    v = [2, 1, -1, 3]    # up codes
    r = [1, 3, -2, 2]    # down codes
    W_gu = np.concatenate([_q8_0_rows([c[e]] * N_ff + [v[e]] * N_ff, K) for e in range(E)])
    W_d = np.concatenate([_q8_0_rows([r[e]] * K, N_ff) for e in range(E)])
    ids = np.array([[2, 0, 3], [1, -1, 1], [3, 4, 0]], dtype=np.int32)   # -1 and 4 are skipped
    w = np.array([[0.5, 0.25, 0.125], [1.0, 7.0, -0.75], [2.0, 9.0, 0.5]], dtype=np.float32)
    g = np.random.default_rng(2)
    X = (g.integers(-2, 3, size=(M, K)) / 64.0).astype(np.float32)   # S_t of a few units
    y, tol = oracle.moe_ffn("Q8_0", W_gu, W_d, E, N_ff, K, ids, w, X)
    assert y.shape == (M, K) and tol.shape == (M, K)
    for t in range(M):
        S = float(X[t].astype(np.float64).sum())
        want = 0.0
        for s in range(topk):
            e = int(ids[t, s])
            if 0 <= e < E:
                gate = c[e] * S
                want += float(w[t, s]) * r[e] * N_ff * (gate / (1.0 + math.exp(-gate))) * (v[e] * S)
        np.testing.assert_allclose(y[t], want, rtol=1e-12, atol=1e-12)
    assert np.all(tol >= 0)


def test_ffn_tolerance_scales_with_the_combine_weights():
    E, N_ff, K, M = 2, 32, 64, 2
    W_gu = np.concatenate([_q8_0_rows([1] * N_ff + [2] * N_ff, K) for _ in range(E)])
    W_d = np.concatenate([_q8_0_rows([1] * K, N_ff) for _ in range(E)])
    ids = np.array([[0, 1], [1, 0]], dtype=np.int32)
    X = np.full((M, K), 1.0 / 32, dtype=np.float32)
    w1 = np.ones((M, 2), dtype=np.float32)
    y1, t1 = oracle.moe_ffn("Q8_0", W_gu, W_d, E, N_ff, K, ids, w1, X)
    y2, t2 = oracle.moe_ffn("Q8_0", W_gu, W_d, E, N_ff, K, ids, 2 * w1, X)
    np.testing.assert_allclose(y2, 2 * y1, rtol=1e-15)
    np.testing.assert_allclose(t2, 2 * t1, rtol=1e-12)
    y0, t0 = oracle.moe_ffn("Q8_0", W_gu, W_d, E, N_ff, K, ids, w1, np.zeros_like(X))
    assert np.all(y0 == 0) and np.all(t0 > 0)
