"""The seeded workload generators: sizes of the stated workloads, scale-field
distributions, determinism and routing."""
import numpy as np

import workloads as wl


def test_weight_bytes_of_the_workloads():
    by_name = {w.name: w.weight_bytes for w in wl.C1 + wl.C2 + wl.C3 + wl.C4}
    assert by_name["c1_q4_0_m1"] == 9_437_184
    assert by_name["c2_q4_k_m1"] == by_name["c2_q4_k_m8"] == 33_030_144
    assert by_name["c2_q6_k_m1"] == 48_168_960
    assert by_name["c3_q8_0_m512"] == 17_825_792
    assert by_name["c3_q5_0_m512"] == 11_534_336
    assert by_name["c4_iq4_nl_m1"] == 25_362_432
    assert by_name["c4_iq4_xs_m256"] == by_name["c4_mxfp4_m1"] == 23_953_408
    e = wl.C5[0]
    assert 1536 * wl.row_bytes("Q4_K", 2048) == 1_769_472
    assert 2048 * wl.row_bytes("Q4_K", 768) == 884_736
    assert e.touched_bytes(np.arange(8).reshape(1, 8)) == 8 * (1_769_472 + 884_736)


def test_scale_fields_follow_the_recipe():
    for name in wl.KINDS:
        bb, be = wl.geometry(name)
        W = wl.random_weights(name, 64, 4 * be, wl.rng("t", name)).reshape(-1, bb)
        for off in wl.F16_FIELDS[name]:
            d = W[:, off:off + 2].copy().view(np.float16).astype(np.float64)
            assert d.min() >= np.float16(1e-3) and d.max() <= np.float16(1e-2), name
        for off in wl.E8M0_FIELDS.get(name, ()):
            assert W[:, off].min() >= 118 and W[:, off].max() <= 130
        S = wl.random_weights(name, 64, 4 * be, wl.rng("t", name), scales="stress").reshape(-1, bb)
        for off in wl.F16_FIELDS[name]:
            h = S[:, off].astype(np.uint16) | (S[:, off + 1].astype(np.uint16) << 8)
            ex = (h >> 10) & 31
            assert ex.min() >= 8 and ex.max() <= 22


def test_streams_are_reproducible_and_distinct():
    a = wl.random_weights("Q4_K", 8, 256, wl.rng("w", "W"))
    b = wl.random_weights("Q4_K", 8, 256, wl.rng("w", "W"))
    c = wl.random_weights("Q4_K", 8, 256, wl.rng("w", "other"))
    assert np.array_equal(a, b) and not np.array_equal(a, c)


def test_routing_draws_distinct_experts():
    ids = wl.routing(300, 128, 8, wl.rng("t", "ids"))
    assert ids.shape == (300, 8) and ids.dtype == np.int32
    assert all(len(set(r)) == 8 for r in ids)
    assert ids.min() >= 0 and ids.max() < 128
