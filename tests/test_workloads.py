"""The seeded generators: determinism and the stated distributions (CPU)."""
import hashlib

import numpy as np

from workloads import (fleet_ids, fleet_ranks, make_config, make_random_workload, round_to_bf16,
                       zipf_ids)


def _digest(wl):
    h = hashlib.sha256()
    for arr in [wl.ids, wl.x, wl.module.ranks, wl.module.scales, *wl.module.A, *wl.module.B]:
        h.update(np.ascontiguousarray(arr).tobytes())
    return h.hexdigest()


def test_deterministic():
    assert _digest(make_config("1")) == _digest(make_config("1"))
    assert _digest(make_config("2")) == _digest(make_config("2"))
    assert _digest(make_random_workload(3, 10, 2, 8, 8, [1, 2])) == \
        _digest(make_random_workload(3, 10, 2, 8, 8, [1, 2]))


def test_cfg1_tiny():
    wl = make_config("1")
    assert wl.dtype == "fp32" and wl.T == 16 and wl.n == 4
    assert list(wl.module.ranks) == [1, 2, 3, 4]
    assert np.all(wl.module.scales == 2.0)
    assert wl.module.A[3].shape == (4, 256) and wl.module.B[3].shape == (256, 4)
    assert 0.03 < wl.module.A[3].std() < 0.1  # std 1/16


def test_cfg2_decode_uniform():
    wl = make_config("2")
    assert wl.dtype == "bf16" and wl.T == 256 and wl.n == 64
    assert np.all(wl.module.ranks == 4) and np.all(wl.module.scales == 2.0)
    assert np.array_equal(round_to_bf16(wl.x), wl.x)
    assert np.array_equal(round_to_bf16(wl.module.B[0]), wl.module.B[0])


def test_cfg3_ranks_and_zipf():
    wl = make_config("3")
    r = wl.module.ranks
    assert r.min() >= 6 and r.max() <= 64 and 15 < r.mean() < 23
    counts = np.bincount(wl.ids, minlength=wl.n)
    assert 0.12 < counts.max() / wl.T < 0.26
    assert np.all(wl.module.scales == 0.5)


def test_cfg4_segments():
    wl = make_config("4")
    assert wl.T == 8192 and wl.module.d_in == 4096 and wl.module.d_out == 14336
    segs = wl.ids.reshape(32, 256)
    assert np.all(segs == segs[:, :1])
    assert sorted(segs[:, 0]) == list(range(32))
    assert set(wl.module.ranks.tolist()) <= {8, 12, 16, 24, 32}
    assert np.allclose(wl.module.scales, 32.0 / wl.module.ranks)


def test_cfg5_ranks():
    ru = fleet_ranks("5U")
    assert ru.shape == (28, 7, 1024) and np.all(ru == 6)
    rs = fleet_ranks("5S")
    assert rs.min() >= 4 and rs.max() <= 16 and 5.5 < rs.mean() < 7.0
    ids = fleet_ids()
    assert ids.shape == (4096,) and ids.min() >= 0 and ids.max() < 1024
    assert 0.12 < np.bincount(ids).max() / 4096 < 0.26


def test_zipf_is_a_distribution_over_all_ids():
    ids = zipf_ids(77, 16, 20000)
    c = np.bincount(ids, minlength=16)
    s = np.sort(c)[::-1]
    assert c.min() > 0 and s[0] > 1.9 * s[1] * 0.8  # P(1)/P(2) = 2^1.1 ~ 2.14


def test_integer_variant_is_exact_and_bounded():
    wl = make_config("2", integer=True)
    assert np.all(np.abs(wl.x) <= 2) and np.all(wl.x == np.round(wl.x))
    assert np.all(wl.module.A[0] == np.round(wl.module.A[0]))
    s = make_config("4", integer=True).module.scales
    assert np.all(np.log2(s) == np.round(np.log2(s)))


def test_jd_workloads_seeded_and_shaped():
    from workloads import JD_CONFIGS, make_jd_config, make_jd_workload
    a = make_jd_workload(4, 40, 9, 3, 32, 16, 4, mode="full")
    b = make_jd_workload(4, 40, 9, 3, 32, 16, 4, mode="full")
    assert np.array_equal(a.ids, b.ids) and np.array_equal(a.sigma, b.sigma)
    assert all(np.array_equal(u, v) for u, v in zip(a.U, b.U))
    assert a.sigma.shape == (9, 4, 4) and a.U[0].shape == (16, 4) and a.V[0].shape == (32, 4)
    d = make_jd_workload(4, 40, 9, 3, 32, 16, 4, mode="diag")
    assert d.sigma.shape == (9, 4)
    assert set(JD_CONFIGS) == {"jd-full", "jd-diag"}
    for name in JD_CONFIGS:
        w = make_jd_config(name)
        assert (w.T, w.n, w.k, w.r, w.d_in, w.d_out) == (2048, 1024, 32, 16, 4096, 4096)
        assert w.cluster_of.min() >= 0 and w.cluster_of.max() < 32
