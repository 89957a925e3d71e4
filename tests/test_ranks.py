"""Retained-rank allocation in the library (host code, CPU): the same pins
as the oracle, and equality with the oracle on random fleets."""
import numpy as np
import pytest

import rank_specialized_amd as rs
from oracle import spectral_ranks_ref, uniform_ranks_ref

import oracle_pins as P


@pytest.mark.parametrize("pin", P.RANK_PINS, ids=lambda f: f.__name__)
def test_library_rank_pin(pin):
    pin(rs.lora_ranks_uniform, rs.lora_ranks_spectral)


@pytest.mark.parametrize("seed", range(6))
def test_library_equals_oracle(seed):
    rng = np.random.default_rng(100 + seed)
    m = int(rng.integers(1, 60))
    r_orig = [int(v) for v in rng.integers(0, 65, size=m)]
    # float32 values, some repeated, so ties occur
    sig = [np.sort(np.round(rng.gamma(2.0, 1.0, size=r), 1).astype(np.float32))[::-1] for r in r_orig]
    for ratio, floor in ((1 / 12, 4), (0.3, 2), (0.0, 0), (1.0, 3)):
        assert rs.lora_ranks_uniform(r_orig, ratio, floor) == uniform_ranks_ref(r_orig, ratio, floor)
        for budget in (0, sum(r_orig) // 3, sum(uniform_ranks_ref(r_orig, ratio, floor)), sum(r_orig) + 5):
            assert rs.lora_ranks_spectral(r_orig, sig, floor, budget) == \
                spectral_ranks_ref(r_orig, [s.astype(np.float64) for s in sig], floor, budget=budget)


def test_library_rejects():
    import rank_specialized_amd._lib as L
    with pytest.raises(L.LoraError):
        rs.lora_ranks_uniform([4, 8], 1.5, 1)
    with pytest.raises(L.LoraError):
        rs.lora_ranks_spectral([2], [np.array([1.0, 2.0], np.float32)], 0, 2)  # increasing
    with pytest.raises(L.LoraError):
        rs.lora_ranks_spectral([2], [np.array([1.0, np.nan], np.float32)], 0, 2)


def test_library_equals_oracle_every_budget_with_ties():
    """Few distinct values (zeros, -0.0 among them) so that the budget's
    last ranks fall on ties at every possible place: every budget from 0 to
    past the total."""
    rng = np.random.default_rng(7)
    m = 9
    r_orig = [int(v) for v in rng.integers(0, 9, size=m)]
    vals = np.array([3.0, 2.0, 2.0, 1.0, 0.5, 0.5, 0.0, -0.0], np.float32)
    sig = [np.sort(rng.choice(vals, size=r))[::-1].copy() for r in r_orig]
    for s in sig:
        s[s == 0] = np.float32(-0.0) if rng.random() < 0.5 else np.float32(0.0)
    for floor in (0, 1, 3):
        for budget in range(0, sum(r_orig) + 3):
            assert rs.lora_ranks_spectral(r_orig, sig, floor, budget) == \
                spectral_ranks_ref(r_orig, [s.astype(np.float64) for s in sig], floor, budget=budget), (floor, budget)


def test_library_equals_oracle_wide_range():
    """Values over many binades, so the selection's two 16-bit passes both
    matter, on a larger fleet."""
    rng = np.random.default_rng(8)
    m = 400
    r_orig = [int(v) for v in rng.integers(1, 65, size=m)]
    sig = [np.sort((10.0 ** rng.uniform(-30, 10, size=r)).astype(np.float32))[::-1].copy() for r in r_orig]
    total = sum(r_orig)
    for budget in (1, 2 * m, total // 2, total - 1):
        assert rs.lora_ranks_spectral(r_orig, sig, 2, budget) == \
            spectral_ranks_ref(r_orig, [s.astype(np.float64) for s in sig], 2, budget=budget), budget


def test_library_rejects_null_sigma():
    import ctypes as C
    import rank_specialized_amd._lib as L
    ro = (C.c_int32 * 1)(3)
    off = (C.c_int64 * 2)(0, 3)
    out = (C.c_int32 * 1)()
    assert L.lib().lora_ranks_spectral(1, ro, None, off, 0, 2, out) == 1
