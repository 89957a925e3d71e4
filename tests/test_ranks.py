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
