"""The oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle
from oracle import apply_ref, base_fused_ref, bf16_round_ref, brute_force, segment_ref, shrink_error_bound, shrink_ref
from workloads import make_random_workload

import oracle_pins as P


@pytest.mark.parametrize("pin", P.APPLY_PINS, ids=lambda f: f.__name__)
def test_apply_pin(pin):
    pin(apply_ref)


def test_apply_brute_force():
    P.pin_brute_force(apply_ref, brute_force)


def test_apply_integer_exact():
    P.pin_integer_exact(apply_ref, brute_force)


def test_merged_weight_bf16_zipf():
    wl = make_random_workload(30, 48, 8, 64, 32, [1, 2, 3, 4, 5, 6, 7, 8], dtype="bf16",
                              id_mode="zipf", invalid_frac=0.1)
    P.pin_merged_weight(apply_ref, wl, seed=1)


@pytest.mark.parametrize("pin", P.SEGMENT_PINS, ids=lambda f: f.__name__)
def test_segment_pin(pin):
    pin(segment_ref)


def test_shrink_matches_per_segment_product():
    """h for every token equals the rows of X_seg A_a^T (numpy product)."""
    wl = make_random_workload(8, 50, 5, 40, 8, [1, 4, 2, 0, 6], dtype="bf16", id_mode="zipf",
                              invalid_frac=0.1)
    m = wl.module
    h = shrink_ref(wl.x, wl.ids, m.A)
    bound = shrink_error_bound(wl.x, wl.ids, m.A)
    for a in range(m.n):
        rows = np.nonzero(wl.ids == a)[0]
        if len(rows) == 0:
            continue
        H = wl.x[rows].astype(np.float64) @ m.A[a].astype(np.float64).T
        for i, t in enumerate(rows):
            assert h[t].shape == (m.ranks[a],)
            assert np.abs(h[t] - H[i]).max(initial=0) <= 1e-12 * max(np.abs(H).max(initial=0), 1e-300)
            assert np.all(bound[t] >= 0)
    for t in np.nonzero(wl.ids < 0)[0]:
        assert h[t].size == 0


@pytest.mark.parametrize("pin", P.SHRINK_BOUND_PINS, ids=lambda f: f.__name__)
def test_shrink_bound_pin(pin):
    pin(shrink_error_bound)


@pytest.mark.parametrize("pin", P.FUSED_PINS, ids=lambda f: f.__name__)
def test_base_fused_pin(pin):
    pin(base_fused_ref)


def test_bf16_round_known_values():
    """Hand-checked roundings: ties go to the even neighbour."""
    one = 1.0
    ulp = 2.0 ** -7  # bfloat16 spacing in [1, 2)
    cases = {
        one: one,
        one + ulp / 2: one,                  # tie, 1.0 is even
        one + 3 * ulp / 2: one + 2 * ulp,    # tie, rounds up to the even neighbour
        one + ulp / 4: one,
        one + 3 * ulp / 4: one + ulp,
        -(one + 3 * ulp / 4): -(one + ulp),
        257.0: 256.0,                        # tie between 256 and 258 -> 256 (even)
        259.0: 260.0,                        # tie between 258 and 260 -> 260 (even)
        0.0: 0.0,
    }
    got = bf16_round_ref(np.array(list(cases.keys())))
    assert list(got) == list(cases.values())


def test_bf16_round_matches_torch_cpu():
    """Library routine: torch's float32 -> bfloat16 conversion (RNE) on the CPU."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(9)
    v = rng.normal(size=20000).astype(np.float32)
    v[:2000] = rng.integers(-2 ** 23, 2 ** 23, size=2000).astype(np.float32)
    bits = v.view(np.uint32) & np.uint32(0xFFFF0000)
    v[2000:4000] = (bits[2000:4000] | np.uint32(0x8000)).view(np.float32)  # exact ties
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf16_round_ref(v.astype(np.float64)), ref)


def test_oracle_header_marks_test_infrastructure():
    assert "TEST INFRASTRUCTURE" in oracle.__doc__


@pytest.mark.parametrize("pin", P.JD_PINS, ids=lambda f: f.__name__)
def test_jd_pin(pin):
    from oracle import jd_apply_ref
    pin(jd_apply_ref)


@pytest.mark.parametrize("pin", P.RANK_PINS, ids=lambda f: f.__name__)
def test_rank_pin(pin):
    from oracle import spectral_ranks_ref, uniform_ranks_ref
    pin(uniform_ranks_ref, lambda r, s, f, b: spectral_ranks_ref(r, s, f, budget=b))


@pytest.mark.parametrize("pin", P.RSVD_PINS, ids=lambda f: f.__name__)
def test_rsvd_pin(pin):
    from oracle import retained_factors_ref
    pin(retained_factors_ref)


def test_tall_skinny_r_pin():
    from oracle import tall_skinny_r_ref
    P.pin_tall_skinny_r(tall_skinny_r_ref)
