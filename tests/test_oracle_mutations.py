"""Plant plausible mistakes in copies of the oracle (CPU only) and check
that the pins catch every one of them."""
import numpy as np
import pytest

from oracle import apply_ref, base_fused_ref, segment_ref, shrink_error_bound

import oracle_pins as P


def _apply_mutant(kind):
    def fn(x, ids, A_list, B_list, scales, y0=None):
        x64 = np.asarray(x, np.float64)
        T = x64.shape[0]
        n = len(A_list)
        d_out = np.asarray(B_list[0]).shape[0]
        y = np.zeros((T, d_out)) if y0 is None else np.asarray(y0, np.float64).copy()
        if kind == "drop_y0" and y0 is not None:
            y = np.zeros_like(y)
        for t in range(T):
            a = int(ids[t])
            if not 0 <= a < n:
                if kind == "invalid_uses_adapter0":
                    a = 0
                else:
                    continue
            if kind == "off_by_one_adapter":
                a = (a + 1) % n
            A = np.asarray(A_list[a], np.float64)
            B = np.asarray(B_list[a], np.float64)
            s = float(scales[a])
            if kind == "drop_scale":
                s = 1.0
            if kind == "neg_sign":
                s = -s
            if kind == "transpose_B" and B.shape[0] == B.shape[1]:
                B = B.T
            if kind == "truncate_rank" and A.shape[0] > 1:
                A, B = A[:-1], B[:, :-1]
            if kind == "scale_squared":
                s = s * s
            h = A @ x64[t]
            if kind == "relu_h":
                h = np.maximum(h, 0)
            y[t] += s * (B @ h)
        return y
    return fn


APPLY_MUTANTS = ["drop_y0", "invalid_uses_adapter0", "off_by_one_adapter", "drop_scale", "neg_sign",
                 "transpose_B", "truncate_rank", "scale_squared", "relu_h"]


@pytest.mark.parametrize("kind", APPLY_MUTANTS)
def test_apply_mutant_is_caught(kind):
    fn = _apply_mutant(kind)
    caught = []
    for pin in P.APPLY_PINS:
        try:
            pin(fn)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {kind} passed every pin"


def test_unmutated_copy_passes():
    fn = _apply_mutant("none")
    for pin in P.APPLY_PINS:
        pin(fn)


def _segment_mutant(kind):
    def fn(ids, n):
        seg_off, perm, n_inv = segment_ref(ids, n)
        perm = list(perm)
        seg_off = list(seg_off)
        if kind == "unstable" and len(perm) > 1:
            # reverse the order inside each group
            for g in range(n + 1):
                perm[seg_off[g]:seg_off[g + 1]] = perm[seg_off[g]:seg_off[g + 1]][::-1]
        elif kind == "invalid_first":
            key = [n if not 0 <= int(v) < n else int(v) for v in ids]
            order = sorted(range(len(ids)), key=lambda t: (-1 if key[t] == n else key[t], t))
            perm = order
        elif kind == "inclusive_offsets":
            seg_off = seg_off[1:] + [seg_off[-1]]
        elif kind == "count_minus_one_as_invalid":
            n_inv = sum(1 for v in ids if not 0 <= int(v) < n)
        return seg_off, perm, n_inv
    return fn


@pytest.mark.parametrize("kind", ["unstable", "invalid_first", "inclusive_offsets",
                                  "count_minus_one_as_invalid"])
def test_segment_mutant_is_caught(kind):
    fn = _segment_mutant(kind)
    caught = []
    for pin in P.SEGMENT_PINS:
        try:
            pin(fn)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"segment mutant {kind} passed every pin"


def _jd_mutant(kind):
    def fn(x, ids, cluster_of, U_list, V_list, sigma, scales, y0=None):
        x64 = np.asarray(x, np.float64)
        T = x64.shape[0]
        n = len(cluster_of)
        d_out = np.asarray(U_list[0]).shape[0]
        y = np.zeros((T, d_out)) if y0 is None else np.asarray(y0, np.float64).copy()
        for t in range(T):
            a = int(ids[t])
            if not 0 <= a < n:
                continue
            c = int(cluster_of[a])
            if kind == "cluster_zero":
                c = 0
            if kind == "cluster_by_adapter":
                c = a % len(U_list)
            if not 0 <= c < len(U_list):
                continue
            U = np.asarray(U_list[c], np.float64)
            V = np.asarray(V_list[c], np.float64)
            S = np.asarray(sigma[a], np.float64)
            if kind == "sigma_of_next_adapter":
                S = np.asarray(sigma[(a + 1) % n], np.float64)
            if S.ndim == 1:
                S = np.diag(S)
            if kind == "sigma_transposed":
                S = S.T
            if kind == "sigma_dropped":
                S = np.eye(S.shape[0])
            s = float(scales[a])
            if kind == "drop_scale":
                s = 1.0
            h = V.T @ x64[t]
            if kind == "h_abs":
                h = np.abs(h)
            g = S @ h
            if kind == "sigma_twice":
                g = S @ g
            y[t] += s * (U @ g)
        return y
    return fn


JD_MUTANTS = ["cluster_zero", "cluster_by_adapter", "sigma_of_next_adapter", "sigma_transposed", "sigma_dropped",
              "drop_scale", "h_abs", "sigma_twice"]


@pytest.mark.parametrize("kind", JD_MUTANTS)
def test_jd_mutant_is_caught(kind):
    fn = _jd_mutant(kind)
    caught = []
    for pin in P.JD_PINS:
        try:
            pin(fn)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"shared-basis mutant {kind} passed every pin"


def test_jd_unmutated_copy_passes():
    fn = _jd_mutant("none")
    for pin in P.JD_PINS:
        pin(fn)


def _rank_mutants(kind):
    import math
    from oracle import spectral_ranks_ref, uniform_ranks_ref

    def uni(r_orig, ratio, floor):
        if kind == "uniform_round":
            return [min(r, max(floor, round(ratio * r))) for r in r_orig]
        if kind == "uniform_no_floor":
            return [min(r, math.ceil(ratio * r)) for r in r_orig]
        if kind == "uniform_floor_beyond_rank":
            return [max(floor, math.ceil(ratio * r)) for r in r_orig]
        return uniform_ranks_ref(r_orig, ratio, floor)

    def spec(r_orig, sig, floor, budget):
        if kind == "spectral_smallest_first":
            # 1/sigma is largest where sigma is smallest
            return spectral_ranks_ref(r_orig, [[1.0 / (1e-9 + abs(v)) for v in s] for s in sig], floor, budget=budget)
        if kind == "spectral_no_floor":
            return spectral_ranks_ref(r_orig, sig, 0, budget=budget)
        if kind == "spectral_budget_minus_one":
            return spectral_ranks_ref(r_orig, sig, floor, budget=budget - 1)
        if kind == "spectral_ties_high_first":
            rev = spectral_ranks_ref(r_orig[::-1], sig[::-1], floor, budget=budget)
            return rev[::-1]
        return spectral_ranks_ref(r_orig, sig, floor, budget=budget)
    return uni, spec


RANK_MUTANTS = ["uniform_round", "uniform_no_floor", "uniform_floor_beyond_rank", "spectral_smallest_first",
                "spectral_no_floor", "spectral_budget_minus_one", "spectral_ties_high_first"]


@pytest.mark.parametrize("kind", RANK_MUTANTS)
def test_rank_mutant_is_caught(kind):
    uni, spec = _rank_mutants(kind)
    caught = []
    for pin in P.RANK_PINS:
        try:
            pin(uni, spec)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"rank-policy mutant {kind} passed every pin"


def _rsvd_mutant(kind):
    def fn(A, B, k):
        A64, B64 = np.asarray(A, np.float64), np.asarray(B, np.float64)
        Q_B, R_B = np.linalg.qr(B64)
        Q_A, R_A = np.linalg.qr(A64.T)
        core = R_B @ R_A if kind == "core_untransposed" else R_B @ R_A.T
        U, s, Vt = np.linalg.svd(core)
        if kind == "smallest_components":
            U, s, Vt = U[:, ::-1], s[::-1], Vt[::-1, :]
        B2 = Q_B @ U[:, :k]
        A2 = (s[:k, None] * Vt[:k, :]) @ Q_A.T
        if kind == "drop_sigma":
            A2 = Vt[:k, :] @ Q_A.T
        if kind == "sigma_on_both":
            B2 = B2 * s[None, :k]
        if kind == "no_q_a":
            A2 = np.pad(s[:k, None] * Vt[:k, :], ((0, 0), (0, A64.shape[1] - Vt.shape[1])))
        return A2, B2, s
    return fn


RSVD_MUTANTS = ["core_untransposed", "smallest_components", "drop_sigma", "sigma_on_both", "no_q_a"]


@pytest.mark.parametrize("kind", RSVD_MUTANTS)
def test_rsvd_mutant_is_caught(kind):
    fn = _rsvd_mutant(kind)
    caught = []
    for pin in P.RSVD_PINS:
        try:
            pin(fn)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"r-SVD mutant {kind} passed every pin"


def _bound_mutant(kind):
    """Copies of the float32 bound of h with a plausible mistake planted."""
    def fn(x, ids, A_list):
        x64 = np.abs(np.asarray(x, np.float64))
        out = []
        for t in range(x64.shape[0]):
            a = int(ids[t])
            if not 0 <= a < len(A_list):
                out.append(np.zeros(0))
                continue
            A = np.asarray(A_list[a], np.float64)
            d = A.shape[1]
            u = 2.0 ** -16 if kind == "unit_2^-16" else 2.0 ** -24
            n = {"no_d_in": 1, "sqrt_d_in": np.sqrt(d), "d_in_squared": d * d}.get(kind, d)
            if kind == "abs_of_sum":
                s = np.abs(A @ np.asarray(x, np.float64)[t])  # |sum| instead of sum of |.|
            else:
                s = np.abs(A) @ x64[t]
            out.append(n * u / (1 - min(n * u, 0.5)) * s)
        return out
    return fn


BOUND_MUTANTS = ["unit_2^-16", "no_d_in", "sqrt_d_in", "d_in_squared", "abs_of_sum"]


@pytest.mark.parametrize("kind", BOUND_MUTANTS)
def test_bound_mutant_is_caught(kind):
    fn = _bound_mutant(kind)
    caught = []
    for pin in P.SHRINK_BOUND_PINS:
        try:
            pin(fn)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {kind} passed every pin"


def test_bound_unmutated_copy_passes():
    fn = _bound_mutant("none")
    for pin in P.SHRINK_BOUND_PINS:
        pin(fn)
    for pin in P.SHRINK_BOUND_PINS:
        pin(shrink_error_bound)


def _fused_mutant(kind):
    """Copies of the base-fused oracle with a plausible mistake planted."""
    def fn(x, ids, W0, A_list, B_list, scales):
        W = np.asarray(W0, np.float64)
        if kind == "base_transposed" and W.shape[0] == W.shape[1]:
            W = W.T
        if kind == "no_base":
            W = np.zeros_like(W)
        y = np.asarray(x, np.float64) @ W.T
        if kind == "base_twice":
            y = 2 * y
        if kind == "base_only_with_adapter":
            keep = np.array([0 <= int(a) < len(A_list) for a in ids])
            y = y * keep[:, None]
        delta = apply_ref(x, ids, A_list, B_list, scales, y0=np.zeros_like(y))
        if kind == "no_branch":
            delta = 0 * delta
        if kind == "branch_twice":
            delta = 2 * delta
        return y + delta
    return fn


FUSED_MUTANTS = ["base_transposed", "no_base", "base_twice", "base_only_with_adapter", "no_branch", "branch_twice"]


@pytest.mark.parametrize("kind", FUSED_MUTANTS)
def test_fused_mutant_is_caught(kind):
    fn = _fused_mutant(kind)
    caught = []
    for pin in P.FUSED_PINS:
        try:
            pin(fn)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {kind} passed every pin"


def test_fused_unmutated_copy_passes():
    for pin in P.FUSED_PINS:
        pin(_fused_mutant("none"))
        pin(base_fused_ref)
