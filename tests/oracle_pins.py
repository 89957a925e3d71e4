"""Pins for the CPU oracle: checks against what the sources and the
mathematics fix, independent of the oracle's own code.

Each check takes the function under test as an argument so that the same
checks can be run on deliberately broken copies of the oracle
(tests/test_oracle_mutations.py) to show that they catch plausible mistakes.
Each check raises AssertionError on failure.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

from workloads import make_config, make_integer_workload, make_random_workload

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_worked_example():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        ex = json.load(f)
    A = [np.array(a, dtype=np.float32).reshape(r, ex["d_in"]) for a, r in zip(ex["A"], ex["ranks"])]
    B = [np.array(b, dtype=np.float32).reshape(ex["d_out"], r) for b, r in zip(ex["B"], ex["ranks"])]
    return ex, A, B


# ---------------------------------------------------------------- apply pins

def pin_worked_example(apply_fn):
    """Hand-worked example from the LoRA definition (tests/golden)."""
    ex, A, B = load_worked_example()
    y = apply_fn(np.array(ex["x"], np.float32), np.array(ex["ids"], np.int32), A, B,
                 np.array(ex["scales"], np.float32), np.array(ex["y0"], np.float32))
    assert np.array_equal(np.asarray(y, np.float64), np.array(ex["expected_y"], np.float64)), y


def pin_merged_weight(apply_fn, wl=None, seed=0):
    """With y0 = 0 the delta equals x (W + s B A)^T - x W^T for any W
    (merged form W0 -> W0 + B_i A_i versus the separate branch, Compress then
    Serve section 11).  The merged form is built with dense numpy products."""
    wl = wl or make_config("1")
    m = wl.module
    rng = np.random.default_rng(seed)
    W = rng.normal(size=(m.d_out, m.d_in))
    x = wl.x.astype(np.float64)
    ref = np.zeros((wl.T, m.d_out))
    for t in range(wl.T):
        a = int(wl.ids[t])
        if not 0 <= a < m.n:
            continue
        merged = W + float(m.scales[a]) * (m.B[a].astype(np.float64) @ m.A[a].astype(np.float64))
        ref[t] = merged @ x[t] - W @ x[t]
    y = np.asarray(apply_fn(wl.x, wl.ids, m.A, m.B, m.scales), np.float64)
    scale = max(np.abs(ref).max(), 1e-300)
    assert np.abs(y - ref).max() <= 1e-10 * scale, np.abs(y - ref).max() / scale


def pin_rank_zero(apply_fn):
    """An adapter with retained rank 0 contributes an exactly zero delta."""
    wl = make_random_workload(1, 24, 3, 16, 8, [0, 2, 0], dtype="fp32")
    m = wl.module
    y = np.asarray(apply_fn(wl.x, wl.ids, m.A, m.B, m.scales), np.float64)
    for t in range(wl.T):
        if m.ranks[wl.ids[t]] == 0:
            assert np.all(y[t] == 0.0), (t, y[t])
    assert np.any(y != 0.0)


def pin_scale_linearity(apply_fn):
    """The delta is linear in s: doubling s doubles it exactly; s1 + s2 adds."""
    wl = make_random_workload(2, 20, 4, 32, 24, [1, 3, 5, 2], dtype="bf16")
    m = wl.module
    y1 = np.asarray(apply_fn(wl.x, wl.ids, m.A, m.B, m.scales), np.float64)
    y2 = np.asarray(apply_fn(wl.x, wl.ids, m.A, m.B, m.scales * 2), np.float64)
    assert np.array_equal(y2, 2 * y1)
    s2 = np.full(m.n, 0.375, np.float32)
    y3 = np.asarray(apply_fn(wl.x, wl.ids, m.A, m.B, s2), np.float64)
    y4 = np.asarray(apply_fn(wl.x, wl.ids, m.A, m.B, m.scales + s2), np.float64)
    assert np.abs(y4 - (y1 + y3)).max() <= 1e-12 * max(np.abs(y4).max(), 1e-300)


def pin_zero_padding(apply_fn):
    """Appending zero rows to A_a and zero columns to B_a (any larger rank)
    leaves the result unchanged: padding is neutral, only wasteful."""
    wl = make_random_workload(3, 30, 5, 40, 24, [1, 2, 3, 4, 7], dtype="bf16")
    m = wl.module
    rng = np.random.default_rng(3)
    Ap, Bp = [], []
    for a in range(m.n):
        r = int(m.ranks[a]) + int(rng.integers(1, 9))
        A = np.zeros((r, m.d_in), np.float32)
        B = np.zeros((m.d_out, r), np.float32)
        A[: m.ranks[a]] = m.A[a]
        B[:, : m.ranks[a]] = m.B[a]
        Ap.append(A)
        Bp.append(B)
    y = np.asarray(apply_fn(wl.x, wl.ids, m.A, m.B, m.scales), np.float64)
    yp = np.asarray(apply_fn(wl.x, wl.ids, Ap, Bp, m.scales), np.float64)
    assert np.abs(y - yp).max() <= 1e-13 * max(np.abs(y).max(), 1e-300)


def pin_brute_force(apply_fn, brute_fn):
    """Exact rational triple loops on tiny inputs, both association orders."""
    for seed, (T, n, di, do, ranks) in enumerate([(5, 2, 3, 4, [1, 2]), (7, 3, 4, 3, [2, 0, 3])]):
        wl = make_random_workload(10 + seed, T, n, di, do, ranks, dtype="bf16", y0=True,
                                  invalid_frac=0.2)
        m = wl.module
        exact = brute_fn(wl.x, wl.ids, m.A, m.B, m.scales, wl.y0, form="B(Ax)")
        merged = brute_fn(wl.x, wl.ids, m.A, m.B, m.scales, wl.y0, form="(BA)x")
        assert exact == merged
        y = np.asarray(apply_fn(wl.x, wl.ids, m.A, m.B, m.scales, wl.y0), np.float64)
        ref = np.array([[float(v) for v in row] for row in exact])
        assert np.abs(y - ref).max() <= 1e-13 * max(np.abs(ref).max(), 1.0)


def pin_integer_exact(apply_fn, brute_fn):
    """Integer inputs and power-of-two scales: the float64 result is exact."""
    wl = make_random_workload(20, 9, 3, 6, 5, [2, 3, 1], dtype="fp32", integer=True,
                              scales=[0.5, 2.0, 1.0])
    m = wl.module
    exact = brute_fn(wl.x, wl.ids, m.A, m.B, m.scales)
    y = np.asarray(apply_fn(wl.x, wl.ids, m.A, m.B, m.scales), np.float64)
    assert all(Fraction(float(y[t, o])) == exact[t][o] for t in range(wl.T) for o in range(m.d_out))


def pin_token_permutation(apply_fn):
    """Tokens are independent: permuting tokens permutes outputs exactly."""
    wl = make_random_workload(4, 33, 4, 24, 16, [3, 1, 4, 2], dtype="bf16", y0=True,
                              invalid_frac=0.1)
    m = wl.module
    p = np.random.default_rng(4).permutation(wl.T)
    y = np.asarray(apply_fn(wl.x, wl.ids, m.A, m.B, m.scales, wl.y0), np.float64)
    yp = np.asarray(apply_fn(wl.x[p], wl.ids[p], m.A, m.B, m.scales, wl.y0[p]), np.float64)
    assert np.array_equal(yp, y[p])


def pin_per_segment(apply_fn):
    """Per adapter group: delta = s_a (X_seg A_a^T) B_a^T with numpy products
    (the stacked-bmm form of Compress then Serve section 11)."""
    wl = make_random_workload(5, 64, 6, 48, 40, [1, 2, 4, 8, 3, 5], dtype="bf16", id_mode="zipf")
    m = wl.module
    y = np.asarray(apply_fn(wl.x, wl.ids, m.A, m.B, m.scales), np.float64)
    for a in range(m.n):
        rows = np.nonzero(wl.ids == a)[0]
        if len(rows) == 0:
            continue
        X = wl.x[rows].astype(np.float64)
        d = float(m.scales[a]) * ((X @ m.A[a].astype(np.float64).T) @ m.B[a].astype(np.float64).T)
        assert np.abs(y[rows] - d).max() <= 1e-12 * max(np.abs(d).max(), 1e-300)


def pin_no_adapter_tokens(apply_fn):
    """Tokens with id -1 keep y0 exactly."""
    wl = make_random_workload(6, 40, 3, 16, 16, [2, 2, 2], dtype="bf16", y0=True, invalid_frac=0.4)
    m = wl.module
    y = np.asarray(apply_fn(wl.x, wl.ids, m.A, m.B, m.scales, wl.y0), np.float64)
    mask = wl.ids < 0
    assert mask.any()
    assert np.array_equal(y[mask], wl.y0[mask].astype(np.float64))
    assert not np.array_equal(y[~mask], wl.y0[~mask].astype(np.float64))


APPLY_PINS = (pin_worked_example, pin_merged_weight, pin_rank_zero, pin_scale_linearity,
              pin_zero_padding, pin_token_permutation, pin_per_segment, pin_no_adapter_tokens)


# ------------------------------------------------------- base-fused pins
# y = W0 x + s_a B_a A_a x per token ("Compress then Serve" sections 3 and
# 11).  Each pin takes fn(x, ids, W0, A_list, B_list, scales).

def _fused_case(seed=0, d_in=24, d_out=40):
    wl = make_random_workload(60 + seed, 37, 5, d_in, d_out, [3, 0, 6, 1, 8], dtype="bf16", id_mode="zipf",
                              invalid_frac=0.15)
    W0 = np.random.default_rng(seed).normal(size=(d_out, d_in)) / np.sqrt(d_in)
    return wl, W0


def pin_fused_merged_weight(fn):
    """Equals x (W0 + s_a B_a A_a)^T per token: the merged weight of the
    token's adapter (W0 alone without one), applied with one numpy product."""
    for seed, (di, do) in enumerate(((24, 40), (32, 32), (48, 16))):
        wl, W0 = _fused_case(seed, di, do)
        m = wl.module
        ref = np.zeros((wl.T, do))
        for t in range(wl.T):
            a = int(wl.ids[t])
            Wm = W0.copy()
            if 0 <= a < m.n:
                Wm = Wm + float(m.scales[a]) * (m.B[a].astype(np.float64) @ m.A[a].astype(np.float64))
            ref[t] = wl.x[t].astype(np.float64) @ Wm.T
        y = np.asarray(fn(wl.x, wl.ids, W0, m.A, m.B, m.scales), np.float64)
        assert y.shape == ref.shape
        assert np.abs(y - ref).max() <= 1e-12 * max(np.abs(ref).max(), 1.0), np.abs(y - ref).max()


def pin_fused_no_adapter_is_base(fn):
    """With every id outside [0, n), the result is the base product x W0^T
    (numpy), whatever the factors."""
    wl, W0 = _fused_case(3)
    m = wl.module
    ids = np.full(wl.T, -1, np.int32)
    ids[::5] = m.n + 2
    y = np.asarray(fn(wl.x, ids, W0, m.A, m.B, m.scales), np.float64)
    ref = wl.x.astype(np.float64) @ W0.T
    assert np.abs(y - ref).max() <= 1e-12 * np.abs(ref).max()


def pin_fused_zero_base(fn):
    """With W0 = 0 only the branch remains: for integer inputs, exactly the
    rational B (A x) of every token (brute force)."""
    wl = make_integer_workload("1")
    m = wl.module
    W0 = np.zeros((m.d_out, m.d_in))
    y = np.asarray(fn(wl.x[:6], wl.ids[:6], W0, m.A, m.B, m.scales), np.float64)
    from oracle import brute_force
    exact = brute_force(wl.x[:6], wl.ids[:6], m.A, m.B, m.scales)
    assert [[float(v) for v in row] for row in exact] == y.tolist()


def pin_fused_linear_in_base(fn):
    """The result is affine in W0: f(W1 + W2) = f(W1) + f(W2) - f(0)."""
    wl, W1 = _fused_case(4)
    m = wl.module
    W2 = np.random.default_rng(9).normal(size=W1.shape)
    f = lambda W: np.asarray(fn(wl.x, wl.ids, W, m.A, m.B, m.scales), np.float64)
    lhs = f(W1 + W2)
    rhs = f(W1) + f(W2) - f(np.zeros_like(W1))
    assert np.abs(lhs - rhs).max() <= 1e-12 * max(np.abs(lhs).max(), 1.0)


FUSED_PINS = (pin_fused_merged_weight, pin_fused_no_adapter_is_base, pin_fused_zero_base, pin_fused_linear_in_base)


# -------------------------------------------------------------- segment pins

def pin_segment_worked_example(segment_fn):
    ex, _, _ = load_worked_example()
    seg_off, perm, n_inv = segment_fn(ex["ids"], ex["n"])
    assert list(seg_off) == ex["expected_seg_off"], seg_off
    assert list(perm) == ex["expected_perm"], perm
    assert n_inv == 0


def pin_segment_vs_stable_argsort(segment_fn):
    """perm equals numpy's stable argsort of ids (out-of-range ids mapped to
    n); seg_off equals the cumulative bincount."""
    rng = np.random.default_rng(7)
    for T, n in [(0, 3), (1, 1), (17, 4), (200, 16), (513, 300), (64, 1)]:
        ids = rng.integers(-1, n, size=T).astype(np.int32)
        if T > 3:
            ids[rng.integers(0, T, size=2)] = [n + 5, -7]
        key = np.where((ids >= 0) & (ids < n), ids, n)
        seg_off, perm, n_inv = segment_fn(ids, n)
        assert list(perm) == list(np.argsort(key, kind="stable"))
        exp_off = np.concatenate([[0], np.cumsum(np.bincount(key, minlength=n + 1))])
        assert list(seg_off) == list(exp_off)
        assert n_inv == int(np.sum((ids != -1) & ((ids < 0) | (ids >= n))))


def pin_segment_invariants(segment_fn):
    """perm is a permutation, ids[perm] is non-decreasing, positions increase
    inside each group, empty groups have zero length."""
    ids = np.array([3, 3, 0, 5, 3, 0, 0, 5, 5, 5], np.int32)
    seg_off, perm, _ = segment_fn(ids, 7)
    assert sorted(perm) == list(range(len(ids)))
    g = ids[np.array(perm)]
    assert np.all(np.diff(g) >= 0)
    for a in range(7):
        members = perm[seg_off[a]:seg_off[a + 1]]
        assert list(members) == sorted(members)
        assert all(ids[t] == a for t in members)
    assert seg_off[1] - seg_off[0] == 3 and seg_off[2] == seg_off[1] and seg_off[-1] == len(ids)


SEGMENT_PINS = (pin_segment_worked_example, pin_segment_vs_stable_argsort, pin_segment_invariants)


# ------------------------------------------------- float32 bound of the shrink
# The intermediate h = A_a x is accumulated in float32 (Compress then Serve
# section 13.4: a float32 buffer).  shrink_error_bound(x, ids, A_list) gives,
# per token and retained rank, the largest |h_float32 - h_exact| that any
# summation order may produce.  The pins below simulate float32 summation in
# several orders (numpy float32 arithmetic, one rounding per addition) on
# inputs chosen to make rounding errors large, and compare with the exact
# sum (bf16 x bf16 products are exact in float64; math.fsum rounds their sum
# once).  They are checked against what rounding actually does, not against
# the bound's formula.

_U32 = 2.0 ** -24  # float32 unit roundoff (round to nearest)


def _bf16_exact(v):
    """Round float64 values to the nearest bfloat16 (ties to even) by bit
    manipulation of their float32 image; the inputs below are chosen exact."""
    f = np.asarray(v, np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return b.astype(np.uint32).view(np.float32)


def _sum32(p, order):
    """float32 sum of the last axis of p (products, exact in float32) in a
    given order: 'fwd', 'rev', 'pairwise' (recursive halving) or 'blocked'
    (64-term blocks summed in turn, then the block sums in turn)."""
    p = np.asarray(p, np.float32)
    if order == "rev":
        p = p[..., ::-1]
    if order in ("fwd", "rev"):
        s = np.zeros(p.shape[:-1], np.float32)
        for k in range(p.shape[-1]):
            s = np.float32(s + p[..., k])
        return s
    if order == "pairwise":
        while p.shape[-1] > 1:
            if p.shape[-1] % 2:
                p = np.concatenate([p, np.zeros(p.shape[:-1] + (1,), np.float32)], axis=-1)
            p = (p[..., 0::2] + p[..., 1::2]).astype(np.float32)
        return p[..., 0]
    if order == "blocked":
        n = p.shape[-1]
        blocks = [_sum32(p[..., i:i + 64], "fwd") for i in range(0, n, 64)]
        return _sum32(np.stack(blocks, axis=-1), "fwd")
    raise ValueError(order)


def _bound_cases(d=18944):
    """Tokens paired with one-row adapters (token t uses adapter t), bf16-exact:
      0 stagnation: 2^24 followed by d-1 ones; each float32 addition of 1 to
        2^24 is a tie that rounds back to 2^24, so sequential summation loses
        every one of them (the error reaches (d-1)/d of the first-order bound);
      1 cancellation: 2^24 + 1 - 2^24 (the exact sum 1 is lost to rounding);
      2 equal terms (1 + 2^-7)^2, whose rounding errors all have one sign;
      3 mixed magnitudes: N(0,1) values scaled by 2^e, e uniform in [-20, 20];
      4 N(0,1) bf16 values."""
    rng = np.random.default_rng(23)
    X = np.zeros((5, d), np.float64)
    A = np.zeros((5, d), np.float64)
    X[0, 0], A[0, 0] = 2.0 ** 12, 2.0 ** 12
    X[0, 1:], A[0, 1:] = 1.0, 1.0
    X[1, :3] = [2.0 ** 12, 1.0, 2.0 ** 12]
    A[1, :3] = [2.0 ** 12, 1.0, -(2.0 ** 12)]
    X[2, :], A[2, :] = 1.0 + 2.0 ** -7, 1.0 + 2.0 ** -7
    X[3] = rng.normal(size=d) * 2.0 ** rng.integers(-20, 21, size=d)
    A[3] = rng.normal(size=d) * 2.0 ** rng.integers(-20, 21, size=d)
    X[4], A[4] = rng.normal(size=d), rng.normal(size=d)
    X, A = _bf16_exact(X), _bf16_exact(A)
    return X, [A[t:t + 1] for t in range(5)], np.arange(5, dtype=np.int32)


def _exact_dots(X, A_list, ids):
    import math
    out = []
    for t, a in enumerate(ids):
        p = np.asarray(A_list[a], np.float64) * np.asarray(X[t], np.float64)  # exact products
        out.append(np.array([math.fsum(row) for row in p]))
    return out


def pin_shrink_bound_sound(bound_fn):
    """No float32 summation order exceeds the bound on the adversarial cases
    (any order the GPU may take: sequential either way, pairwise, blocked)."""
    X, A_list, ids = _bound_cases()
    bound = bound_fn(X, ids, A_list)
    exact = _exact_dots(X, A_list, ids)
    for order in ("fwd", "rev", "pairwise", "blocked"):
        for t, a in enumerate(ids):
            p = (np.asarray(A_list[a], np.float32) * np.asarray(X[t], np.float32))
            h32 = _sum32(p, order).astype(np.float64)
            err = np.abs(h32 - exact[t])
            assert np.all(err <= np.asarray(bound[t])), (order, t, err, bound[t])


def pin_shrink_bound_attained(bound_fn):
    """The bound is nearly reached: sequential summation of the stagnation
    case loses d - 1 of a first-order bound of d u (2^24 + d - 1)."""
    X, A_list, ids = _bound_cases()
    bound = bound_fn(X, ids, A_list)
    exact = _exact_dots(X, A_list, ids)
    p = np.asarray(A_list[0], np.float32) * np.asarray(X[0], np.float32)
    err = abs(float(_sum32(p, "fwd")[0]) - float(exact[0][0]))
    assert err == X.shape[1] - 1, err
    assert err >= 0.99 * float(np.asarray(bound[0])[0]), (err, bound[0])


def pin_shrink_bound_shape(bound_fn):
    """One non-negative value per retained rank for tokens with an adapter,
    none for the others; zero for a zero input."""
    wl = make_random_workload(6, 12, 3, 16, 4, [2, 0, 3], dtype="bf16", id_mode="uniform", invalid_frac=0.3)
    m = wl.module
    b = bound_fn(wl.x, wl.ids, m.A)
    for t, a in enumerate(wl.ids):
        if 0 <= a < m.n:
            assert np.asarray(b[t]).shape == (m.ranks[a],) and np.all(np.asarray(b[t]) >= 0)
        else:
            assert np.asarray(b[t]).size == 0
    z = bound_fn(np.zeros_like(wl.x), wl.ids, m.A)
    assert all(np.all(np.asarray(v) == 0) for v in z)


SHRINK_BOUND_PINS = (pin_shrink_bound_sound, pin_shrink_bound_attained, pin_shrink_bound_shape)


# ------------------------------------------------------- shared-basis pins
# The shared-basis (joint-diagonalization) apply of "Compress then Serve"
# sections 3.1-3.2 and 11: y += s_i U_j Sigma_i V_j^T x for adapter i in
# cluster j.  Each pin takes the function under test (the signature of
# oracle.jd_apply_ref).

def _jd_small(mode, seed=0, **kw):
    from workloads import make_jd_workload
    args = dict(T=30, n=7, k=3, d_in=24, d_out=20, r=5)
    args.update(kw)
    return make_jd_workload(seed, args["T"], args["n"], args["k"], args["d_in"], args["d_out"], args["r"],
                            mode=mode, dtype="fp32", id_mode="uniform", invalid_frac=0.1)


def _jd_call(fn, w, **over):
    args = dict(x=w.x, ids=w.ids, cluster_of=w.cluster_of, U_list=w.U, V_list=w.V, sigma=w.sigma,
                scales=w.scales)
    args.update(over)
    return np.asarray(fn(args["x"], args["ids"], args["cluster_of"], args["U_list"], args["V_list"],
                         args["sigma"], args["scales"], over.get("y0")), np.float64)


def pin_jd_merged_weight(fn):
    """With y0 = 0 the delta equals x (W + s U Sigma V^T)^T - x W^T for any W
    (the merged form of section 11 with B_i A_i = U Sigma_i V^T), for full
    and diagonal Sigma; the merged matrix is built with dense products."""
    for mode in ("full", "diag"):
        w = _jd_small(mode, seed=1)
        rng = np.random.default_rng(2)
        W = rng.normal(size=(w.d_out, w.d_in))
        ref = np.zeros((w.T, w.d_out))
        for t in range(w.T):
            a = int(w.ids[t])
            if not 0 <= a < w.n:
                continue
            c = int(w.cluster_of[a])
            S = w.sigma[a].astype(np.float64)
            S = S if S.ndim == 2 else np.diag(S)
            M = W + float(w.scales[a]) * (w.U[c].astype(np.float64) @ S @ w.V[c].astype(np.float64).T)
            ref[t] = M @ w.x[t].astype(np.float64) - W @ w.x[t].astype(np.float64)
        y = _jd_call(fn, w)
        assert np.abs(y - ref).max() <= 1e-10 * max(np.abs(ref).max(), 1e-300), mode


def pin_jd_diag_is_lora(fn):
    """A diagonal Sigma_i is a LoRA adapter with B_i = U_j diag(Sigma_i) and
    A_i = V_j^T (section 3.1): the result equals the LoRA oracle's on those
    factors."""
    from oracle import apply_ref
    w = _jd_small("diag", seed=3)
    A = [w.V[int(w.cluster_of[a])].astype(np.float64).T for a in range(w.n)]
    B = [w.U[int(w.cluster_of[a])].astype(np.float64) * w.sigma[a].astype(np.float64)[None, :] for a in range(w.n)]
    ref = apply_ref(w.x, w.ids, A, B, w.scales)
    y = _jd_call(fn, w)
    assert np.abs(y - ref).max() <= 1e-12 * max(np.abs(ref).max(), 1e-300)


def pin_jd_exact_reconstruction(fn):
    """JD-Full with orthonormal U, V: for adapters whose B_i A_i lies in
    span(U) x span(V), the optimal Sigma_i = U^T B_i A_i V (section 8.1,
    equation 6) reproduces B_i A_i exactly, so the apply equals the LoRA
    oracle on the original B_i, A_i."""
    from oracle import apply_ref
    rng = np.random.default_rng(4)
    T, n, k, d_in, d_out, r = 25, 5, 2, 18, 14, 4
    U = [np.linalg.qr(rng.normal(size=(d_out, r)))[0] for _ in range(k)]
    V = [np.linalg.qr(rng.normal(size=(d_in, r)))[0] for _ in range(k)]
    cluster_of = rng.integers(0, k, size=n)
    A_l, B_l, sig = [], [], []
    for a in range(n):
        c = cluster_of[a]
        ra = 1 + a % 3
        Ba = U[c] @ rng.normal(size=(r, ra))
        Aa = rng.normal(size=(ra, r)) @ V[c].T
        A_l.append(Aa)
        B_l.append(Ba)
        sig.append(U[c].T @ (Ba @ Aa) @ V[c])
    x = rng.normal(size=(T, d_in))
    ids = rng.integers(-1, n, size=T)
    scales = rng.random(n) + 0.5
    ref = apply_ref(x, ids, A_l, B_l, scales)
    y = np.asarray(fn(x, ids, cluster_of, U, V, np.array(sig), scales, None), np.float64)
    assert np.abs(y - ref).max() <= 1e-10 * max(np.abs(ref).max(), 1e-300)


def pin_jd_brute_force(fn):
    """Tiny integer inputs: equal to exact rational loops in both association
    orders, U (Sigma (V^T x)) and (U Sigma V^T) x, for full and diagonal Sigma."""
    from oracle import jd_brute_force
    from workloads import make_jd_workload
    for mode in ("full", "diag"):
        w = make_jd_workload(5, 6, 4, 2, 5, 4, 3, mode=mode, dtype="fp32", id_mode="uniform",
                             invalid_frac=0.2, integer=True)
        y = _jd_call(fn, w)
        for form in ("U(S(Vx))", "(USV)x"):
            ex = jd_brute_force(w.x, w.ids, w.cluster_of, w.U, w.V, w.sigma, w.scales, form=form)
            assert np.array_equal(y, np.array([[float(v) for v in row] for row in ex])), (mode, form)


def pin_jd_zero_scale_invalid(fn):
    """Sigma = 0 gives an exactly zero delta; doubling every scale doubles the
    delta bit for bit; a token without adapter (-1) keeps y0."""
    w = _jd_small("full", seed=6)
    y0 = np.random.default_rng(7).normal(size=(w.T, w.d_out))
    y = _jd_call(fn, w, sigma=np.zeros_like(w.sigma), y0=y0)
    assert np.array_equal(y, y0)
    d1 = _jd_call(fn, w)
    d2 = _jd_call(fn, w, scales=w.scales * 2)
    assert np.array_equal(d2, 2 * d1)
    none = np.full(w.T, -1, np.int32)
    assert np.array_equal(_jd_call(fn, w, ids=none, y0=y0), y0)
    # an adapter outside every cluster (cluster -1 or k) adds nothing; the others are unchanged
    cl = w.cluster_of.copy()
    cl[0], cl[1] = -1, w.k
    y_cut = _jd_call(fn, w, cluster_of=cl, y0=y0)
    y_all = _jd_call(fn, w, y0=y0)
    cut = np.isin(w.ids, [0, 1])
    assert np.array_equal(y_cut[cut], y0[cut]) and np.array_equal(y_cut[~cut], y_all[~cut])


def pin_jd_cluster_relabel(fn):
    """Renaming the clusters (and permuting U, V alike) changes nothing."""
    w = _jd_small("full", seed=8)
    perm = np.array([2, 0, 1])  # new label of old cluster c
    inv = np.argsort(perm)
    y1 = _jd_call(fn, w)
    y2 = _jd_call(fn, w, cluster_of=perm[w.cluster_of], U_list=[w.U[inv[c]] for c in range(w.k)],
                  V_list=[w.V[inv[c]] for c in range(w.k)])
    assert np.array_equal(y1, y2)


JD_PINS = [pin_jd_merged_weight, pin_jd_diag_is_lora, pin_jd_exact_reconstruction, pin_jd_brute_force,
           pin_jd_zero_scale_invalid, pin_jd_cluster_relabel]


# ------------------------------------------------------------ rank policies
# Retained-rank allocation (LoRAForge core design section: uniform ratio with
# a floor, spectral budget).  Pins take (uniform_fn, spectral_fn).

def _rank_units(seed, n=12, r_hi=16):
    rng = np.random.default_rng(seed)
    r_orig = [int(v) for v in rng.integers(1, r_hi + 1, size=n)]
    sig = [sorted(rng.gamma(2.0, 1.0, size=r).tolist(), reverse=True) for r in r_orig]
    return r_orig, sig


def _energy(r, sig):
    return sum(sum(s * s for s in sig[u][: r[u]]) for u in range(len(r)))


def pin_uniform_closed_form(uniform_fn, spectral_fn):
    """ratio 1 keeps every rank, ratio 0 keeps the floor (or all if fewer),
    and the fleet reading: 64 ranks at 1/12 with floor 4 keep 6."""
    assert list(uniform_fn([64, 16, 3], 1.0, 4)) == [64, 16, 3]
    assert list(uniform_fn([64, 16, 3], 0.0, 4)) == [4, 4, 3]
    assert list(uniform_fn([64], 1 / 12, 4)) == [6]
    assert list(uniform_fn([16, 10], 0.25, 1)) == [4, 3]


def pin_spectral_budget_and_floors(uniform_fn, spectral_fn):
    """The budget is met exactly (or every unit is at its original rank),
    floors are kept, no unit exceeds its original rank."""
    for seed in range(4):
        r_orig, sig = _rank_units(seed)
        for floor in (0, 2, 5):
            lo = sum(min(floor, r) for r in r_orig)
            for budget in (lo, lo + 7, lo + 30, sum(r_orig), sum(r_orig) + 9):
                r = list(spectral_fn(r_orig, sig, floor, budget))
                assert sum(r) == min(budget, sum(r_orig)), (seed, floor, budget)
                assert all(min(floor, ro) <= v <= ro for v, ro in zip(r, r_orig))


def pin_spectral_monotone(uniform_fn, spectral_fn):
    """One more rank of budget adds exactly one rank to one unit."""
    r_orig, sig = _rank_units(7)
    prev = list(spectral_fn(r_orig, sig, 2, sum(min(2, r) for r in r_orig)))
    for budget in range(sum(prev) + 1, sum(r_orig) + 1):
        cur = list(spectral_fn(r_orig, sig, 2, budget))
        diff = [c - p for c, p in zip(cur, prev)]
        assert sorted(diff)[-1] == 1 and sum(diff) == 1 and min(diff) == 0, budget
        prev = cur


def pin_spectral_beats_uniform(uniform_fn, spectral_fn):
    """At the uniform policy's total budget, the spectral allocation keeps at
    least as much energy (the uniform allocation is one of its candidates)."""
    for seed in range(5):
        r_orig, sig = _rank_units(10 + seed, n=20, r_hi=32)
        u = list(uniform_fn(r_orig, 0.3, 2))
        s = list(spectral_fn(r_orig, sig, 2, sum(u)))
        assert sum(s) == sum(u)
        assert _energy(s, sig) >= _energy(u, sig) - 1e-12


def pin_spectral_optimal_brute_force(uniform_fn, spectral_fn):
    """On tiny fleets, the spectral allocation keeps the most energy of every
    allocation with the same floors and total (exhaustive enumeration)."""
    import itertools
    for seed in range(3):
        r_orig, sig = _rank_units(20 + seed, n=4, r_hi=5)
        floor = 1
        for budget in range(sum(min(floor, r) for r in r_orig), sum(r_orig) + 1):
            best = max(_energy(list(c), sig) for c in itertools.product(*[range(min(floor, r), r + 1) for r in r_orig])
                       if sum(c) == budget)
            s = list(spectral_fn(r_orig, sig, floor, budget))
            assert abs(_energy(s, sig) - best) <= 1e-12 * max(best, 1.0), (seed, budget)


def pin_spectral_ties(uniform_fn, spectral_fn):
    """Equal singular values everywhere: ranks go to the lower unit first."""
    r_orig = [3, 3, 3]
    sig = [[1.0, 1.0, 1.0]] * 3
    assert list(spectral_fn(r_orig, sig, 0, 4)) == [3, 1, 0]
    assert list(spectral_fn(r_orig, sig, 1, 4)) == [2, 1, 1]


RANK_PINS = [pin_uniform_closed_form, pin_spectral_budget_and_floors, pin_spectral_monotone,
             pin_spectral_beats_uniform, pin_spectral_optimal_brute_force, pin_spectral_ties]


# ------------------------------------------------- retained-factor (r-SVD) pins
# Retained factors of one adapter by the SVD of B A through the thin QRs of B
# and A^T (LoRAForge FlashTSQR section; Compress then Serve section 4).  Pins
# take fn(A, B, k) -> (A', B', sigma) and, for R, r_fn(M) -> R.

def _rsvd_factors(seed, r=8, d_in=40, d_out=30):
    rng = np.random.default_rng(seed)
    return rng.normal(size=(r, d_in)), rng.normal(size=(d_out, r))


def pin_rsvd_eckart_young(fn):
    """sigma equals the dense SVD of B A (numpy, on the d_out x d_in product),
    and the rank-k residual's squared Frobenius norm is the sum of the
    discarded sigma^2, for every k."""
    for seed in range(3):
        A, B = _rsvd_factors(seed)
        dense = B @ A
        sv = np.linalg.svd(dense, compute_uv=False)[: A.shape[0]]
        for k in range(1, A.shape[0] + 1):
            A2, B2, s = fn(A, B, k)
            assert np.allclose(np.asarray(s), sv, rtol=1e-10, atol=1e-12 * sv[0]), seed
            res = np.linalg.norm(dense - np.asarray(B2) @ np.asarray(A2)) ** 2
            assert abs(res - float(np.sum(sv[k:] ** 2))) <= 1e-9 * float(np.sum(sv ** 2)), (seed, k)


def pin_rsvd_orthonormal(fn):
    """B' has orthonormal columns and A' A'^T = diag(sigma_k^2)."""
    A, B = _rsvd_factors(5)
    for k in (1, 4, 8):
        A2, B2, s = fn(A, B, k)
        B2, A2 = np.asarray(B2), np.asarray(A2)
        assert np.allclose(B2.T @ B2, np.eye(k), atol=1e-10)
        assert np.allclose(A2 @ A2.T, np.diag(np.asarray(s)[:k] ** 2), rtol=1e-10, atol=1e-9)


def pin_rsvd_full_rank_exact(fn):
    """Keeping every component reproduces B A."""
    A, B = _rsvd_factors(6, r=6, d_in=20, d_out=25)
    A2, B2, _ = fn(A, B, 6)
    assert np.allclose(np.asarray(B2) @ np.asarray(A2), B @ A, rtol=1e-11, atol=1e-11)


def pin_rsvd_worked_example(fn):
    """By hand: B = [[3, 0], [0, 1], [0, 0]], A = [[1, 0, 0], [0, 2, 0]]
    give B A = diag(3, 2, 0) (3 x 3 with a zero row and column): singular
    values 3 and 2; keeping one, B' A' = diag(3, 0, 0)."""
    B = np.array([[3.0, 0.0], [0.0, 1.0], [0.0, 0.0]])
    A = np.array([[1.0, 0.0, 0.0], [0.0, 2.0, 0.0]])
    A2, B2, s = fn(A, B, 1)
    assert np.allclose(np.asarray(s), [3.0, 2.0], atol=1e-14)
    assert np.allclose(np.asarray(B2) @ np.asarray(A2), np.diag([3.0, 0.0, 0.0]), atol=1e-14)


def pin_tall_skinny_r(r_fn):
    """R is upper triangular with a positive diagonal, R^T R = M^T M, and it
    equals the transposed Cholesky factor of M^T M (numpy)."""
    rng = np.random.default_rng(9)
    for shape in ((50, 8), (200, 16), (16, 16)):
        M = rng.normal(size=shape)
        R = np.asarray(r_fn(M))
        assert np.allclose(np.tril(R, -1), 0.0) and np.all(np.diag(R) > 0)
        G = M.T @ M
        assert np.allclose(R.T @ R, G, rtol=1e-12, atol=1e-10)
        assert np.allclose(R, np.linalg.cholesky(G).T, rtol=1e-9, atol=1e-10)


RSVD_PINS = [pin_rsvd_eckart_young, pin_rsvd_orthonormal, pin_rsvd_full_rank_exact, pin_rsvd_worked_example]
