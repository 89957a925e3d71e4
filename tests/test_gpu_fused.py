"""GPU: the base layer with the adapter branch in its epilogue
(lora_apply_base_fused) against the oracle's base_fused_ref,
y[t] = W0 x[t] + s_a B_a (A_a x[t])  ("Compress then Serve" sections 3, 11).

Float data: max |y - ref| <= 2e-2 max |ref| over the call, and element by
element |y - ref| <= 2^-8 |ref| + 2 E with
    E = g(K + 1024) (|x| |W0|^T + s |B| (|h| + e_h))
        + s |B| (e_h + 2^-15 (|h| + e_h)),
g(k) = k u / (1 - k u), u = 2^-24: every product of the GEMM and of the
branch is exact in float32 and all of them are summed in float32 (at most
K + 1024 terms, any order); h carries the shrink's error e_h (the oracle's
shrink_error_bound) and enters as hi + lo (within 2^-16 of s h, plus the
rounding of s h); y adds its own bf16 rounding.  Integer data (x, W0, A, B in
[-2, 2], s = 0.5): every sum is an exact integer or half-integer below
2^24, and h = hi + lo exactly, so y equals the bf16 rounding of the exact
result bit for bit.
"""
import numpy as np
import pytest
import torch

import rank_specialized_amd as rs
from oracle import base_fused_ref, bf16_round_ref, shrink_error_bound
from workloads import base_weight, fleet_base_weight, make_fleet_module, make_random_workload

from gpu_helpers import device, inputs, note, pack, to_dev, y_host

pytestmark = pytest.mark.gpu

CASES = {
    # ragged everything: d_out below one tile, d_in off the K stage, odd
    # ranks and rank 0, ids -1, a Zipf mix
    "ragged": dict(seed=1, T=300, n=9, d_in=264, d_out=136, ranks=[3, 0, 6, 1, 8, 5, 2, 7, 4], id_mode="zipf",
                   invalid_frac=0.1),
    # ranks up to 64: 8 rank groups per adapter
    "rank64": dict(seed=2, T=200, n=6, d_in=512, d_out=264, ranks=[64, 33, 17, 9, 63, 40], id_mode="uniform"),
    # one token per adapter: 32 adapters in every 32-token block
    "distinct": dict(seed=3, T=96, n=128, d_in=256, d_out=512, ranks=None, id_mode="distinct"),
    # one adapter everywhere, several tiles of tokens and outputs
    "all_same": dict(seed=4, T=700, n=3, d_in=320, d_out=520, ranks=[16, 4, 12], id_mode="all_same"),
    # tiny T
    "one_token": dict(seed=5, T=1, n=2, d_in=64, d_out=64, ranks=[5, 3], id_mode="uniform"),
}


def _make(name, integer=False):
    kw = dict(CASES[name])
    seed, T, n = kw.pop("seed"), kw.pop("T"), kw.pop("n")
    d_in, d_out, ranks = kw.pop("d_in"), kw.pop("d_out"), kw.pop("ranks")
    if ranks is None:
        ranks = [1 + (7 * a) % 16 for a in range(n)]
    scales = np.full(n, 0.5, np.float32) if integer else None
    wl = make_random_workload(400 + seed, T, n, d_in, d_out, ranks, dtype="bf16", integer=integer, scales=scales,
                              **kw)
    W0 = base_weight(seed, d_out, d_in, integer=integer)
    return wl, W0


def _run(wl, W0, dev, with_ids=True):
    store = pack(wl, dev)
    x, ids, _ = inputs(wl, dev)
    W = to_dev(W0, torch.bfloat16, dev)
    y = torch.full((wl.T, wl.module.d_out), float("nan"), dtype=torch.bfloat16, device=dev)
    note(f"base fused T={wl.T} n={wl.module.n} d={wl.module.d_in}->{wl.module.d_out} ids={with_ids}")
    rs.lora_apply_base_fused(store, W, x, y, ids=ids if with_ids else None)
    torch.cuda.synchronize()
    return y_host(y)


def _g(k):
    u = 2.0 ** -24
    return k * u / (1 - k * u)


def _bound(wl, W0, toks):
    m = wl.module
    x = wl.x[toks].astype(np.float64)
    W = W0.astype(np.float64)
    E = _g(m.d_in + 1024) * (np.abs(x) @ np.abs(W).T)
    ids = wl.ids[toks]
    eh_all = shrink_error_bound(wl.x[toks], ids, m.A)
    for i, a in enumerate(ids):
        a = int(a)
        if not (0 <= a < m.n) or int(m.ranks[a]) == 0:
            continue
        s = float(m.scales[a])
        A = m.A[a].astype(np.float64)
        B = np.abs(m.B[a].astype(np.float64))
        h = np.abs(A @ x[i])
        eh = np.asarray(eh_all[i], np.float64)
        E[i] += _g(m.d_in + 1024) * s * (B @ (h + eh))
        E[i] += s * (B @ (eh + 2.0 ** -15 * (h + eh)))
    return E


def _check_float(got, ref, E):
    assert np.abs(got - ref).max() <= 2e-2 * np.abs(ref).max()
    lim = 2.0 ** -8 * np.abs(ref) + 2 * E + 1e-30
    bad = np.abs(got - ref) > lim
    assert not bad.any(), (int(bad.sum()), float((np.abs(got - ref) - lim).max()))


@pytest.mark.parametrize("name", list(CASES))
def test_fused_parity(name):
    dev = device()
    wl, W0 = _make(name)
    m = wl.module
    got = _run(wl, W0, dev)
    ref = base_fused_ref(wl.x, wl.ids, W0, m.A, m.B, m.scales)
    _check_float(got, ref, _bound(wl, W0, np.arange(wl.T)))


@pytest.mark.parametrize("name", list(CASES))
def test_fused_integer_exact(name):
    dev = device()
    wl, W0 = _make(name, integer=True)
    m = wl.module
    got = _run(wl, W0, dev)
    ref = base_fused_ref(wl.x, wl.ids, W0, m.A, m.B, m.scales)
    assert np.abs(ref).max() < 2 ** 24
    assert np.array_equal(got, bf16_round_ref(ref))


def test_fused_without_ids_is_the_base_product():
    """ids = NULL: y = x W0^T alone (integer data: bit for bit)."""
    dev = device()
    wl, W0 = _make("ragged", integer=True)
    got = _run(wl, W0, dev, with_ids=False)
    ref = wl.x.astype(np.float64) @ W0.astype(np.float64).T
    assert np.array_equal(got, bf16_round_ref(ref))


def test_fused_no_valid_id_equals_base_only():
    """Every id -1 or >= n: the branch adds nothing, bit for bit the result
    without ids."""
    dev = device()
    wl, W0 = _make("ragged")
    wl.ids[:] = -1
    wl.ids[::3] = wl.module.n + 4
    a = _run(wl, W0, dev)
    b = _run(wl, W0, dev, with_ids=False)
    assert np.array_equal(a, b)


FLEET = [("5S", 0, 0), ("5S", 0, 4), ("5U", 3, 0)]  # q 3584->3584, gate 3584->18944


def _fleet_tokens(wl, k=40):
    rng = np.random.default_rng(11)
    top = int(np.bincount(wl.ids).argmax())
    picks = {0, wl.T - 1, int(np.flatnonzero(wl.ids == top)[0])}
    counts = np.bincount(wl.ids, minlength=wl.module.n)
    single = np.flatnonzero(counts[wl.ids] == 1)  # tokens alone with their adapter
    picks.update(int(t) for t in single[:8])
    picks.update(int(t) for t in rng.choice(wl.T, size=k, replace=False))
    return np.array(sorted(picks))


@pytest.mark.parametrize("key,layer,proj", FLEET)
@pytest.mark.parametrize("integer", [False, True])
def test_fused_fleet_module(key, layer, proj, integer):
    """Full-size fleet modules (4096 tokens, 1024 adapters): the whole call
    in the launch configuration timed, checked on sampled tokens (the
    oracle's rows are independent per token)."""
    dev = device()
    wl = make_fleet_module(key, layer, proj, integer=integer)
    W0 = fleet_base_weight(layer, proj, integer=integer)
    m = wl.module
    got = _run(wl, W0, dev)
    toks = _fleet_tokens(wl)
    ref = base_fused_ref(wl.x[toks], wl.ids[toks], W0, m.A, m.B, m.scales)
    if integer:
        assert np.abs(ref).max() < 2 ** 24
        assert np.array_equal(got[toks], bf16_round_ref(ref))
    else:
        _check_float(got[toks], ref, _bound(wl, W0, toks))
