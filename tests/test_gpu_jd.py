"""GPU: the shared-basis (joint-diagonalization) apply against the oracle.

y[t] += s_a U_c Sigma_a V_c^T x[t] ("Compress then Serve" sections 3.1, 3.2,
11): full and diagonal Sigma, bf16 and float32, ranks 1..64.  Float data:
max |err| <= tol * max |ref| with y0 = 0 (bf16 2e-2, float32 1e-5).  Integer
data (x, U, V, Sigma in [-2, 2], scales 0.5): every partial sum is an exact
integer below 2**24, so the GPU result equals the round-to-nearest-even of
the exact one bit for bit.
"""
import numpy as np
import pytest
import torch

import rank_specialized_amd as rs
from oracle import bf16_round_ref, jd_apply_ref
from workloads import make_jd_config, make_jd_workload

from gpu_helpers import TOL, TORCH_DTYPE, device, note, to_dev, y_host

pytestmark = pytest.mark.gpu


def _pack(w, dev):
    dt = TORCH_DTYPE[w.dtype]
    return rs.lora_jd_pack([to_dev(u, dt, dev) for u in w.U], [to_dev(v, dt, dev) for v in w.V], w.cluster_of,
                           w.sigma, w.scales)


def _inputs(w, dev):
    dt = TORCH_DTYPE[w.dtype]
    x = to_dev(w.x, dt, dev)
    ids = torch.from_numpy(w.ids.astype(np.int32)).to(dev)
    y = to_dev(w.y0, dt, dev) if w.y0 is not None else torch.zeros(w.T, w.d_out, dtype=dt, device=dev)
    return x, ids, y


def _ref(w):
    return jd_apply_ref(w.x, w.ids, w.cluster_of, w.U, w.V, w.sigma, w.scales, w.y0)


CASES = {
    "small": dict(seed=10, T=60, n=9, k=3, d_in=64, d_out=40, r=5, invalid_frac=0.1),
    "rank1": dict(seed=11, T=50, n=6, k=2, d_in=32, d_out=24, r=1),
    "rank16_zipf": dict(seed=12, T=300, n=40, k=5, d_in=264, d_out=136, r=16, id_mode="zipf"),
    "rank33": dict(seed=13, T=120, n=12, k=3, d_in=128, d_out=72, r=33),
    "rank64": dict(seed=14, T=90, n=8, k=2, d_in=96, d_out=64, r=64),
    "one_cluster_many_tiles": dict(seed=15, T=400, n=20, k=1, d_in=128, d_out=128, r=8),
    "wide_in": dict(seed=16, T=40, n=6, k=2, d_in=18944, d_out=64, r=12),
    # rank 64 over a wide input: 16 partial sums per h value (the shrink's
    # chunks shrink with the rank), more than one batch of their loads.
    "rank64_wide_in": dict(seed=17, T=70, n=7, k=2, d_in=8192, d_out=72, r=64),
}


def _make(name, mode, dtype, integer=False, y0=False):
    kw = dict(CASES[name])
    kw.setdefault("id_mode", "uniform")
    return make_jd_workload(kw.pop("seed"), kw.pop("T"), kw.pop("n"), kw.pop("k"), kw.pop("d_in"), kw.pop("d_out"),
                            kw.pop("r"), mode=mode, dtype=dtype, integer=integer, y0=y0, **kw)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("mode", ["full", "diag"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_jd_parity(name, mode, dtype):
    dev = device()
    w = _make(name, mode, dtype)
    st = _pack(w, dev)
    x, ids, y = _inputs(w, dev)
    note(f"jd {name} {mode} {dtype} T={w.T} n={w.n} k={w.k} r={w.r}")
    rs.lora_jd_apply(st, x, y, ids)
    torch.cuda.synchronize()
    ref = _ref(w)
    assert np.abs(y_host(y) - ref).max() <= TOL[dtype] * max(np.abs(ref).max(), 1e-30)


@pytest.mark.parametrize("name", ["small", "rank16_zipf", "rank33", "one_cluster_many_tiles"])
@pytest.mark.parametrize("mode", ["full", "diag"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_jd_integer_exact(name, mode, dtype):
    dev = device()
    w = _make(name, mode, dtype, integer=True)
    st = _pack(w, dev)
    x, ids, y = _inputs(w, dev)
    note(f"jd integer {name} {mode} {dtype}")
    rs.lora_jd_apply(st, x, y, ids)
    torch.cuda.synchronize()
    ref = _ref(w)
    assert np.abs(ref).max() < 2 ** 24
    want = bf16_round_ref(ref) if dtype == "bf16" else ref.astype(np.float32)
    assert np.array_equal(y_host(y), want)


def test_jd_accumulates_into_y0_fp32():
    dev = device()
    w = _make("rank16_zipf", "full", "fp32", y0=True)
    st = _pack(w, dev)
    x, ids, y = _inputs(w, dev)
    note("jd y0 fp32")
    rs.lora_jd_apply(st, x, y, ids)
    torch.cuda.synchronize()
    ref = _ref(w)
    assert np.abs(y_host(y) - ref).max() <= 1e-5 * np.abs(ref).max()


def test_jd_unassigned_clusters_and_invalid_ids():
    """Adapters whose cluster is -1 or k, and ids -1 or >= n, add nothing."""
    dev = device()
    w = _make("small", "full", "bf16", integer=True)
    w.cluster_of[0], w.cluster_of[1] = -1, w.k
    w.ids[::7] = -1
    w.ids[3::11] = w.n + 5
    st = _pack(w, dev)
    x, ids, y = _inputs(w, dev)
    note("jd unassigned")
    rs.lora_jd_apply(st, x, y, ids)
    torch.cuda.synchronize()
    assert np.array_equal(y_host(y), bf16_round_ref(_ref(w)))


@pytest.mark.parametrize("name", ["jd-full", "jd-diag"])
def test_jd_configs(name):
    """The measured shared-basis workloads at full size (T = 2048, 1024
    adapters in 32 clusters of rank 16, d = 4096), float and integer data."""
    dev = device()
    for integer in (False, True):
        w = make_jd_config(name, integer=integer)
        st = _pack(w, dev)
        x, ids, y = _inputs(w, dev)
        note(f"jd config {name} integer={integer}")
        rs.lora_jd_apply(st, x, y, ids)
        torch.cuda.synchronize()
        ref = _ref(w)
        if integer:
            assert np.abs(ref).max() < 2 ** 24
            assert np.array_equal(y_host(y), bf16_round_ref(ref))
        else:
            assert np.abs(y_host(y) - ref).max() <= TOL["bf16"] * np.abs(ref).max()


def test_jd_graph_replay_matches_eager():
    dev = device()
    w = make_jd_config("jd-full")
    st = _pack(w, dev)
    x, ids, y0 = _inputs(w, dev)
    y0.normal_()
    ws = torch.empty(rs.lora_jd_workspace_bytes(st, w.T), dtype=torch.uint8, device=dev)
    note("jd graph: eager")
    y_eager = y0.clone()
    rs.lora_jd_apply(st, x, y_eager, ids, ws=ws)
    y = y0.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        y.copy_(y0)
        rs.lora_jd_apply(st, x, y, ids, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    note("jd graph: capture")
    with torch.cuda.graph(g):
        y.copy_(y0)
        rs.lora_jd_apply(st, x, y, ids, ws=ws)
    other = y0.clone()
    for k in range(3):
        note(f"jd graph: replay {k}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_eager.view(torch.int16)), k
        rs.lora_jd_apply(st, x, other, ids, ws=ws)
        torch.cuda.synchronize()
