"""GPU parity of the HIP path against the CPU oracle.

Float configs: max |y_gpu - y_ref| <= 2e-2 max |y_ref| (bf16) or 1e-5 max |y_ref|
(f32) over the call, y0 = 0.  Integer configs (x, A, B integers in [-2, 2],
power-of-two scales): every partial sum is an exact integer below 2**24, so
the GPU result must equal the round-to-nearest-even bf16 of the exact result
bit for bit, whatever the summation order.
"""
import numpy as np
import pytest
import torch

import rank_specialized_amd as rs
from oracle import apply_ref, bf16_round_ref, shrink_error_bound, shrink_ref
from workloads import make_config, make_random_workload

from gpu_helpers import (TOL, TORCH_DTYPE, device, hbits, inputs, note, pack, rel_err, to_dev, ws_offsets,
                         y_host)

pytestmark = pytest.mark.gpu

FLOAT_CONFIGS = ["1", "2", "3", "4"]
FLEET_SAMPLES = [("5U", 0, 0), ("5U", 27, 6), ("5S", 3, 1), ("5S", 14, 4)]


def _run_apply(wl, dev, pad_to=0, **kw):
    store = pack(wl, dev, pad_to)
    x, ids, y = inputs(wl, dev)
    note(f"apply {wl.key} T={wl.T} n={wl.n} d={wl.module.d_in}->{wl.module.d_out} pad_to={pad_to}")
    rs.lora_apply_batched(store, x, y, ids=ids, **kw)
    torch.cuda.synchronize()
    return store, x, ids, y


def _ref(wl):
    m = wl.module
    return apply_ref(wl.x, wl.ids, m.A, m.B, m.scales, wl.y0)


@pytest.mark.parametrize("key", FLOAT_CONFIGS)
def test_apply_parity(key):
    dev = device()
    wl = make_config(key)
    _, _, _, y = _run_apply(wl, dev)
    err = rel_err(y_host(y), _ref(wl))
    assert err <= TOL[wl.dtype], err


@pytest.mark.parametrize("key,layer,proj", FLEET_SAMPLES)
def test_apply_parity_fleet_module(key, layer, proj):
    dev = device()
    wl = make_config(key, layer=layer, proj=proj)
    _, _, _, y = _run_apply(wl, dev)
    err = rel_err(y_host(y), _ref(wl))
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("key", FLOAT_CONFIGS + ["5U", "5S"])
def test_apply_integer_exact(key):
    dev = device()
    wl = make_config(key, integer=True, layer=2, proj=6) if key.startswith("5") else \
        make_config(key, integer=True)
    _, _, _, y = _run_apply(wl, dev)
    ref = _ref(wl)
    assert np.abs(ref).max() < 2 ** 24
    want = bf16_round_ref(ref) if wl.dtype == "bf16" else ref
    got = y_host(y)
    bad = np.argwhere(got != want)
    assert bad.size == 0, (len(bad), bad[:5], got[tuple(bad[0])], want[tuple(bad[0])])


@pytest.mark.parametrize("key,layer,proj", [("5S", 5, 4), ("5S", 20, 5), ("5U", 9, 4)])
def test_apply_integer_exact_run_form(key, layer, proj):
    """gate/up modules (3584 -> 18944): calls large enough for the expand's
    run form, where sub-tiles of up to 8 tokens and rank up to 16 take the
    vector path; integer data, bit for bit."""
    dev = device()
    wl = make_config(key, integer=True, layer=layer, proj=proj)
    _, _, _, y = _run_apply(wl, dev)
    ref = _ref(wl)
    assert np.abs(ref).max() < 2 ** 24
    got, want = y_host(y), bf16_round_ref(ref)
    bad = np.argwhere(got != want)
    assert bad.size == 0, (len(bad), bad[:5])


@pytest.mark.parametrize("key", ["1", "2", "3", "4"])
def test_shrink_h_within_fp32_bound(key):
    dev = device()
    wl = make_config(key)
    m = wl.module
    store = pack(wl, dev)
    x, ids, _ = inputs(wl, dev)
    note(f"shrink {key}")
    seg = rs.lora_segment(ids, m.n)
    h = torch.full((wl.T, store.r_max), float("nan"), dtype=torch.float32, device=dev)
    rs.lora_shrink(store, x, seg, h)
    torch.cuda.synchronize()
    hg = h.cpu().numpy().astype(np.float64)
    perm = seg.perm.cpu().numpy()
    href = shrink_ref(wl.x, wl.ids, m.A)
    bound = shrink_error_bound(wl.x, wl.ids, m.A)
    for i, t in enumerate(perm):
        a = wl.ids[t]
        r = m.ranks[a]
        assert np.all(np.abs(hg[i, :r] - href[t]) <= bound[t] + 1e-30), (i, t)
        assert np.all(np.isnan(hg[i, r:])), "columns beyond the rank must stay untouched"


@pytest.mark.parametrize("key", ["1", "2", "3", "4"])
def test_shrink_then_expand_equals_apply(key):
    """lora_segment + lora_shrink + lora_expand and the two-launch apply
    (shrink, then expand: phases 1 and 2) compute the same y bit for bit
    (same sub-tiles, same partial sums, same order)."""
    dev = device()
    for integer in (False, True):
        wl = make_config(key, integer=integer)
        store = pack(wl, dev)
        x, ids, y1 = inputs(wl, dev)
        y2 = y1.clone()
        ws = torch.empty(rs.lora_workspace_bytes(store, wl.T), dtype=torch.uint8, device=dev)
        note(f"compose {key} integer={integer}")
        rs.lora_apply_batched_phases(store, x, y1, 1, ids=ids, ws=ws)
        rs.lora_apply_batched_phases(store, x, y1, 2, ids=ids, ws=ws)
        seg = rs.lora_segment(ids, store.n)
        h = rs.lora_shrink(store, x, seg)
        rs.lora_expand(store, h, seg, y2)
        torch.cuda.synchronize()
        assert np.array_equal(hbits(y1), hbits(y2)), (key, integer)


# Decode-sized calls with ids (T <= 512, ranks <= 8 in bf16 or 4 in float32,
# d_in at most one 16-byte chunk per thread of a 512-thread workgroup) run as
# one launch, a workgroup per (token, 4096 output features).
FUSED = {
    "r4": dict(seed=90, T=256, n=64, d_in=4096, d_out=4096, ranks=[4] * 64),
    "r6_ragged_out": dict(seed=91, T=200, n=30, d_in=1024, d_out=2056, ranks=[6, 5, 1, 0, 3, 6] * 5),
    "r8_short_in": dict(seed=92, T=150, n=12, d_in=64, d_out=520, ranks=[8, 7, 2, 8, 1, 3, 5, 8, 6, 4, 2, 7]),
    "many_tiles": dict(seed=93, T=512, n=3, d_in=2048, d_out=1024, ranks=[3, 4, 2], id_mode="zipf"),
    "invalid_ids": dict(seed=94, T=300, n=9, d_in=512, d_out=768, ranks=[2, 4, 1, 3, 4, 2, 1, 3, 4],
                        invalid_frac=0.3),
    "wide_out_many_adapters": dict(seed=95, T=96, n=5000, d_in=256, d_out=9000,
                                   ranks=[(a * 7) % 5 for a in range(5000)]),
}


@pytest.mark.parametrize("name", list(FUSED))
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("grouped", [False, True])
def test_decode_fused_matches_split(name, dtype, grouped):
    """The one-launch decode form (phases 3 with ids) against the oracle and
    against the same call as two launches (phases 1 and 2): bit for bit on
    exact integer data, within the tolerance on float data.  With a grouping
    given, or a float32 store of rank above 4, both are the two launches."""
    dev = device()
    for integer in (True, False):
        kw = dict(FUSED[name])
        wl = make_random_workload(kw.pop("seed"), kw.pop("T"), kw.pop("n"), kw.pop("d_in"), kw.pop("d_out"),
                                  kw.pop("ranks"), dtype=dtype, integer=integer, **kw)
        store = pack(wl, dev)
        x, ids, y1 = inputs(wl, dev)
        y2 = y1.clone()
        ws = torch.empty(rs.lora_workspace_bytes(store, wl.T), dtype=torch.uint8, device=dev)
        grp = dict(seg=rs.lora_segment(ids, store.n)) if grouped else dict(ids=ids)
        note(f"fused vs split {name} {dtype} grouped={grouped} integer={integer}")
        rs.lora_apply_batched(store, x, y1, ws=ws, **grp)
        rs.lora_apply_batched_phases(store, x, y2, 1, ws=ws, **grp)
        rs.lora_apply_batched_phases(store, x, y2, 2, ws=ws, **grp)
        torch.cuda.synchronize()
        ref = _ref(wl)
        if integer:
            want = bf16_round_ref(ref) if dtype == "bf16" else ref.astype(np.float32)
            assert np.array_equal(y_host(y1), want), "fused"
            assert np.array_equal(y_host(y2), want), "split"
        else:
            tol = TOL[dtype] * max(np.abs(ref).max(), 1e-30)
            assert np.abs(y_host(y1) - ref).max() <= tol, "fused"
            assert np.abs(y_host(y2) - ref).max() <= tol, "split"


def test_decode_float32_half_feature_group():
    """float32 rows of 4 (mod 8) output features, where the row's last
    thread holds 4 features (half its B block and y chunks in range), with
    one adapter and with 64 (the largest fleet whose metadata comes from lane
    copies), d_in down to one 4-element chunk: the one-launch form, bit for
    bit on exact integer data."""
    dev = device()
    for n, d_in, d_out, ranks in ((1, 4, 4100, [3]), (64, 2044, 12, [1, 2, 3, 4] * 16)):
        wl = make_random_workload(97 + n, 70, n, d_in, d_out, ranks, dtype="fp32", integer=True)
        store = pack(wl, dev)
        assert rs.lora_apply_launches(store, wl.T, True) == 1
        x, ids, y = inputs(wl, dev)
        note(f"decode f32 half group n={n} d={d_in}->{d_out}")
        rs.lora_apply_batched(store, x, y, ids=ids)
        torch.cuda.synchronize()
        assert np.array_equal(y_host(y), _ref(wl).astype(np.float32)), (n, d_in, d_out)


# The matrix-path expand takes runs of feature blocks per wave when a call has
# at least 48 Ki one-block items (plan sub-tile bound x 128-feature blocks);
# prefill and the fleet's wide projections do.
RUN_MIN_ITEMS = 48 * 1024


@pytest.mark.parametrize("dtype,d_out", [("bf16", 17408), ("fp32", 17408), ("bf16", 17416), ("fp32", 17412)])
def test_expand_runs_integer_exact(dtype, d_out):
    """A call past the run threshold (T=4096, 128 adapters, d_out about 17 K):
    the two-launch apply from ids, and the standalone shrink + expand from a
    grouping, both bit for bit on exact integer data.  d_out = 17408 fills 136
    feature blocks, 68 full runs; 17416 and 17412 add a 137th block of 8 or 4
    features, alone in the last run."""
    dev = device()
    T, n, d_in = 4096, 128, 32
    assert (T + 15 * n) // 16 * ((d_out + 127) // 128) >= RUN_MIN_ITEMS
    ranks = [1 + (a * 5) % 16 for a in range(n)] if dtype == "bf16" else [1 + (a * 3) % 4 for a in range(n)]
    wl = make_random_workload(99, T, n, d_in, d_out, ranks, dtype=dtype, integer=True)
    store = pack(wl, dev)
    x, ids, y1 = inputs(wl, dev)
    y2 = y1.clone()
    note(f"expand runs {dtype} T={T} n={n} d_out={d_out}")
    rs.lora_apply_batched(store, x, y1, ids=ids)
    seg = rs.lora_segment(ids, store.n)
    h = rs.lora_shrink(store, x, seg)
    rs.lora_expand(store, h, seg, y2)
    torch.cuda.synchronize()
    ref = _ref(wl)
    want = bf16_round_ref(ref) if dtype == "bf16" else ref.astype(np.float32)
    assert np.array_equal(y_host(y1), want)
    assert np.array_equal(y_host(y2), want)


def test_shrink_batches_integer_exact():
    """The fleet's down projection (d_in 18944: eight K chunks per sub-tile)
    gives each resident shrink workgroup more than one batch of items: from
    ids and from a supplied grouping, bit for bit on exact integer data."""
    dev = device()
    wl = make_config("5U", integer=True, layer=27, proj=6)
    assert wl.module.d_in == 18944
    store = pack(wl, dev)
    x, ids, y1 = inputs(wl, dev)
    y2 = y1.clone()
    note("shrink batches: 5U down, ids and grouping")
    rs.lora_apply_batched(store, x, y1, ids=ids)
    rs.lora_apply_batched(store, x, y2, seg=rs.lora_segment(ids, store.n))
    torch.cuda.synchronize()
    want = bf16_round_ref(_ref(wl))
    assert np.array_equal(y_host(y1), want)
    assert np.array_equal(y_host(y2), want)


def test_separate_kernels_integer_exact_decode():
    """The standalone shrink + expand (not the fused path) on a decode shape."""
    dev = device()
    wl = make_config("3", integer=True)
    store = pack(wl, dev)
    x, ids, y = inputs(wl, dev)
    note("separate kernels decode integer")
    seg = rs.lora_segment(ids, store.n)
    h = rs.lora_shrink(store, x, seg)
    rs.lora_expand(store, h, seg, y)
    torch.cuda.synchronize()
    assert np.array_equal(y_host(y), bf16_round_ref(_ref(wl)))


@pytest.mark.parametrize("key", ["1", "3", "4"])
def test_padded_equals_specialized(key):
    """The rank-padded store (zero rows and columns up to r_max) gives the
    same y: bit for bit on exact integer data; on float data to float32
    rounding (the shrink cuts d_in into chunks per rank bucket, so a padded
    adapter's sum over d_in is formed in another order): within one output
    ulp plus 1e-5 of the largest output for sums that cancel."""
    dev = device()
    for integer in (True, False):
        wl = make_config(key, integer=integer)
        _, _, _, y1 = _run_apply(wl, dev)
        _, _, _, y2 = _run_apply(wl, dev, pad_to=int(wl.module.ranks.max()))
        if integer:
            assert np.array_equal(hbits(y1), hbits(y2)), key
        else:
            a, b = y_host(y1), y_host(y2)
            ulp = 2.0 ** -7 if wl.dtype == "bf16" else 2.0 ** -22
            floor = 1e-5 * np.abs(a).max()  # float32 rounding of sums that cancel
            assert np.all(np.abs(a - b) <= ulp * np.maximum(np.abs(a), np.abs(b)) + floor), key
            assert rel_err(a, _ref(wl)) <= TOL[wl.dtype] and rel_err(b, _ref(wl)) <= TOL[wl.dtype]


def test_deterministic():
    dev = device()
    wl = make_config("3")
    store = pack(wl, dev)
    x, ids, y = inputs(wl, dev)
    ys = []
    for _ in range(3):
        yy = y.clone()
        note("determinism run")
        rs.lora_apply_batched(store, x, yy, ids=ids)
        ys.append(hbits(yy))
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[2])


def test_given_segmentation_equals_ids():
    dev = device()
    wl = make_config("3")
    store = pack(wl, dev)
    x, ids, y1 = inputs(wl, dev)
    y2 = y1.clone()
    note("given segmentation")
    rs.lora_apply_batched(store, x, y1, ids=ids)
    seg = rs.lora_segment(ids, store.n)
    rs.lora_apply_batched(store, x, y2, seg=seg)
    torch.cuda.synchronize()
    assert np.array_equal(hbits(y1), hbits(y2))


def test_accumulate_fp32():
    dev = device()
    wl = make_config("1", with_y0=True)
    assert wl.y0 is not None and np.abs(wl.y0).max() > 0
    _, _, _, y = _run_apply(wl, dev)
    err = rel_err(y_host(y), _ref(wl))
    assert err <= 1e-5, err


def test_accumulate_bf16():
    """y0 + delta rounded once to bf16: within half a bf16 ulp plus float32 slack."""
    dev = device()
    wl = make_config("2", with_y0=True)
    _, _, _, y = _run_apply(wl, dev)
    ref = _ref(wl)
    got = y_host(y)
    tol = np.abs(ref) * 2.0 ** -8 + 1e-3 * np.abs(ref).max() * 2.0 ** -8 + 1e-6
    assert np.all(np.abs(got - ref) <= tol)


def test_strided_y_slice_and_canaries():
    """y as a column slice of a wider buffer (offset + row stride); everything
    outside the slice, and rows of tokens without an adapter, stay untouched."""
    dev = device()
    wl = make_random_workload(50, 200, 7, 264, 136, [3, 9, 1, 0, 17, 33, 64], dtype="bf16",
                              id_mode="zipf", invalid_frac=0.15)
    store = pack(wl, dev)
    x, ids, _ = inputs(wl, dev)
    wide = torch.randn(wl.T, 136 + 64 + 16, device=dev).to(torch.bfloat16)
    before = wide.clone()
    y = wide[:, 64: 64 + 136]
    note("strided y")
    rs.lora_apply_batched(store, x, y, ids=ids)
    torch.cuda.synchronize()
    assert torch.equal(wide[:, :64], before[:, :64]) and torch.equal(wide[:, 200:], before[:, 200:])
    invalid = torch.from_numpy(wl.ids < 0).to(dev)
    assert torch.equal(wide[invalid], before[invalid])
    zero_rank = torch.from_numpy(np.isin(wl.ids, [3])).to(dev)
    assert torch.equal(wide[zero_rank], before[zero_rank])
    m = wl.module
    ref = apply_ref(wl.x, wl.ids, m.A, m.B, m.scales, y_host(before[:, 64:200]))
    got = y_host(wide[:, 64:200])
    tol = np.abs(ref) * 2.0 ** -8 + 2e-2 * np.abs(ref - y_host(before[:, 64:200])).max()
    assert np.all(np.abs(got - ref) <= tol)


def test_strided_x():
    dev = device()
    wl = make_random_workload(51, 90, 3, 128, 64, [5, 12, 2], dtype="bf16")
    store = pack(wl, dev)
    _, ids, y = inputs(wl, dev)
    xw = torch.zeros(wl.T, 128 + 40, dtype=torch.bfloat16, device=dev)
    xw[:, 8:136] = to_dev(wl.x, torch.bfloat16, dev)
    note("strided x")
    rs.lora_apply_batched(store, xw[:, 8:136], y, ids=ids)
    torch.cuda.synchronize()
    assert rel_err(y_host(y), _ref(wl)) <= TOL["bf16"]


EDGE = {
    "one_adapter_many_tiles": dict(seed=60, T=333, n=1, d_in=64, d_out=64, ranks=[7], id_mode="uniform"),
    "tile_boundaries": dict(seed=61, T=64 + 65 + 1 + 128, n=4, d_in=96, d_out=40, ranks=[16, 32, 48, 64],
                            id_mode="sorted"),
    "ragged_dims": dict(seed=62, T=77, n=5, d_in=8, d_out=8, ranks=[1, 2, 3, 4, 8], id_mode="uniform"),
    "wide_out": dict(seed=63, T=20, n=3, d_in=520, d_out=3000, ranks=[13, 27, 64], id_mode="uniform"),
    "zero_ranks": dict(seed=64, T=50, n=4, d_in=64, d_out=64, ranks=[0, 5, 0, 2], id_mode="uniform"),
    "all_invalid": dict(seed=65, T=40, n=3, d_in=64, d_out=64, ranks=[1, 2, 3], id_mode="uniform",
                        invalid_frac=1.0),
    "distinct": dict(seed=66, T=100, n=200, d_in=256, d_out=128, ranks=list(range(1, 65)) * 3 + [8] * 8,
                     id_mode="distinct"),
    # d_in = 18944 splits K into the most chunks (8 partial sums per h value).
    "wide_in_decode": dict(seed=67, T=48, n=12, d_in=18944, d_out=520, ranks=[6, 3, 8, 1, 5, 2, 7, 4, 16, 40, 6, 3],
                           id_mode="uniform"),
    "wide_in_tiles": dict(seed=68, T=70, n=3, d_in=18944, d_out=136, ranks=[6, 24, 64], id_mode="sorted"),
}


@pytest.mark.parametrize("name", list(EDGE))
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_edge_cases(name, dtype):
    dev = device()
    kw = dict(EDGE[name])
    wl = make_random_workload(kw.pop("seed"), kw.pop("T"), kw.pop("n"), kw.pop("d_in"), kw.pop("d_out"),
                              kw.pop("ranks"), dtype=dtype, y0=True, **kw)
    _, _, _, y = _run_apply(wl, dev)
    ref = _ref(wl)
    got = y_host(y)
    y0 = wl.y0.astype(np.float64)
    delta = np.abs(ref - y0).max()
    if dtype == "fp32":
        assert np.abs(got - ref).max() <= 1e-5 * max(np.abs(ref).max(), 1e-30)
    else:
        tol = np.abs(ref) * 2.0 ** -8 + 2e-2 * delta + 1e-30
        assert np.all(np.abs(got - ref) <= tol)


def test_empty_batch():
    dev = device()
    wl = make_random_workload(70, 0, 3, 64, 64, [1, 2, 3], dtype="bf16")
    store = pack(wl, dev)
    x = torch.empty(0, 64, dtype=torch.bfloat16, device=dev)
    y = torch.empty(0, 64, dtype=torch.bfloat16, device=dev)
    ids = torch.empty(0, dtype=torch.int32, device=dev)
    note("empty batch")
    rs.lora_apply_batched(store, x, y, ids=ids)
    torch.cuda.synchronize()


def test_fp32_output_width_not_multiple_of_8():
    """f32 rows of d_out = 4 (mod 8): a lane's last 16 bytes of features fall
    past the row end and must be neither read nor written."""
    dev = device()
    wl = make_random_workload(71, 37, 3, 20, 44, [3, 17, 40], dtype="fp32", y0=True)
    store = pack(wl, dev)
    x, ids, _ = inputs(wl, dev)
    wide = torch.randn(wl.T, 48, dtype=torch.float32, device=dev)
    wide[:, :44] = to_dev(wl.y0, torch.float32, dev)
    before = wide.clone()
    note("f32 d_out=44")
    rs.lora_apply_batched(store, x, wide[:, :44], ids=ids)
    torch.cuda.synchronize()
    assert torch.equal(wide[:, 44:], before[:, 44:])
    ref = _ref(wl)
    assert np.abs(y_host(wide[:, :44]) - ref).max() <= 1e-5 * np.abs(ref).max()


@pytest.mark.parametrize("key", ["2", "3"])
def test_graph_replay_matches_eager(key):
    """The apply captured in a HIP graph (as the benchmark times it) and
    replayed several times, with eager work and synchronizations between the
    replays: every replay equals the eager result bit for bit (decode-uniform
    runs the fused launch, decode-spectral the two launches)."""
    dev = device()
    wl = make_config(key, with_y0=True)
    store = pack(wl, dev)
    x, ids, y0 = inputs(wl, dev)
    ws = torch.empty(rs.lora_workspace_bytes(store, wl.T), dtype=torch.uint8, device=dev)
    note("graph: eager reference")
    y_eager = y0.clone()
    rs.lora_apply_batched(store, x, y_eager, ids=ids, ws=ws)
    y = y0.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up on the capture stream
        y.copy_(y0)
        rs.lora_apply_batched(store, x, y, ids=ids, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    note("graph: capture")
    with torch.cuda.graph(g):
        y.copy_(y0)
        rs.lora_apply_batched(store, x, y, ids=ids, ws=ws)
    other = y0.clone()
    for k in range(4):
        note(f"graph: replay {k}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_eager.view(torch.int16)), k
        rs.lora_apply_batched(store, x, other, ids=ids, ws=ws)  # eager work between replays
        torch.cuda.synchronize()


def test_ids_not_16_byte_aligned():
    """ids as a slice starting one element into a buffer (4-byte aligned
    only): the grouping reads them element by element and gives the same y."""
    dev = device()
    wl = make_config("3", integer=True)
    store = pack(wl, dev)
    x, ids, y1 = inputs(wl, dev)
    y2 = y1.clone()
    big = torch.empty(wl.T + 1, dtype=torch.int32, device=dev)
    big[1:] = ids
    note("ids offset by one element")
    rs.lora_apply_batched(store, x, y1, ids=ids)
    rs.lora_apply_batched(store, x, y2, ids=big[1:])
    torch.cuda.synchronize()
    assert np.array_equal(hbits(y1), hbits(y2))
    assert np.array_equal(y_host(y2), bf16_round_ref(_ref(wl)))


def test_phases_compose_to_apply():
    """The shrink-only and expand-only calls (the benchmark's per-kernel
    timing) give the apply's y when run in order on one workspace."""
    dev = device()
    wl = make_config("3")
    store = pack(wl, dev)
    x, ids, y1 = inputs(wl, dev)
    y2 = y1.clone()
    ws = torch.empty(rs.lora_workspace_bytes(store, wl.T), dtype=torch.uint8, device=dev)
    note("phases 1 then 2")
    rs.lora_apply_batched(store, x, y1, ids=ids, ws=ws)
    rs.lora_apply_batched_phases(store, x, y2, 1, ids=ids, ws=ws)
    rs.lora_apply_batched_phases(store, x, y2, 2, ids=ids, ws=ws)
    torch.cuda.synchronize()
    assert np.array_equal(hbits(y1), hbits(y2))


def _two_stores(dev):
    """Two stores with the same shapes and ids but different rank totals."""
    big = make_random_workload(80, 300, 8, 256, 192, [64, 60, 33, 17, 64, 5, 48, 41], dtype="bf16")
    small = make_random_workload(80, 300, 8, 256, 192, [3, 1, 5, 2, 7, 4, 1, 6], dtype="bf16")
    return big, pack(big, dev), small, pack(small, dev)


def test_expand_skips_plan_of_another_store():
    """The expand-only call on a workspace whose sub-tile metadata was made
    for another store (larger row offsets and ranks): sub-tiles that do not
    fit the store are skipped, nothing outside its buffers is read, and the
    call succeeds."""
    dev = device()
    big, sb, small, ss = _two_stores(dev)
    x, ids, y = inputs(big, dev)
    ws = torch.empty(max(rs.lora_workspace_bytes(sb, big.T), rs.lora_workspace_bytes(ss, big.T)),
                     dtype=torch.uint8, device=dev)
    note("plan of the large store, expand on the small one")
    rs.lora_apply_batched_phases(sb, x, y, 1, ids=ids, ws=ws)
    rs.lora_apply_batched_phases(ss, x, y, 2, ids=ids, ws=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all()


@pytest.mark.parametrize("fill", ["ones", "random"])
def test_expand_on_garbage_workspace(fill):
    """An expand-only call on a workspace of arbitrary bytes never reads
    outside the store's buffers (every plan entry and sub-tile metadata is
    checked against T and the store before use)."""
    dev = device()
    big, sb, _, _ = _two_stores(dev)
    x, ids, y = inputs(big, dev)
    ws = torch.empty(rs.lora_workspace_bytes(sb, big.T), dtype=torch.uint8, device=dev)
    if fill == "ones":
        ws.fill_(0xFF)
    else:
        ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, generator=torch.Generator().manual_seed(5)))
        _, plan_off, _ = ws_offsets(big.T, 8, 256, sb.r_max, 2)
        ws[plan_off:plan_off + 4].copy_(torch.tensor([20, 0, 0, 0], dtype=torch.uint8))  # a plausible sub-tile count
    note(f"expand on a workspace of {fill}")
    rs.lora_apply_batched_phases(sb, x, y, 2, ids=ids, ws=ws)
    torch.cuda.synchronize()
    assert y.shape == (big.T, 192)


# One plan (lora_group) shared by several stores of the same adapters, as a
# decode step's projections share it: each store's result must equal the
# same store applied with ids (the grouping formed per call), bit for bit,
# and the oracle within the bf16 bar.  The fleet modules span every input and
# output width of the step and ranks 4..16 (5S) or 6 (5U).
PLANNED_MODULES = [("5S", 0, 0), ("5S", 0, 1), ("5S", 5, 3), ("5S", 9, 4), ("5S", 27, 6), ("5U", 1, 5)]


def test_planned_apply_shares_one_plan():
    dev = device()
    wls = [make_config(k, layer=l, proj=p) for k, l, p in PLANNED_MODULES]
    ids = torch.from_numpy(wls[0].ids.astype(np.int32)).to(dev)
    n = wls[0].n
    note(f"lora_group T={wls[0].T} n={n}")
    seg = rs.lora_group(ids, n)
    for wl, (k, l, p) in zip(wls, PLANNED_MODULES):
        assert np.array_equal(wl.ids, wls[0].ids)
        store = pack(wl, dev)
        x, _, y = inputs(wl, dev)
        y_ids = y.clone()
        note(f"planned apply {k} L{l} p{p} {wl.module.d_in}->{wl.module.d_out}")
        rs.lora_apply_planned(store, x, y, seg)
        rs.lora_apply_batched(store, x, y_ids, ids=ids)
        torch.cuda.synchronize()
        assert np.array_equal(hbits(y), hbits(y_ids)), (k, l, p)
        err = rel_err(y_host(y), _ref(wl))
        assert err <= TOL["bf16"], (k, l, p, err)


@pytest.mark.parametrize("key", ["3", "4"])
def test_planned_phases_compose(key):
    """Shrink alone, then expand alone, on a plan: the same bits as the
    planned apply."""
    dev = device()
    wl = make_config(key, integer=True)
    store = pack(wl, dev)
    x, ids, y = inputs(wl, dev)
    y2 = y.clone()
    seg = rs.lora_group(ids, wl.n)
    ws = torch.empty(rs.lora_workspace_bytes(store, wl.T), dtype=torch.uint8, device=dev)
    note(f"planned phases {key}")
    rs.lora_apply_planned(store, x, y, seg, ws=ws, phases=1)
    rs.lora_apply_planned(store, x, y, seg, ws=ws, phases=2)
    rs.lora_apply_planned(store, x, y2, seg)
    torch.cuda.synchronize()
    assert np.array_equal(hbits(y), hbits(y2))
    ref = _ref(wl)
    want = bf16_round_ref(ref) if wl.dtype == "bf16" else ref
    assert np.array_equal(y_host(y), want)


def test_planned_apply_on_plan_of_other_grouping():
    """A plan made for another grouping of the same T and n (other ids) gives
    wrong values but reads nothing outside the call's buffers: every entry and
    token is checked against T and the store."""
    dev = device()
    wl = make_config("3")
    store = pack(wl, dev)
    x, ids, y = inputs(wl, dev)
    other = torch.from_numpy(np.roll(wl.ids, 7).astype(np.int32)).to(dev)
    seg = rs.lora_group(other, wl.n)
    note("planned apply on another grouping's plan")
    rs.lora_apply_planned(store, x, y, seg)
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all()


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_eight_partial_sums_integer_exact(dtype):
    """Ranks up to 64 over a 16384-wide input: the shrink cuts d_in into 8
    chunks (bf16; float32 chunks are half as wide, 16 K values twice over).
    The apply, and shrink + expand through h, are bit for bit the exact
    result."""
    from gpu_helpers import chunks_of
    dev = device()
    ranks = [64, 40, 3, 17, 64, 0, 9]
    e = 2 if dtype == "bf16" else 4
    assert chunks_of(16384, 64, e) == 8
    wl = make_random_workload(41, 200, len(ranks), 16384, 136, ranks, dtype=dtype, integer=True,
                              scales=[0.5] * len(ranks), id_mode="zipf", invalid_frac=0.05)
    store, x, ids, y = _run_apply(wl, dev)
    ref = _ref(wl)
    assert np.abs(ref).max() < 2 ** 24
    want = bf16_round_ref(ref) if dtype == "bf16" else ref
    assert np.array_equal(y_host(y), want)
    seg = rs.lora_segment(ids, wl.n)
    h = rs.lora_shrink(store, x, seg)
    y2 = torch.zeros_like(y)
    rs.lora_expand(store, h, seg, y2)
    torch.cuda.synchronize()
    assert np.array_equal(y_host(y2), want)


@pytest.mark.parametrize("case", ["small", "run_form_pairs"])
def test_expand_h_split_per_element_bound(case):
    """The bf16 expand feeds h to the matrix cores as the pair hi + lo of bf16
    values (hi = nearest bf16 of h, lo = nearest bf16 of h - hi), so
    |h - (hi + lo)| <= 2^-16 |h| (two roundings of relative size 2^-8).
    The 2r products are exact in float32 and summed in float32, then scaled
    once, so before the output rounding the error in y[t, o] is at most
        E = s (2^-16 + (2r + 2) 2^-24 (1 + 2^-6)) sum_j |B[o, j] h[t, j]|,
    and the bf16 output adds at most half an ulp of the result.  Checked
    element by element against the exact s B h (float64) on h with 24
    significant bits and on outputs that cancel: with B = [b, -b] pairs the
    exact sums are small next to sum |B h|, where a single bf16 copy of h
    (error 2^-8 |h|) breaks the bound.  Case run_form_pairs: a call large
    enough for the expand's run form (1024 adapters, 2048 tokens, 6144
    features) whose tokens all go to 4 adapters, so that consecutive
    sub-tiles pair up (ranks 2, 8, 17; rank 40 takes two K chunks and stays
    single)."""
    dev = device()
    rng = np.random.default_rng(77)
    if case == "small":
        n, T, d_out = 4, 64, 256
        ranks = [2, 8, 17, 40]
    else:
        n, T, d_out = 1024, 2048, 6144
        ranks = [2, 8, 17, 40] + [1] * (n - 4)
        max_sub = (T + 15 * min(n, T)) // 16
        assert max_sub * (d_out // 128) >= 48 * 1024  # the run form
    wl = make_random_workload(78, T, n, 64, d_out, ranks, dtype="bf16", id_mode="uniform")
    if case != "small":
        wl.ids = rng.integers(0, 4, size=T).astype(wl.ids.dtype)
    m = wl.module
    # B columns in cancelling pairs (column 2i+1 = -column 2i + small bf16 noise).
    for a in range(4):
        B = m.B[a].astype(np.float64)
        for j in range(0, ranks[a] - 1, 2):
            B[:, j + 1] = -B[:, j] + 2.0 ** -10 * np.sign(rng.normal(size=d_out))
        m.B[a] = B.astype(np.float32)
        m.B[a] = torch.from_numpy(m.B[a]).to(torch.bfloat16).float().numpy()
    store = pack(wl, dev)
    ids = torch.from_numpy(wl.ids.astype(np.int32)).to(dev)
    seg = rs.lora_segment(ids, n)
    so = seg.seg_off.cpu().numpy()
    perm = seg.perm.cpu().numpy()
    # h: float32 values with full 24-bit significands, equal within each
    # cancelling pair up to a relative 2^-12, in grouped rows.
    r_max = max(ranks)
    h = np.zeros((T, r_max), np.float32)
    base = rng.uniform(0.5, 2.0, size=(T, r_max)) * (1 + rng.integers(0, 2 ** 23, size=(T, r_max)) * 2.0 ** -23)
    h[:] = base.astype(np.float32)
    h[:, 1::2] = (h[:, 0::2][:, : h[:, 1::2].shape[1]] * (1 + 2.0 ** -12)).astype(np.float32)
    y = torch.zeros(T, d_out, dtype=torch.bfloat16, device=dev)
    note("expand from a float32 h: per-element bound of the hi + lo split")
    rs.lora_expand(store, torch.from_numpy(h).to(dev), seg, y)
    torch.cuda.synchronize()
    got = y_host(y)
    worst, n_cancel = 0.0, 0
    for a in range(4):
        r = ranks[a]
        s = float(m.scales[a])
        Ba = m.B[a].astype(np.float64)
        for i in range(so[a], so[a + 1]):
            t = perm[i]
            hv = h[i, :r].astype(np.float64)
            exact = s * (Ba @ hv)
            mag = s * (np.abs(Ba) @ np.abs(hv))
            E = (2.0 ** -16 + (2 * r + 2) * 2.0 ** -24 * (1 + 2.0 ** -6)) * mag
            half_ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(exact) + E, 1e-300))) - 8)
            err = np.abs(got[t] - exact)
            assert np.all(err <= E + half_ulp), (a, t, float((err - E - half_ulp).max()))
            # Where the sum cancels to below 2^-6 of its magnitude, the output
            # rounding is below 2^-15 of it, so the error seen is h's: a single
            # bf16 copy of h (2^-8 |h| per term) would exceed 2^-12 there.
            c = np.abs(exact) <= 2.0 ** -6 * mag
            n_cancel += int(c.sum())
            if c.any():
                worst = max(worst, float((err[c] / mag[c]).max()))
    assert n_cancel > 1000, n_cancel
    assert worst < 2.0 ** -12, worst
