"""GPU: the multi-slice apply (projections sharing one input) against the
oracle, slice by slice.

"Compress then Serve" section 13.4 adds each projection's delta into a slice
of y (offset, width).  For every slice s, y_s must equal the oracle apply of
that slice's factors on the shared x and ids: bf16 within 2e-2 and float32
within 1e-5 of max |ref| (y0 = 0); integer data bit for bit (every partial sum
is an exact integer below 2**24).
"""
import numpy as np
import pytest
import torch

import rank_specialized_amd as rs
from oracle import apply_ref, bf16_round_ref
from workloads import make_random_workload

from gpu_helpers import TOL, TORCH_DTYPE, device, note, pack, to_dev, y_host

pytestmark = pytest.mark.gpu


def _slices(seed, T, n, d_in, d_outs, ranks, dtype, integer=False, id_mode="uniform"):
    """Workloads of the same adapters: slice 0 supplies x and ids for all."""
    return [make_random_workload(seed + 17 * k, T, n, d_in, d_out, r, dtype=dtype, integer=integer,
                                 id_mode=id_mode, scales=[0.5] * n if integer else None)
            for k, (d_out, r) in enumerate(zip(d_outs, ranks))]


CASES = {
    "qkv_small": dict(seed=1, T=50, n=7, d_in=64, d_outs=(64, 16, 16),
                      ranks=([3, 0, 5, 12, 1, 7, 2], [2, 4, 0, 6, 1, 3, 8], [5, 5, 1, 0, 9, 2, 4])),
    "gate_up": dict(seed=2, T=120, n=5, d_in=128, d_outs=(256, 256),
                    ranks=([16, 8, 4, 12, 2], [1, 16, 9, 3, 7])),
    "odd_offsets_matrix": dict(seed=3, T=400, n=4, d_in=96, d_outs=(40, 72, 24),
                               ranks=([3, 5, 7, 1], [5, 3, 9, 13], [7, 1, 3, 11]), id_mode="zipf"),
    "high_rank": dict(seed=4, T=200, n=3, d_in=256, d_outs=(128, 64),
                      ranks=([33, 20, 1], [31, 44, 63])),
    "one_slice": dict(seed=5, T=90, n=6, d_in=64, d_outs=(48,), ranks=([1, 2, 3, 4, 5, 6],)),
    # Every adapter at rank 4 in both slices: a stacked rank of 8, so the
    # partial-sum rows are 8 floats wide and slice 1 starts at column 4; its
    # sub-tiles (~67 tokens per adapter) take the matrix path, whose h chunk
    # must not read past the row.
    "rank4_pairs": dict(seed=6, T=200, n=3, d_in=64, d_outs=(64, 32), ranks=([4, 4, 4], [4, 4, 4])),
    # Four rank-8 slices (stacked rank 32) over a 12288-wide input: 12
    # partial sums per h value, read by the expand's vector path (few tokens
    # per adapter, slice ranks <= 8).
    "wide_stacked": dict(seed=7, T=60, n=12, d_in=12288, d_outs=(64, 32, 32, 96),
                         ranks=([8] * 12, [7] * 12, [8] * 12, [5] * 12)),
}


def _run(name, dtype, integer=False, fused=False, grouping=False):
    dev = device()
    c = dict(CASES[name])
    ws = _slices(c["seed"], c["T"], c["n"], c["d_in"], c["d_outs"], c["ranks"], dtype, integer,
                 c.get("id_mode", "uniform"))
    stores = [pack(w, dev) for w in ws]
    ms = rs.lora_pack_multi(stores)
    dt = TORCH_DTYPE[dtype]
    x = to_dev(ws[0].x, dt, dev)
    ids = torch.from_numpy(ws[0].ids.astype(np.int32)).to(dev)
    T = c["T"]
    if fused:
        fused_y = torch.zeros(T, sum(c["d_outs"]) + 8, dtype=dt, device=dev)
        ys, off = [], 0
        for d in c["d_outs"]:
            ys.append(fused_y[:, off:off + d])
            off += d
    else:
        ys = [torch.zeros(T, d, dtype=dt, device=dev) for d in c["d_outs"]]
    note(f"multi {name} {dtype} integer={integer} fused={fused} grouping={grouping}")
    if grouping == "plan":
        seg = rs.lora_group(ids, c["n"])
        rs.lora_apply_multi(ms, x, ys, seg=seg)
    elif grouping:
        seg = rs.lora_segment(ids, c["n"])
        rs.lora_apply_multi(ms, x, ys, seg=seg)
    else:
        rs.lora_apply_multi(ms, x, ys, ids=ids)
    torch.cuda.synchronize()
    for k, w in enumerate(ws):
        m = w.module
        ref = apply_ref(ws[0].x, ws[0].ids, m.A, m.B, m.scales)
        got = y_host(ys[k])
        if integer:
            assert np.abs(ref).max() < 2 ** 24
            want = bf16_round_ref(ref) if dtype == "bf16" else ref.astype(np.float32)
            assert np.array_equal(got, want), (name, k)
        else:
            assert np.abs(got - ref).max() <= TOL[dtype] * max(np.abs(ref).max(), 1e-30), (name, k)
    if fused:  # the padding columns past the last slice are untouched
        assert torch.count_nonzero(fused_y[:, sum(c["d_outs"]):]).item() == 0


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_multi_parity(name, dtype):
    _run(name, dtype)


@pytest.mark.parametrize("name", ["qkv_small", "odd_offsets_matrix", "high_rank", "rank4_pairs", "wide_stacked"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_multi_integer_exact(name, dtype):
    _run(name, dtype, integer=True)


@pytest.mark.parametrize("name", ["qkv_small", "gate_up"])
def test_multi_fused_output(name):
    _run(name, "bf16", fused=True)


@pytest.mark.parametrize("name", ["odd_offsets_matrix", "gate_up"])
def test_multi_from_grouping(name):
    _run(name, "bf16", integer=True, grouping=True)


@pytest.mark.parametrize("name", ["qkv_small", "odd_offsets_matrix", "rank4_pairs"])
def test_multi_from_plan(name):
    _run(name, "bf16", integer=True, grouping="plan")


def test_multi_equals_separate_applies_integer():
    """On integer data the multi-slice result equals each slice applied
    alone, bit for bit."""
    dev = device()
    c = CASES["odd_offsets_matrix"]
    ws = _slices(c["seed"], c["T"], c["n"], c["d_in"], c["d_outs"], c["ranks"], "bf16", True, "zipf")
    stores = [pack(w, dev) for w in ws]
    ms = rs.lora_pack_multi(stores)
    x = to_dev(ws[0].x, torch.bfloat16, dev)
    ids = torch.from_numpy(ws[0].ids.astype(np.int32)).to(dev)
    ys = [torch.zeros(c["T"], d, dtype=torch.bfloat16, device=dev) for d in c["d_outs"]]
    note("multi vs separate")
    rs.lora_apply_multi(ms, x, ys, ids=ids)
    for k, st in enumerate(stores):
        y1 = torch.zeros_like(ys[k])
        rs.lora_apply_batched(st, x, y1, ids=ids)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), ys[k].view(torch.int16)), k


def test_multi_stacked_rank_limit():
    dev = device()
    ws = _slices(9, 10, 2, 32, (16, 16), ([40, 1], [30, 1]), "bf16")
    stores = [pack(w, dev) for w in ws]
    note("multi rank limit")
    with pytest.raises(rs.LoraError) as e:
        rs.lora_pack_multi(stores)
    assert e.value.status == 2


def test_multi_runs_integer_exact():
    """Slices wide enough that each slice's expand takes runs of feature
    blocks (T=4096, 128 adapters, d_out 17408 and 2048): bit for bit on exact
    integer data."""
    dev = device()
    T, n, d_in = 4096, 128, 32
    ranks = ([1 + (a * 5) % 16 for a in range(n)], [1 + (a * 7) % 12 for a in range(n)])
    ws = _slices(11, T, n, d_in, (17408, 2048), ranks, "bf16", integer=True)
    stores = [pack(w, dev) for w in ws]
    ms = rs.lora_pack_multi(stores)
    x = to_dev(ws[0].x, torch.bfloat16, dev)
    ids = torch.from_numpy(ws[0].ids.astype(np.int32)).to(dev)
    ys = [torch.zeros(T, d, dtype=torch.bfloat16, device=dev) for d in (17408, 2048)]
    note("multi runs")
    rs.lora_apply_multi(ms, x, ys, ids=ids)
    torch.cuda.synchronize()
    for k, w in enumerate(ws):
        ref = apply_ref(ws[0].x, ws[0].ids, w.module.A, w.module.B, w.module.scales)
        assert np.array_equal(y_host(ys[k]), bf16_round_ref(ref)), k
