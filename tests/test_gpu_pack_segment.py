"""GPU: the packed store and the token grouping, both bit-exact."""
import zlib

import numpy as np
import pytest
import torch

import rank_specialized_amd as rs
from oracle import segment_ref
from workloads import make_config, make_random_workload

from gpu_helpers import TORCH_DTYPE, device, note, pack

pytestmark = pytest.mark.gpu


def _expected_store(wl, pad_to=0):
    m = wl.module
    rows_a, rows_b, row_off = [], [], [0]
    for a in range(m.n):
        r = int(m.ranks[a])
        stored = pad_to if pad_to else r
        A = np.zeros((stored, m.d_in), np.float32)
        Bt = np.zeros((stored, m.d_out), np.float32)
        A[:r] = m.A[a]
        Bt[:r] = m.B[a].T
        rows_a.append(A)
        rows_b.append(Bt)
        row_off.append(row_off[-1] + stored)
    return np.concatenate(rows_a), np.concatenate(rows_b), np.array(row_off, np.int32)


@pytest.mark.parametrize("case", ["1", "2", "ragged", "ragged-pad", "3-pad"])
def test_pack_roundtrip(case):
    dev = device()
    pad_to = 0
    if case in ("1", "2"):
        wl = make_config(case)
    elif case == "3-pad":
        wl = make_config("3")
        pad_to = int(wl.module.ranks.max())
    else:
        wl = make_random_workload(40, 10, 6, 136, 264, [3, 0, 17, 64, 1, 8], dtype="bf16")
        pad_to = 64 if case == "ragged-pad" else 0
    note(f"pack {case} pad_to={pad_to}")
    store = pack(wl, dev, pad_to)
    torch.cuda.synchronize()
    A_exp, Bt_exp, row_off = _expected_store(wl, pad_to)
    dt = TORCH_DTYPE[wl.dtype]
    R = A_exp.shape[0]
    assert store.c.R == R and store.r_max == (pad_to or int(wl.module.ranks.max()))
    A_got = store.A_pack[: R * wl.module.d_in * dt.itemsize].view(dt).float().cpu().numpy()
    Bt_got = store.Bt_pack[: R * wl.module.d_out * dt.itemsize].view(dt).float().cpu().numpy()
    assert np.array_equal(A_got.reshape(A_exp.shape), A_exp)
    assert np.array_equal(Bt_got.reshape(Bt_exp.shape), Bt_exp)
    ro, rk, sc = store.device_meta()
    assert np.array_equal(ro.cpu().numpy(), row_off)
    assert np.array_equal(rk.cpu().numpy(), np.diff(row_off))
    assert np.array_equal(sc.cpu().numpy(), wl.module.scales)


def _plan_offsets(T, n):
    max_tiles = (T + 63 * min(n, T)) // 64 if T > 0 else 0
    return 64, 64 + 16 * max_tiles


def _check_plan(seg, n):
    """Expand tiles (<= 64 tokens; tiles of more than 4 tokens first) and
    shrink sub-tiles (<= 16 tokens) each cover every grouped token of a real
    adapter exactly once; each list is in (adapter, position) order."""
    ws = seg.ws.cpu().numpy()
    hdr = ws[:64].view(np.int32)
    count, n_large, n_small, n_sub = int(hdr[0]), int(hdr[1]), int(hdr[2]), int(hdr[3])
    assert count == n_large + n_small
    t_off, s_off = _plan_offsets(seg.T, n)
    tiles = ws[t_off: t_off + 16 * count].view(np.int32).reshape(count, 4)
    subs = ws[s_off: s_off + 16 * n_sub].view(np.int32).reshape(n_sub, 4)
    so = seg.seg_off.cpu().numpy()
    for lst, cap, large in ((tiles, rs._lib.LORA_TILE_TOKENS, n_large), (subs, 16, None)):
        covered = []
        for k, (a, p0, m, _) in enumerate(lst):
            assert 0 <= a < n and 1 <= m <= cap
            if large is not None:
                assert (m > 4) == (k < large)
            assert so[a] <= p0 and p0 + m <= so[a + 1]
            assert (p0 - so[a]) % cap == 0
            covered.extend(range(p0, p0 + m))
        assert sorted(covered) == list(range(int(so[n])))
    for part in (tiles[:n_large], tiles[n_large:], subs):
        keys = [(int(a), int(p)) for a, p, _, _ in part]
        assert keys == sorted(keys)
    return np.concatenate([tiles.ravel(), subs.ravel()])


def _segment_case(name):
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    if name in ("1", "2", "3", "4"):
        wl = make_config(name)
        return wl.ids, wl.n
    if name == "5":
        from workloads import fleet_ids
        return fleet_ids(), 1024
    if name == "all_same":
        return np.full(1000, 7, np.int32), 9
    if name == "all_invalid":
        return np.full(300, -1, np.int32), 5
    if name == "out_of_range":
        ids = rng.integers(-1, 12, size=777).astype(np.int32)
        ids[::13] = 99
        ids[::17] = -5
        return ids, 12
    if name == "distinct":
        return rng.permutation(4096)[:3000].astype(np.int32), 4096
    if name == "max_T":
        return rng.integers(0, 100, size=rs._lib.LORA_SEGMENT_MAX_T).astype(np.int32), 100
    if name == "many_adapters":
        return rng.integers(-1, 16000, size=5000).astype(np.int32), 16000
    if name == "one_token":
        return np.array([2], np.int32), 3
    if name == "n1":
        return rng.integers(-1, 1, size=129).astype(np.int32), 1
    if name == "sorted_desc":
        return np.sort(rng.integers(0, 50, size=2000))[::-1].astype(np.int32).copy(), 50
    raise KeyError(name)


SEGMENT_CASES = ["1", "2", "3", "4", "5", "all_same", "all_invalid", "out_of_range", "distinct",
                 "max_T", "many_adapters", "one_token", "n1", "sorted_desc"]


@pytest.mark.parametrize("name", SEGMENT_CASES)
def test_segment_exact(name):
    dev = device()
    ids, n = _segment_case(name)
    note(f"segment {name} T={len(ids)} n={n}")
    seg = rs.lora_segment(torch.from_numpy(ids).to(dev), n)
    torch.cuda.synchronize()
    so_ref, perm_ref, inv_ref = segment_ref(ids.tolist(), n)
    assert seg.seg_off.cpu().tolist() == so_ref
    assert seg.perm.cpu().tolist() == perm_ref
    assert int(seg.n_invalid.cpu()[0]) == inv_ref
    _check_plan(seg, n)


def test_segment_empty():
    dev = device()
    note("segment T=0")
    seg = rs.lora_segment(torch.empty(0, dtype=torch.int32, device=dev), 4)
    torch.cuda.synchronize()
    assert seg.seg_off.cpu().tolist() == [0] * 6
    assert int(seg.ws.cpu().numpy()[:4].view(np.int32)[0]) == 0


@pytest.mark.parametrize("name", ["3", "out_of_range", "all_same"])
def test_plan_from_offsets_matches(name):
    dev = device()
    ids, n = _segment_case(name)
    note(f"plan_from_offsets {name}")
    seg = rs.lora_segment(torch.from_numpy(ids).to(dev), n)
    seg2 = rs.lora_segment_from_offsets(seg.seg_off, seg.perm, n)
    torch.cuda.synchronize()
    assert np.array_equal(_check_plan(seg, n), _check_plan(seg2, n))


def test_segment_repeatable():
    dev = device()
    ids, n = _segment_case("3")
    t = torch.from_numpy(ids).to(dev)
    note("segment repeat")
    a = rs.lora_segment(t, n)
    b = rs.lora_segment(t, n)
    torch.cuda.synchronize()
    assert torch.equal(a.perm, b.perm) and torch.equal(a.seg_off, b.seg_off)
    assert np.array_equal(_check_plan(a, n), _check_plan(b, n))
