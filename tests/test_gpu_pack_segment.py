"""GPU: the packed store, the token grouping and the work plan the shrink
builds from ids, all bit-exact."""
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
    """A_pack rows and B_pack blocks as the store layout defines them: A_a
    ([r, d_in]) then zero rows, B_a ([d_out, r]) widened with zero columns,
    to the stored rank; adapters end to end."""
    m = wl.module
    rows_a, blocks_b, row_off = [], [], [0]
    for a in range(m.n):
        r = int(m.ranks[a])
        stored = pad_to if pad_to else r
        A = np.zeros((stored, m.d_in), np.float32)
        B = np.zeros((m.d_out, stored), np.float32)
        A[:r] = m.A[a]
        B[:, :r] = m.B[a]
        rows_a.append(A)
        blocks_b.append(B.ravel())
        row_off.append(row_off[-1] + stored)
    return np.concatenate(rows_a), np.concatenate(blocks_b), np.array(row_off, np.int32)


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
    A_exp, B_exp, row_off = _expected_store(wl, pad_to)
    dt = TORCH_DTYPE[wl.dtype]
    R = A_exp.shape[0]
    assert store.c.R == R and store.r_max == (pad_to or int(wl.module.ranks.max()))
    A_got = store.A_pack[: R * wl.module.d_in * dt.itemsize].view(dt).float().cpu().numpy()
    B_got = store.B_pack[: R * wl.module.d_out * dt.itemsize].view(dt).float().cpu().numpy()
    assert np.array_equal(A_got.reshape(A_exp.shape), A_exp)
    assert np.array_equal(B_got, B_exp)
    ro, rk, sc = store.device_meta()
    assert np.array_equal(ro.cpu().numpy(), row_off)
    assert np.array_equal(rk.cpu().numpy(), np.diff(row_off))
    assert np.array_equal(sc.cpu().numpy(), wl.module.scales)


def _read_plan(ws):
    """(count, entries) of the work plan at the start of a workspace: a
    256-byte header (int32 count), then 128-byte entries {adapter, first
    grouped position, tokens, stored rank, row offset, scale, -, -,
    token indices[16], -}."""
    raw = ws.cpu().numpy()
    count = int(raw[:4].view(np.int32)[0])
    ent = raw[256: 256 + 128 * count].view(np.int32).reshape(count, 32)
    return count, ent


def _expected_plan(seg_off, perm, ranks, row_off, scales):
    """Every adapter with tokens and a non-zero stored rank, cut into runs of
    16 grouped positions, in adapter order."""
    out = []
    for a in range(len(ranks)):
        c = seg_off[a + 1] - seg_off[a]
        if ranks[a] <= 0:
            continue
        for j in range(0, c, 16):
            p0 = seg_off[a] + j
            m = min(16, c - j)
            tok = list(perm[p0: p0 + m]) + [-1] * (16 - m)
            out.append([a, p0, m, int(ranks[a]), int(row_off[a]), scales[a], tok])
    return out


def _check_plan(ws, expect):
    count, ent = _read_plan(ws)
    assert count == len(expect)
    for k, (a, p0, m, r, ro, sc, tok) in enumerate(expect):
        e = ent[k]
        assert [int(e[0]), int(e[1]), int(e[2]), int(e[3]), int(e[4])] == [a, p0, m, r, ro], k
        assert np.float32(e[5:6].view(np.float32)[0]) == np.float32(sc)
        assert e[8:24].tolist() == tok, k


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


def test_segment_empty():
    dev = device()
    note("segment T=0")
    seg = rs.lora_segment(torch.empty(0, dtype=torch.int32, device=dev), 4)
    torch.cuda.synchronize()
    assert seg.seg_off.cpu().tolist() == [0] * 6


def test_segment_repeatable():
    dev = device()
    ids, n = _segment_case("3")
    t = torch.from_numpy(ids).to(dev)
    note("segment repeat")
    a = rs.lora_segment(t, n)
    b = rs.lora_segment(t, n)
    torch.cuda.synchronize()
    assert torch.equal(a.perm, b.perm) and torch.equal(a.seg_off, b.seg_off)


PLAN_CASES = ["1", "2", "3", "4", "5", "all_same", "all_invalid", "out_of_range", "distinct", "max_T",
              "many_adapters", "one_token", "n1", "sorted_desc"]


def _plan_store(n, dev, seed):
    """A small bf16 store over n adapters with ranks 0..64 (some zero)."""
    rng = np.random.default_rng(seed)
    ranks = rng.integers(0, 65, size=n)
    ranks[rng.random(n) < 0.1] = 0
    A = [torch.zeros(int(r), 64, dtype=torch.bfloat16, device=dev) for r in ranks]
    B = [torch.zeros(64, int(r), dtype=torch.bfloat16, device=dev) for r in ranks]
    scales = rng.random(n).astype(np.float32)
    store = rs.lora_pack_retained(A, B, scales)
    return store, ranks, scales


@pytest.mark.parametrize("name", PLAN_CASES)
def test_plan_from_ids(name):
    """The plan the shrink (phase 1 of the two-launch apply) forms from ids
    inside its workgroups (or, beyond 4096 adapters, from the sort it runs
    first) equals the sub-tiles of the oracle's grouping, token for token."""
    dev = device()
    ids, n = _segment_case(name)
    T = len(ids)
    store, ranks, scales = _plan_store(n, dev, zlib.crc32(name.encode()))
    x = torch.zeros(T, 64, dtype=torch.bfloat16, device=dev)
    y = torch.zeros(T, 64, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(rs.lora_workspace_bytes(store, T), dtype=torch.uint8, device=dev)
    note(f"plan from ids {name} T={T} n={n}")
    rs.lora_apply_batched_phases(store, x, y, 1, ids=torch.from_numpy(ids).to(dev), ws=ws)
    torch.cuda.synchronize()
    so_ref, perm_ref, _ = segment_ref(ids.tolist(), n)
    row_off = np.concatenate([[0], np.cumsum(ranks)])
    _check_plan(ws, _expected_plan(so_ref, perm_ref, ranks, row_off, scales))


@pytest.mark.parametrize("name", ["3", "out_of_range", "all_same", "many_adapters"])
def test_plan_from_grouping(name):
    """The same plan from a caller-supplied grouping: the apply's shrink with
    (seg_off, perm), and the plan kernel of the standalone expand."""
    dev = device()
    ids, n = _segment_case(name)
    T = len(ids)
    store, ranks, scales = _plan_store(n, dev, zlib.crc32(name.encode()) + 1)
    seg = rs.lora_segment(torch.from_numpy(ids).to(dev), n)
    x = torch.zeros(T, 64, dtype=torch.bfloat16, device=dev)
    y = torch.zeros(T, 64, dtype=torch.bfloat16, device=dev)
    h = torch.zeros(T, max(store.r_max, 1), dtype=torch.float32, device=dev)
    so_ref, perm_ref, _ = segment_ref(ids.tolist(), n)
    row_off = np.concatenate([[0], np.cumsum(ranks)])
    want = _expected_plan(so_ref, perm_ref, ranks, row_off, scales)
    ws = torch.empty(rs.lora_workspace_bytes(store, T), dtype=torch.uint8, device=dev)
    note(f"plan from grouping {name}")
    rs.lora_apply_batched_phases(store, x, y, 1, seg=seg, ws=ws)
    torch.cuda.synchronize()
    _check_plan(ws, want)
    ws.fill_(0xAB)
    rs.lora_expand(store, h, seg, y, ws=ws)
    torch.cuda.synchronize()
    _check_plan(ws, want)
