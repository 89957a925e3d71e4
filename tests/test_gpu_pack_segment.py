"""GPU: the packed store, the token grouping and the work plan the shrink
builds from ids, all bit-exact."""
import zlib

import numpy as np
import pytest
import torch

import rank_specialized_amd as rs
from oracle import apply_ref, bf16_round_ref, segment_ref
from workloads import make_config, make_random_workload

from gpu_helpers import chunks_of, ws_offsets, y_host, TORCH_DTYPE, device, note, pack

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


def _read_plan(buf, off=0):
    """(count, entries) of a plan: a 256-byte header (int32 count, T, n),
    then 128-byte entries {adapter, first grouped position, tokens, index of
    the sub-tile within its adapter, -, -, -, -, token indices[16], -}."""
    raw = buf.cpu().numpy()[off:]
    count = int(raw[:4].view(np.int32)[0])
    ent = raw[256: 256 + 128 * count].view(np.int32).reshape(count, 32)
    return count, ent, raw[:12].view(np.int32).tolist()


def _expected_plan(seg_off, perm, n):
    """Every adapter with tokens cut into runs of 16 grouped positions, in
    adapter order (the plan depends on the grouping only)."""
    out = []
    for a in range(n):
        c = seg_off[a + 1] - seg_off[a]
        for j, q in enumerate(range(0, c, 16)):
            p0 = seg_off[a] + q
            m = min(16, c - q)
            tok = list(perm[p0: p0 + m]) + [-1] * (16 - m)
            out.append([a, p0, m, j, tok])
    return out


def _check_plan(buf, expect, T, n, off=0):
    count, ent, hdr = _read_plan(buf, off)
    assert count == len(expect)
    assert hdr[1:3] == [T, n]
    for k, (a, p0, m, j, tok) in enumerate(expect):
        e = ent[k]
        assert [int(e[0]), int(e[1]), int(e[2]), int(e[3])] == [a, p0, m, j], k
        assert e[8:24].tolist() == tok, k


def _check_meta(ws, expect, ranks, row_off, scales, S_of):
    """The per-sub-tile metadata of a call: the store's rank, row offset and
    scale of the sub-tile's adapter, and the partial-sum count S_of(rank)."""
    raw = ws.cpu().numpy()
    meta = raw[: 16 * len(expect)].view(np.int32).reshape(-1, 4)
    for k, (a, _p0, _m, _j, _tok) in enumerate(expect):
        want = [int(ranks[a]), int(row_off[a]), S_of(int(ranks[a]))]
        assert [int(meta[k, 0]), int(meta[k, 1]), int(meta[k, 3])] == want, k
        assert np.float32(meta[k, 2:3].view(np.float32)[0]) == np.float32(scales[a]), k


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
    # The one-workgroup grouping at its limits (T = 8192, n = 2048):
    if name == "max_subtiles":
        # 384 adapters of 17 tokens and 1664 of one: 8192 tokens in 2432
        # sub-tiles, the most any grouping of that size has.
        ids = np.concatenate([np.repeat(np.arange(384), 17), np.arange(384, 2048)]).astype(np.int32)
        return rng.permutation(ids).astype(np.int32), 2048
    if name == "one_adapter_max_T":
        ids = np.full(8192, 2047, np.int32)
        ids[rng.random(8192) < 0.01] = -1
        return ids, 2048
    if name == "no_adapter_max_T":
        return np.full(8192, -1, np.int32), 2048
    raise KeyError(name)


SEGMENT_CASES = ["1", "2", "3", "4", "5", "all_same", "all_invalid", "out_of_range", "distinct",
                 "max_T", "many_adapters", "one_token", "n1", "sorted_desc", "max_subtiles",
                 "one_adapter_max_T", "no_adapter_max_T"]


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
              "many_adapters", "one_token", "n1", "sorted_desc", "max_subtiles", "one_adapter_max_T",
              "no_adapter_max_T"]


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


@pytest.mark.parametrize("name", SEGMENT_CASES)
def test_group_exact(name):
    """lora_group: seg_off and perm equal the oracle's grouping, and the plan
    holds its sub-tiles, token for token (one launch up to 8192 tokens and
    2048 adapters; beyond, the sort and the plan kernel)."""
    dev = device()
    ids, n = _segment_case(name)
    T = len(ids)
    note(f"group {name} T={T} n={n}")
    seg = rs.lora_group(torch.from_numpy(ids).to(dev), n)
    torch.cuda.synchronize()
    so_ref, perm_ref, inv_ref = segment_ref(ids.tolist(), n)
    assert seg.seg_off.cpu().tolist() == so_ref
    assert seg.perm.cpu().tolist() == perm_ref
    assert int(seg.n_invalid.cpu()[0]) == inv_ref
    _check_plan(seg.plan, _expected_plan(so_ref, perm_ref, n), T, n)


@pytest.mark.parametrize("name", PLAN_CASES)
def test_plan_from_ids(name):
    """The plan the apply forms from ids (phase 1 of the two-kernel form:
    grouping, then shrink) equals the sub-tiles of the oracle's grouping,
    token for token, and the shrink records each sub-tile's store metadata."""
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
    want = _expected_plan(so_ref, perm_ref, n)
    _, plan_off, S = ws_offsets(T, n, 64, store.r_max, 2)
    _check_plan(ws, want, T, n, plan_off)
    _check_meta(ws, want, ranks, row_off, scales, lambda r: chunks_of(64, r, 2))


def test_plan_meta_one_chunk_large_call():
    """A call with room for 1024 sub-tiles or more and d_in of two chunk
    units (the fleet's 4096 tokens over 1024 adapters, d_in 3584): every
    sub-tile records one partial sum (d_in in one chunk, where a smaller call
    has two), and the apply is the exact result rounded once (integer data,
    ranks 0..24 on both sides of 16)."""
    from workloads import fleet_ids
    dev = device()
    ids = fleet_ids()
    n, T, d_in, d_out = 1024, len(ids), 3584, 64
    rng = np.random.default_rng(57)
    ranks = rng.integers(0, 25, size=n)
    Ah = [rng.integers(-2, 3, size=(int(r), d_in)).astype(np.float32) for r in ranks]
    Bh = [rng.integers(-2, 3, size=(d_out, int(r))).astype(np.float32) for r in ranks]
    scales = np.full(n, 0.25, np.float32)
    store = rs.lora_pack_retained([torch.from_numpy(a).to(torch.bfloat16).to(dev) for a in Ah],
                                  [torch.from_numpy(b).to(torch.bfloat16).to(dev) for b in Bh], scales)
    xh = rng.integers(-2, 3, size=(T, d_in)).astype(np.float32)
    x = torch.from_numpy(xh).to(torch.bfloat16).to(dev)
    y = torch.zeros(T, d_out, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(rs.lora_workspace_bytes(store, T), dtype=torch.uint8, device=dev)
    note(f"one chunk T={T} n={n} d_in={d_in}")
    rs.lora_apply_batched(store, x, y, ids=torch.from_numpy(ids).to(dev), ws=ws)
    torch.cuda.synchronize()
    so_ref, perm_ref, _ = segment_ref(ids.tolist(), n)
    row_off = np.concatenate([[0], np.cumsum(ranks)])
    want = _expected_plan(so_ref, perm_ref, n)
    assert chunks_of(d_in, 16, 2) == 2 and chunks_of(d_in, 16, 2, T, n) == 1
    assert any(m == 16 and ranks[a] > 16 for a, _p, m, _j, _t in want)
    _check_meta(ws, want, ranks, row_off, scales, lambda r: chunks_of(d_in, r, 2, T, n))
    # Integers: h and every float32 sum are exact, so y is the exact result
    # rounded once to bf16.
    ref = apply_ref(xh, ids, Ah, Bh, scales)
    assert np.abs(ref).max() < 2 ** 24
    assert np.array_equal(y_host(y), bf16_round_ref(ref))


@pytest.mark.parametrize("name", ["3", "out_of_range", "all_same", "many_adapters"])
def test_plan_from_grouping(name):
    """The same plan from a caller-supplied grouping: the apply's phase 1
    with (seg_off, perm), and the plan kernel of the standalone expand (which
    records the store metadata itself, with one partial sum: h is given)."""
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
    want = _expected_plan(so_ref, perm_ref, n)
    _, plan_off, S = ws_offsets(T, n, 64, store.r_max, 2)
    ws = torch.empty(rs.lora_workspace_bytes(store, T), dtype=torch.uint8, device=dev)
    note(f"plan from grouping {name}")
    rs.lora_apply_batched_phases(store, x, y, 1, seg=seg, ws=ws)
    torch.cuda.synchronize()
    _check_plan(ws, want, T, n, plan_off)
    _check_meta(ws, want, ranks, row_off, scales, lambda r: chunks_of(64, r, 2))
    ws.fill_(0xAB)
    rs.lora_expand(store, h, seg, y, ws=ws)
    torch.cuda.synchronize()
    _check_plan(ws, want, T, n, plan_off)
    _check_meta(ws, want, ranks, row_off, scales, lambda r: 1)
