"""GPU: the batched apply that allocates nothing (lora_apply_batched_noalloc)
against lora_apply_batched with a caller workspace.

Both run the same kernels on the same inputs, so their outputs must agree bit
for bit (the integer-exact and bf16 bars of the apply are then met too).  Each
case makes two no-allocation calls in a row, the second on a smaller input:
the library's scratch array keeps the first call's contents, and nothing in
it may leak into the second call's result.  The second call is also checked
against the CPU oracle.
"""
import numpy as np
import pytest
import torch

import rank_specialized_amd as rs
from oracle import apply_ref
from workloads import make_config, make_random_workload

from gpu_helpers import TOL, device, hbits, note, pack, to_dev, y_host

pytestmark = pytest.mark.gpu


def _pair(store, wl, dev, T, grouping):
    """(y from the workspace form, y from the no-allocation form) for the
    first T tokens of the workload, y0 = 0."""
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    x = to_dev(wl.x[:T], dt, dev)
    ids = torch.from_numpy(np.ascontiguousarray(wl.ids[:T], dtype=np.int32)).to(dev)
    y_ws = torch.zeros(T, wl.module.d_out, dtype=dt, device=dev)
    y_na = torch.zeros_like(y_ws)
    if grouping:
        seg = rs.lora_segment(ids, wl.module.n)
        rs.lora_apply_batched(store, x, y_ws, seg=seg)
        rs.lora_apply_batched_noalloc(store, x, y_na, seg=seg)
    else:
        rs.lora_apply_batched(store, x, y_ws, ids=ids)
        rs.lora_apply_batched_noalloc(store, x, y_na, ids=ids)
    torch.cuda.synchronize()
    return y_ws, y_na


def _workload(name):
    if name == "decode-spectral":   # two launches: shrink (grouping from ids) + expand
        return make_config("3")
    if name == "prefill":           # two launches, MFMA expand runs
        return make_config("4")
    if name == "decode-uniform":    # one launch (no scratch used)
        return make_config("2")
    if name == "many-adapters":     # three launches: the sort writes seg_off/perm into the scratch
        return make_random_workload(31, 3000, 5000, 256, 128, [1 + a % 12 for a in range(5000)], dtype="bf16",
                                    id_mode="zipf", invalid_frac=0.05)
    if name == "tiny-fp32":
        return make_config("1")
    raise KeyError(name)


SECOND_T = {"decode-spectral": 700, "prefill": 1000, "decode-uniform": 100, "many-adapters": 333,
            "tiny-fp32": 9}


@pytest.mark.parametrize("grouping", [False, True], ids=["ids", "grouping"])
@pytest.mark.parametrize("name", list(SECOND_T))
def test_noalloc_equals_workspace_form(name, grouping):
    dev = device()
    wl = _workload(name)
    store = pack(wl, dev)
    for T in (wl.T, SECOND_T[name]):
        note(f"noalloc {name} grouping={grouping} T={T}")
        y_ws, y_na = _pair(store, wl, dev, T, grouping)
        assert np.array_equal(hbits(y_ws), hbits(y_na)), (name, T)
    m = wl.module
    T = SECOND_T[name]
    ref = apply_ref(wl.x[:T], wl.ids[:T], m.A, m.B, m.scales)
    got = y_host(y_na)
    assert np.abs(got - ref).max() <= TOL[wl.dtype] * max(np.abs(ref).max(), 1e-30), name


def test_noalloc_rejects_oversize_before_launch():
    """A call whose workspace would exceed the scratch array is refused with
    UNSUPPORTED, nothing enqueued (T = 16384 tokens at rank 64, 8 chunks of a
    16384-wide input: 33.5 MB of partial sums)."""
    dev = device()
    wl = make_random_workload(5, 8, 2, 16384, 64, [64, 1], dtype="bf16")
    store = pack(wl, dev)
    T = 16384
    assert rs.lora_workspace_bytes(store, T) > rs._lib.LORA_NOALLOC_SCRATCH_BYTES
    x = torch.zeros(T, 16384, dtype=torch.bfloat16, device=dev)
    y = torch.zeros(T, 64, dtype=torch.bfloat16, device=dev)
    ids = torch.zeros(T, dtype=torch.int32, device=dev)
    note("noalloc oversize")
    with pytest.raises(rs.LoraError) as e:
        rs.lora_apply_batched_noalloc(store, x, y, ids=ids)
    assert e.value.status == 2
    assert torch.count_nonzero(y).item() == 0
