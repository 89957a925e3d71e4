"""The C ABI on the CPU: the library loads, exports every symbol that
include/lora.h declares, and rejects bad arguments before touching the GPU.
No compute call is made here."""
import ctypes as C
import os
import re

import pytest

from rank_specialized_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lora.h")

FAKE = 0x10000  # a 16-byte aligned non-null address; never dereferenced on error paths


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    src = "\n".join(line for line in src.splitlines() if not line.lstrip().startswith("#"))
    return sorted(set(re.findall(r"\b(lora_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return L.lib()


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ["lora_pack_retained", "lora_segment", "lora_shrink", "lora_expand",
                 "lora_apply_batched", "lora_store_bytes", "lora_status_string"]:
        assert want in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in L.SIGNATURES, f"binding lacks {name}"


def test_binding_matches_header():
    assert set(L.SIGNATURES) == set(declared_functions())


def test_status_strings(lib):
    assert lib.lora_status_string(0) == b"ok"
    assert b"invalid" in lib.lora_status_string(1)
    assert b"unsupported" in lib.lora_status_string(2)
    assert b"HIP" in lib.lora_status_string(3)
    assert lib.lora_abi_version() == 5
    assert lib.lora_last_hip_error() == 0


def _sizes(lib, n, d_in, d_out, dtype, ranks, pad_to=0):
    r = (C.c_int32 * max(n, 1))(*ranks)
    a, b, m = C.c_size_t(), C.c_size_t(), C.c_size_t()
    st = lib.lora_store_bytes(n, d_in, d_out, dtype, r, pad_to, C.byref(a), C.byref(b), C.byref(m))
    return st, a.value, b.value, m.value


def test_store_bytes(lib):
    st, a, b, m = _sizes(lib, 3, 64, 32, L.LORA_DTYPE_BF16, [1, 0, 5])
    assert st == 0 and a == 6 * 64 * 2 and b == 6 * 32 * 2
    assert m >= (4 * 3 + 1) * 4 + 16 * 3
    st, a, b, _ = _sizes(lib, 3, 64, 32, L.LORA_DTYPE_F32, [1, 0, 5], pad_to=8)
    assert st == 0 and a == 24 * 64 * 4 and b == 24 * 32 * 4


@pytest.mark.parametrize("args,status", [
    ((-1, 64, 64, 1, [1]), 1),
    ((1, 0, 64, 1, [1]), 1),
    ((1, 64, -8, 1, [1]), 1),
    ((2, 64, 64, 1, [1, -2]), 1),
    ((1, 64, 64, 1, [65]), 2),          # above LORA_MAX_RANK
    ((1, 60, 64, 1, [4]), 2),           # d_in not a multiple of 8 (bf16)
    ((1, 64, 66, 0, [4]), 2),           # d_out not a multiple of 4 (f32)
    ((1, 64, 64, 7, [4]), 2),           # unknown dtype
])
def test_store_bytes_errors(lib, args, status):
    assert _sizes(lib, *args)[0] == status


def test_store_bytes_pad_below_rank(lib):
    assert _sizes(lib, 2, 64, 64, 1, [4, 9], pad_to=8)[0] == 1
    assert _sizes(lib, 2, 64, 64, 1, [4, 9], pad_to=72)[0] == 2


def test_store_bytes_null_outputs(lib):
    r = (C.c_int32 * 1)(4)
    assert lib.lora_store_bytes(1, 64, 64, 1, r, 0, None, None, None) == 1


def test_pack_rejects_before_launch(lib):
    st = L.lora_store()
    r = (C.c_int32 * 2)(2, 3)
    s = (C.c_float * 2)(1.0, 1.0)
    ptrs = (C.c_void_p * 2)(FAKE, FAKE)
    nulls = (C.c_void_p * 2)(FAKE, None)
    f = lib.lora_pack_retained
    assert f(None, 2, 64, 64, 1, r, s, ptrs, ptrs, FAKE, FAKE, FAKE, 0, None) == 1
    assert f(C.byref(st), 0, 64, 64, 1, r, s, ptrs, ptrs, FAKE, FAKE, FAKE, 0, None) == 1
    assert f(C.byref(st), 2, 64, 64, 1, r, s, ptrs, nulls, FAKE, FAKE, FAKE, 0, None) == 1
    assert f(C.byref(st), 2, 64, 64, 1, r, s, ptrs, ptrs, None, FAKE, FAKE, 0, None) == 1
    assert f(C.byref(st), 2, 64, 64, 1, r, s, ptrs, ptrs, FAKE, FAKE, None, 0, None) == 1
    assert f(C.byref(st), 2, 64, 64, 1, r, s, ptrs, ptrs, FAKE + 4, FAKE, FAKE, 0, None) == 2
    assert f(C.byref(st), 2, 64, 64, 1, r, s, ptrs, ptrs, FAKE, FAKE, FAKE, 2, None) == 1
    # metadata only takes both pointer arrays NULL, not one of them
    assert f(C.byref(st), 2, 64, 64, 1, r, s, None, ptrs, FAKE, FAKE, FAKE, 0, None) == 1
    assert f(C.byref(st), 2, 64, 64, 1, r, s, ptrs, None, FAKE, FAKE, FAKE, 0, None) == 1
    assert f(C.byref(st), 2, 64, 64, 1, r, s, None, None, None, FAKE, FAKE, 0, None) == 1
    assert f(C.byref(st), 2, 64, 64, 1, r, s, None, None, FAKE, FAKE, None, 0, None) == 1


def test_segment_rejects_before_launch(lib):
    f = lib.lora_segment
    assert f(FAKE, -1, 4, FAKE, FAKE, None, None) == 1
    assert f(FAKE, 16, 0, FAKE, FAKE, None, None) == 1
    assert f(None, 16, 4, FAKE, FAKE, None, None) == 1
    assert f(FAKE, 16, 4, None, FAKE, None, None) == 1
    assert f(FAKE, 16, 4, FAKE, None, None, None) == 1
    assert f(FAKE, L.LORA_SEGMENT_MAX_T + 1, 4, FAKE, FAKE, None, None) == 2
    assert f(FAKE, 16, L.LORA_SEGMENT_MAX_N + 1, FAKE, FAKE, None, None) == 2


def _store(n=4, d_in=64, d_out=32, dtype=1, r_max=8, R=20):
    st = L.lora_store()
    st.n, st.d_in, st.d_out, st.dtype, st.r_max, st.R = n, d_in, d_out, dtype, r_max, R
    st.A_pack = st.B_pack = st.row_off = st.rank = st.scale = FAKE
    return st


def test_shrink_expand_reject_before_launch(lib):
    big = 1 << 30
    for fn in (lib.lora_shrink, lib.lora_expand):
        good = _store()
        d = 64 if fn is lib.lora_shrink else 32

        def call(st=good, p=FAKE, ld=d, T=16, so=FAKE, pm=FAKE, ws=FAKE, wsb=big, h=FAKE, ldh=8):
            if fn is lib.lora_shrink:
                return fn(C.byref(st) if st is not None else None, p, ld, T, so, pm, h, ldh, ws, wsb, None)
            return fn(C.byref(st) if st is not None else None, h, ldh, T, so, pm, p, ld, ws, wsb, None)

        assert call(T=0) == 0                       # no-op, nothing launched
        assert call(st=None) == 1
        assert call(st=_store(n=0)) == 1
        assert call(st=_store(r_max=65)) == 2
        assert call(st=_store(dtype=9)) == 2
        assert call(st=_store(d_in=60, d_out=36)) == 2
        assert call(T=-1) == 1
        assert call(ld=d - 8) == 1                  # row stride below the row length
        assert call(ld=d + 4) == 2                  # stride not a multiple of 8 bf16 elements
        assert call(p=FAKE + 2) == 2                # misaligned rows
        assert call(p=None) == 1
        assert call(ldh=4) == 1                     # ldh < r_max
        assert call(h=None) == 1
        assert call(wsb=8) == 1
        assert call(ws=None) == 1
        assert call(ws=FAKE + 8) == 2
        assert call(so=None) == 1
        assert call(pm=None) == 1
        assert call(st=_store(n=L.LORA_SEGMENT_MAX_N + 1)) == 2


def test_apply_rejects_before_launch(lib):
    big = 1 << 30
    st = _store()
    f = lib.lora_apply_batched

    def call(T=16, ids=FAKE, so=None, pm=None, ws=FAKE, wsb=big, x=FAKE, y=FAKE, ldx=64, ldy=32, s=st):
        return f(C.byref(s) if s is not None else None, x, ldx, y, ldy, T, ids, so, pm, ws, wsb, None)

    assert call(s=None) == 1
    assert call(T=-3) == 1
    assert call(x=None) == 1
    assert call(ldy=16) == 1
    assert call(ws=None) == 1
    assert call(wsb=16) == 1
    assert call(ws=FAKE + 8) == 2
    assert call(T=L.LORA_SEGMENT_MAX_T + 1) == 2
    # no ids: a grouping must be supplied
    assert call(ids=None) == 1
    assert call(ids=None, so=FAKE) == 1
    # T = 0: nothing to group or apply, with or without ids
    assert call(T=0, ids=None, so=FAKE, pm=FAKE) == 0
    assert call(T=0, ids=None) == 0
    assert call(T=0, x=None, y=None, ws=None, wsb=0) == 0


def test_noalloc_rejects_before_any_hip_call(lib):
    """lora_apply_batched_noalloc checks every argument, and the size its call
    needs against the scratch array, before any HIP call (so here, without a
    GPU, no HIP error is recorded)."""
    st = _store()
    f = lib.lora_apply_batched_noalloc

    def call(T=16, ids=FAKE, so=None, pm=None, x=FAKE, y=FAKE, ldx=64, ldy=32, s=st):
        return f(C.byref(s) if s is not None else None, x, ldx, y, ldy, T, ids, so, pm, None)

    assert call(s=None) == 1
    assert call(s=_store(n=0)) == 1
    assert call(T=-3) == 1
    assert call(x=None) == 1
    assert call(ldy=16) == 1
    assert call(ldx=68) == 2
    assert call(T=L.LORA_SEGMENT_MAX_T + 1) == 2
    assert call(ids=None) == 1
    assert call(ids=None, so=FAKE) == 1
    assert call(T=0) == 0
    assert call(T=0, ids=None, x=None, y=None) == 0
    big = _store(n=16000, d_in=16384, r_max=64, R=16000 * 64)
    T = 16384
    assert lib.lora_workspace_bytes(C.byref(big), T) > L.LORA_NOALLOC_SCRATCH_BYTES
    assert call(s=big, T=T, ldx=16384) == 2
    assert lib.lora_last_hip_error() == 0


def test_concurrent_validation_from_threads(lib):
    """Eight host threads run the apply's argument checks at once, each with
    its own arguments and expected status (ctypes releases the GIL during the
    call, so the calls overlap).  The checks keep no shared mutable state, so
    every call returns its own status.  Without a GPU, a call that reaches
    the HIP runtime fails there; its error code is kept per thread, so only
    the failing thread sees it."""
    import threading

    st = _store()
    f = lib.lora_apply_batched
    big = 1 << 30
    cases = [dict(s=None, want=1), dict(T=-3, want=1), dict(ws=FAKE + 8, want=2),
             dict(T=L.LORA_SEGMENT_MAX_T + 1, want=2), dict(ids=None, want=1), dict(T=0, want=0),
             dict(wsb=16, want=1), dict(ldy=16, want=1)]
    errors = []

    def worker(c):
        kw = dict(T=16, ids=FAKE, ws=FAKE, wsb=big, x=FAKE, y=FAKE, ldx=64, ldy=32, s=st)
        kw.update({k: v for k, v in c.items() if k != "want"})
        s = kw["s"]
        for _ in range(3000):
            got = f(C.byref(s) if s is not None else None, kw["x"], kw["ldx"], kw["y"], kw["ldy"], kw["T"],
                    kw["ids"], None, None, kw["ws"], kw["wsb"], None)
            if got != c["want"]:
                errors.append((c, got))
                return
        if lib.lora_last_hip_error() != 0:
            errors.append((c, "hip error seen by a thread that made no HIP call"))

    hip_seen = {}

    def hip_worker():
        # Reaches the HIP runtime (the current device's LDS limit); only where
        # no GPU is present, so nothing is ever launched.
        got = lib.lora_segment(FAKE, 16, 4, FAKE, FAKE, None, None)
        hip_seen["status"], hip_seen["err"] = got, lib.lora_last_hip_error()

    threads = [threading.Thread(target=worker, args=(c,)) for c in cases]
    no_gpu = not os.path.exists("/dev/kfd")
    if no_gpu:
        threads.append(threading.Thread(target=hip_worker))
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    if no_gpu:
        assert hip_seen["status"] == 3 and hip_seen["err"] != 0, hip_seen


def _layout_bytes(T, n, d_in, r_max, e):
    """The workspace layout restated: 16 bytes of metadata per possible
    sub-tile of <= 16 tokens; float32 partial sums for the S chunks of d_in
    (a chunk is 8 waves x 8 K steps of 64 bytes, or the smallest multiple of
    that keeping S at most 8; one chunk for up to two units when the call can
    hold 1024 sub-tiles or has at least 16 tokens per adapter) at row stride
    r_max rounded up to 8; the plan (256-byte
    header + one 128-byte entry per possible sub-tile); seg_off [n + 2] and
    perm [T]; s h as two bf16 values per rank for the base-fused apply
    ([T][2][ldp]); each part 256-byte aligned."""
    up = lambda v: -(-v // 256) * 256
    max_sub = (T + 15 * min(n, T)) // 16 if T > 0 else 0
    unit = 8 * 8 * 4 * (16 // e)  # 8 waves x 8 K steps of 64 bytes
    units = -(-d_in // unit)
    mult = max(1, -(-units // 8))
    if units <= 2 and (max_sub >= 1024 or T >= 16 * n):  # one chunk: sub-tiles enough, or full ones
        mult = units
    S = max(1, -(-d_in // (mult * unit)))
    ldp = -(-max(r_max, 1) // 8) * 8
    return (up(16 * max_sub) + up(S * T * ldp * 4) + up(256 + 128 * max_sub) + up((n + 2) * 4) + up(T * 4)
            + up(T * ldp * 4))


def test_plan_bytes(lib):
    for T, n in ((100, 4), (4096, 1024), (16384, 16382), (1, 1)):
        assert lib.lora_plan_bytes(T, n) == 256 + 128 * ((T + 15 * min(n, T)) // 16)
    assert lib.lora_plan_bytes(0, 4) == 256
    assert lib.lora_plan_bytes(-1, 4) == 0
    assert lib.lora_plan_bytes(4, 0) == 0


def test_group_rejects_before_launch(lib):
    f = lib.lora_group
    big = 1 << 30

    def call(ids=FAKE, T=16, n=4, so=FAKE, pm=FAKE, plan=FAKE, pb=big):
        return f(ids, T, n, so, pm, plan, pb, None, None)

    assert call(T=-1) == 1
    assert call(n=0) == 1
    assert call(so=None) == 1
    assert call(pm=None) == 1
    assert call(ids=None) == 1
    assert call(plan=None) == 1
    assert call(pb=8) == 1
    assert call(plan=FAKE + 4) == 2
    assert call(T=L.LORA_SEGMENT_MAX_T + 1) == 2
    assert call(n=L.LORA_SEGMENT_MAX_N + 1) == 2


def test_base_fused_rejects_before_any_hip_call(lib):
    """lora_apply_base_fused checks every argument before any HIP call."""
    st = _store()  # bf16, d_in 64, d_out 32
    f = lib.lora_apply_base_fused
    big = 1 << 30

    def call(s=st, w=FAKE, ldw=64, x=FAKE, ldx=64, y=FAKE, ldy=32, T=16, ids=FAKE, ws=FAKE, wsb=big):
        return f(C.byref(s) if s is not None else None, w, ldw, x, ldx, y, ldy, T, ids, ws, wsb, None)

    assert call(s=None) == 1
    assert call(s=_store(dtype=0)) == 2          # float32 store
    assert call(T=-1) == 1
    assert call(w=None) == 1
    assert call(ldw=56) == 1                      # W0 rows shorter than d_in
    assert call(ldw=68) == 2                      # W0 rows off 16 bytes
    assert call(w=FAKE + 8) == 2
    assert call(ldw=1 << 22) == 2                 # a 256-row tile of W0 spans 2^31 bytes
    assert call(T=1 << 14, ldx=1 << 16) == 2      # x spans 2^31 bytes
    assert call(s=_store(d_out=1 << 20, R=1 << 10), ldy=1 << 20) == 2   # B spans 2^31 bytes
    assert call(x=None) == 1
    assert call(ldy=16) == 1
    assert call(ws=None) == 1
    assert call(wsb=16) == 1
    assert call(T=L.LORA_SEGMENT_MAX_T + 1) == 2
    assert call(T=0) == 0
    assert call(T=0, ids=None, ws=None, wsb=0, x=None, y=None) == 0
    assert lib.lora_last_hip_error() == 0


def test_apply_planned_rejects_before_launch(lib):
    st = _store()
    big = 1 << 30
    for f in (lib.lora_apply_planned, lambda *a: lib.lora_apply_planned_phases(*a, 3)):
        def call(s=st, x=FAKE, ldx=64, y=FAKE, ldy=32, T=16, plan=FAKE, pb=big, ws=FAKE, wsb=big):
            return f(C.byref(s) if s is not None else None, x, ldx, y, ldy, T, plan, pb, ws, wsb, None)

        assert call(s=None) == 1
        assert call(T=-1) == 1
        assert call(plan=None) == 1
        assert call(pb=100) == 1
        assert call(plan=FAKE + 8) == 2
        assert call(x=None) == 1
        assert call(ldy=16) == 1
        assert call(ws=None) == 1
        assert call(wsb=16) == 1
        assert call(T=0, plan=None, x=None, y=None, ws=None, wsb=0) == 0
    for bad in (0, 4):
        assert lib.lora_apply_planned_phases(C.byref(st), FAKE, 64, FAKE, 32, 16, FAKE, big, FAKE, big, None,
                                             bad) == 1


@pytest.mark.parametrize("T,n,d_in,r_max,dtype", [(100, 4, 64, 6, 1), (2048, 512, 3584, 64, 1),
                                                  (4096, 1024, 18944, 16, 1), (4096, 1024, 3584, 16, 1),
                                                  (1024, 1024, 4096, 8, 1), (16, 4, 256, 4, 0),
                                                  (300, 5000, 4096, 8, 1), (0, 3, 64, 4, 1),
                                                  (8192, 32, 4096, 32, 1), (8192, 512, 4096, 16, 1),
                                                  (511, 32, 4096, 8, 1), (512, 32, 4096, 8, 1)])
def test_workspace_bytes(lib, T, n, d_in, r_max, dtype):
    st = _store(n=n, d_in=d_in, r_max=r_max, dtype=dtype)
    assert lib.lora_workspace_bytes(C.byref(st), T) == _layout_bytes(T, n, d_in, r_max, 2 if dtype == 1 else 4)
    assert lib.lora_workspace_bytes(None, T) == 0
    assert lib.lora_workspace_bytes(C.byref(st), -1) == 0


def test_apply_phases_rejects_before_launch(lib):
    st = _store()
    f = lib.lora_apply_batched_phases
    args = (FAKE, 64, FAKE, 32, 16, FAKE, None, None, FAKE, 1 << 30, None)
    for bad in (0, 4, -1):
        assert f(C.byref(st), *args, bad) == 1
    assert f(None, *args, 3) == 1
    assert f(C.byref(st), FAKE, 64, FAKE, 32, 0, FAKE, None, None, FAKE, 1 << 30, None, 1) == 0


@pytest.mark.parametrize("T,n,d_in,r_max,dtype,with_ids,want", [
    (256, 64, 4096, 4, 1, 1, 1),      # decode-uniform: one launch, a workgroup per token
    (512, 64, 4096, 8, 1, 1, 1),      # the largest T and rank of that path
    (512, 64, 4096, 8, 1, 0, 3),      # a grouping given: its plan, shrink, expand
    (512, 64, 4096, 8, 1, 2, 2),      # a plan given: shrink + expand
    (513, 64, 4096, 8, 1, 1, 3),      # one token more: grouping, shrink, expand
    (256, 64, 4104, 4, 1, 1, 3),      # d_in beyond one 16-byte step per thread
    (256, 64, 4096, 9, 1, 1, 3),      # rank above the fused path's
    (16, 4, 256, 4, 0, 1, 1),         # float32 up to rank 4 ...
    (16, 4, 256, 5, 0, 1, 3),         # ... not beyond
    (16, 4, 2052, 4, 0, 1, 3),        # float32 d_in above 2048
    (2048, 512, 3584, 64, 1, 1, 3),   # decode-spectral
    (300, 5000, 64, 4, 1, 1, 1),      # per-token path: any number of adapters
    (600, 5000, 64, 4, 1, 1, 4),      # beyond it, more adapters than the one-workgroup grouping: sort first
    (300, 5000, 64, 9, 1, 0, 3),      # ... unless the grouping is given
    (8193, 64, 4096, 16, 1, 1, 4),    # more tokens than the one-workgroup grouping
    (0, 4, 64, 4, 1, 1, 0),
])
def test_apply_launches(lib, T, n, d_in, r_max, dtype, with_ids, want):
    st = _store(n=n, d_in=d_in, d_out=32, r_max=r_max, dtype=dtype)
    assert lib.lora_apply_launches(C.byref(st), T, with_ids) == want


def test_apply_launches_errors(lib):
    assert lib.lora_apply_launches(None, 16, 1) == -1
    assert lib.lora_apply_launches(C.byref(_store()), -1, 1) == -1
    assert lib.lora_apply_launches(C.byref(_store(r_max=65)), 16, 1) == -2
    assert lib.lora_apply_launches(C.byref(_store()), L.LORA_SEGMENT_MAX_T + 1, 1) == -2
    assert lib.lora_apply_launches(C.byref(_store()), 16, 3) == -1
    assert lib.lora_apply_launches(C.byref(_store()), 16, -1) == -1


def _jd(k=4, r=8, n=10, diag=0, d_in=64, d_out=32):
    j = L.lora_jd_store()
    j.basis = _store(n=k, d_in=d_in, d_out=d_out, r_max=r, R=k * r)
    j.n_adapters, j.r, j.diag = n, r, diag
    j.cluster_of = j.sigma = j.scale = FAKE
    return j


def test_jd_workspace_bytes(lib):
    j = _jd()
    T = 100
    up = lambda v: -(-v // 256) * 256
    want = up(T * 8 * 4) + lib.lora_workspace_bytes(C.byref(j.basis), T)
    assert lib.lora_jd_workspace_bytes(C.byref(j), T) == want
    assert lib.lora_jd_workspace_bytes(None, T) == 0
    bad = _jd()
    bad.r = 7  # must equal the basis r_max (8)
    assert lib.lora_jd_workspace_bytes(C.byref(bad), T) == 0


def test_jd_apply_rejects_before_launch(lib):
    big = 1 << 30
    f = lib.lora_jd_apply

    def call(j=None, T=16, ids=FAKE, ws=FAKE, wsb=big, x=FAKE, y=FAKE, ldx=64, ldy=32):
        j = j if j is not None else _jd()
        return f(C.byref(j), x, ldx, y, ldy, T, ids, ws, wsb, None)

    assert f(None, FAKE, 64, FAKE, 32, 16, FAKE, FAKE, big, None) == 1
    assert call(T=-1) == 1
    assert call(T=0) == 0
    assert call(ids=None) == 1
    assert call(ws=None) == 1
    assert call(wsb=64) == 1
    assert call(ws=FAKE + 8) == 2
    assert call(x=None) == 1
    assert call(ldy=16) == 1
    j = _jd()
    j.basis.R = 31  # not k * r
    assert call(j=j) == 1
    assert call(j=_jd(diag=2)) == 1
    assert call(j=_jd(r=65)) == 2
    assert call(j=_jd(k=5000, n=6000)) == 2  # more clusters than the one-workgroup grouping takes
    assert call(j=_jd(k=2049, n=3000)) == 2
    assert call(T=8193) == 2                   # more tokens than it takes
    assert call(T=L.LORA_SEGMENT_MAX_T + 1) == 2


def _rsvd_ws(n, d_in, d_out):
    return n * 7 * 64 * 64 * 8


@pytest.mark.parametrize("n,d_in,d_out", [(1, 16, 16), (1024, 3584, 3584), (7, 520, 264), (3, 64, 200),
                                          (0, 64, 64)])
def test_rsvd_workspace_bytes(lib, n, d_in, d_out):
    assert lib.lora_rsvd_workspace_bytes(n, d_in, d_out) == _rsvd_ws(n, d_in, d_out)


def test_rsvd_workspace_bytes_invalid(lib):
    assert lib.lora_rsvd_workspace_bytes(-1, 64, 64) == 0
    assert lib.lora_rsvd_workspace_bytes(4, 0, 64) == 0
    assert lib.lora_rsvd_workspace_bytes(4, 64, 0) == 0


def test_rsvd_factor_rejects_before_launch(lib):
    f = lib.lora_rsvd_factor
    big = 1 << 40

    def call(n=4, d_in=256, d_out=128, dtype=1, r=16, A=FAKE, B=FAKE, sig=FAKE, st=FAKE, ws=FAKE, wsb=big):
        return f(n, d_in, d_out, dtype, r, A, B, sig, st, ws, wsb, None)

    assert call(n=0) == 0
    assert call(n=-1) == 1
    assert call(r=0) == 1
    assert call(d_in=0) == 1
    assert call(r=65) == 2
    assert call(d_in=15) == 2  # fewer rows than the rank
    assert call(d_out=8) == 2
    assert call(dtype=7) == 2
    for k in ("A", "B", "sig", "st", "ws"):
        assert call(**{k: None}) == 1
    assert call(wsb=_rsvd_ws(4, 256, 128) - 1) == 1
    assert call(ws=FAKE + 8) == 2
    assert call(A=FAKE + 2) == 2
    assert call(B=FAKE + 4) == 2
    assert call(d_in=260) == 2  # rows read as 16-byte vectors: bf16 d a multiple of 8
    assert call(d_out=132, dtype=1) == 2
    assert call(n=1 << 24) == 2  # grid too large
    g = lib.lora_rsvd_factor_phases
    for bad in (0, 16, -1):
        assert g(4, 256, 128, 1, 16, FAKE, FAKE, FAKE, FAKE, FAKE, big, None, bad) == 1
    for good in (1, 2, 4, 8, 6, 15):
        assert g(0, 256, 128, 1, 16, FAKE, FAKE, FAKE, FAKE, FAKE, big, None, good) == 0
    assert g(0, 256, 128, 1, 16, FAKE, FAKE, FAKE, FAKE, FAKE, big, None, 1) == 0
    assert g(4, 256, 128, 1, 65, FAKE, FAKE, FAKE, FAKE, FAKE, big, None, 2) == 2


def test_rsvd_write_rejects_before_launch(lib):
    f = lib.lora_rsvd_write
    big = 1 << 40
    st = _store(n=4, d_in=64, d_out=32, r_max=8)
    assert f(None, 8, FAKE, FAKE, FAKE, big, None) == 1
    assert f(C.byref(st), 0, FAKE, FAKE, FAKE, big, None) == 1
    assert f(C.byref(st), 33, FAKE, FAKE, FAKE, big, None) == 2  # d_out below r
    assert f(C.byref(st), 8, None, FAKE, FAKE, big, None) == 1
    assert f(C.byref(st), 8, FAKE, None, FAKE, big, None) == 1
    assert f(C.byref(st), 8, FAKE, FAKE, None, big, None) == 1
    assert f(C.byref(st), 8, FAKE, FAKE, FAKE, _rsvd_ws(4, 64, 32) - 1, None) == 1
    assert f(C.byref(st), 8, FAKE, FAKE, FAKE + 8, big, None) == 2
    assert f(C.byref(st), 8, FAKE + 2, FAKE, FAKE, big, None) == 2
    empty = _store(n=4, d_in=64, d_out=32, r_max=0, R=0)
    assert f(C.byref(empty), 8, None, None, None, 0, None) == 0


def _multi(k=2, n=4, d_in=64, d_outs=(32, 16), r_max=8):
    m = L.lora_multi_store()
    m.n_slices = k
    m.stacked = _store(n=n, d_in=d_in, d_out=d_in, r_max=2 * r_max, R=40)
    for s in range(k):
        m.slice[s] = _store(n=n, d_in=d_in, d_out=d_outs[s % len(d_outs)], r_max=r_max, R=20)
    m.hoff = FAKE
    return m


def test_multi_bytes_and_rejects(lib):
    arr = (L.lora_store * 2)(_store(n=4, d_in=64, d_out=32, R=20), _store(n=4, d_in=64, d_out=16, R=12))
    a, mb, hb = C.c_size_t(), C.c_size_t(), C.c_size_t()
    assert lib.lora_multi_bytes(2, arr, C.byref(a), C.byref(mb), C.byref(hb)) == 0
    assert a.value == (20 + 12) * 64 * 2 and hb.value == 2 * 4 * 4
    assert lib.lora_multi_bytes(0, arr, C.byref(a), C.byref(mb), C.byref(hb)) == 1
    assert lib.lora_multi_bytes(5, arr, C.byref(a), C.byref(mb), C.byref(hb)) == 1
    assert lib.lora_multi_bytes(2, None, C.byref(a), C.byref(mb), C.byref(hb)) == 1
    bad = (L.lora_store * 2)(_store(n=4, d_in=64), _store(n=5, d_in=64))  # different adapters
    assert lib.lora_multi_bytes(2, bad, C.byref(a), C.byref(mb), C.byref(hb)) == 1
    bad = (L.lora_store * 2)(_store(n=4, d_in=64), _store(n=4, d_in=128))
    assert lib.lora_multi_bytes(2, bad, C.byref(a), C.byref(mb), C.byref(hb)) == 1
    bad = (L.lora_store * 2)(_store(n=4, d_in=64, dtype=1), _store(n=4, d_in=64, dtype=0))
    assert lib.lora_multi_bytes(2, bad, C.byref(a), C.byref(mb), C.byref(hb)) == 1
    st = L.lora_multi_store()
    assert lib.lora_pack_multi(C.byref(st), 2, arr, FAKE, None, FAKE, None) == 1
    assert lib.lora_pack_multi(C.byref(st), 2, arr, FAKE, FAKE, None, None) == 1
    assert lib.lora_pack_multi(C.byref(st), 2, arr, FAKE, FAKE + 4, FAKE, None) == 2
    assert lib.lora_pack_multi(None, 2, arr, FAKE, FAKE, FAKE, None) == 1


def test_multi_workspace_and_apply_rejects(lib):
    m = _multi()
    # The stacked store's workspace, then 16 bytes per slice and possible
    # sub-tile of <= 16 tokens (the slice records), 256-byte aligned.
    for T in (16, 1000):
        max_sub = (T + 15 * min(4, T)) // 16
        want = lib.lora_workspace_bytes(C.byref(m.stacked), T) + -(-(16 * max_sub * 2) // 256) * 256
        assert lib.lora_multi_workspace_bytes(C.byref(m), T) == want
    assert lib.lora_multi_workspace_bytes(None, 16) == 0
    assert lib.lora_multi_workspace_bytes(C.byref(m), -1) == 0
    big = 1 << 30
    ys = (C.c_void_p * 2)(FAKE, FAKE)
    lds = (C.c_int64 * 2)(32, 16)
    f = lib.lora_apply_multi

    def call(mm=None, T=16, ids=FAKE, x=FAKE, ldx=64, y=ys, ld=lds, ws=FAKE, wsb=big):
        mm = mm if mm is not None else _multi()
        return f(C.byref(mm), x, ldx, y, ld, T, ids, None, None, ws, wsb, None)

    assert call(T=0) == 0
    assert call(T=-1) == 1
    assert call(x=None) == 1
    assert call(ldx=32) == 1
    assert call(y=None) == 1
    assert call(ld=(C.c_int64 * 2)(32, 8)) == 1  # slice 1's row shorter than its d_out
    assert call(y=(C.c_void_p * 2)(FAKE, FAKE + 2)) == 2
    assert call(ws=None) == 1
    assert call(wsb=64) == 1
    assert call(wsb=lib.lora_multi_workspace_bytes(C.byref(_multi()), 16) - 1) == 1  # no room for the slice records
    assert call(T=L.LORA_SEGMENT_MAX_T + 1) == 2
    mm = _multi()
    mm.hoff = None
    assert call(mm=mm) == 1
    mm = _multi()
    mm.n_slices = 0
    assert call(mm=mm) == 1
    mm = _multi()
    mm.slice[1].d_in = 128  # slices disagree
    assert call(mm=mm) == 1
    assert f(None, FAKE, 64, ys, lds, 16, FAKE, None, None, FAKE, big, None) == 1
