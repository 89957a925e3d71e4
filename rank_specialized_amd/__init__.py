"""Batched, rank-specialized LoRA-delta apply on AMD Instinct MI355X.

Thin PyTorch binding over the C ABI (include/lora.h).  Torch provides device
memory and the current stream; every step of the apply runs in the HIP
kernels of librank_specialized.so.  The entry points keep the C names:

    store = lora_pack_retained(A_list, B_list, scales)        # pack
    seg   = lora_segment(ids, store.n)                        # group tokens
    h     = lora_shrink(store, x, seg)                        # h = A_a x (grouped rows)
    lora_expand(store, h, seg, y)                             # y += s_a B_a h
    lora_apply_batched(store, x, y, ids=ids)                  # all of the above

Workspaces (lora_workspace_bytes) are allocated here with torch when the
caller passes none.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass
from typing import List, Optional, Sequence

import torch

from . import _lib as L
from ._lib import LoraError, lora_store  # noqa: F401

__all__ = [
    "Store", "Segmentation", "LoraError", "lora_store_bytes", "lora_pack_retained",
    "lora_segment", "lora_plan_bytes", "lora_group", "lora_apply_planned", "lora_workspace_bytes", "lora_shrink", "lora_expand", "lora_apply_batched",
    "lora_apply_batched_phases", "lora_apply_batched_noalloc", "lora_apply_launches", "lora_apply_base_fused", "JDStore", "lora_jd_pack", "lora_jd_workspace_bytes",
    "lora_jd_apply", "lora_ranks_uniform", "lora_ranks_spectral", "RsvdFactors", "lora_rsvd_workspace_bytes",
    "lora_rsvd_factor", "lora_rsvd_write", "MultiStore", "lora_pack_multi", "lora_multi_workspace_bytes",
    "lora_apply_multi", "load_library",
]

_DTYPES = {torch.bfloat16: L.LORA_DTYPE_BF16, torch.float32: L.LORA_DTYPE_F32}


def load_library():
    """Load librank_specialized.so (raises ImportError if it was not built)."""
    return L.lib()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _p(t: Optional[torch.Tensor]):
    return None if t is None or t.numel() == 0 else t.data_ptr()


def _rows(t: torch.Tensor, name: str):
    if t.dim() != 2 or (t.shape[0] > 0 and t.stride(1) != 1):
        raise ValueError(f"{name} must be 2-D with unit column stride")
    return t.stride(0) if t.shape[0] > 0 else t.shape[1]


@dataclass
class Store:
    """A packed retained-rank store: the C struct plus the buffers it references."""

    c: lora_store
    A_pack: torch.Tensor
    B_pack: torch.Tensor
    meta: torch.Tensor
    ranks: List[int]
    dtype: torch.dtype

    @property
    def n(self) -> int:
        return self.c.n

    @property
    def d_in(self) -> int:
        return self.c.d_in

    @property
    def d_out(self) -> int:
        return self.c.d_out

    @property
    def r_max(self) -> int:
        return self.c.r_max

    @property
    def pad_to(self) -> int:
        return self.c.pad_to

    def ref(self):
        return C.byref(self.c)

    def clone(self) -> "Store":
        """An independent copy in fresh device memory (same layout)."""
        A, B, meta = self.A_pack.clone(), self.B_pack.clone(), self.meta.clone()
        c = lora_store.from_buffer_copy(self.c)
        n = self.c.n
        c.A_pack, c.B_pack = A.data_ptr(), B.data_ptr()
        c.row_off = meta.data_ptr()
        c.rank = meta.data_ptr() + (n + 1) * 4
        c.scale = meta.data_ptr() + (2 * n + 1) * 4
        return Store(c, A, B, meta, list(self.ranks), self.dtype)

    def device_meta(self):
        """(row_off, rank, scale) as device tensors (views of the meta buffer)."""
        n = self.n
        i32 = self.meta[: (3 * n + 1) * 4].view(torch.int32)
        return i32[: n + 1], i32[n + 1: 2 * n + 1], i32[2 * n + 1: 3 * n + 1].view(torch.float32)


def lora_store_bytes(n: int, d_in: int, d_out: int, dtype: torch.dtype, ranks: Sequence[int],
                     pad_to: int = 0):
    r = (C.c_int32 * max(n, 1))(*[int(v) for v in ranks])
    a, b, m = C.c_size_t(), C.c_size_t(), C.c_size_t()
    L.check("lora_store_bytes", L.lib().lora_store_bytes(n, d_in, d_out, _DTYPES[dtype], r, pad_to,
                                                         C.byref(a), C.byref(b), C.byref(m)))
    return a.value, b.value, m.value


def lora_pack_retained(A_list: Sequence[torch.Tensor], B_list: Sequence[torch.Tensor], scales,
                       pad_to: int = 0) -> Store:
    """Pack per-adapter factors (A_a [r_a, d_in], B_a [d_out, r_a], device tensors,
    row-major contiguous, one dtype) into a store.  pad_to > 0 builds the
    rank-padded comparison store."""
    n = len(A_list)
    if n == 0 or len(B_list) != n:
        raise ValueError("need one A and one B per adapter")
    dtype = A_list[0].dtype
    device = A_list[0].device
    d_in = A_list[0].shape[1]
    d_out = B_list[0].shape[0]
    ranks = [int(a.shape[0]) for a in A_list]
    for a, b, r in zip(A_list, B_list, ranks):
        if a.dtype != dtype or b.dtype != dtype or a.shape != (r, d_in) or b.shape != (d_out, r):
            raise ValueError("factor shapes/dtypes are inconsistent")
        if not (a.is_contiguous() and b.is_contiguous()):
            raise ValueError("factors must be contiguous")
    return _pack(n, d_in, d_out, dtype, ranks, scales, pad_to, device,
                 (C.c_void_p * n)(*[_p(a) for a in A_list]), (C.c_void_p * n)(*[_p(b) for b in B_list]))


def _pack(n, d_in, d_out, dtype, ranks, scales, pad_to, device, a_ptrs, b_ptrs) -> Store:
    """Allocate a store's buffers and call lora_pack_retained (a_ptrs and
    b_ptrs None: metadata only)."""
    a_bytes, b_bytes, m_bytes = lora_store_bytes(n, d_in, d_out, dtype, ranks, pad_to)
    A_pack = torch.empty(max(a_bytes, 16), dtype=torch.uint8, device=device)
    B_pack = torch.empty(max(b_bytes, 16), dtype=torch.uint8, device=device)
    meta = torch.empty(m_bytes, dtype=torch.uint8, device=device)
    r_arr = (C.c_int32 * n)(*ranks)
    s_arr = (C.c_float * n)(*[float(v) for v in scales])
    st = lora_store()
    L.check("lora_pack_retained", L.lib().lora_pack_retained(
        C.byref(st), n, d_in, d_out, _DTYPES[dtype], r_arr, s_arr, a_ptrs, b_ptrs,
        A_pack.data_ptr(), B_pack.data_ptr(), meta.data_ptr(), pad_to, _stream(meta)))
    return Store(st, A_pack, B_pack, meta, list(ranks), dtype)


@dataclass
class Segmentation:
    """Grouped order of T tokens over n adapters (as lora_segment writes it)."""

    T: int
    n: int
    seg_off: torch.Tensor  # int32 [n + 2]
    perm: torch.Tensor  # int32 [T]
    n_invalid: Optional[torch.Tensor] = None
    plan: Optional[torch.Tensor] = None  # uint8 [lora_plan_bytes(T, n)] (lora_group)


def lora_segment(ids: torch.Tensor, n: int, *, seg: Optional[Segmentation] = None) -> Segmentation:
    """Stable grouping of tokens by adapter id (ids: int32 device tensor [T])."""
    if ids.dtype != torch.int32 or ids.dim() != 1 or not ids.is_contiguous():
        raise ValueError("ids must be a contiguous int32 vector")
    T = ids.shape[0]
    dev = ids.device
    if seg is None:
        seg = Segmentation(T, n, torch.empty(n + 2, dtype=torch.int32, device=dev),
                           torch.empty(max(T, 1), dtype=torch.int32, device=dev)[:T],
                           torch.empty(1, dtype=torch.int32, device=dev))
    L.check("lora_segment", L.lib().lora_segment(
        _p(ids), T, n, seg.seg_off.data_ptr(), _p(seg.perm), seg.n_invalid.data_ptr(), _stream(seg.seg_off)))
    return seg


def lora_plan_bytes(T: int, n: int) -> int:
    return int(L.lib().lora_plan_bytes(T, n))


def lora_group(ids: torch.Tensor, n: int, *, seg: Optional[Segmentation] = None) -> Segmentation:
    """lora_segment plus the plan of the grouping (its sub-tiles), which
    lora_apply_planned reuses across stores."""
    if ids.dtype != torch.int32 or ids.dim() != 1 or not ids.is_contiguous():
        raise ValueError("ids must be a contiguous int32 vector")
    T = ids.shape[0]
    dev = ids.device
    nb = lora_plan_bytes(T, n)
    if seg is None or seg.plan is None:
        seg = Segmentation(T, n, torch.empty(n + 2, dtype=torch.int32, device=dev),
                           torch.empty(max(T, 1), dtype=torch.int32, device=dev)[:T],
                           torch.empty(1, dtype=torch.int32, device=dev),
                           torch.empty(max(nb, 16), dtype=torch.uint8, device=dev))
    L.check("lora_group", L.lib().lora_group(
        _p(ids), T, n, seg.seg_off.data_ptr(), _p(seg.perm), seg.plan.data_ptr(), seg.plan.numel(),
        seg.n_invalid.data_ptr(), _stream(seg.seg_off)))
    return seg


def lora_workspace_bytes(store: Store, T: int) -> int:
    return int(L.lib().lora_workspace_bytes(store.ref(), T))


def _ws(store: Store, T: int, ws: Optional[torch.Tensor], device) -> torch.Tensor:
    if ws is None:
        ws = torch.empty(max(lora_workspace_bytes(store, T), 16), dtype=torch.uint8, device=device)
    return ws


def lora_shrink(store: Store, x: torch.Tensor, seg: Segmentation, h: Optional[torch.Tensor] = None,
                ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """h[i, :r_a] = A_a x[perm[i]] in float32 (grouped rows).  Columns >= r_a
    and rows of tokens without an adapter are left as they were in ``h``."""
    T = x.shape[0]
    if h is None:
        h = torch.zeros(T, max(store.r_max, 1), dtype=torch.float32, device=x.device)
    ws = _ws(store, T, ws, x.device)
    L.check("lora_shrink", L.lib().lora_shrink(
        store.ref(), _p(x), _rows(x, "x"), T, seg.seg_off.data_ptr(), _p(seg.perm), _p(h), _rows(h, "h"),
        ws.data_ptr(), ws.numel(), _stream(x)))
    return h


def lora_expand(store: Store, h: torch.Tensor, seg: Segmentation, y: torch.Tensor,
                ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y[perm[i]] += s_a B_a h[i] in place."""
    T = y.shape[0]
    ws = _ws(store, T, ws, y.device)
    L.check("lora_expand", L.lib().lora_expand(
        store.ref(), _p(h), _rows(h, "h"), T, seg.seg_off.data_ptr(), _p(seg.perm), _p(y), _rows(y, "y"),
        ws.data_ptr(), ws.numel(), _stream(y)))
    return y


def lora_apply_batched(store: Store, x: torch.Tensor, y: torch.Tensor, *,
                       ids: Optional[torch.Tensor] = None, seg: Optional[Segmentation] = None,
                       ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y[t] += s_a B_a (A_a x[t]) in place, for ids (grouped here) or a prior grouping."""
    T = x.shape[0]
    if (ids is None) == (seg is None):
        raise ValueError("pass exactly one of ids or seg")
    ws = _ws(store, T, ws, x.device)
    if seg is not None:
        so, pm = seg.seg_off.data_ptr(), _p(seg.perm)
    else:
        if ids.dtype != torch.int32 or not ids.is_contiguous():
            raise ValueError("ids must be a contiguous int32 vector")
        so = pm = None
    L.check("lora_apply_batched", L.lib().lora_apply_batched(
        store.ref(), _p(x), _rows(x, "x"), _p(y), _rows(y, "y"), T, _p(ids) if ids is not None else None,
        so, pm, ws.data_ptr(), ws.numel(), _stream(x)))
    return y


def lora_apply_batched_phases(store: Store, x: torch.Tensor, y: torch.Tensor, phases: int, *,
                              ids: Optional[torch.Tensor] = None, seg: Optional[Segmentation] = None,
                              ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One kernel of lora_apply_batched at a time (phases 1 = shrink, 2 =
    expand from the plan a phase-1 call left in ``ws``, 3 = the apply, a
    single fused kernel for decode-sized calls)."""
    T = x.shape[0]
    if (ids is None) == (seg is None):
        raise ValueError("pass exactly one of ids or seg")
    ws = _ws(store, T, ws, x.device)
    so = seg.seg_off.data_ptr() if seg is not None else None
    pm = _p(seg.perm) if seg is not None else None
    if ids is not None and (ids.dtype != torch.int32 or not ids.is_contiguous()):
        raise ValueError("ids must be a contiguous int32 vector")
    L.check("lora_apply_batched_phases", L.lib().lora_apply_batched_phases(
        store.ref(), _p(x), _rows(x, "x"), _p(y), _rows(y, "y"), T, _p(ids) if ids is not None else None,
        so, pm, ws.data_ptr(), ws.numel(), _stream(x), phases))
    return y


def lora_apply_batched_noalloc(store: Store, x: torch.Tensor, y: torch.Tensor, *,
                               ids: Optional[torch.Tensor] = None,
                               seg: Optional[Segmentation] = None) -> torch.Tensor:
    """lora_apply_batched without a workspace: the library's own per-device
    scratch array serves as one (nothing is allocated, here or in the
    library).  Calls that overlap on one device race on that array."""
    T = x.shape[0]
    if (ids is None) == (seg is None):
        raise ValueError("pass exactly one of ids or seg")
    if seg is not None:
        so, pm = seg.seg_off.data_ptr(), _p(seg.perm)
    else:
        if ids.dtype != torch.int32 or not ids.is_contiguous():
            raise ValueError("ids must be a contiguous int32 vector")
        so = pm = None
    L.check("lora_apply_batched_noalloc", L.lib().lora_apply_batched_noalloc(
        store.ref(), _p(x), _rows(x, "x"), _p(y), _rows(y, "y"), T, _p(ids) if ids is not None else None,
        so, pm, _stream(x)))
    return y


def lora_apply_base_fused(store: Store, W0: torch.Tensor, x: torch.Tensor, y: torch.Tensor, *,
                          ids: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = x W0^T + s_a B_a (A_a x) per token (overwrites y): the base layer
    W0 [d_out, d_in] with the adapter branch added in its epilogue, y written
    once.  Without ids: the base product alone.  bf16 stores only."""
    T = x.shape[0]
    if W0.dim() != 2 or W0.shape[0] != store.d_out or W0.shape[1] < store.d_in:
        raise ValueError("W0 must be [d_out, >= d_in]")
    if ids is not None:
        if ids.dtype != torch.int32 or not ids.is_contiguous():
            raise ValueError("ids must be a contiguous int32 vector")
        ws = _ws(store, T, ws, x.device)
    L.check("lora_apply_base_fused", L.lib().lora_apply_base_fused(
        store.ref(), _p(W0), _rows(W0, "W0"), _p(x), _rows(x, "x"), _p(y), _rows(y, "y"), T,
        _p(ids) if ids is not None else None, ws.data_ptr() if ws is not None else None,
        ws.numel() if ws is not None else 0, _stream(x)))
    return y


def lora_apply_planned(store: Store, x: torch.Tensor, y: torch.Tensor, seg: Segmentation, *,
                       ws: Optional[torch.Tensor] = None, phases: int = 3) -> torch.Tensor:
    """y[t] += s_a B_a (A_a x[t]) in place on the plan of ``seg`` (from
    lora_group): the shrink and the expand only (phases 1 / 2: one of them)."""
    T = x.shape[0]
    if seg.plan is None:
        raise ValueError("seg has no plan (use lora_group)")
    ws = _ws(store, T, ws, x.device)
    L.check("lora_apply_planned_phases", L.lib().lora_apply_planned_phases(
        store.ref(), _p(x), _rows(x, "x"), _p(y), _rows(y, "y"), T, seg.plan.data_ptr(), seg.plan.numel(),
        ws.data_ptr(), ws.numel(), _stream(x), phases))
    return y


def lora_apply_launches(store: Store, T: int, with_ids=True) -> int:
    """Kernel launches an apply makes for this store and T: with_ids True / 1
    (ids), False / 0 (a caller's seg_off, perm), 2 (a plan).  1 = the fused
    decode kernel, 2 = shrink + expand, 3 = grouping + shrink + expand,
    4 = sort + plan + shrink + expand."""
    v = L.lib().lora_apply_launches(store.ref(), int(T), int(with_ids))
    if v < 0:
        L.check("lora_apply_launches", -v)
    return v


@dataclass
class JDStore:
    """A shared-basis store: the basis store over clusters (A = V_j^T, B = U_j,
    rank r, scale 1) plus per-adapter cluster, Sigma and scale buffers."""

    c: L.lora_jd_store
    basis: Store
    cluster_of: torch.Tensor
    sigma: torch.Tensor
    scale: torch.Tensor

    @property
    def n(self) -> int:
        return self.c.n_adapters

    @property
    def k(self) -> int:
        return self.basis.n

    @property
    def r(self) -> int:
        return self.c.r

    def ref(self):
        return C.byref(self.c)

    def clone(self) -> "JDStore":
        return _jd_store(self.basis.clone(), self.cluster_of.clone(), self.sigma.clone(), self.scale.clone(),
                         self.c.diag)


def _jd_store(basis: Store, cluster_of, sigma, scale, diag: int) -> JDStore:
    c = L.lora_jd_store()
    c.basis = basis.c
    c.n_adapters = int(cluster_of.numel())
    c.r = basis.r_max
    c.diag = int(diag)
    c.cluster_of, c.sigma, c.scale = cluster_of.data_ptr(), sigma.data_ptr(), scale.data_ptr()
    return JDStore(c, basis, cluster_of, sigma, scale)


def lora_jd_pack(U_list: Sequence[torch.Tensor], V_list: Sequence[torch.Tensor], cluster_of, sigma, scales) -> JDStore:
    """Shared-basis store from per-cluster U_j [d_out, r] and V_j [d_in, r]
    (device tensors of one dtype), cluster_of [n], Sigma [n, r, r] (full) or
    [n, r] (diagonal) and scales [n]."""
    k = len(U_list)
    if k == 0 or len(V_list) != k:
        raise ValueError("need one U and one V per cluster")
    device = U_list[0].device
    basis = lora_pack_retained([V.t().contiguous() for V in V_list], [U.contiguous() for U in U_list], [1.0] * k)
    r = basis.r_max
    sig = torch.as_tensor(sigma, dtype=torch.float32).to(device).contiguous()
    n = sig.shape[0]
    if sig.shape not in ((n, r, r), (n, r)):
        raise ValueError("sigma must be [n, r, r] or [n, r]")
    cl = torch.as_tensor(cluster_of, dtype=torch.int32).to(device).contiguous()
    sc = torch.as_tensor(scales, dtype=torch.float32).to(device).contiguous()
    if cl.shape != (n,) or sc.shape != (n,):
        raise ValueError("cluster_of and scales need one entry per adapter")
    return _jd_store(basis, cl, sig, sc, 1 if sig.dim() == 2 else 0)


def lora_jd_workspace_bytes(store: JDStore, T: int) -> int:
    return int(L.lib().lora_jd_workspace_bytes(store.ref(), int(T)))


def lora_jd_apply(store: JDStore, x: torch.Tensor, y: torch.Tensor, ids: torch.Tensor,
                  ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y[t] += s_a U_c Sigma_a V_c^T x[t] in place (a = ids[t], c = its cluster)."""
    T = x.shape[0]
    if ids.dtype != torch.int32 or not ids.is_contiguous():
        raise ValueError("ids must be a contiguous int32 vector")
    if ws is None:
        ws = torch.empty(max(lora_jd_workspace_bytes(store, T), 16), dtype=torch.uint8, device=x.device)
    L.check("lora_jd_apply", L.lib().lora_jd_apply(store.ref(), _p(x), _rows(x, "x"), _p(y), _rows(y, "y"), T,
                                                   _p(ids), ws.data_ptr(), ws.numel(), _stream(x)))
    return y


def lora_ranks_uniform(r_orig: Sequence[int], ratio: float, floor: int) -> List[int]:
    """Retained ranks by a uniform ratio of the original rank, with a floor."""
    m = len(r_orig)
    ro = (C.c_int32 * max(m, 1))(*[int(v) for v in r_orig])
    out = (C.c_int32 * max(m, 1))()
    L.check("lora_ranks_uniform", L.lib().lora_ranks_uniform(m, ro, float(ratio), int(floor), out))
    return list(out)[:m]


def lora_ranks_spectral(r_orig: Sequence[int], sigmas, floor: int, budget: int) -> List[int]:
    """Retained ranks by a spectral budget: floors first, then the largest
    remaining singular values over all units, `budget` ranks in total."""
    import numpy as np
    m = len(r_orig)
    ro = np.ascontiguousarray(np.asarray(r_orig, np.int32))
    flat = np.ascontiguousarray(np.concatenate([np.asarray(s, np.float32) for s in sigmas]) if m else
                                np.zeros(1, np.float32))
    off = np.zeros(m + 1, np.int64)
    off[1:] = np.cumsum(ro)
    out = np.zeros(max(m, 1), np.int32)
    L.check("lora_ranks_spectral", L.lib().lora_ranks_spectral(
        m, ro.ctypes.data, flat.ctypes.data, off.ctypes.data, int(floor), int(budget), out.ctypes.data))
    return [int(v) for v in out[:m]]


@dataclass
class RsvdFactors:
    """What lora_rsvd_factor leaves for lora_rsvd_write: the original factors
    (kept referenced), the singular values, the status flags and the
    workspace holding W_B, W_A."""

    A_all: torch.Tensor  # [n, r, d_in]
    B_all: torch.Tensor  # [n, d_out, r]
    sigma: torch.Tensor  # float32 [n, r], descending
    status: torch.Tensor  # int32 [n]
    ws: torch.Tensor

    @property
    def n(self) -> int:
        return self.A_all.shape[0]

    @property
    def r(self) -> int:
        return self.A_all.shape[1]


def lora_rsvd_workspace_bytes(n: int, d_in: int, d_out: int) -> int:
    return int(L.lib().lora_rsvd_workspace_bytes(n, d_in, d_out))


def lora_rsvd_factor(A_all: torch.Tensor, B_all: torch.Tensor, ws: Optional[torch.Tensor] = None,
                     phases: int = 15, out: Optional[RsvdFactors] = None) -> RsvdFactors:
    """Stage 1 of retained-factor construction for n adapters of one rank r:
    A_all [n, r, d_in], B_all [n, d_out, r] (contiguous, bf16 or float32).
    phases: a bit mask of its kernels (lora_rsvd_factor_phases; 15 = all);
    ``out`` reuses the sigma, status and workspace buffers of a previous call."""
    if A_all.dim() != 3 or B_all.dim() != 3:
        raise ValueError("A_all is [n, r, d_in] and B_all [n, d_out, r]")
    n, r, d_in = A_all.shape
    d_out = B_all.shape[1]
    if B_all.shape != (n, d_out, r) or A_all.dtype != B_all.dtype:
        raise ValueError("A_all and B_all are inconsistent")
    if not (A_all.is_contiguous() and B_all.is_contiguous()):
        raise ValueError("factors must be contiguous")
    if out is not None:
        sigma, status, ws = out.sigma, out.status, out.ws
    else:
        sigma = torch.empty(n, r, dtype=torch.float32, device=A_all.device)
        status = torch.empty(n, dtype=torch.int32, device=A_all.device)
    if ws is None:
        ws = torch.empty(max(lora_rsvd_workspace_bytes(n, d_in, d_out), 16), dtype=torch.uint8, device=A_all.device)
    L.check("lora_rsvd_factor", L.lib().lora_rsvd_factor_phases(
        n, d_in, d_out, _DTYPES[A_all.dtype], r, _p(A_all), _p(B_all), _p(sigma), _p(status), ws.data_ptr(),
        ws.numel(), _stream(A_all), int(phases)))
    return RsvdFactors(A_all, B_all, sigma, status, ws)


def lora_rsvd_write(f: RsvdFactors, ranks: Sequence[int], scales, pad_to: int = 0,
                    store: Optional[Store] = None) -> Store:
    """Stage 2: a store of the retained factors at `ranks` (one per adapter,
    e.g. from lora_ranks_uniform / lora_ranks_spectral over f.sigma).  With
    ``store`` (built by an earlier call for the same adapters), its buffers are
    rewritten in place and ranks / scales / pad_to are taken from it."""
    n, r, d_in = f.A_all.shape
    d_out = f.B_all.shape[1]
    if store is None:
        ranks = [int(v) for v in ranks]
        if len(ranks) != n:
            raise ValueError("one retained rank per adapter")
        store = _pack(n, d_in, d_out, f.A_all.dtype, ranks, scales, pad_to, f.A_all.device, None, None)
    L.check("lora_rsvd_write", L.lib().lora_rsvd_write(store.ref(), r, _p(f.A_all), _p(f.B_all), f.ws.data_ptr(),
                                                       f.ws.numel(), _stream(f.A_all)))
    return store


@dataclass
class MultiStore:
    """Slices of one input (q/k/v, gate/up) for the multi-slice apply: the
    slices' stores (kept referenced), the stacked A buffer, its metadata and
    hoff."""

    c: L.lora_multi_store
    slices: List[Store]
    A: torch.Tensor
    meta: torch.Tensor
    hoff: torch.Tensor

    @property
    def n(self) -> int:
        return self.c.stacked.n

    @property
    def n_slices(self) -> int:
        return self.c.n_slices

    def ref(self):
        return C.byref(self.c)


def lora_pack_multi(slices: Sequence[Store]) -> MultiStore:
    """Stack the A rows of stores of the same adapters (same n, d_in, dtype)."""
    k = len(slices)
    arr = (L.lora_store * max(k, 1))(*[st.c for st in slices])
    a, m, h = C.c_size_t(), C.c_size_t(), C.c_size_t()
    L.check("lora_multi_bytes", L.lib().lora_multi_bytes(k, arr, C.byref(a), C.byref(m), C.byref(h)))
    dev = slices[0].meta.device
    A = torch.empty(max(a.value, 16), dtype=torch.uint8, device=dev)
    meta = torch.empty(m.value, dtype=torch.uint8, device=dev)
    hoff = torch.empty(max(h.value // 4, 4), dtype=torch.int32, device=dev)
    c = L.lora_multi_store()
    L.check("lora_pack_multi", L.lib().lora_pack_multi(C.byref(c), k, arr, A.data_ptr(), meta.data_ptr(),
                                                       hoff.data_ptr(), _stream(meta)))
    return MultiStore(c, list(slices), A, meta, hoff)


def lora_multi_workspace_bytes(store: MultiStore, T: int) -> int:
    return int(L.lib().lora_multi_workspace_bytes(store.ref(), T))


def lora_apply_multi(store: MultiStore, x: torch.Tensor, ys: Sequence[torch.Tensor], ids=None,
                     seg: Optional[Segmentation] = None, ws: Optional[torch.Tensor] = None):
    """y_s += s B_s A_s x for every slice, x read once; ys may be column
    slices of one fused buffer (row stride taken from each view).  A ``seg``
    from lora_group carries a plan, which is then used as it is."""
    T = x.shape[0]
    k = store.n_slices
    if len(ys) != k:
        raise ValueError("one y per slice")
    if (ids is None) == (seg is None):
        raise ValueError("pass exactly one of ids or seg")
    yp = (C.c_void_p * k)(*[_p(y) for y in ys])
    ld = (C.c_int64 * k)(*[_rows(y, "y") for y in ys])
    if ids is not None and (ids.dtype != torch.int32 or not ids.is_contiguous()):
        raise ValueError("ids must be a contiguous int32 vector")
    if ws is None:
        ws = torch.empty(max(lora_multi_workspace_bytes(store, T), 16), dtype=torch.uint8, device=x.device)
    if seg is not None and seg.plan is not None:
        L.check("lora_apply_multi_planned", L.lib().lora_apply_multi_planned(
            store.ref(), _p(x), _rows(x, "x"), yp, ld, T, seg.plan.data_ptr(), seg.plan.numel(), ws.data_ptr(),
            ws.numel(), _stream(x)))
        return ys
    so = seg.seg_off if seg is not None else None
    pm = seg.perm if seg is not None else None
    L.check("lora_apply_multi", L.lib().lora_apply_multi(
        store.ref(), _p(x), _rows(x, "x"), yp, ld, T, _p(ids), _p(so), _p(pm), ws.data_ptr(), ws.numel(),
        _stream(x)))
    return ys
