"""GPU: retained-factor construction (r-SVD) against the oracle.

"LoRAForge" (section "FlashTSQR: An Accelerator for Batched Factor
Construction") and "Compress then Serve" section 4: per adapter, the rank-k
SVD of B A, kept as B' = Q_B U_k and A' = S_k V_k^T Q_A^T.  Checked against
oracle.retained_factors_ref (numpy QR and SVD in float64):

* singular values: max |sigma - sigma_ref| <= 1e-5 max sigma_ref (they are
  computed in float64 and rounded once to float32);
* the retained product B' A' (unique while sigma_k > sigma_k+1): max error
  <= 1e-5 (float32) / 2e-2 (bf16) of its largest entry, as for the apply;
* float32: B'^T B' = I to 1e-5, and each component (a column of B' and the
  row of A') equal to the oracle's up to its sign, to 1e-4;
* zeros where the store pads, and past r when a retained rank exceeds r;
* status 1 exactly for rank-deficient adapters.
"""
import numpy as np
import pytest
import torch

import rank_specialized_amd as rs
from oracle import apply_ref, retained_factors_ref, rsvd_ref, spectral_ranks_ref, uniform_ranks_ref
from workloads import make_random_workload, make_rsvd_config, make_rsvd_workload

from gpu_helpers import TOL, TORCH_DTYPE, device, note, to_dev, y_host

pytestmark = pytest.mark.gpu


def _upload(w, dev):
    dt = TORCH_DTYPE[w.dtype]
    return to_dev(w.A, dt, dev), to_dev(w.B, dt, dev)


def _retained(store, a):
    """(A'_a [stored, d_in], B'_a [d_out, stored]) read back from a store."""
    row_off, rank, _ = store.device_meta()
    ro, st = int(row_off[a]), int(rank[a])
    R = store.c.R
    A = store.A_pack.view(store.dtype)[: R * store.d_in].view(R, store.d_in)[ro: ro + st]
    B = store.B_pack.view(store.dtype)[ro * store.d_out: (ro + st) * store.d_out].view(store.d_out, st)
    return A.double().cpu().numpy(), B.double().cpu().numpy()


CASES = {
    "small": dict(seed=1, n=5, r=8, d_in=40, d_out=24),
    "rank1": dict(seed=2, n=3, r=1, d_in=16, d_out=16),
    "rank33": dict(seed=3, n=4, r=33, d_in=200, d_out=136),
    "rank64_ragged": dict(seed=4, n=6, r=64, d_in=520, d_out=264),
    "rank5_tall": dict(seed=12, n=7, r=5, d_in=1032, d_out=8),
    "square": dict(seed=5, n=3, r=16, d_in=16, d_out=16),
    "k_proj": dict(seed=6, n=4, r=64, d_in=3584, d_out=512),
    "flat": dict(seed=7, n=4, r=32, d_in=256, d_out=128, spectrum="flat"),
}


def _make(name, dtype):
    kw = dict(CASES[name])
    return make_rsvd_workload(kw.pop("seed"), kw.pop("n"), kw.pop("r"), kw.pop("d_in"), kw.pop("d_out"),
                              dtype=dtype, **kw)


def _keep(w):
    """A spread of retained ranks: 0, 1, r, r - 1, then r // 2 ..."""
    r = w.r
    base = [0, 1, r, max(r - 1, 0)]
    return [base[a] if a < len(base) else max(1, r // (a - 2)) for a in range(w.n)]


def _check_adapter(w, store, a, k, tol_prod, components):
    A2, B2 = _retained(store, a)
    stored = A2.shape[0]
    kk = min(k, w.r)
    rA, rB, s = retained_factors_ref(w.A[a].astype(np.float64), w.B[a].astype(np.float64), kk)
    assert np.all(A2[kk:] == 0) and np.all(B2[:, kk:] == 0), "components past min(k, r) and padding are zero"
    if kk == 0:
        return
    prod, ref = B2[:, :kk] @ A2[:kk], rB @ rA
    assert np.abs(prod - ref).max() <= tol_prod * np.abs(ref).max(), (a, k)
    if components:
        Bk = B2[:, :kk]
        assert np.abs(Bk.T @ Bk - np.eye(kk)).max() <= 1e-5, (a, k)
        for c in range(kk):
            sg = 1.0 if Bk[:, c] @ rB[:, c] >= 0 else -1.0
            assert np.abs(sg * Bk[:, c] - rB[:, c]).max() <= 1e-4, (a, c)
            assert np.abs(sg * A2[c] - rA[c]).max() <= 1e-4 * max(s[0], 1e-30), (a, c)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_rsvd_parity(name, dtype):
    dev = device()
    w = _make(name, dtype)
    A, B = _upload(w, dev)
    note(f"rsvd {name} {dtype} n={w.n} r={w.r} d={w.d_in}->{w.d_out}")
    f = rs.lora_rsvd_factor(A, B)
    torch.cuda.synchronize()
    sig = f.sigma.cpu().numpy().astype(np.float64)
    assert np.all(f.status.cpu().numpy() == 0)
    for a in range(w.n):
        s_ref = rsvd_ref(w.A[a], w.B[a])[0]
        assert np.abs(sig[a] - s_ref).max() <= 1e-5 * s_ref.max(), a
        assert np.all(np.diff(sig[a]) <= 0)
    keep = _keep(w)
    for pad_to in (0, w.r):
        note(f"rsvd write {name} {dtype} pad_to={pad_to}")
        store = rs.lora_rsvd_write(f, keep, w.scales, pad_to=pad_to)
        torch.cuda.synchronize()
        for a in range(w.n):
            _check_adapter(w, store, a, keep[a], TOL[dtype], dtype == "fp32" and w.r > 1)


def test_rsvd_phases_match_whole():
    """The four kernels run one call at a time give the same bits."""
    dev = device()
    w = _make("rank64_ragged", "bf16")
    A, B = _upload(w, dev)
    note("rsvd phases")
    f = rs.lora_rsvd_factor(A, B)
    g = rs.lora_rsvd_factor(A, B, phases=1)
    for ph in (2, 4, 8):
        rs.lora_rsvd_factor(A, B, phases=ph, out=g)
    torch.cuda.synchronize()
    assert torch.equal(f.sigma, g.sigma) and torch.equal(f.status, g.status)
    assert torch.equal(f.ws, g.ws)


def test_rsvd_ranks_above_r():
    """A retained rank above r keeps the whole product; the rest is zero."""
    dev = device()
    w = make_rsvd_workload(8, 3, 8, 64, 48, dtype="fp32")
    A, B = _upload(w, dev)
    note("rsvd ranks above r")
    f = rs.lora_rsvd_factor(A, B)
    store = rs.lora_rsvd_write(f, [8, 10, 12], w.scales)
    torch.cuda.synchronize()
    for a, k in enumerate([8, 10, 12]):
        A2, B2 = _retained(store, a)
        assert A2.shape[0] == k and np.all(A2[8:] == 0) and np.all(B2[:, 8:] == 0)
        ref = w.B[a].astype(np.float64) @ w.A[a].astype(np.float64)
        assert np.abs(B2 @ A2 - ref).max() <= 1e-5 * np.abs(ref).max()


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_rsvd_rank_deficient_and_zero(dtype):
    """Adapters 0, 1: B with its last 3 columns zero (rank r - 3); adapter 2:
    all-zero B.  Their status is 1; the others' 0; the zero adapter's values
    and retained factors are zero, the deficient ones' trailing values tiny
    and their leading product still right."""
    dev = device()
    w = make_rsvd_workload(9, 5, 12, 96, 80, dtype=dtype, zero_cols=3, zero_adapters=2)
    w.B[2] = 0.0
    A, B = _upload(w, dev)
    note(f"rsvd rank-deficient {dtype}")
    f = rs.lora_rsvd_factor(A, B)
    torch.cuda.synchronize()
    st = f.status.cpu().numpy()
    assert list(st) == [1, 1, 1, 0, 0]
    sig = f.sigma.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(sig))
    assert np.all(sig[2] == 0)
    for a in (0, 1):
        assert sig[a][-3:].max() <= 1e-6 * sig[a][0]
        s_ref = rsvd_ref(w.A[a], w.B[a])[0]
        assert np.abs(sig[a] - s_ref).max() <= 1e-5 * s_ref.max()
    store = rs.lora_rsvd_write(f, [6] * 5, w.scales)
    torch.cuda.synchronize()
    A2, B2 = _retained(store, 2)
    assert np.all(A2 == 0) and np.all(B2 == 0)
    for a in (0, 1, 3):
        _check_adapter(w, store, a, 6, TOL[dtype], False)


def test_rsvd_spectral_store_serves():
    """Factor, choose ranks by the spectral budget from the GPU's singular
    values (the library's policy equals the oracle's on them), write the
    store, and apply it: the result matches the oracle apply of the oracle's
    retained factors at those ranks."""
    dev = device()
    w = make_rsvd_workload(10, 24, 16, 512, 384, dtype="bf16")
    A, B = _upload(w, dev)
    note("rsvd spectral store serves")
    f = rs.lora_rsvd_factor(A, B)
    torch.cuda.synchronize()
    sig = f.sigma.cpu().numpy()
    budget = sum(uniform_ranks_ref([w.r] * w.n, 0.25, 2))
    ranks = rs.lora_ranks_spectral([w.r] * w.n, list(sig), 2, budget)
    assert ranks == spectral_ranks_ref([w.r] * w.n, [list(map(float, s)) for s in sig], 2, budget)
    store = rs.lora_rsvd_write(f, ranks, w.scales)
    wl = make_random_workload(11, 300, w.n, w.d_in, w.d_out, ranks, dtype="bf16", id_mode="zipf")
    Ar, Br = [], []
    for a in range(w.n):
        a2, b2, _ = retained_factors_ref(w.A[a].astype(np.float64), w.B[a].astype(np.float64), ranks[a])
        Ar.append(a2)
        Br.append(b2)
    x = to_dev(wl.x, torch.bfloat16, dev)
    ids = torch.from_numpy(wl.ids.astype(np.int32)).to(dev)
    y = torch.zeros(wl.T, w.d_out, dtype=torch.bfloat16, device=dev)
    rs.lora_apply_batched(store, x, y, ids=ids)
    torch.cuda.synchronize()
    ref = apply_ref(wl.x, wl.ids, Ar, Br, w.scales)
    assert np.abs(y_host(y) - ref).max() <= TOL["bf16"] * np.abs(ref).max()


def test_rsvd_config_sampled():
    """The measured configuration at full size (1024 adapters of rank 64,
    3584 -> 3584, bf16) in the measured launch: sampled adapters against the
    oracle (singular values, the retained product at the spectral ranks)."""
    dev = device()
    w = make_rsvd_config("rsvd-q")
    A, B = _upload(w, dev)
    note("rsvd-q full size")
    f = rs.lora_rsvd_factor(A, B)
    torch.cuda.synchronize()
    sig = f.sigma.cpu().numpy()
    assert np.all(f.status.cpu().numpy() == 0)
    budget = sum(uniform_ranks_ref([w.r] * w.n, 1.0 / 12.0, 4))
    ranks = rs.lora_ranks_spectral([w.r] * w.n, list(sig), 4, budget)
    store = rs.lora_rsvd_write(f, ranks, w.scales)
    torch.cuda.synchronize()
    for a in (0, 1, 517, 1023):
        s_ref = rsvd_ref(w.A[a], w.B[a])[0]
        assert np.abs(sig[a].astype(np.float64) - s_ref).max() <= 1e-5 * s_ref.max(), a
        _check_adapter(w, store, a, ranks[a], TOL["bf16"], False)
