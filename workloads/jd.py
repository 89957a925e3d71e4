"""Seeded synthetic inputs of the shared-basis (joint-diagonalization) apply.

Draws only: clusters, shared bases U_j and V_j, per-adapter Sigma_i and
scales, ids and activations.  None of the apply's arithmetic is here.

Shapes follow "Compress then Serve" section 3.1 (U Sigma_i V^T with U of
d_out x r, V of d_in x r; JD-Full: U, V with orthonormal columns and a full
r x r Sigma_i; JD-Diag: unconstrained U, V and a diagonal Sigma_i) and
section 3.2 (k clusters, each with its own U_j, V_j).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional

import numpy as np

from .configs import BASE_SEED, round_to_bf16


@dataclass
class JDWorkload:
    key: str
    dtype: str              # "bf16" or "fp32"
    mode: str               # "full" or "diag"
    ids: np.ndarray         # int32 [T]
    x: np.ndarray           # float32 [T, d_in] (bf16 values when dtype is bf16)
    cluster_of: np.ndarray  # int32 [n]
    U: List[np.ndarray]     # k x float32 [d_out, r]
    V: List[np.ndarray]     # k x float32 [d_in, r]
    sigma: np.ndarray       # float32 [n, r, r] (full) or [n, r] (diag)
    scales: np.ndarray      # float32 [n]
    y0: Optional[np.ndarray] = None

    @property
    def T(self):
        return len(self.ids)

    @property
    def n(self):
        return len(self.cluster_of)

    @property
    def k(self):
        return len(self.U)

    @property
    def r(self):
        return self.U[0].shape[1]

    @property
    def d_in(self):
        return self.V[0].shape[0]

    @property
    def d_out(self):
        return self.U[0].shape[0]


def _q(a, dtype):
    a32 = np.asarray(a, dtype=np.float32)
    return round_to_bf16(a32) if dtype == "bf16" else np.ascontiguousarray(a32)


def _orthonormal(rng, d, r):
    q, _ = np.linalg.qr(rng.normal(size=(d, r)))
    return q


def make_jd_workload(seed: int, T: int, n: int, k: int, d_in: int, d_out: int, r: int, *, mode: str = "full",
                     dtype: str = "bf16", id_mode: str = "zipf", invalid_frac: float = 0.0,
                     integer: bool = False, y0: bool = False) -> JDWorkload:
    """Clusters uniform over k; ids Zipf(1.1) over a seeded popularity order
    (or uniform); U, V orthonormal (full) or N(0, 1/sqrt(d)) (diag); Sigma
    entries N(0, 1) (diag) or N(0, 1/sqrt(r)) (full); scales 0.5.  Integer
    mode: U, V, Sigma and x integers in [-2, 2] (exact in every format)."""
    assert mode in ("full", "diag")
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, 950, seed])))
    cluster_of = rng.integers(0, k, size=n).astype(np.int32)
    if id_mode == "zipf":
        p = np.arange(1, n + 1, dtype=np.float64) ** -1.1
        ids = rng.permutation(n)[rng.choice(n, size=T, p=p / p.sum())]
    elif id_mode == "uniform":
        ids = rng.integers(0, n, size=T)
    else:
        raise ValueError(id_mode)
    ids = np.asarray(ids, dtype=np.int32)
    if invalid_frac > 0 and T > 0:
        ids[rng.random(T) < invalid_frac] = -1
    U, V = [], []
    for _ in range(k):
        if integer:
            U.append(rng.integers(-2, 3, size=(d_out, r)).astype(np.float32))
            V.append(rng.integers(-2, 3, size=(d_in, r)).astype(np.float32))
        elif mode == "full":
            U.append(_q(_orthonormal(rng, d_out, r), dtype))
            V.append(_q(_orthonormal(rng, d_in, r), dtype))
        else:
            U.append(_q(rng.normal(0, 1 / math.sqrt(d_out), size=(d_out, r)), dtype))
            V.append(_q(rng.normal(0, 1 / math.sqrt(d_in), size=(d_in, r)), dtype))
    shape = (n, r, r) if mode == "full" else (n, r)
    if integer:
        sigma = rng.integers(-2, 3, size=shape).astype(np.float32)
        x = rng.integers(-2, 3, size=(T, d_in)).astype(np.float32)
    else:
        sd = 1 / math.sqrt(r) if mode == "full" else 1.0
        sigma = rng.normal(0, sd, size=shape).astype(np.float32)
        x = _q(rng.normal(0, 1, size=(T, d_in)), dtype)
    scales = np.full(n, 0.5, dtype=np.float32)
    y0a = _q(rng.normal(0, 1, size=(T, d_out)), dtype) if y0 else None
    return JDWorkload(f"jd{seed}", dtype, mode, ids, x, cluster_of, U, V, sigma, scales, y0a)


# Measured shared-basis workloads: a decode batch over 1024 adapters in 32
# clusters of rank 16 (the pages serve 1000+ adapters with about 25 clusters
# of rank 15-16), d = 4096, Zipf(1.1) ids.
JD_CONFIGS = {
    "jd-full": dict(seed=1, T=2048, n=1024, k=32, d_in=4096, d_out=4096, r=16, mode="full"),
    "jd-diag": dict(seed=2, T=2048, n=1024, k=32, d_in=4096, d_out=4096, r=16, mode="diag"),
}


def make_jd_config(name: str, *, integer: bool = False, with_y0: bool = False) -> JDWorkload:
    kw = dict(JD_CONFIGS[name])
    wl = make_jd_workload(kw.pop("seed"), kw.pop("T"), kw.pop("n"), kw.pop("k"), kw.pop("d_in"), kw.pop("d_out"),
                          kw.pop("r"), integer=integer, y0=with_y0, **kw)
    wl.key = name
    return wl
