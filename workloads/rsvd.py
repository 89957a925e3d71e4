"""Seeded original adapters for retained-factor construction (r-SVD).

A module's n adapters, all at one original rank r (the fleet's adapters are
rank 64), stored as A_all [n, r, d_in] and B_all [n, d_out, r] float32
arrays (bf16-exact for bf16 workloads).  Stream ``[2611, 950, seed]``: per
adapter in id order, the spectrum exponent, then A_a, then B_a (standard
normals drawn in float32, scaled in float32):

  A_a ~ N(0, 1/sqrt(d_in)),  B_a[:, j] ~ N(0, 1/sqrt(d_out)) * (j + 1)^-alpha_a

alpha_a is 0 for every adapter with ``spectrum="flat"`` and uniform in
[0, 1.5) with ``spectrum="decay"``, so that the adapters' singular values
fall at different rates (the case a spectral budget tells apart from a
uniform ratio).  ``zero_cols`` zeroes the last columns of B_a for the first
adapters (rank-deficient factors).

The module draws inputs only; nothing here computes a decomposition.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from .configs import BASE_SEED, FLEET_HIDDEN, round_to_bf16


@dataclass
class RsvdWorkload:
    name: str
    dtype: str  # "bf16" or "fp32"
    A: np.ndarray  # float32 [n, r, d_in]
    B: np.ndarray  # float32 [n, d_out, r]
    scales: np.ndarray  # float32 [n]

    @property
    def n(self) -> int:
        return self.A.shape[0]

    @property
    def r(self) -> int:
        return self.A.shape[1]

    @property
    def d_in(self) -> int:
        return self.A.shape[2]

    @property
    def d_out(self) -> int:
        return self.B.shape[1]


def _q(a: np.ndarray, dtype: str) -> np.ndarray:
    a32 = np.asarray(a, dtype=np.float32)
    return round_to_bf16(a32) if dtype == "bf16" else a32


def make_rsvd_workload(seed: int, n: int, r: int, d_in: int, d_out: int, *, dtype: str = "bf16",
                       spectrum: str = "decay", zero_cols: int = 0, zero_adapters: int = 0,
                       name: str = "") -> RsvdWorkload:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, 950, seed])))
    A = np.empty((n, r, d_in), np.float32)
    B = np.empty((n, d_out, r), np.float32)
    sa, sb = 1.0 / math.sqrt(d_in), 1.0 / math.sqrt(d_out)
    for a in range(n):
        alpha = rng.uniform(0.0, 1.5) if spectrum == "decay" else 0.0
        A[a] = _q(rng.standard_normal((r, d_in), dtype=np.float32) * np.float32(sa), dtype)
        col = ((np.arange(r, dtype=np.float64) + 1.0) ** -alpha * sb).astype(np.float32)
        B[a] = _q(rng.standard_normal((d_out, r), dtype=np.float32) * col[None, :], dtype)
        if a < zero_adapters and zero_cols > 0:
            B[a][:, r - zero_cols:] = 0.0
    scales = np.full(n, 0.5, np.float32)
    return RsvdWorkload(name or f"rsvd-{seed}", dtype, A, B, scales)


# The measured case: one q projection of the fleet (3584 -> 3584), 1024
# adapters of original rank 64, bf16, decaying spectra.
RSVD_CONFIGS = {
    "rsvd-q": dict(seed=1, n=1024, r=64, d_in=FLEET_HIDDEN, d_out=FLEET_HIDDEN, dtype="bf16", spectrum="decay"),
}


def make_rsvd_config(name: str, n: int = 0) -> RsvdWorkload:
    """The named configuration; ``n`` > 0 takes only its first n adapters
    (the same draws: adapters are drawn one after another)."""
    kw = dict(RSVD_CONFIGS[name])
    if n > 0:
        kw["n"] = min(n, kw["n"])
    return make_rsvd_workload(kw.pop("seed"), kw.pop("n"), kw.pop("r"), kw.pop("d_in"), kw.pop("d_out"),
                              name=name, **kw)
