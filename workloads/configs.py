"""Seeded synthetic inputs for the five adapter-fleet workloads.

Every random quantity comes from ``numpy.random.Generator(PCG64(SeedSequence(
[2611, cfg, stream, ...])))`` with fixed streams:

  stream 0    retained ranks / spectral draws ``e``
  stream 1    adapter popularity permutation (Zipf workloads) or the
              segment -> adapter permutation (prefill workload)
  stream 2    token adapter ids
  stream 3    activations ``x`` (fleet: one stream per (layer, input kind))
  stream 4    starting outputs ``y0`` (timing runs only; parity uses zeros)
  100 + m     factors of module ``m``: for each adapter in id order,
              ``A_a`` is drawn, then ``B_a``

Values are drawn in float64, cast to float32 and, for bf16 workloads,
rounded to the nearest bfloat16 (ties to even) and kept as float32 arrays
whose values are exactly representable in bfloat16.

Factor orientation follows the LoRA definition in "Compress then Serve:
Serving Thousands of LoRA Adapters with Little Overhead", section 3: for an
adapter of rank r, ``A`` is ``r x d_in`` and ``B`` is ``d_out x r``; the
delta on an input row ``x`` is ``s * B (A x)``.

The module draws inputs only; nothing here computes the delta.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np

BASE_SEED = 2611

CONFIG_KEYS = ("1", "2", "3", "4", "5U", "5S")

# Fleet projection table (Qwen2-7B-like shapes): name, d_in, d_out, input kind.
# Input kinds: 0 = attention input (shared by q, k, v), 1 = o-proj input,
# 2 = MLP input (shared by gate, up), 3 = down-proj input.
FLEET_LAYERS = 28
FLEET_HIDDEN = 3584
FLEET_KV = 512
FLEET_MLP = 18944
FLEET_PROJECTIONS: Tuple[Tuple[str, int, int, int], ...] = (
    ("q", FLEET_HIDDEN, FLEET_HIDDEN, 0),
    ("k", FLEET_HIDDEN, FLEET_KV, 0),
    ("v", FLEET_HIDDEN, FLEET_KV, 0),
    ("o", FLEET_HIDDEN, FLEET_HIDDEN, 1),
    ("gate", FLEET_HIDDEN, FLEET_MLP, 2),
    ("up", FLEET_HIDDEN, FLEET_MLP, 2),
    ("down", FLEET_MLP, FLEET_HIDDEN, 3),
)
FLEET_INPUT_DIMS = (FLEET_HIDDEN, FLEET_HIDDEN, FLEET_HIDDEN, FLEET_MLP)


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, *key])))


def round_to_bf16(a) -> np.ndarray:
    """float array -> float32 array of the nearest bfloat16 values (ties to even).

    Input preparation only: the workloads are defined on bfloat16 values.
    """
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).reshape(f.shape)


def bf16_bits(a) -> np.ndarray:
    """Raw bfloat16 bit patterns (uint16) of a float32 array of bf16 values."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("array holds values that are not exact bfloat16")
    return (u >> 16).astype(np.uint16)


@dataclass
class Module:
    """One adapted projection: per-adapter retained factors of one module."""

    d_in: int
    d_out: int
    ranks: np.ndarray  # int32 [n]
    scales: np.ndarray  # float32 [n]
    A: List[np.ndarray]  # float32 [r_a, d_in] per adapter
    B: List[np.ndarray]  # float32 [d_out, r_a] per adapter
    orig_rank: Optional[int] = None
    name: str = ""

    @property
    def n(self) -> int:
        return len(self.A)

    @property
    def r_max(self) -> int:
        return int(self.ranks.max()) if len(self.ranks) else 0


@dataclass
class Workload:
    key: str
    dtype: str  # "fp32" or "bf16"
    ids: np.ndarray  # int32 [T]
    x: np.ndarray  # float32 [T, d_in]
    module: Module
    y0: Optional[np.ndarray] = None  # float32 [T, d_out]; None means zeros
    meta: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return int(self.ids.shape[0])

    @property
    def n(self) -> int:
        return self.module.n


def _quant(a: np.ndarray, dtype: str) -> np.ndarray:
    a32 = np.asarray(a, dtype=np.float32)
    return round_to_bf16(a32) if dtype == "bf16" else np.ascontiguousarray(a32)


def _draw_factors(module_stream: int, cfg: int, ranks: Sequence[int], d_in: int, d_out: int,
                  dtype: str, integer: bool = False) -> Tuple[List[np.ndarray], List[np.ndarray]]:
    """Factors of one module, adapter by adapter: A_a then B_a.

    A_a ~ N(0, 1/sqrt(d_in)) and B_a ~ N(0, 1/sqrt(d_out)) (standard
    deviations); with ``integer`` they are uniform integers in [-2, 2].
    """
    rng = _rng(cfg, 100 + module_stream)
    As, Bs = [], []
    sa, sb = 1.0 / math.sqrt(d_in), 1.0 / math.sqrt(d_out)
    for r in ranks:
        r = int(r)
        if integer:
            a = rng.integers(-2, 3, size=(r, d_in)).astype(np.float32)
            b = rng.integers(-2, 3, size=(d_out, r)).astype(np.float32)
        else:
            a = _quant(rng.normal(0.0, sa, size=(r, d_in)), dtype)
            b = _quant(rng.normal(0.0, sb, size=(d_out, r)), dtype)
        As.append(np.ascontiguousarray(a))
        Bs.append(np.ascontiguousarray(b))
    return As, Bs


def zipf_ids(cfg: int, n: int, T: int, exponent: float = 1.1) -> np.ndarray:
    """Adapter ids with Zipf popularity P(k) ~ k^-exponent over k = 1..n.

    Popularity ranks are mapped to adapter ids through a seeded permutation.
    """
    k = np.arange(1, n + 1, dtype=np.float64)
    p = k ** (-exponent)
    p /= p.sum()
    pop = _rng(cfg, 1).permutation(n)
    draws = _rng(cfg, 2).choice(n, size=T, p=p)
    return pop[draws].astype(np.int32)


def _x(cfg: int, T: int, d_in: int, dtype: str, integer: bool, *extra: int) -> np.ndarray:
    rng = _rng(cfg, 3, *extra)
    if integer:
        return rng.integers(-2, 3, size=(T, d_in)).astype(np.float32)
    return _quant(rng.normal(0.0, 1.0, size=(T, d_in)), dtype)


def timing_y0(cfg: int, T: int, d_out: int, dtype: str) -> np.ndarray:
    """Non-zero starting outputs for timing runs: N(0, 1)."""
    return _quant(_rng(cfg, 4).normal(0.0, 1.0, size=(T, d_out)), dtype)


def _pow2_scale(s: float) -> float:
    return float(2.0 ** round(math.log2(s)))


def make_config(key: str, *, integer: bool = False, layer: int = 0, proj: int = 0,
                with_y0: bool = False) -> Workload:
    """Build workload ``key`` in ``CONFIG_KEYS``.

    ``integer``: same shapes, ranks and ids, but x and factors are integers
    in [-2, 2] and scales are powers of two, so every partial sum of the apply
    is an exact integer below 2**24 (exactness pin).
    For the fleet workloads (``5U``/``5S``) one module, ``(layer, proj)``, is
    returned at full shape.
    """
    key = str(key)
    if key == "1":
        cfg, n, T, d, dtype = 1, 4, 16, 256, "fp32"
        ranks = np.arange(1, n + 1, dtype=np.int32)
        scales = np.full(n, 2.0, np.float32)
        ids = _rng(cfg, 2).integers(0, n, size=T).astype(np.int32)
        A, B = _draw_factors(0, cfg, ranks, d, d, dtype, integer)
        mod = Module(d, d, ranks, scales, A, B, orig_rank=8, name="tiny")
        x = _x(cfg, T, d, dtype, integer)
    elif key == "2":
        cfg, n, T, d, dtype = 2, 64, 256, 4096, "bf16"
        ranks = np.full(n, 4, np.int32)
        scales = np.full(n, 32.0 / 16.0, np.float32)
        ids = _rng(cfg, 2).integers(0, n, size=T).astype(np.int32)
        A, B = _draw_factors(0, cfg, ranks, d, d, dtype, integer)
        mod = Module(d, d, ranks, scales, A, B, orig_rank=16, name="decode-uniform")
        x = _x(cfg, T, d, dtype, integer)
    elif key == "3":
        cfg, n, T, d, dtype = 3, 512, 2048, 3584, "bf16"
        e = _rng(cfg, 0).beta(2.0, 5.0, size=n)
        ranks = np.maximum(6, np.ceil(64.0 * e)).astype(np.int32)
        scales = np.full(n, 32.0 / 64.0, np.float32)
        ids = zipf_ids(cfg, n, T)
        A, B = _draw_factors(0, cfg, ranks, d, d, dtype, integer)
        mod = Module(d, d, ranks, scales, A, B, orig_rank=64, name="decode-spectral")
        x = _x(cfg, T, d, dtype, integer)
    elif key == "4":
        cfg, n, T, d_in, d_out, dtype = 4, 32, 8192, 4096, 14336, "bf16"
        ranks = _rng(cfg, 0).choice(np.array([8, 12, 16, 24, 32]), size=n).astype(np.int32)
        seg_adapter = _rng(cfg, 1).permutation(n)
        ids = np.repeat(seg_adapter, T // n).astype(np.int32)
        s = 32.0 / ranks.astype(np.float64)
        if integer:
            s = np.array([_pow2_scale(v) for v in s])
        scales = s.astype(np.float32)
        A, B = _draw_factors(0, cfg, ranks, d_in, d_out, dtype, integer)
        mod = Module(d_in, d_out, ranks, scales, A, B, orig_rank=None, name="prefill")
        x = _x(cfg, T, d_in, dtype, integer)
    elif key in ("5U", "5S"):
        return make_fleet_module(key, layer, proj, integer=integer, with_y0=with_y0)
    else:
        raise KeyError(f"unknown workload {key!r}; expected one of {CONFIG_KEYS}")
    y0 = timing_y0(cfg, T, mod.d_out, dtype) if with_y0 else None
    return Workload(key, dtype, ids, x, mod, y0=y0, meta={"cfg": cfg})


def fleet_ranks(key: str, n: int = 1024) -> np.ndarray:
    """Retained ranks of the fleet, int32 [layers, projections, n].

    5U: ceil(64 / 12) = 6 everywhere (floor 4 inactive).
    5S: clamp(ceil(64 * e * 7/24), 4, 16) with e ~ Beta(2, 5) per
        (layer, projection, adapter); 7/24 maps Beta(2,5)'s mean 2/7 to 1/12.
    """
    shape = (FLEET_LAYERS, len(FLEET_PROJECTIONS), n)
    if key == "5U":
        return np.full(shape, max(4, math.ceil(64 / 12)), np.int32)
    if key == "5S":
        e = _rng(5, 0).beta(2.0, 5.0, size=shape)
        return np.clip(np.ceil(64.0 * e * 7.0 / 24.0), 4, 16).astype(np.int32)
    raise KeyError(key)


def fleet_module_shapes():
    """[(layer, proj, name, d_in, d_out, input_kind)] for all 196 modules."""
    return [(l, p, nm, di, do, kind)
            for l in range(FLEET_LAYERS)
            for p, (nm, di, do, kind) in enumerate(FLEET_PROJECTIONS)]


def fleet_ids(T: int = 4096, n: int = 1024) -> np.ndarray:
    return zipf_ids(5, n, T)


def fleet_x(layer: int, kind: int, T: int = 4096, integer: bool = False) -> np.ndarray:
    return _x(5, T, FLEET_INPUT_DIMS[kind], "bf16", integer, layer, kind)


def make_fleet_module(key: str, layer: int, proj: int, *, integer: bool = False,
                      with_y0: bool = False, T: int = 4096, n: int = 1024) -> Workload:
    """One module of the fleet decode step at full shape."""
    name, d_in, d_out, kind = FLEET_PROJECTIONS[proj]
    ranks = fleet_ranks(key, n)[layer, proj]
    scales = np.full(n, 32.0 / 64.0, np.float32)
    module_index = layer * len(FLEET_PROJECTIONS) + proj
    A, B = _draw_factors(module_index, 5, ranks, d_in, d_out, "bf16", integer)
    mod = Module(d_in, d_out, ranks, scales, A, B, orig_rank=64, name=f"L{layer}.{name}")
    ids = fleet_ids(T, n)
    x = fleet_x(layer, kind, T, integer)
    y0 = _quant(_rng(5, 4, layer, proj).normal(0.0, 1.0, size=(T, d_out)), "bf16") if with_y0 else None
    return Workload(key, "bf16", ids, x, mod, y0=y0,
                    meta={"cfg": 5, "layer": layer, "proj": proj, "input_kind": kind})


def make_integer_workload(key: str, **kw) -> Workload:
    return make_config(key, integer=True, **kw)


def make_random_workload(seed: int, T: int, n: int, d_in: int, d_out: int, ranks,
                         dtype: str = "bf16", *, scales=None, id_mode: str = "uniform",
                         invalid_frac: float = 0.0, integer: bool = False,
                         y0: bool = False) -> Workload:
    """Small custom workload for edge cases (ragged shapes, empty adapters, -1 ids).

    id_mode: "uniform", "zipf", "sorted", "all_same", "distinct".
    """
    ranks = np.asarray(ranks, dtype=np.int32)
    assert ranks.shape == (n,)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, 900, seed])))
    if id_mode == "uniform":
        ids = rng.integers(0, n, size=T)
    elif id_mode == "zipf":
        p = np.arange(1, n + 1, dtype=np.float64) ** -1.1
        ids = rng.permutation(n)[rng.choice(n, size=T, p=p / p.sum())]
    elif id_mode == "sorted":
        ids = np.sort(rng.integers(0, n, size=T))
    elif id_mode == "all_same":
        ids = np.full(T, int(rng.integers(0, n)))
    elif id_mode == "distinct":
        assert T <= n
        ids = rng.permutation(n)[:T]
    else:
        raise ValueError(id_mode)
    ids = np.asarray(ids, dtype=np.int32)
    if invalid_frac > 0 and T > 0:
        mask = rng.random(T) < invalid_frac
        ids[mask] = -1
    if scales is None:
        scales = rng.choice(np.array([0.25, 0.5, 1.0, 2.0]), size=n)
    scales = np.asarray(scales, dtype=np.float32)
    As, Bs = [], []
    for r in ranks:
        if integer:
            As.append(rng.integers(-2, 3, size=(int(r), d_in)).astype(np.float32))
            Bs.append(rng.integers(-2, 3, size=(d_out, int(r))).astype(np.float32))
        else:
            As.append(_quant(rng.normal(0, 1 / math.sqrt(d_in), size=(int(r), d_in)), dtype))
            Bs.append(_quant(rng.normal(0, 1 / math.sqrt(d_out), size=(d_out, int(r))), dtype))
    if integer:
        x = rng.integers(-2, 3, size=(T, d_in)).astype(np.float32)
    else:
        x = _quant(rng.normal(0, 1, size=(T, d_in)), dtype)
    y0a = _quant(rng.normal(0, 1, size=(T, d_out)), dtype) if y0 else None
    mod = Module(d_in, d_out, ranks, scales, As, Bs, name=f"random{seed}")
    return Workload(f"rand{seed}", dtype, ids, x, mod, y0=y0a, meta={"seed": seed})


def base_weight(seed: int, d_out: int, d_in: int, *, integer: bool = False) -> np.ndarray:
    """Frozen base weight W0 [d_out, d_in] of a layer (the layer computes
    W0 x): N(0, 1/d_in) entries rounded to bf16, or integers in [-2, 2]."""
    rng = _rng(7, seed, d_out, d_in)
    if integer:
        return rng.integers(-2, 3, size=(d_out, d_in)).astype(np.float32)
    return _quant(rng.normal(0.0, 1.0 / math.sqrt(d_in), size=(d_out, d_in)), "bf16")


def fleet_base_weight(layer: int, proj: int, *, integer: bool = False) -> np.ndarray:
    """W0 of one fleet module (the Qwen2-7B-like shapes), seeded by its place."""
    _, d_in, d_out, _ = FLEET_PROJECTIONS[proj]
    return base_weight(1000 + layer * len(FLEET_PROJECTIONS) + proj, d_out, d_in, integer=integer)
