"""Reference (oracle) of the retained-rank allocation policies.

Test infrastructure: see the package docstring.  Source:

[LF]   "LoRAForge: Co-Designing Compression and Execution for More Efficient
       Multi-LoRA Serving", section "LoRAForge's Core Design: Explicit
       Retained-Rank Representation and Dual Strategies": two ways to choose
       how many ranks each adapter factor keeps after compression, a uniform
       ratio of the original rank (with a floor) and a spectral budget that
       keeps the components carrying the most energy.

The pages give no formula for either; the readings taken:

* unit: one adapter factor pair (one adapter of one module) with original
  rank r_orig and singular values sigma_1 >= sigma_2 >= ... (their squares
  are the energy each component carries).
* uniform (U): r = min(r_orig, max(floor, ceil(ratio * r_orig))).
* spectral (S): every unit first keeps min(floor, r_orig) ranks; the rest
  of a total budget goes, one rank at a time, to the unit whose next
  component has the largest sigma^2 (ties: lower unit index), never beyond
  r_orig.  The default budget is the uniform policy's total, so both keep the
  same number of ranks.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence


def uniform_ranks_ref(r_orig: Sequence[int], ratio: float, floor: int) -> List[int]:
    """The uniform policy, unit by unit."""
    return [min(int(r), max(int(floor), math.ceil(ratio * int(r) - 1e-12))) for r in r_orig]


def spectral_ranks_ref(r_orig: Sequence[int], sigmas: Sequence[Sequence[float]], floor: int,
                       budget: Optional[int] = None, ratio: Optional[float] = None) -> List[int]:
    """The spectral-budget policy by repeated selection: while ranks remain in
    the budget, give one more rank to the unit whose next sigma^2 is largest.
    ``budget`` defaults to the uniform policy's total at ``ratio``."""
    n = len(r_orig)
    if budget is None:
        budget = sum(uniform_ranks_ref(r_orig, ratio, floor))
    r = [min(int(floor), int(r_orig[u])) for u in range(n)]
    left = int(budget) - sum(r)
    while left > 0:
        best, best_e = -1, -1.0
        for u in range(n):
            if r[u] < int(r_orig[u]):
                e = float(sigmas[u][r[u]]) ** 2
                if e > best_e:  # strict: the lower index keeps a tie
                    best, best_e = u, e
        if best < 0:
            break  # every unit at its original rank
        r[best] += 1
        left -= 1
    return r
