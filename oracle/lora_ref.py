"""Reference (oracle) implementation of the multi-adapter LoRA delta.

Test infrastructure: see the package docstring.  Sources:

[CtS]  "Compress then Serve: Serving Thousands of LoRA Adapters with Little
       Overhead" (arXiv 2407.00066), section 3 (the LoRA-updated layer output
       (W0 + B A) x with B of shape d_B x r, A of shape r x d_A), section 11
       (each request names its adapter; W0 x and B_i A_i x are computed
       separately and merged), section 2 (SGMV groups the requests that use
       the same adapter), section 13.4 (adapter selection by a per-token
       index array; step 1 applies A into a float32 buffer with scale 1,
       step 3 applies B with the scale and adds into a slice of y).
[LF]   "LoRAForge: Co-Designing Compression and Execution for More Efficient
       Multi-LoRA Serving", section "LoRAForge's Core Design: Explicit
       Retained-Rank Representation and Dual Strategies" (execution runs on
       each adapter's retained factors at its own rank, without padding).
"""
from __future__ import annotations

from fractions import Fraction
from typing import List, Optional, Sequence, Tuple

import numpy as np


def segment_ref(ids: Sequence[int], n: int) -> Tuple[List[int], List[int], int]:
    """Group tokens by adapter: a stable counting sort of ``ids``.

    [CtS] section 2 (grouping the requests that use the same adapter) and
    section 13.4 (per-token adapter index).  Reading taken where the sources
    are silent: adapters are ordered by ascending id, tokens inside a group
    keep ascending token index, and any id outside [0, n) (-1 = no adapter)
    goes to one extra trailing group ``n`` that receives no delta.

    Returns ``seg_off`` (n + 2 entries: group g holds sorted positions
    seg_off[g] .. seg_off[g+1]-1), ``perm`` (perm[i] = original token index
    at sorted position i) and the number of ids that are neither -1 nor in
    [0, n).
    """
    T = len(ids)
    group = []
    n_invalid = 0
    for v in ids:
        v = int(v)
        if 0 <= v < n:
            group.append(v)
        else:
            group.append(n)
            if v != -1:
                n_invalid += 1
    count = [0] * (n + 1)
    for g in group:
        count[g] += 1
    seg_off = [0] * (n + 2)
    for g in range(n + 1):
        seg_off[g + 1] = seg_off[g] + count[g]
    cursor = list(seg_off[: n + 1])
    perm = [0] * T
    for t in range(T):
        g = group[t]
        perm[cursor[g]] = t
        cursor[g] += 1
    return seg_off, perm, n_invalid


def _as64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def shrink_ref(x, ids, A_list) -> List[np.ndarray]:
    """Per token t with adapter a = ids[t] in range: h_t = A_a x_t (float64).

    [CtS] section 13.4, step 1 (A applied with scale 1 into the float32
    intermediate; here in float64).  Tokens without an adapter get an empty
    vector.
    """
    x64 = _as64(x)
    n = len(A_list)
    cache = {}
    out = []
    for t in range(x64.shape[0]):
        a = int(ids[t])
        if not 0 <= a < n:
            out.append(np.zeros(0))
            continue
        if a not in cache:
            cache[a] = _as64(A_list[a])
        out.append(cache[a] @ x64[t])
    return out


def shrink_error_bound(x, ids, A_list, unit_roundoff: float = 2.0 ** -24) -> List[np.ndarray]:
    """Largest error of h = A_a x when it is accumulated in float32.

    [CtS] section 13.4 keeps h in a float32 buffer.  Each of the d_in
    products and d_in - 1 additions rounds at most once, with relative error
    at most the unit roundoff u = 2^-24 (round to nearest; products of bf16
    values are exact, so there only the additions round).  For any order of
    the additions the textbook dot-product bound (Higham, "Accuracy and
    Stability of Numerical Algorithms", 2nd ed., section 3.1) gives

        |h_float32[j] - h[j]|  <=  gamma_n * sum_k |A_a[j, k] x[k]|,
        gamma_n = n u / (1 - n u),   n = d_in,

    whose first-order term is d_in * u * sum_k |A_a[j, k] x[k]|.  Returns one
    array of r_a bounds per token (empty for tokens without an adapter).
    """
    x64 = np.abs(_as64(x))
    n = len(A_list)
    out = []
    for t in range(x64.shape[0]):
        a = int(ids[t])
        if not 0 <= a < n:
            out.append(np.zeros(0))
            continue
        Aa = np.abs(_as64(A_list[a]))
        nu = Aa.shape[1] * unit_roundoff
        out.append(nu / (1.0 - nu) * (Aa @ x64[t]))
    return out


def apply_ref(x, ids, A_list, B_list, scales, y0=None) -> np.ndarray:
    """y[t] = y0[t] + s_a * B_a (A_a x[t]) for every token t with a = ids[t].

    [CtS] section 3 (the LoRA branch B A x beside W0 x), section 11 (the
    branch is computed per request's adapter and merged), section 13.4
    (shrink with A, then expand with B and the scale, accumulated into y).
    [LF]: each adapter's own retained rank r_a is used as is.  Tokens with no
    adapter (id outside [0, n)) keep y0.  float64 throughout, on the exact
    values of the inputs.
    """
    x64 = _as64(x)
    T = x64.shape[0]
    n = len(A_list)
    d_out = int(np.asarray(B_list[0]).shape[0]) if n else 0
    if y0 is None:
        y = np.zeros((T, d_out), dtype=np.float64)
    else:
        y = _as64(y0).copy()
        d_out = y.shape[1]
    cache = {}
    for t in range(T):
        a = int(ids[t])
        if not 0 <= a < n:
            continue
        if a not in cache:
            cache[a] = (_as64(A_list[a]), _as64(B_list[a]))
        Aa, Ba = cache[a]
        h = Aa @ x64[t]
        y[t] += float(scales[a]) * (Ba @ h)
    return y


def base_fused_ref(x, ids, W0, A_list, B_list, scales) -> np.ndarray:
    """y[t] = W0 x[t] + s_a B_a (A_a x[t]) for every token t, a = ids[t].

    [CtS] section 3: the LoRA-updated layer computes (W0 + B A) x; section
    11: the base product W0 x is computed once for all requests and each
    request's branch B_i A_i x is added to it.  W0 has the layer's [d_out,
    d_in] orientation (y = W0 x).  Tokens without an adapter (id outside
    [0, n)) get W0 x alone.  float64, a per-token loop.
    """
    x64 = _as64(x)
    W = _as64(W0)
    T = x64.shape[0]
    y = np.zeros((T, W.shape[0]), dtype=np.float64)
    for t in range(T):
        y[t] = W @ x64[t]
    return apply_ref(x, ids, A_list, B_list, scales, y0=y)


def brute_force(x, ids, A_list, B_list, scales, y0=None, form: str = "B(Ax)") -> List[List[Fraction]]:
    """Exact rational evaluation with explicit triple loops (tiny inputs only).

    ``form="B(Ax)"`` forms h = A x first (the served branch, [CtS] section
    11); ``form="(BA)x"`` forms the merged update B A first (the merged form
    W0 -> W0 + B A of the same section).  Both must agree exactly.
    """
    T = len(ids)
    n = len(A_list)
    X = [[Fraction(float(v)) for v in row] for row in np.asarray(x)]
    d_in = len(X[0]) if T else 0
    d_out = int(np.asarray(B_list[0]).shape[0]) if n else 0
    if y0 is None:
        Y = [[Fraction(0)] * d_out for _ in range(T)]
    else:
        Y = [[Fraction(float(v)) for v in row] for row in np.asarray(y0)]
    for t in range(T):
        a = int(ids[t])
        if not 0 <= a < n:
            continue
        A = [[Fraction(float(v)) for v in row] for row in np.asarray(A_list[a])]
        B = [[Fraction(float(v)) for v in row] for row in np.asarray(B_list[a])]
        r = len(A)
        s = Fraction(float(scales[a]))
        if form == "B(Ax)":
            h = [sum((A[j][k] * X[t][k] for k in range(d_in)), Fraction(0)) for j in range(r)]
            for o in range(d_out):
                Y[t][o] += s * sum((B[o][j] * h[j] for j in range(r)), Fraction(0))
        elif form == "(BA)x":
            for o in range(d_out):
                row = [sum((B[o][j] * A[j][k] for j in range(r)), Fraction(0)) for k in range(d_in)]
                Y[t][o] += s * sum((row[k] * X[t][k] for k in range(d_in)), Fraction(0))
        else:
            raise ValueError(form)
    return Y


def bf16_round_ref(v) -> np.ndarray:
    """Nearest bfloat16 value of each entry, ties to even, returned as float64.

    Written from the format: bfloat16 keeps the sign, the 8 exponent bits and
    the top 7 fraction bits of a binary32 value.  The value is first made
    exact in binary32 (the callers pass values that are exactly
    representable there, e.g. integers below 2**24), then the low 16 bits are
    rounded away by comparing the discarded part with half an ulp.
    """
    f = np.asarray(v, dtype=np.float64)
    f32 = f.astype(np.float32)
    if not np.array_equal(f32.astype(np.float64), f):
        raise ValueError("bf16_round_ref expects values exact in binary32")
    bits = f32.view(np.uint32).astype(np.int64)
    low = bits & 0xFFFF
    high = bits >> 16
    half = 0x8000
    up = (low > half) | ((low == half) & ((high & 1) == 1))
    high = high + up.astype(np.int64)
    out = (high << 16).astype(np.uint32).view(np.float32)
    return out.astype(np.float64)
