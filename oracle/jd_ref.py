"""Reference (oracle) of the shared-basis (joint-diagonalization) apply.

Test infrastructure: see the package docstring.  Source:

[CtS]  "Compress then Serve: Serving Thousands of LoRA Adapters with Little
       Overhead": section 3.1 (each adapter's product B_i A_i is represented
       as U Sigma_i V^T with U and V shared and Sigma_i either a full r x r
       matrix (JD-Full) or diagonal (JD-Diag)), section 3.2 (adapters are
       split into clusters, each cluster j with its own U_j and V_j),
       section 11 (the served branch is U (Sigma (V^T x)): V^T x and the U
       product are shared by all the tokens of a cluster, Sigma is per
       token's adapter), section 13.4 (the three steps A, Sigma, B of the
       apply with a per-token adapter index; the scale is applied with B).

Shapes: U_j is d_out x r and V_j is d_in x r (U plays B's role, V^T plays
A's), Sigma_i is r x r (full) or a vector of r values (diagonal), s_i is
the adapter's scale.
"""
from __future__ import annotations

from fractions import Fraction
from typing import List

import numpy as np


def _as64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def _sigma_times(sig, h):
    """Sigma_i h for a full (r x r) or diagonal (r values) Sigma_i."""
    sig = _as64(sig)
    return sig @ h if sig.ndim == 2 else sig * h


def jd_apply_ref(x, ids, cluster_of, U_list, V_list, sigma, scales, y0=None) -> np.ndarray:
    """y[t] = y0[t] + s_a U_c (Sigma_a (V_c^T x[t])), a = ids[t], c = cluster_of[a].

    Tokens whose id is outside [0, n) (-1 = no adapter) keep y0, and so do
    tokens whose adapter's cluster is outside [0, k) (a reading: the pages
    assign every adapter a cluster; an unassigned one adds nothing).
    float64 throughout, on the exact values of the inputs, in the served
    order of [CtS] section 11 (V^T x, then Sigma, then U).
    """
    x64 = _as64(x)
    T = x64.shape[0]
    n = len(cluster_of)
    d_out = _as64(U_list[0]).shape[0] if len(U_list) else 0
    y = np.zeros((T, d_out)) if y0 is None else _as64(y0).copy()
    for t in range(T):
        a = int(ids[t])
        if not 0 <= a < n:
            continue
        c = int(cluster_of[a])
        if not 0 <= c < len(U_list):
            continue
        U = _as64(U_list[c])
        V = _as64(V_list[c])
        h = V.T @ x64[t]
        y[t] += float(scales[a]) * (U @ _sigma_times(sigma[a], h))
    return y


def jd_brute_force(x, ids, cluster_of, U_list, V_list, sigma, scales, y0=None,
                   form: str = "U(S(Vx))") -> List[List[Fraction]]:
    """Exact rational evaluation with explicit loops (tiny inputs only), in
    the served order U (Sigma (V^T x)) or as the merged update (U Sigma V^T) x
    applied to x (the merged form W0 -> W0 + B_i A_i of section 11 with
    B_i A_i = U Sigma_i V^T)."""
    T = len(ids)
    n = len(cluster_of)
    X = [[Fraction(float(v)) for v in row] for row in np.asarray(x)]
    d_out = np.asarray(U_list[0]).shape[0]
    d_in = np.asarray(V_list[0]).shape[0]
    if y0 is None:
        Y = [[Fraction(0)] * d_out for _ in range(T)]
    else:
        Y = [[Fraction(float(v)) for v in row] for row in np.asarray(y0)]
    for t in range(T):
        a = int(ids[t])
        if not 0 <= a < n:
            continue
        c = int(cluster_of[a])
        if not 0 <= c < len(U_list):
            continue
        U = [[Fraction(float(v)) for v in row] for row in np.asarray(U_list[c])]
        V = [[Fraction(float(v)) for v in row] for row in np.asarray(V_list[c])]
        r = len(U[0])
        sg = np.asarray(sigma[a])
        if sg.ndim == 2:
            S = [[Fraction(float(sg[i, j])) for j in range(r)] for i in range(r)]
        else:
            S = [[Fraction(float(sg[i])) if i == j else Fraction(0) for j in range(r)] for i in range(r)]
        s = Fraction(float(scales[a]))
        if form == "U(S(Vx))":
            h = [sum((V[k][j] * X[t][k] for k in range(d_in)), Fraction(0)) for j in range(r)]
            g = [sum((S[i][j] * h[j] for j in range(r)), Fraction(0)) for i in range(r)]
            for o in range(d_out):
                Y[t][o] += s * sum((U[o][i] * g[i] for i in range(r)), Fraction(0))
        elif form == "(USV)x":
            for o in range(d_out):
                US = [sum((U[o][i] * S[i][j] for i in range(r)), Fraction(0)) for j in range(r)]
                row = [sum((US[j] * V[k][j] for j in range(r)), Fraction(0)) for k in range(d_in)]
                Y[t][o] += s * sum((row[k] * X[t][k] for k in range(d_in)), Fraction(0))
        else:
            raise ValueError(form)
    return Y
