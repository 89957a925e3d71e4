"""Reference (oracle) of retained-factor construction (r-SVD).

Test infrastructure: see the package docstring.  Sources:

[LF]   "LoRAForge: Co-Designing Compression and Execution for More Efficient
       Multi-LoRA Serving": post-hoc compression decomposes each adapter's
       original factors into retained ones; FlashTSQR (section "FlashTSQR: An
       Accelerator for Batched Factor Construction", and the glossary before
       it) is a tall-and-skinny QR by local QR on row blocks then a merge,
       parallel across modules and row blocks.
[CtS]  "Compress then Serve", section 4: compressing one adapter alone is
       the rank-r SVD of its product B A (Eckart-Young), saved as U_r and
       Sigma_r V_r^T.

For an adapter with B (d_out x r) and A (r x d_in): B = Q_B R_B and
A^T = Q_A R_A (thin QR), so B A = Q_B (R_B R_A^T) Q_A^T; the SVD of the small
core R_B R_A^T = U S V^T gives the SVD of B A with left vectors Q_B U and
right vectors Q_A V.  Keeping k components: B' = Q_B U_k (d_out x k) and
A' = S_k V_k^T Q_A^T (k x d_in), so B' A' is the best rank-k approximation.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def tall_skinny_r_ref(M) -> np.ndarray:
    """R of the thin QR of M (rows >= columns) with a non-negative diagonal
    (the sign convention that makes R unique for full column rank)."""
    _, R = np.linalg.qr(np.asarray(M, dtype=np.float64))
    sgn = np.where(np.diag(R) < 0, -1.0, 1.0)
    return sgn[:, None] * R


def rsvd_ref(A, B) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """(sigma, U_full, V_full, Q_B, Q_A) pieces of B A = (Q_B U) S (Q_A V)^T:
    returns sigma (descending), the left vectors Q_B U (d_out x r) and the
    right vectors Q_A V (d_in x r)."""
    A64 = np.asarray(A, dtype=np.float64)
    B64 = np.asarray(B, dtype=np.float64)
    Q_B, R_B = np.linalg.qr(B64)
    Q_A, R_A = np.linalg.qr(A64.T)
    U, s, Vt = np.linalg.svd(R_B @ R_A.T)
    return s, Q_B @ U, Q_A @ Vt.T, R_B @ R_A.T


def retained_factors_ref(A, B, k: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(A', B', sigma): the retained factors of rank k, A' = S_k V_k^T Q_A^T
    (k x d_in), B' = Q_B U_k (d_out x k), and all r singular values."""
    s, left, right, _ = rsvd_ref(A, B)
    B2 = left[:, :k]
    A2 = s[:k, None] * right[:, :k].T
    return A2, B2, s
