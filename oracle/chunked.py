"""Exact chunk-parallel (WY/UT) form of the gated delta rule, fp64 numpy.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Follows the gated branch of ``chunked_delta`` on the "Prizma seq/delta.py" page
step by step, transposed to our state layout H = S^T ([d_k][d_v]). Within each
chunk of C tokens, with a_i = log alpha_i:

  1. b_i = sum_{s<=i} a_s (log space, the page's underflow remark), b'_i = b_i - a_i.
  2. A_ij = beta_i (k_i . k_j) exp(b_i - b_j) for j < i, else 0.
  3. rhs = diag(beta) V - diag(beta * exp(b)) K H.
  4. U = (I + A)^{-1} rhs (unit lower-triangular solve; ``_solve_unit_lower``).
  5. post read: O = diag(exp(b)) Q H + [(q_i . k_j) exp(b_i - b_j)]_{j<=i} U
     pre read:  O = diag(exp(b')) Q H + [(q_i . k_j) exp(b'_i - b_j)]_{j<i} U
  6. carry: H <- exp(b_C) H + K^T diag(exp(b_C - b)) U.

The page only gives the pre-write read; the post-write read is the same algebra
with the diagonal kept and b in place of b' (a token's own write is visible to
its read). Every exponent formed is <= 0 when a <= 0: the masks are applied to
the exponent before exp, never after.

It is an oracle for the chunk algebra, checked in the CPU tests against the
per-token recurrence in ``gdr_oracle.c``; it never sees GPU output.
"""
from __future__ import annotations

import numpy as np
import scipy.linalg


def solve_unit_lower(A: np.ndarray, rhs: np.ndarray) -> np.ndarray:
    """(I + A) X = rhs for strictly lower-triangular A ("Prizma seq/delta.py", ``_solve_unit_lower``)."""
    C = A.shape[0]
    return scipy.linalg.solve_triangular(np.eye(C) + A, rhs, lower=True, unit_diagonal=True)


def neumann_inverse(A: np.ndarray) -> np.ndarray:
    """(I + A)^{-1} = sum_{j<C} (-A)^j for nilpotent strictly-lower A (the same page's fallback)."""
    C = A.shape[0]
    X = np.eye(C)
    term = np.eye(C)
    for _ in range(1, C):
        term = -A @ term
        X = X + term
    return X


def _masked_exp(diff: np.ndarray, mask: np.ndarray) -> np.ndarray:
    return np.exp(np.where(mask, diff, -np.inf))


def chunked_sequence(q, k, v, log_alpha, beta, h0=None, *, chunk: int = 64, read: str = "post"):
    """One sequence, one head. q, k: [T, dk]; v: [T, dv]; log_alpha, beta: [T]; h0: [dk, dv].

    Returns (o [T, dv], hT [dk, dv]), all float64."""
    q, k, v, a, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, log_alpha, beta))
    T, dk = k.shape
    dv = v.shape[1]
    H = np.zeros((dk, dv)) if h0 is None else np.array(h0, dtype=np.float64)
    out = np.zeros((T, dv))
    for c0 in range(0, T, chunk):
        c1 = min(c0 + chunk, T)
        C = c1 - c0
        K, Q, V = k[c0:c1], q[c0:c1], v[c0:c1]
        ac, bc = a[c0:c1], beta[c0:c1]
        b = np.cumsum(ac)                      # step 1
        bp = b - ac
        ii, jj = np.meshgrid(np.arange(C), np.arange(C), indexing="ij")
        strict = jj < ii
        Gam = _masked_exp(b[:, None] - b[None, :], strict)
        A = bc[:, None] * (K @ K.T) * Gam      # step 2
        rhs = bc[:, None] * V - (bc * np.exp(b))[:, None] * (K @ H)   # step 3
        U = solve_unit_lower(A, rhs)           # step 4
        if read == "post":                     # step 5
            P = (Q @ K.T) * _masked_exp(b[:, None] - b[None, :], jj <= ii)
            O = np.exp(b)[:, None] * (Q @ H) + P @ U
        else:
            P = (Q @ K.T) * _masked_exp(bp[:, None] - b[None, :], strict)
            O = np.exp(bp)[:, None] * (Q @ H) + P @ U
        out[c0:c1] = O
        H = np.exp(b[-1]) * H + K.T @ (np.exp(b[-1] - b)[:, None] * U)   # step 6
    return out, H


def chunked(q, k, v, log_alpha, beta, h0=None, *, chunk: int = 64, read: str = "post"):
    """Batched wrapper: q, k [B, Hk, T, dk]; v [B, Hv, T, dv]; gates [B, Hv, T]; h0 [B, Hv, dk, dv]."""
    q, k, v, a, b = (np.asarray(x, dtype=np.float64) for x in (q, k, v, log_alpha, beta))
    B, Hk, T, dk = q.shape
    Hv, dv = v.shape[1], v.shape[3]
    g = Hv // Hk
    out = np.zeros((B, Hv, T, dv))
    hT = np.zeros((B, Hv, dk, dv))
    for bi in range(B):
        for h in range(Hv):
            o, s = chunked_sequence(q[bi, h // g], k[bi, h // g], v[bi, h], a[bi, h], b[bi, h],
                                    None if h0 is None else h0[bi, h], chunk=chunk, read=read)
            out[bi, h] = o
            hT[bi, h] = s
    return out, hT
