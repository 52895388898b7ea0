"""DeltaProduct (n_delta >= 2 delta sub-steps per token) as a plain fp64 per-token recurrence.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The "Prizma seq/delta.py" page (`_delta_reference`, the n_delta branch) applies n sub-steps per
token: the decay alpha_t once, on sub-step 0, then pure delta sub-steps. In the layout H = S^T
[dk][dv], for token t and sub-step j = 0 .. n-1 with a_tj = alpha_t when j = 0 and 1 otherwise:

    u_tj = beta_tj (v_tj - a_tj H^T k_tj),    H <- a_tj H + k_tj u_tj^T

The page reads before the token's sub-steps, o_t = H_{t-1}^T q_t (pre-write read); the
post-write read o_t = H_t^T q_t (after the last sub-step) is the same reading as for the scalar
rule. Key heads are shared by groups of value heads as in ``oracle.scan``; q and k rows (every
sub-step's key) are normalised first when ``l2norm``.
"""
from __future__ import annotations

import numpy as np

from .prologue import l2_normalize, _f64


def scan(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, *, read: str = "pre", out=None,
         want_state: bool = True, l2norm: bool = False):
    """q [B, Hk, T, dk]; k [B, Hk, T, n, dk]; v [B, Hv, T, n, dv]; log_alpha [B, Hv, T];
    beta [B, Hv, T, n]; h0 [S, Hv, dk, dv] or None; cu_seqlens [S + 1] or None (then B must be 1
    for packed rows). Returns (o [B, Hv, T, dv], hT [S, Hv, dk, dv] or None), float64."""
    q, k, v, la, beta = (_f64(x) for x in (q, k, v, log_alpha, beta))
    if l2norm:
        q, k = l2_normalize(q), l2_normalize(k)
    B, Hk, T, dk = q.shape
    n = k.shape[3]
    Hv, dv = v.shape[1], v.shape[4]
    assert k.shape == (B, Hk, T, n, dk) and v.shape == (B, Hv, T, n, dv)
    assert la.shape == (B, Hv, T) and beta.shape == (B, Hv, T, n) and Hv % Hk == 0
    if cu_seqlens is None:
        segs = [(row, 0, T) for row in range(B)]
    else:
        cu = [int(x) for x in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
        assert B == 1
        segs = [(0, cu[i], cu[i + 1]) for i in range(len(cu) - 1)]
    h0a = None if h0 is None else _f64(h0)
    o = out if out is not None else np.zeros((B, Hv, T, dv))
    hT = np.zeros((len(segs), Hv, dk, dv)) if want_state else None
    grp = Hv // Hk
    for si, (row, t0, t1) in enumerate(segs):
        for h in range(Hv):
            kh = h // grp
            H = np.zeros((dk, dv)) if h0a is None else h0a[si, h].copy()
            for t in range(t0, t1):
                if read == "pre":
                    ot = H.T @ q[row, kh, t]
                for j in range(n):
                    a = np.exp(la[row, h, t]) if j == 0 else 1.0
                    kk = k[row, kh, t, j]
                    u = beta[row, h, t, j] * (v[row, h, t, j] - a * (H.T @ kk))
                    H = a * H + np.outer(kk, u)
                if read == "post":
                    ot = H.T @ q[row, kh, t]
                if out is not None:
                    o[row, h, t] += ot
                else:
                    o[row, h, t] = ot
            if want_state:
                hT[si, h] = H
    return o, hT
