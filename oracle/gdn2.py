"""GDN-2 (decoupled gates, per-key-channel decay) as a plain fp64 per-token recurrence.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The update is the one in the BidirectionalGatedDeltaNet2 docstring on the "tiny_gdn/fugue.py"
page, written for a state H of shape [dk][dv] (the page's S, which the page multiplies by k
on the left):

    H_t = (I - k_t (b_t * k_t)^T) Diag(exp g_t) H_{t-1} + k_t (w_t * v_t)^T

with g_t (log decay), b_t (erase gate) per key channel and w_t (write gate) per value
channel. Expanded, with H' = Diag(exp g_t) H_{t-1}:

    u_t = w_t * v_t - H'^T (b_t * k_t),   H_t = H' + k_t u_t^T

Reads: post-write o_t = H_t^T q_t, pre-write o_t = H_{t-1}^T q_t (the page's kernels read
after the write; its reverse scan reads one step early, which is the pre-write read of the
reversed sequence). g and b belong to the key head (the page repeats them with q and k to the
value heads); w and v to the value head. q and k are normalised per row first when
``l2norm`` (the page calls its kernels with use_qk_l2norm_in_kernel=True), with the
x / max(||x||, 1e-6) reading of ``oracle.prologue``.

With g = log(alpha) on every channel and b = w = beta on every channel this is exactly the
gated delta rule of ``oracle.scan`` (a pin checks it).
"""
from __future__ import annotations

import numpy as np

from .prologue import l2_normalize, _f64


def scan(q, k, v, g, b, w, h0=None, cu_seqlens=None, *, read: str = "post", reverse: bool = False,
         out=None, want_state: bool = True, l2norm: bool = False):
    """q, k [B, Hk, T, dk]; v [B, Hv, T, dv]; g, b [B, Hk, T, dk]; w [B, Hv, T, dv];
    h0 [S, Hv, dk, dv] or None; cu_seqlens [S + 1] or None (then B must be 1).
    ``out`` (float64 [B, Hv, T, dv]) turns on accumulation into it.
    Returns (o [B, Hv, T, dv], hT [S, Hv, dk, dv] or None), float64."""
    q, k, v, g, b, w = (_f64(x) for x in (q, k, v, g, b, w))
    if l2norm:
        q, k = l2_normalize(q), l2_normalize(k)
    B, Hk, T, dk = q.shape
    Hv, dv = v.shape[1], v.shape[3]
    assert k.shape == q.shape and g.shape == q.shape and b.shape == q.shape
    assert v.shape == (B, Hv, T, dv) and w.shape == v.shape and Hv % Hk == 0
    if cu_seqlens is None:
        segs = [(row, 0, T) for row in range(B)]
    else:
        cu = [int(x) for x in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
        assert B == 1
        segs = [(0, cu[i], cu[i + 1]) for i in range(len(cu) - 1)]
    S = len(segs)
    h0a = None if h0 is None else _f64(h0)
    o = out if out is not None else np.zeros((B, Hv, T, dv))
    hT = np.zeros((S, Hv, dk, dv)) if want_state else None
    grp = Hv // Hk
    for si, (row, t0, t1) in enumerate(segs):
        order = range(t1 - 1, t0 - 1, -1) if reverse else range(t0, t1)
        for j in range(Hv):
            kh = j // grp
            H = np.zeros((dk, dv)) if h0a is None else h0a[si, j].copy()
            for t in order:
                if read == "pre":
                    ot = H.T @ q[row, kh, t]
                Hd = np.exp(g[row, kh, t])[:, None] * H
                u = w[row, j, t] * v[row, j, t] - Hd.T @ (b[row, kh, t] * k[row, kh, t])
                H = Hd + np.outer(k[row, kh, t], u)
                if read == "post":
                    ot = H.T @ q[row, kh, t]
                if out is not None:
                    o[row, j, t] += ot
                else:
                    o[row, j, t] = ot
            if want_state:
                hT[si, j] = H
    return o, hT


def decode(q, k, v, g, b, w, state, *, read: str = "post", l2norm: bool = False):
    """One token per sequence: q, k, g, b [N, Hk, dk]; v, w [N, Hv, dv]; state [N, Hv, dk, dv].
    Returns (o [N, Hv, dv], new state [N, Hv, dk, dv]), float64."""
    q, k, v, g, b, w = (_f64(x)[:, :, None] for x in (q, k, v, g, b, w))
    o, hT = scan(q, k, v, g, b, w, h0=state, read=read, l2norm=l2norm)
    return o[:, :, 0], hT
