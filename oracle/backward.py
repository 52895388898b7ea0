"""Gradients of the gated delta rule forward, in fp64, by reverse-mode differentiation of the plain
per-token recurrence.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages give no backward equations ("Prizma seq/delta.py" requires the chunked form to agree
with the recurrence in forward and gradient; the other pages train through the operation with
autograd). The definition used here is therefore the derivative of the recurrence itself, taken
by torch autograd in float64 on the CPU over ``recurrence`` below: a direct transcription of the
update (H = S^T, [dk][dv]):

    u_t = beta_t (v_t - alpha_t H^T k_t),   H <- alpha_t H + k_t u_t^T,   alpha_t = exp(log_alpha_t)
    o_t = H_t^T q_t (post-write) or H_{t-1}^T q_t (pre-write)

Given upstream gradients dout (of o) and dhT (of the final state), ``grads`` returns
dq, dk, dv, dlog_alpha, dbeta and dh0. Key heads shared by several value heads receive the sum
over their value heads.
"""
from __future__ import annotations

import numpy as np
import torch


def _t(x):
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).clone()
    return torch.as_tensor(np.asarray(x, dtype=np.float64))


def recurrence(q, k, v, log_alpha, beta, h0, segs, grp, read="post", reverse=False):
    """Torch float64 forward over segments ``segs`` = [(row, t0, t1)]; returns (o, hT)."""
    B, Hk, T, dk = q.shape
    Hv, dv = v.shape[1], v.shape[3]
    outs = [[[None] * T for _ in range(Hv)] for _ in range(B)]
    finals = []
    for si, (row, t0, t1) in enumerate(segs):
        hs = []
        for h in range(Hv):
            kh = h // grp
            H = h0[si, h]
            order = range(t1 - 1, t0 - 1, -1) if reverse else range(t0, t1)
            for t in order:
                if read == "pre":
                    outs[row][h][t] = H.T @ q[row, kh, t]
                a = torch.exp(log_alpha[row, h, t])
                u = beta[row, h, t] * (v[row, h, t] - a * (H.T @ k[row, kh, t]))
                H = a * H + torch.outer(k[row, kh, t], u)
                if read == "post":
                    outs[row][h][t] = H.T @ q[row, kh, t]
            hs.append(H)
        finals.append(torch.stack(hs))
    zero = torch.zeros(dv, dtype=torch.float64)
    o = torch.stack([torch.stack([torch.stack([x if x is not None else zero for x in outs[b][h]])
                                  for h in range(Hv)]) for b in range(B)])
    return o, torch.stack(finals)


def grads(q, k, v, log_alpha, beta, h0, cu_seqlens, dout, dhT, *, read="post", reverse=False):
    """q, k [B, Hk, T, dk]; v [B, Hv, T, dv]; log_alpha, beta [B, Hv, T]; h0 [S, Hv, dk, dv] or
    None; cu_seqlens [S + 1] or None; dout [B, Hv, T, dv]; dhT [S, Hv, dk, dv] or None.
    Returns numpy float64 (dq, dk, dv, dlog_alpha, dbeta, dh0)."""
    q, k, v, la, be = (_t(x).requires_grad_(True) for x in (q, k, v, log_alpha, beta))
    B, Hk, T, dk = q.shape
    Hv, dv = v.shape[1], v.shape[3]
    if cu_seqlens is None:
        segs = [(row, 0, T) for row in range(B)]
    else:
        cu = [int(x) for x in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
        segs = [(0, cu[i], cu[i + 1]) for i in range(len(cu) - 1)]
    S = len(segs)
    h0t = (torch.zeros(S, Hv, dk, dv, dtype=torch.float64) if h0 is None else _t(h0)).requires_grad_(True)
    o, hT = recurrence(q, k, v, la, be, h0t, segs, Hv // Hk, read=read, reverse=reverse)
    loss = (o * _t(dout)).sum()
    if dhT is not None:
        loss = loss + (hT * _t(dhT)).sum()
    loss.backward()
    return tuple(x.grad.numpy() for x in (q, k, v, la, be, h0t))
