"""Pins of the backward oracle (``oracle.backward``) to facts it does not compute itself.

* central finite differences of L = sum(o * dout) + sum(hT * dhT), where o and hT come from the
  C oracle (``oracle.scan``, independent code, pinned on its own), for every input element of
  small cases, both reads, reversed scans and packed segments with key-head sharing;
* linearity of the gradients in (dout, dhT);
* the closed form at beta = 0 (post-write read): o_t = e^{sum_{s<=t} a_s} H_0^T q_t, so
  dq_t = e^{sum a} H_0 dout_t, dlog_alpha_s = sum_{t>=s} <dout_t, o_t> + <dhT, hT>,
  dh0 = sum_t e^{sum a} q_t dout_t^T + e^{sum a} dhT, dk = dv = 0.
Mutants at the end plant mistakes in a copy of ``oracle/backward.py``.
"""
from __future__ import annotations

import os
import types

import numpy as np
import pytest

import oracle
from oracle import backward as bw

SRC = os.path.join(os.path.dirname(oracle.__file__), "backward.py")


def _case(seed, B=1, Hk=1, Hv=2, T=6, dk=3, dv=2, nseg=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hk, T, dk))
    k = rng.standard_normal((B, Hk, T, dk)) * 0.6
    v = rng.standard_normal((B, Hv, T, dv))
    la = -rng.uniform(0.05, 0.8, (B, Hv, T))
    beta = rng.uniform(0.1, 1.0, (B, Hv, T))
    S = B if nseg is None else nseg
    h0 = rng.standard_normal((S, Hv, dk, dv)) * 0.5
    dout = rng.standard_normal((B, Hv, T, dv))
    dhT = rng.standard_normal((S, Hv, dk, dv))
    return q, k, v, la, beta, h0, dout, dhT


def _loss(inputs, cu, dout, dhT, read, reverse):
    q, k, v, la, beta, h0 = inputs
    o, hT = oracle.scan(q, k, v, la, beta, h0, cu, read=read, reverse=reverse)
    return float(np.sum(o * dout) + np.sum(hT * dhT))


def pin_finite_differences(mod, seed=0, read="post", reverse=False, packed=False):
    if packed:
        q, k, v, la, beta, h0, dout, dhT = _case(seed, T=7, Hk=1, Hv=2, nseg=3)
        cu = np.array([0, 2, 2, 7], dtype=np.int64)
    else:
        q, k, v, la, beta, h0, dout, dhT = _case(seed, B=2)
        cu = None
    g = mod.grads(q, k, v, la, beta, h0, cu, dout, dhT, read=read, reverse=reverse)
    inputs = [q, k, v, la, beta, h0]
    eps = 1e-6
    for idx, (x, gx) in enumerate(zip(inputs, g)):
        flat = x.reshape(-1)
        fd = np.zeros(flat.size)
        for i in range(flat.size):
            keep = flat[i]
            flat[i] = keep + eps
            lp = _loss(inputs, cu, dout, dhT, read, reverse)
            flat[i] = keep - eps
            lm = _loss(inputs, cu, dout, dhT, read, reverse)
            flat[i] = keep
            fd[i] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(fd - gx.reshape(-1)))
        scale = max(1.0, np.max(np.abs(fd)))
        assert err <= 1e-6 * scale, "input %d (%s, rev=%s, packed=%s): fd err %.3e" % (idx, read, reverse, packed, err)


def pin_linearity(mod):
    q, k, v, la, beta, h0, dout, dhT = _case(5, B=1, Hk=1, Hv=1, T=9, dk=4, dv=3)
    rng = np.random.default_rng(6)
    dout2, dhT2 = rng.standard_normal(dout.shape), rng.standard_normal(dhT.shape)
    g1 = mod.grads(q, k, v, la, beta, h0, None, dout, dhT)
    g2 = mod.grads(q, k, v, la, beta, h0, None, dout2, dhT2)
    g3 = mod.grads(q, k, v, la, beta, h0, None, 2.0 * dout - dout2, 2.0 * dhT - dhT2)
    for a, b, c in zip(g1, g2, g3):
        assert np.max(np.abs(2.0 * a - b - c)) <= 1e-10 * max(1.0, np.max(np.abs(c))), "not linear"


def pin_beta_zero(mod):
    q, k, v, la, beta, h0, dout, dhT = _case(7, B=1, Hk=1, Hv=1, T=8, dk=4, dv=3)
    beta = np.zeros_like(beta)
    dq, dk_, dv_, dla, dbeta, dh0 = mod.grads(q, k, v, la, beta, h0, None, dout, dhT)
    G = np.cumsum(la[0, 0])
    H0 = h0[0, 0]
    o = np.stack([np.exp(G[t]) * (H0.T @ q[0, 0, t]) for t in range(8)])
    hT = np.exp(G[-1]) * H0
    for t in range(8):
        assert np.allclose(dq[0, 0, t], np.exp(G[t]) * (H0 @ dout[0, 0, t]), atol=1e-12), "dq"
    ref_la = np.array([sum(np.dot(dout[0, 0, t], o[t]) for t in range(s, 8)) + np.sum(dhT[0, 0] * hT)
                       for s in range(8)])
    assert np.allclose(dla[0, 0], ref_la, atol=1e-12), "dlog_alpha"
    ref_h0 = sum(np.exp(G[t]) * np.outer(q[0, 0, t], dout[0, 0, t]) for t in range(8)) + np.exp(G[-1]) * dhT[0, 0]
    assert np.allclose(dh0[0, 0], ref_h0, atol=1e-12), "dh0"
    assert np.max(np.abs(dk_)) == 0.0 and np.max(np.abs(dv_)) == 0.0, "dk, dv"


ALL_PINS = [
    ("fd_post", lambda m: pin_finite_differences(m, 0, "post")),
    ("fd_pre", lambda m: pin_finite_differences(m, 1, "pre")),
    ("fd_reverse", lambda m: pin_finite_differences(m, 2, "post", reverse=True)),
    ("fd_packed_pre", lambda m: pin_finite_differences(m, 3, "pre", packed=True)),
    ("linearity", pin_linearity),
    ("beta_zero", pin_beta_zero),
]


@pytest.mark.parametrize("name,fn", ALL_PINS, ids=[p[0] for p in ALL_PINS])
def test_pin(oracle_lib, name, fn):
    fn(bw)


MUTANTS = [
    ("erase_not_decayed", "u = beta[row, h, t] * (v[row, h, t] - a * (H.T @ k[row, kh, t]))",
     "u = beta[row, h, t] * (v[row, h, t] - (H.T @ k[row, kh, t]))"),
    ("state_not_decayed", "H = a * H + torch.outer(k[row, kh, t], u)", "H = H + torch.outer(k[row, kh, t], u)"),
    ("post_reads_old", "if read == \"post\":\n                    outs[row][h][t] = H.T @ q[row, kh, t]",
     "if read == \"post\":\n                    outs[row][h][t] = (H - torch.outer(k[row, kh, t], u)).T @ q[row, kh, t]"),
    ("decay_linear", "a = torch.exp(log_alpha[row, h, t])", "a = 1.0 + log_alpha[row, h, t]"),
    ("head_modulo", "kh = h // grp", "kh = h % grp"),
    ("reverse_ignored", "order = range(t1 - 1, t0 - 1, -1) if reverse else range(t0, t1)", "order = range(t0, t1)"),
    ("dhT_ignored", "loss = loss + (hT * _t(dhT)).sum()", "loss = loss"),
]


def _load_mutant(text):
    mod = types.ModuleType("bw_mutant")
    exec(compile(text, "bw_mutant.py", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(oracle_lib, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation anchor for %s not found" % name
    mod = _load_mutant(src.replace(old, new, 1))
    for _, fn in ALL_PINS:
        try:
            fn(mod)
        except (AssertionError, ValueError, IndexError, RuntimeError):
            return
    pytest.fail("no pin catches mutant %s" % name)
