"""Pins of the GDN-2 oracle (``oracle.gdn2``) to facts it does not compute itself.

* an exact-rational brute force that applies the page's matrix statement literally,
  H <- (I - k (b*k)^T) Diag(a) H + k (w*v)^T with dense Fraction matrices;
* the reduction to the scalar gated delta rule of the C oracle (already pinned on its own)
  when every channel of g, b and w carries the same value;
* one-hot keys, where every row of the state follows its own scalar recursion;
* b = 0, where the state has an explicit sum form;
* b = 2 with unit keys, no decay and no write: a Householder reflection, which keeps the
  Frobenius norm and undoes itself when applied twice;
* structural identities: pre/post shift, reversal, segments, key-head sharing, accumulation,
  decode = one-token scan, row-scale invariance under the q/k normalisation.

The mutants at the end plant plausible mistakes in a copy of ``oracle/gdn2.py`` and check
that some pin fails for each.
"""
from __future__ import annotations

import math
import os
import random
import types
from fractions import Fraction as F

import numpy as np
import pytest

import oracle
from oracle import gdn2

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdn2.py")


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, "%s: max abs err %.3e > %.1e (scale %.3g)" % (what, err, tol, scale)


def _case(seed, B=1, Hk=2, Hv=4, T=23, dk=5, dv=3, bmax=2.0, h0=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hk, T, dk))
    k = rng.standard_normal((B, Hk, T, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, Hv, T, dv))
    g = -rng.uniform(0.0, 1.5, (B, Hk, T, dk))
    b = rng.uniform(0.0, bmax, (B, Hk, T, dk))
    w = rng.uniform(0.0, 1.0, (B, Hv, T, dv))
    H0 = 0.5 * rng.standard_normal((B, Hv, dk, dv)) if h0 else None
    return q, k, v, g, b, w, H0


# --------------------------------------------------------------------------- the pins

def _fr(rng, lo=-3, hi=3):
    return F(rng.randint(lo, hi), rng.choice((1, 2, 3, 4)))


def pin_brute_rational(mod, seed=0, read="post"):
    """Exact Fraction evaluation of the page's matrix form, T = 5, dk = 3, dv = 2, Hv = 2 Hk."""
    rng = random.Random(seed)
    T, dk, dv, Hk, Hv = 5, 3, 2, 1, 2
    q = [[[_fr(rng) for _ in range(dk)] for _ in range(T)] for _ in range(Hk)]
    k = [[[_fr(rng) for _ in range(dk)] for _ in range(T)] for _ in range(Hk)]
    a = [[[rng.choice((F(1), F(1, 2), F(3, 4), F(2, 3))) for _ in range(dk)] for _ in range(T)]
         for _ in range(Hk)]
    b = [[[rng.choice((F(0), F(1, 2), F(1), F(3, 2), F(2))) for _ in range(dk)] for _ in range(T)]
         for _ in range(Hk)]
    v = [[[_fr(rng) for _ in range(dv)] for _ in range(T)] for _ in range(Hv)]
    w = [[[rng.choice((F(0), F(1, 4), F(1, 2), F(1))) for _ in range(dv)] for _ in range(T)]
         for _ in range(Hv)]
    H0 = [[[_fr(rng) for _ in range(dv)] for _ in range(dk)] for _ in range(Hv)]
    arr = lambda x: np.array([[[float(e) for e in r] for r in h] for h in x])[None]
    G = np.log(arr(a))
    o, hT = mod.scan(arr(q), arr(k), arr(v), G, arr(b), arr(w), arr(H0)[0][None], read=read)
    for h in range(Hv):
        kh = h // (Hv // Hk)
        H = [row[:] for row in H0[h]]
        for t in range(T):
            if read == "pre":
                ref = [sum(H[i][j] * q[kh][t][i] for i in range(dk)) for j in range(dv)]
            # M = (I - k (b*k)^T) Diag(a): M[i][j] = (delta_ij - k_i b_j k_j) a_j
            M = [[((F(1) if i == j else F(0)) - k[kh][t][i] * b[kh][t][j] * k[kh][t][j]) * a[kh][t][j]
                  for j in range(dk)] for i in range(dk)]
            H = [[sum(M[i][m] * H[m][j] for m in range(dk)) + k[kh][t][i] * w[h][t][j] * v[h][t][j]
                  for j in range(dv)] for i in range(dk)]
            if read == "post":
                ref = [sum(H[i][j] * q[kh][t][i] for i in range(dk)) for j in range(dv)]
            _close(o[0, h, t], [float(x) for x in ref], 1e-12, "brute o head %d tok %d" % (h, t))
        _close(hT[0, h], [[float(x) for x in r] for r in H], 1e-12, "brute hT head %d" % h)


def pin_reduces_to_scalar_rule(mod, read="post"):
    """g = log(alpha), b = w = beta on every channel: the C oracle's gated delta rule."""
    q, k, v, g, b, w, H0 = _case(3)
    B, Hk, T, dk = q.shape
    Hv, dv = v.shape[1], v.shape[3]
    rng = np.random.default_rng(4)
    la = -rng.uniform(0.0, 1.5, (B, Hk, T))
    beta = rng.uniform(0.0, 1.0, (B, Hk, T))
    grp = Hv // Hk
    la_v, beta_v = np.repeat(la, grp, axis=1), np.repeat(beta, grp, axis=1)
    g = np.repeat(la[..., None], dk, axis=-1)
    bb = np.repeat(beta[..., None], dk, axis=-1)
    ww = np.repeat(beta_v[..., None], dv, axis=-1)
    o, hT = mod.scan(q, k, v, g, bb, ww, H0, read=read)
    o_ref, h_ref = oracle.scan(q, k, v, la_v, beta_v, H0, read=read)
    _close(o, o_ref, 1e-12, "scalar reduction o (%s)" % read)
    _close(hT, h_ref, 1e-12, "scalar reduction hT (%s)" % read)


def pin_one_hot_keys(mod):
    """k_t = e_{c_t}: row c of H is scaled by (1 - b_t[c]) a_t[c] and gains w_t * v_t when c = c_t,
    and only decays by a_t[c] otherwise."""
    rng = np.random.default_rng(7)
    B, Hk, Hv, T, dk, dv = 1, 1, 2, 17, 4, 3
    idx = rng.integers(0, dk, T)
    k = np.zeros((B, Hk, T, dk))
    k[0, 0, np.arange(T), idx] = 1.0
    q = rng.standard_normal((B, Hk, T, dk))
    v = rng.standard_normal((B, Hv, T, dv))
    g = -rng.uniform(0, 1, (B, Hk, T, dk))
    b = rng.uniform(0, 2, (B, Hk, T, dk))
    w = rng.uniform(0, 1, (B, Hv, T, dv))
    H0 = rng.standard_normal((B, Hv, dk, dv))
    o, hT = mod.scan(q, k, v, g, b, w, H0)
    for h in range(Hv):
        H = H0[0, h].copy()
        for t in range(T):
            for c in range(dk):
                a = math.exp(g[0, 0, t, c])
                if c == idx[t]:
                    H[c] = (1.0 - b[0, 0, t, c]) * a * H[c] + w[0, h, t] * v[0, h, t]
                else:
                    H[c] = a * H[c]
            ref = np.array([sum(H[c, j] * q[0, 0, t, c] for c in range(dk)) for j in range(dv)])
            _close(o[0, h, t], ref, 1e-12, "one-hot o head %d tok %d" % (h, t))
        _close(hT[0, h], H, 1e-12, "one-hot hT head %d" % h)


def pin_no_erase_sum_form(mod):
    """b = 0: H_T = Diag(e^{G_T}) H_0 + sum_t Diag(e^{G_T - G_t}) k_t (w_t * v_t)^T, G the cumsum of g."""
    q, k, v, g, b, w, H0 = _case(11, Hk=1, Hv=2)
    b = np.zeros_like(b)
    o, hT = mod.scan(q, k, v, g, b, w, H0)
    G = np.cumsum(g[0, 0], axis=0)
    T = q.shape[2]
    for h in range(2):
        for t in (0, T // 2, T - 1):
            Ht = np.exp(G[t])[:, None] * H0[0, h]
            for s in range(t + 1):
                Ht = Ht + np.exp(G[t] - G[s])[:, None] * np.outer(k[0, 0, s], w[0, h, s] * v[0, h, s])
            _close(o[0, h, t], Ht.T @ q[0, 0, t], 1e-12, "sum form o head %d tok %d" % (h, t))
            if t == T - 1:
                _close(hT[0, h], Ht, 1e-12, "sum form hT head %d" % h)


def pin_householder(mod):
    """b = 2, g = 0, w = 0, unit k: each step reflects H; norms are kept and a repeated key undoes it."""
    rng = np.random.default_rng(13)
    B, Hk, Hv, T, dk, dv = 1, 1, 1, 6, 4, 3
    k = rng.standard_normal((B, Hk, T, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    k[0, 0, 1] = k[0, 0, 0]  # tokens 0 and 1 share a key: their reflections cancel
    q = rng.standard_normal((B, Hk, T, dk))
    v = rng.standard_normal((B, Hv, T, dv))
    g = np.zeros((B, Hk, T, dk))
    b = np.full((B, Hk, T, dk), 2.0)
    w = np.zeros((B, Hv, T, dv))
    H0 = rng.standard_normal((B, Hv, dk, dv))
    _, h2 = mod.scan(q[:, :, :2], k[:, :, :2], v[:, :, :2], g[:, :, :2], b[:, :, :2], w[:, :, :2], H0)
    _close(h2, H0, 1e-12, "reflection applied twice")
    _, hT = mod.scan(q, k, v, g, b, w, H0)
    assert abs(np.linalg.norm(hT) - np.linalg.norm(H0)) < 1e-12 * np.linalg.norm(H0), "norm not kept"
    assert np.max(np.abs(hT - H0)) > 1e-3, "reflections did nothing"


def pin_pre_post_shift(mod):
    """The pre-write read of token t equals the post-write read of token t - 1 with q_t."""
    q, k, v, g, b, w, H0 = _case(17)
    o_pre, h_pre = mod.scan(q, k, v, g, b, w, H0, read="pre")
    qs = np.concatenate([q[:, :, 1:], q[:, :, :1]], axis=2)
    o_post, h_post = mod.scan(qs, k, v, g, b, w, H0, read="post")
    _close(o_pre[:, :, 1:], o_post[:, :, :-1], 1e-12, "pre/post shift")
    grp = v.shape[1] // q.shape[1]
    for h in range(v.shape[1]):
        _close(o_pre[0, h, 0], H0[0, h].T @ q[0, h // grp, 0], 1e-12, "pre read of token 0")
    _close(h_pre, h_post, 1e-12, "state independent of the read")


def pin_reverse_is_flip(mod):
    q, k, v, g, b, w, H0 = _case(19)
    o_r, h_r = mod.scan(q, k, v, g, b, w, H0, reverse=True)
    fl = lambda x: x[:, :, ::-1].copy()
    o_f, h_f = mod.scan(fl(q), fl(k), fl(v), fl(g), fl(b), fl(w), H0)
    _close(o_r, fl(o_f), 1e-12, "reverse o")
    _close(h_r, h_f, 1e-12, "reverse hT")


def pin_segments(mod):
    """cu_seqlens: each segment is an independent scan from its own initial state."""
    lengths = [5, 1, 9]
    q, k, v, g, b, w, _ = _case(23, T=sum(lengths))
    rng = np.random.default_rng(24)
    H0 = rng.standard_normal((len(lengths), v.shape[1], q.shape[3], v.shape[3]))
    cu = np.cumsum([0] + lengths)
    o, hT = mod.scan(q, k, v, g, b, w, H0, cu)
    for s in range(len(lengths)):
        sl = slice(cu[s], cu[s + 1])
        o_s, h_s = mod.scan(q[:, :, sl], k[:, :, sl], v[:, :, sl], g[:, :, sl], b[:, :, sl], w[:, :, sl],
                            H0[s:s + 1])
        _close(o[:, :, sl], o_s, 1e-12, "segment %d o" % s)
        _close(hT[s], h_s[0], 1e-12, "segment %d hT" % s)


def pin_key_head_sharing(mod):
    """Hv = 2 Hk equals the same scan with q, k, g, b repeated to every value head."""
    q, k, v, g, b, w, H0 = _case(29, Hk=2, Hv=4)
    o, hT = mod.scan(q, k, v, g, b, w, H0)
    rep = lambda x: np.repeat(x, 2, axis=1)
    o2, h2 = mod.scan(rep(q), rep(k), v, rep(g), rep(b), w, H0)
    _close(o, o2, 1e-12, "head sharing o")
    _close(hT, h2, 1e-12, "head sharing hT")
    # the value head h reads key head h // 2, not h % 2
    o3, _ = mod.scan(np.tile(q, (1, 2, 1, 1)), np.tile(k, (1, 2, 1, 1)), v, np.tile(g, (1, 2, 1, 1)),
                     np.tile(b, (1, 2, 1, 1)), w, H0)
    assert np.max(np.abs(o3 - o)) > 1e-6, "head mapping is not observable"


def pin_accumulate_and_decode(mod):
    q, k, v, g, b, w, H0 = _case(31, B=3, T=1)
    base = np.random.default_rng(32).standard_normal((3, v.shape[1], 1, v.shape[3]))
    o_s, h_s = mod.scan(q, k, v, g, b, w, H0)
    acc = base.copy()
    mod.scan(q, k, v, g, b, w, H0, out=acc)
    _close(acc, base + o_s, 1e-12, "accumulate")
    o_d, h_d = mod.decode(q[:, :, 0], k[:, :, 0], v[:, :, 0], g[:, :, 0], b[:, :, 0], w[:, :, 0], H0)
    _close(o_d, o_s[:, :, 0], 1e-12, "decode o")
    _close(h_d, h_s, 1e-12, "decode state")


def pin_l2norm_row_scale(mod):
    q, k, v, g, b, w, H0 = _case(37)
    rng = np.random.default_rng(38)
    sq = rng.uniform(0.05, 20.0, q.shape[:-1] + (1,))
    sk = rng.uniform(0.05, 20.0, k.shape[:-1] + (1,))
    qn = q / np.linalg.norm(q, axis=-1, keepdims=True)
    o1, h1 = mod.scan(qn, k, v, g, b, w, H0)
    o2, h2 = mod.scan(q * sq, k * sk, v, g, b, w, H0, l2norm=True)
    _close(o2, o1, 1e-12, "l2norm o")
    _close(h2, h1, 1e-12, "l2norm hT")


ALL_PINS = [
    ("brute_post", lambda m: pin_brute_rational(m, 0, "post")),
    ("brute_pre", lambda m: pin_brute_rational(m, 1, "pre")),
    ("scalar_post", lambda m: pin_reduces_to_scalar_rule(m, "post")),
    ("scalar_pre", lambda m: pin_reduces_to_scalar_rule(m, "pre")),
    ("one_hot", pin_one_hot_keys),
    ("no_erase", pin_no_erase_sum_form),
    ("householder", pin_householder),
    ("pre_post", pin_pre_post_shift),
    ("reverse", pin_reverse_is_flip),
    ("segments", pin_segments),
    ("heads", pin_key_head_sharing),
    ("acc_decode", pin_accumulate_and_decode),
    ("l2norm", pin_l2norm_row_scale),
]


@pytest.mark.parametrize("name,fn", ALL_PINS, ids=[p[0] for p in ALL_PINS])
def test_pin(oracle_lib, name, fn):
    fn(gdn2)


# --------------------------------------------------------------------------- mutants

MUTANTS = [
    ("decay_ignored", "Hd = np.exp(g[row, kh, t])[:, None] * H", "Hd = H"),
    ("decay_sign", "Hd = np.exp(g[row, kh, t])[:, None] * H", "Hd = np.exp(-g[row, kh, t])[:, None] * H"),
    ("decay_on_columns", "Hd = np.exp(g[row, kh, t])[:, None] * H",
     "Hd = H * np.exp(g[row, kh, t])[None, :H.shape[1]]"),
    ("erase_not_decayed", "- Hd.T @ (b[row, kh, t]", "- H.T @ (b[row, kh, t]"),
    ("erase_gate_ignored", "(b[row, kh, t] * k[row, kh, t])", "(k[row, kh, t])"),
    ("erase_gate_scalar", "(b[row, kh, t] * k[row, kh, t])", "(b[row, kh, t].mean() * k[row, kh, t])"),
    ("erase_uses_query", "(b[row, kh, t] * k[row, kh, t])", "(b[row, kh, t] * q[row, kh, t])"),
    ("erase_sign", "u = w[row, j, t] * v[row, j, t] - Hd.T", "u = w[row, j, t] * v[row, j, t] + Hd.T"),
    ("write_gate_ignored", "u = w[row, j, t] * v[row, j, t]", "u = v[row, j, t]"),
    ("write_gate_on_erase", "u = w[row, j, t] * v[row, j, t] - Hd.T @ (b[row, kh, t] * k[row, kh, t])",
     "u = w[row, j, t] * (v[row, j, t] - Hd.T @ (b[row, kh, t] * k[row, kh, t]))"),
    ("state_not_decayed", "H = Hd + np.outer(", "H = H + np.outer("),
    ("write_decayed", "H = Hd + np.outer(k[row, kh, t], u)",
     "H = Hd + np.exp(g[row, kh, t])[:, None] * np.outer(k[row, kh, t], u)"),
    ("post_reads_old_state", "if read == \"post\":\n                    ot = H.T", "if read == \"post\":\n                    ot = Hd.T"),
    ("pre_reads_new_state", "if read == \"pre\":\n                    ot = H.T @ q[row, kh, t]",
     "if read == \"pre\":\n                    ot = (np.exp(g[row, kh, t])[:, None] * H).T @ q[row, kh, t]"),
    ("read_uses_key", "ot = H.T @ q[row, kh, t]\n                if out", "ot = H.T @ k[row, kh, t]\n                if out"),
    ("key_head_modulo", "kh = j // grp", "kh = j % Hk"),
    ("reverse_ignored", "order = range(t1 - 1, t0 - 1, -1) if reverse else range(t0, t1)", "order = range(t0, t1)"),
    ("h0_ignored", "H = np.zeros((dk, dv)) if h0a is None else h0a[si, j].copy()", "H = np.zeros((dk, dv))"),
    ("h0_first_segment", "h0a[si, j].copy()", "h0a[0, j].copy()"),
    ("accumulate_ignored", "o[row, j, t] += ot", "o[row, j, t] = ot"),
    ("l2norm_ignored", "q, k = l2_normalize(q), l2_normalize(k)", "pass"),
    ("l2norm_query_only", "q, k = l2_normalize(q), l2_normalize(k)", "q = l2_normalize(q)"),
]


def _load_mutant(text):
    mod = types.ModuleType("gdn2_mutant")
    mod.__dict__["__name__"] = "gdn2_mutant"
    text = text.replace("from .prologue import l2_normalize, _f64", "from oracle.prologue import l2_normalize, _f64")
    exec(compile(text, "gdn2_mutant.py", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(oracle_lib, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation anchor for %s not found" % name
    mod = _load_mutant(src.replace(old, new, 1))
    for pin_name, fn in ALL_PINS:
        try:
            fn(mod)
        except (AssertionError, ValueError, IndexError):
            return
    pytest.fail("no pin catches mutant %s" % name)


def test_unmutated_copy_passes(oracle_lib):
    mod = _load_mutant(open(SRC).read())
    for _, fn in ALL_PINS:
        fn(mod)
