"""Pins of the DeltaProduct oracle (``oracle.delta_product``) to facts it does not compute itself.

* an exact-rational brute force through per-token transition matrices
  Phi_t = (I - b_{n-1} k_{n-1} k_{n-1}^T) ... (I - b_0 k_0 k_0^T) alpha_t and the write terms;
* n = 1 is the scalar rule of the C oracle;
* the expansion identity: n sub-steps per token are the scalar rule (C oracle) on the sequence of
  T n sub-steps, with the decay on each token's first sub-step and the read at its first
  sub-step (pre-write) or last sub-step (post-write);
* Householder products: alpha = 1, beta = 2, v = 0 and unit keys reflect the state, keeping its
  norm, and a token whose two sub-steps share a key leaves it unchanged;
* segments and accumulation.
Mutants at the end plant mistakes in a copy of ``oracle/delta_product.py``.
"""
from __future__ import annotations

import os
import random
import types
from fractions import Fraction as F

import numpy as np
import pytest

import oracle
from oracle import delta_product as dp

SRC = os.path.join(os.path.dirname(oracle.__file__), "delta_product.py")


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, "%s: max abs err %.3e > %.1e (scale %.3g)" % (what, err, tol, scale)


def _case(seed, B=1, Hk=1, Hv=2, T=13, n=3, dk=5, dv=3):
    rng = np.random.default_rng(seed)
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    q = unit(rng.standard_normal((B, Hk, T, dk)))
    k = unit(rng.standard_normal((B, Hk, T, n, dk)))
    v = rng.standard_normal((B, Hv, T, n, dv))
    la = -rng.uniform(0.0, 1.0, (B, Hv, T))
    beta = rng.uniform(0.0, 1.5, (B, Hv, T, n))
    h0 = rng.standard_normal((B, Hv, dk, dv)) * 0.5
    return q, k, v, la, beta, h0


def _fr(rng):
    return F(rng.randint(-3, 3), rng.choice((1, 2, 3)))


def pin_brute(mod, seed=0, read="pre"):
    rng = random.Random(seed)
    T, n, dk, dv = 4, 2, 3, 2
    q = [[_fr(rng) for _ in range(dk)] for _ in range(T)]
    k = [[[_fr(rng) for _ in range(dk)] for _ in range(n)] for _ in range(T)]
    v = [[[_fr(rng) for _ in range(dv)] for _ in range(n)] for _ in range(T)]
    al = [rng.choice((F(1), F(1, 2), F(3, 4))) for _ in range(T)]
    be = [[rng.choice((F(0), F(1, 2), F(1), F(2))) for _ in range(n)] for _ in range(T)]
    H0 = [[_fr(rng) for _ in range(dv)] for _ in range(dk)]
    o, hT = mod.scan(np.array([[q]], dtype=float).astype(float),
                     np.array([[[[[float(x) for x in r] for r in kk] for kk in k]]])[0][None],
                     np.array([[[[[float(x) for x in r] for r in vv] for vv in v]]])[0][None],
                     np.log(np.array([[[float(a) for a in al]]])),
                     np.array([[[[float(b) for b in bb] for bb in be]]]),
                     np.array([[[[float(x) for x in r] for r in H0]]]), read=read)
    H = [r[:] for r in H0]
    mm = lambda A, Bm: [[sum(A[i][m] * Bm[m][j] for m in range(len(Bm))) for j in range(len(Bm[0]))]
                        for i in range(len(A))]
    for t in range(T):
        if read == "pre":
            ref = [sum(H[i][j] * q[t][i] for i in range(dk)) for j in range(dv)]
        # Phi = (I - b_{n-1} k k^T) ... (I - b_0 k k^T) alpha; write W = sum_j (later factors) b_j k_j v_j^T
        for j in range(n):
            a = al[t] if j == 0 else F(1)
            kk, b = k[t][j], be[t][j]
            P = [[((F(1) if i == m else F(0)) - b * kk[i] * kk[m]) * a for m in range(dk)] for i in range(dk)]
            H = mm(P, H)
            H = [[H[i][c] + b * kk[i] * v[t][j][c] for c in range(dv)] for i in range(dk)]
        if read == "post":
            ref = [sum(H[i][j] * q[t][i] for i in range(dk)) for j in range(dv)]
        _close(o[0, 0, t], [float(x) for x in ref], 1e-12, "brute o tok %d" % t)
    _close(hT[0, 0], [[float(x) for x in r] for r in H], 1e-12, "brute hT")


def pin_one_substep_is_scalar(mod):
    q, k, v, la, beta, h0 = _case(3, n=1)
    for read in ("pre", "post"):
        o, hT = mod.scan(q, k, v, la, beta, h0, read=read)
        o2, h2 = oracle.scan(q, k[:, :, :, 0], v[:, :, :, 0], la, beta[..., 0], h0, read=read)
        _close(o, o2, 1e-12, "n=1 o " + read)
        _close(hT, h2, 1e-12, "n=1 hT " + read)


def pin_expansion(mod):
    """n sub-steps per token = the scalar rule over the T n sub-steps."""
    q, k, v, la, beta, h0 = _case(5, Hk=1, Hv=2, n=3)
    B, Hk, T, n, dk = k.shape
    Hv, dv = v.shape[1], v.shape[4]
    ke = k.reshape(B, Hk, T * n, dk)
    ve = v.reshape(B, Hv, T * n, dv)
    be = beta.reshape(B, Hv, T * n)
    lae = np.zeros((B, Hv, T, n))
    lae[..., 0] = la
    lae = lae.reshape(B, Hv, T * n)
    for read, j in (("pre", 0), ("post", n - 1)):
        qe = np.zeros((B, Hk, T, n, dk))
        qe[:, :, :, j] = q
        qe = qe.reshape(B, Hk, T * n, dk)
        oe, he = oracle.scan(qe, ke, ve, lae, be, h0, read=read)
        o, hT = mod.scan(q, k, v, la, beta, h0, read=read)
        _close(o, oe.reshape(B, Hv, T, n, dv)[:, :, :, j], 1e-12, "expansion o " + read)
        _close(hT, he, 1e-12, "expansion hT " + read)


def pin_householder(mod):
    rng = np.random.default_rng(9)
    T, n, dk, dv = 5, 2, 4, 3
    k = rng.standard_normal((1, 1, T, n, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    k[0, 0, 2, 1] = k[0, 0, 2, 0]  # token 2: the same reflection twice
    q = rng.standard_normal((1, 1, T, dk))
    v = np.zeros((1, 1, T, n, dv))
    la = np.zeros((1, 1, T))
    beta = np.full((1, 1, T, n), 2.0)
    h0 = rng.standard_normal((1, 1, dk, dv))
    _, h2 = mod.scan(q[:, :, :2], k[:, :, :2], v[:, :, :2], la[:, :, :2], beta[:, :, :2], h0)
    _, h3 = mod.scan(q[:, :, :3], k[:, :, :3], v[:, :, :3], la[:, :, :3], beta[:, :, :3], h0)
    _close(h3, h2, 1e-12, "repeated reflection is the identity")
    _, hT = mod.scan(q, k, v, la, beta, h0)
    assert abs(np.linalg.norm(hT) - np.linalg.norm(h0)) < 1e-12 * np.linalg.norm(h0), "norm not kept"
    assert np.max(np.abs(hT - h0)) > 1e-3, "no reflection happened"


def pin_segments_accumulate(mod):
    lengths = [4, 1, 7]
    q, k, v, la, beta, _ = _case(11, T=sum(lengths), n=2)
    h0 = np.random.default_rng(12).standard_normal((3, 2, 5, 3))
    cu = np.cumsum([0] + lengths)
    base = np.random.default_rng(13).standard_normal((1, 2, sum(lengths), 3))
    acc = base.copy()
    o, hT = mod.scan(q, k, v, la, beta, h0, cu, out=acc)
    for s in range(3):
        sl = slice(cu[s], cu[s + 1])
        o_s, h_s = mod.scan(q[:, :, sl], k[:, :, sl], v[:, :, sl], la[:, :, sl], beta[:, :, sl], h0[s:s + 1])
        _close(acc[:, :, sl] - base[:, :, sl], o_s, 1e-12, "segment %d o" % s)
        _close(hT[s], h_s[0], 1e-12, "segment %d hT" % s)


def pin_key_heads(mod):
    """Hv = 2 Hk equals the same scan with q and k repeated to every value head (head j reads j // 2)."""
    q, k, v, la, beta, h0 = _case(17, Hk=2, Hv=4, n=2)
    o, hT = mod.scan(q, k, v, la, beta, h0)
    rep = lambda x: np.repeat(x, 2, axis=1)
    o2, h2 = mod.scan(rep(q), rep(k), v, la, beta, h0)
    _close(o, o2, 1e-12, "head sharing o")
    _close(hT, h2, 1e-12, "head sharing hT")


ALL_PINS = [
    ("heads", pin_key_heads),
    ("brute_pre", lambda m: pin_brute(m, 0, "pre")),
    ("brute_post", lambda m: pin_brute(m, 1, "post")),
    ("one_substep", pin_one_substep_is_scalar),
    ("expansion", pin_expansion),
    ("householder", pin_householder),
    ("segments", pin_segments_accumulate),
]


@pytest.mark.parametrize("name,fn", ALL_PINS, ids=[p[0] for p in ALL_PINS])
def test_pin(oracle_lib, name, fn):
    fn(dp)


MUTANTS = [
    ("decay_every_substep", "a = np.exp(la[row, h, t]) if j == 0 else 1.0", "a = np.exp(la[row, h, t])"),
    ("decay_last_substep", "a = np.exp(la[row, h, t]) if j == 0 else 1.0", "a = np.exp(la[row, h, t]) if j == n - 1 else 1.0"),
    ("decay_never", "a = np.exp(la[row, h, t]) if j == 0 else 1.0", "a = 1.0"),
    ("erase_not_decayed", "(v[row, h, t, j] - a * (H.T @ kk))", "(v[row, h, t, j] - (H.T @ kk))"),
    ("beta_first_substep", "u = beta[row, h, t, j] *", "u = beta[row, h, t, 0] *"),
    ("key_first_substep", "kk = k[row, kh, t, j]", "kk = k[row, kh, t, 0]"),
    ("value_first_substep", "(v[row, h, t, j]", "(v[row, h, t, 0]"),
    ("write_decayed", "H = a * H + np.outer(kk, u)", "H = a * (H + np.outer(kk, u))"),
    ("read_swapped", "if read == \"pre\":\n                    ot", "if read == \"post\":\n                    ot"),
    ("head_modulo", "kh = h // grp", "kh = h % Hk"),
    ("accumulate_ignored", "o[row, h, t] += ot", "o[row, h, t] = ot"),
]


def _load_mutant(text):
    mod = types.ModuleType("dp_mutant")
    text = text.replace("from .prologue import l2_normalize, _f64", "from oracle.prologue import l2_normalize, _f64")
    exec(compile(text, "dp_mutant.py", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(oracle_lib, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation anchor for %s not found" % name
    mod = _load_mutant(src.replace(old, new, 1))
    for _, fn in ALL_PINS:
        try:
            fn(mod)
        except (AssertionError, ValueError, IndexError, UnboundLocalError, NameError):
            return
    pytest.fail("no pin catches mutant %s" % name)


def test_unmutated_copy_passes(oracle_lib):
    mod = _load_mutant(open(SRC).read())
    for _, fn in ALL_PINS:
        fn(mod)
