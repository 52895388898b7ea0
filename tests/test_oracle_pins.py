"""Pins of the CPU oracle to facts fixed by the pages and by mathematics.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with a
value it does not compute itself: an exact-rational brute force written as a
product of transition matrices, a hand-worked example, closed forms (beta = 0,
orthonormal keys), an autograd gradient step, and structural identities
(linearity, pre/post shift, segment independence, reversal, resume, decode vs
scan, key-head sharing). ``tests/test_oracle_mutants.py`` re-runs these pins
against deliberately broken copies of the oracle to show that each plausible
mistake is caught.
"""
from __future__ import annotations

import json
import math
import os
import random
from fractions import Fraction as F

import numpy as np
import pytest
import torch

import oracle
from oracle import chunked as chunked_oracle
from tests import _brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, "%s: max abs err %.3e > %.1e (scale %.3g)" % (what, err, tol, scale)


# --------------------------------------------------------------------------- random tiny rationals

def _rat(rng, lo=-4, hi=4, dens=(1, 2, 3, 4, 5)):
    return F(rng.randint(lo, hi), rng.choice(dens))


def _tiny_case(seed, T, dk, dv, Hk=1, Hv=1, with_h0=True):
    rng = random.Random(seed)
    q = [[[_rat(rng) for _ in range(dk)] for _ in range(T)] for _ in range(Hk)]
    k = [[[_rat(rng) for _ in range(dk)] for _ in range(T)] for _ in range(Hk)]
    v = [[[_rat(rng) for _ in range(dv)] for _ in range(T)] for _ in range(Hv)]
    alpha = [[rng.choice([F(1), F(1, 2), F(3, 4), F(2, 3), F(9, 10)]) for _ in range(T)]
             for _ in range(Hv)]
    beta = [[rng.choice([F(1, 2), F(1, 3), F(1), F(3, 4), F(1, 5), F(0)]) for _ in range(T)]
            for _ in range(Hv)]
    h0 = [[[_rat(rng) if with_h0 else F(0) for _ in range(dv)] for _ in range(dk)]
          for _ in range(Hv)]
    return q, k, v, alpha, beta, h0


def _np(x):
    return np.array([[float(e) for e in row] for row in x]) if isinstance(x[0], list) \
        else np.array([float(e) for e in x])


def _to_oracle(q, k, v, alpha, beta):
    Q = np.stack([_np(h) for h in q])[None]
    K = np.stack([_np(h) for h in k])[None]
    V = np.stack([_np(h) for h in v])[None]
    LA = np.array([[math.log(float(a)) for a in h] for h in alpha])[None]
    B = np.array([[float(b) for b in h] for h in beta])[None]
    return Q, K, V, LA, B


def pin_brute_force(orc, seed=0, T=6, dk=3, dv=2, Hk=1, Hv=2, read="post", reverse=False,
                    lengths=None):
    """Oracle == exact rational transition-matrix expansion (T <= 8)."""
    if lengths is None:
        lengths = [T]
    T = sum(lengths)
    q, k, v, alpha, beta, h0 = _tiny_case(seed, T, dk, dv, Hk, Hv)
    nseq = len(lengths)
    h0s = [[_tiny_case(seed + 100 + s, 1, dk, dv, 1, Hv)[5][h] for h in range(Hv)]
           for s in range(nseq)]
    Q, K, V, LA, B = _to_oracle(q, k, v, alpha, beta)
    H0 = np.array([[_np(h0s[s][h]) for h in range(Hv)] for s in range(nseq)])
    cu = np.array([0] + list(np.cumsum(lengths)), dtype=np.int64) if nseq > 1 else None
    if cu is None:
        H0 = H0.reshape(1, Hv, dk, dv)
    o, hT = orc.scan(Q, K, V, LA, B, H0, cu, read=read, reverse=reverse)
    g = Hv // Hk
    starts = [0] + list(np.cumsum(lengths))
    for s in range(nseq):
        toks = list(range(starts[s], starts[s + 1]))
        order = toks[::-1] if reverse else toks
        for h in range(Hv):
            kh = h // g
            ref_o, ref_H = _brute.run(order, q[kh], k[kh], v[h], alpha[h], beta[h], h0s[s][h],
                                      read_mode=read)
            for t in toks:
                _close(o[0, h, t], [float(x) for x in ref_o[t]], 1e-12,
                       "brute o (seg %d head %d tok %d %s rev=%s)" % (s, h, t, read, reverse))
            _close(hT[s, h], [[float(x) for x in r] for r in ref_H], 1e-12,
                   "brute hT (seg %d head %d)" % (s, h))


def pin_hand_example(orc):
    """Oracle == the hand-worked T=2 example in tests/golden/hand_T2.json."""
    with open(os.path.join(GOLDEN, "hand_T2.json")) as f:
        g = json.load(f)
    inp, exp = g["inputs"], g["expected"]
    fr = lambda rows: [[F(x) for x in r] for r in rows]
    Q, K, V, LA, B = _to_oracle([fr(inp["q"])], [fr(inp["k"])], [fr(inp["v"])],
                                [[F(a) for a in inp["alpha"]]], [[F(b) for b in inp["beta"]]])
    for mode in ("post", "pre"):
        o, hT = orc.scan(Q, K, V, LA, B, None, None, read=mode)
        _close(o[0, 0], [[float(F(x)) for x in r] for r in exp["o_" + mode]], 1e-14, "hand o " + mode)
        _close(hT[0, 0], [[float(F(x)) for x in r] for r in exp["hT"]], 1e-14, "hand hT " + mode)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _float_case(seed, B=1, Hk=2, Hv=2, T=40, dk=8, dv=6, decay="p5"):
    rng = np.random.default_rng(seed)
    q = _unit(_rand(rng, B, Hk, T, dk))
    k = _unit(_rand(rng, B, Hk, T, dk))
    v = _rand(rng, B, Hv, T, dv)
    if decay == "p5":
        la = np.log(rng.uniform(0.5, 1.0, (B, Hv, T)))
    elif decay == "zero":
        la = np.zeros((B, Hv, T))
    else:
        la = -rng.uniform(0.0, 3.0, (B, Hv, T))
    beta = rng.uniform(0.0, 1.0, (B, Hv, T))
    h0 = _rand(rng, B, Hv, dk, dv) * 0.5
    return q, k, v, la, beta, h0


def pin_beta_zero(orc):
    """beta = 0: H_T = exp(sum a) H_0 and o_t = exp(sum_{s<=t} a) H_0^T q_t (post), s<t (pre)."""
    q, k, v, la, beta, h0 = _float_case(1, decay="strong")
    beta[:] = 0.0
    for mode in ("post", "pre"):
        o, hT = orc.scan(q, k, v, la, beta, h0, read=mode)
        cs = np.cumsum(la, axis=-1)
        if mode == "pre":
            cs = cs - la
        for h in range(2):
            ref_o = np.exp(cs[0, h])[:, None] * (q[0, h] @ h0[0, h])
            _close(o[0, h], ref_o, 1e-12, "beta=0 o " + mode)
            _close(hT[0, h], np.exp(la[0, h].sum()) * h0[0, h], 1e-12, "beta=0 hT")
    # beta = 0 and alpha = 1: the state is untouched (the "tiny_gdn/fugue.py" page's edge
    # capture relies on a zero key with zero decay leaving the state unchanged)
    la[:] = 0.0
    _, hT = orc.scan(q, k, v, la, beta, h0)
    _close(hT, h0, 0.0, "beta=0, alpha=1 leaves the state")
    beta = np.random.default_rng(2).uniform(0, 1, beta.shape)
    _, hT = orc.scan(q, np.zeros_like(k), v, la, beta, h0)
    _close(hT, h0, 0.0, "k=0, alpha=1 leaves the state")


def pin_gradient_step(orc):
    """alpha = 1 is one gradient step on 1/2 ||H^T k - v||^2 with step beta ("Prizma seq/delta.py",
    module docstring): H <- H - beta * dF/dH, the gradient taken by torch autograd."""
    rng = np.random.default_rng(3)
    dk, dv = 5, 3
    H = rng.standard_normal((dk, dv))
    kk = _unit(rng.standard_normal(dk))
    vv = rng.standard_normal(dv)
    qq = rng.standard_normal(dk)
    b = 0.7
    Ht = torch.tensor(H, requires_grad=True)
    loss = 0.5 * ((Ht.T @ torch.tensor(kk) - torch.tensor(vv)) ** 2).sum()
    loss.backward()
    H_ref = H - b * Ht.grad.numpy()
    o, hT = orc.scan(qq[None, None, None], kk[None, None, None], vv[None, None, None],
                     np.zeros((1, 1, 1)), np.full((1, 1, 1), b), H[None, None])
    _close(hT[0, 0], H_ref, 1e-13, "gradient step state")
    _close(o[0, 0, 0], H_ref.T @ qq, 1e-13, "gradient step read")
    od, sd = orc.decode(qq[None, None], kk[None, None], vv[None, None], np.zeros((1, 1)),
                        np.full((1, 1), b), H[None, None])
    _close(sd[0, 0], H_ref, 1e-13, "gradient step decode state")
    _close(od[0, 0], H_ref.T @ qq, 1e-13, "gradient step decode read")


def pin_orthonormal_retrieval(orc):
    """beta = 1 with orthonormal keys overwrites: H_T^T k_j = exp(sum_{s>j} a_s) v_j."""
    rng = np.random.default_rng(4)
    dk, dv, T = 8, 5, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm[:, :T].T                       # T orthonormal rows
    v = rng.standard_normal((T, dv))
    h0 = rng.standard_normal((dk, dv))
    for decay in ("zero", "strong"):
        la = np.zeros(T) if decay == "zero" else -rng.uniform(0, 1, T)
        o, hT = orc.scan(keys[None, None], keys[None, None], v[None, None], la[None, None],
                         np.ones((1, 1, T)), h0[None, None])
        # post read with q_t = k_t returns v_t exactly, whatever the decay
        _close(o[0, 0], v, 1e-12, "overwrite-and-retrieve read")
        for j in range(T):
            _close(hT[0, 0].T @ keys[j], np.exp(la[j + 1:].sum()) * v[j], 1e-12,
                   "retrieve key %d (%s)" % (j, decay))


def pin_linearity(orc):
    """(o, H_T) is linear in (H_0, V) for fixed K, beta, alpha."""
    q, k, v, la, beta, h0 = _float_case(5)
    _, _, v2, _, _, h02 = _float_case(6)
    c1, c2 = 0.75, -1.25
    o1, s1 = orc.scan(q, k, v, la, beta, h0)
    o2, s2 = orc.scan(q, k, v2, la, beta, h02)
    o3, s3 = orc.scan(q, k, c1 * v + c2 * v2, la, beta, c1 * h0 + c2 * h02)
    _close(o3, c1 * o1 + c2 * o2, 1e-12, "linearity o")
    _close(s3, c1 * s1 + c2 * s2, 1e-12, "linearity state")


def pin_pre_post_shift(orc):
    """Pre-write read == post-write read one token earlier with the next query
    ("tiny_gdn/fugue.py", ``scan``: the query is shifted one step and the output back),
    and the first pre-write read is H_0^T q_0."""
    q, k, v, la, beta, h0 = _float_case(7, decay="p5")
    o_pre, s_pre = orc.scan(q, k, v, la, beta, h0, read="pre")
    q_next = np.concatenate([q[:, :, 1:], q[:, :, -1:]], axis=2)
    o_post, s_post = orc.scan(q_next, k, v, la, beta, h0, read="post")
    _close(o_pre[:, :, 1:], o_post[:, :, :-1], 1e-12, "pre == shifted post")
    _close(o_pre[0, :, 0], np.einsum("hd,hdv->hv", q[0, :, 0], h0[0]), 1e-12, "first pre read")
    _close(s_pre, s_post, 0.0, "state does not depend on the read mode")


def pin_segments_independent(orc):
    """Packed segments == separate calls, each with its own h0 (state resets at boundaries)."""
    rng = np.random.default_rng(8)
    lengths = [5, 0, 17, 9]
    T = sum(lengths)
    q, k, v, la, beta, _ = _float_case(8, T=T)
    h0 = rng.standard_normal((len(lengths), 2, 8, 6))
    cu = np.array([0] + list(np.cumsum(lengths)))
    for mode in ("post", "pre"):
        for rev in (False, True):
            o, hT = orc.scan(q, k, v, la, beta, h0, cu, read=mode, reverse=rev)
            for s, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
                if b == a:
                    _close(hT[s], h0[s], 0.0, "empty segment keeps h0")
                    continue
                os_, hs = orc.scan(q[:, :, a:b], k[:, :, a:b], v[:, :, a:b], la[:, :, a:b],
                                   beta[:, :, a:b], h0[s:s + 1], read=mode, reverse=rev)
                _close(o[:, :, a:b], os_, 1e-13, "segment %d output" % s)
                _close(hT[s], hs[0], 1e-13, "segment %d state" % s)


def pin_reverse_is_flip(orc):
    """Reverse scan == forward scan of the time-flipped sequence, output flipped back."""
    q, k, v, la, beta, h0 = _float_case(9)
    flip = lambda x: np.ascontiguousarray(x[:, :, ::-1])
    for mode in ("post", "pre"):
        o_r, s_r = orc.scan(q, k, v, la, beta, h0, read=mode, reverse=True)
        o_f, s_f = orc.scan(flip(q), flip(k), flip(v), flip(la), flip(beta), h0, read=mode)
        _close(o_r, flip(o_f), 1e-13, "reverse output " + mode)
        _close(s_r, s_f, 1e-13, "reverse state " + mode)


def pin_resume(orc):
    """scan(T1 || T2) == scan(T2) started from the final state of scan(T1)."""
    q, k, v, la, beta, h0 = _float_case(10, T=50)
    cut = 23
    for mode in ("post", "pre"):
        o, s = orc.scan(q, k, v, la, beta, h0, read=mode)
        o1, s1 = orc.scan(q[:, :, :cut], k[:, :, :cut], v[:, :, :cut], la[:, :, :cut],
                          beta[:, :, :cut], h0, read=mode)
        o2, s2 = orc.scan(q[:, :, cut:], k[:, :, cut:], v[:, :, cut:], la[:, :, cut:],
                          beta[:, :, cut:], s1, read=mode)
        _close(np.concatenate([o1, o2], axis=2), o, 1e-13, "resume output")
        _close(s2, s, 1e-13, "resume state")


def pin_decode_matches_scan(orc):
    """T decode steps from state S == one scan over the same T tokens with h0 = S."""
    q, k, v, la, beta, h0 = _float_case(11, B=3, Hk=1, Hv=2, T=12)
    for mode in ("post", "pre"):
        o_scan, s_scan = orc.scan(q, k, v, la, beta, h0, read=mode)
        state = h0.copy()
        for t in range(q.shape[2]):
            o_t, state = orc.decode(q[:, :, t], k[:, :, t], v[:, :, t], la[:, :, t],
                                    beta[:, :, t], state, read=mode)
            _close(o_t, o_scan[:, :, t], 1e-12, "decode step %d %s" % (t, mode))
        _close(state, s_scan, 1e-12, "decode final state " + mode)


def pin_key_head_sharing(orc):
    """Value head j reads key/query head j // (Hv/Hk): equals the run with q, k repeated."""
    q, k, v, la, beta, h0 = _float_case(12, Hk=2, Hv=6)
    o, s = orc.scan(q, k, v, la, beta, h0)
    o2, s2 = orc.scan(np.repeat(q, 3, axis=1), np.repeat(k, 3, axis=1), v, la, beta, h0)
    _close(o, o2, 0.0, "GQA output")
    _close(s, s2, 0.0, "GQA state")
    # decode: same mapping
    od, sd = orc.decode(q[:, :, 0], k[:, :, 0], v[:, :, 0], la[:, :, 0], beta[:, :, 0], h0)
    od2, sd2 = orc.decode(np.repeat(q[:, :, 0], 3, axis=1), np.repeat(k[:, :, 0], 3, axis=1),
                          v[:, :, 0], la[:, :, 0], beta[:, :, 0], h0)
    _close(od, od2, 0.0, "GQA decode output")
    _close(sd, sd2, 0.0, "GQA decode state")


def pin_accumulate(orc):
    """Accumulate mode adds the scan's output to what the buffer already holds."""
    q, k, v, la, beta, h0 = _float_case(13)
    base = np.random.default_rng(13).standard_normal(v.shape)
    o, _ = orc.scan(q, k, v, la, beta, h0, read="pre", reverse=True)
    acc = base.copy()
    orc.scan(q, k, v, la, beta, h0, read="pre", reverse=True, out=acc)
    _close(acc, base + o, 1e-14, "accumulate")


BRUTE_CASES = [
    dict(read="post"),
    dict(read="pre"),
    dict(read="post", reverse=True),
    dict(read="pre", reverse=True, seed=1),
    dict(read="post", lengths=[3, 4], seed=2),
    dict(read="pre", lengths=[2, 0, 5], reverse=True, seed=3),
    dict(read="post", dk=2, dv=4, Hk=2, Hv=4, T=5, seed=4),
]

ALL_PINS = [
    ("hand_example", pin_hand_example),
    ("beta_zero", pin_beta_zero),
    ("gradient_step", pin_gradient_step),
    ("orthonormal_retrieval", pin_orthonormal_retrieval),
    ("linearity", pin_linearity),
    ("pre_post_shift", pin_pre_post_shift),
    ("segments_independent", pin_segments_independent),
    ("reverse_is_flip", pin_reverse_is_flip),
    ("resume", pin_resume),
    ("decode_matches_scan", pin_decode_matches_scan),
    ("key_head_sharing", pin_key_head_sharing),
    ("accumulate", pin_accumulate),
] + [("brute_%d" % i, (lambda orc, c=c: pin_brute_force(orc, **c))) for i, c in
     enumerate(BRUTE_CASES)]


@pytest.mark.parametrize("name,fn", ALL_PINS, ids=[n for n, _ in ALL_PINS])
def test_oracle_pin(oracle_lib, name, fn):
    fn(oracle_lib)


# --------------------------------------------------------------------------- chunked form

def test_neumann_equals_triangular_solve():
    """(I + A)^{-1} == sum_{j<C} (-A)^j for strictly lower A ("Prizma seq/delta.py",
    ``_solve_unit_lower`` fallback), against scipy's triangular solve."""
    rng = np.random.default_rng(20)
    for C in (16, 32, 64):
        A = np.tril(rng.uniform(-0.3, 0.3, (C, C)), -1)
        X = chunked_oracle.neumann_inverse(A)
        ref = chunked_oracle.solve_unit_lower(A, np.eye(C))
        _close(X, ref, 1e-10, "Neumann C=%d" % C)
        _close((np.eye(C) + A) @ X, np.eye(C), 1e-10, "inverse C=%d" % C)


@pytest.mark.parametrize("read", ["post", "pre"])
@pytest.mark.parametrize("decay", ["p5", "strong", "zero"])
def test_chunked_form_equals_recurrence(oracle_lib, read, decay):
    """The exact chunk form reaches the recurrence's result for every chunk size, incl. a
    ragged tail ("sparse-delta-memory layer.py", module docstring: chunk size changes the
    output only through rounding)."""
    q, k, v, la, beta, h0 = _float_case(21, B=2, Hk=1, Hv=2, T=150, dk=12, dv=10, decay=decay)
    o_ref, s_ref = oracle_lib.scan(q, k, v, la, beta, h0, read=read)
    for C in (16, 32, 64):
        o, s = chunked_oracle.chunked(q, k, v, la, beta, h0, chunk=C, read=read)
        _close(o, o_ref, 1e-10, "chunked C=%d o" % C)
        _close(s, s_ref, 1e-10, "chunked C=%d state" % C)


def test_chunked_form_survives_harsh_gates(oracle_lib):
    """Per-token log decay down to about -48 (the workload gates): every exponent stays <= 0,
    so nothing overflows and the result still equals the recurrence."""
    q, k, v, la, beta, h0 = _float_case(22, B=1, Hk=1, Hv=1, T=128, dk=16, dv=8)
    la = -np.random.default_rng(22).uniform(0.0, 48.0, la.shape)
    o_ref, s_ref = oracle_lib.scan(q, k, v, la, beta, h0)
    with np.errstate(over="raise", invalid="raise"):
        o, s = chunked_oracle.chunked(q, k, v, la, beta, h0, chunk=64)
    _close(o, o_ref, 1e-10, "harsh gates o")
    _close(s, s_ref, 1e-10, "harsh gates state")
