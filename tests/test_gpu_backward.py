"""Parity of the backward (``gdr_chunk_bwd``) with the fp64 oracle ``oracle.backward`` (reverse-mode
derivative of the per-token recurrence, pinned by finite differences of the C oracle).

The kernel computes in fp32 throughout (the inputs, bf16 or fp32, are read as they are; the
oracle sees the same rounded inputs), so every gradient is held to a relative Frobenius error of
1e-4 against the oracle, per tensor."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from gated_delta_rule_70_amd import inputs
from oracle import backward as bw

pytestmark = pytest.mark.gpu

REL = 1e-4
NAMES = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dh0")


@pytest.fixture(scope="module")
def gdr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_70_amd import binding
    binding.lib()
    return binding


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check(x, ref, what):
    x = np.asarray(x, dtype=np.float64)
    assert np.all(np.isfinite(x)), "%s: non-finite values" % what
    e = float(np.linalg.norm(x - ref)) / max(float(np.linalg.norm(ref)), 1e-30)
    assert e <= REL, "%s: rel Frobenius err %.3e > %.1e" % (what, e, REL)
    return e


def _upstream(case, seed, S):
    g = torch.Generator().manual_seed(seed)
    B, Hv, T, dv = case.v.shape
    dk = case.q.shape[3]
    dout = torch.randn(B, Hv, T, dv, generator=g).to(case.v.dtype)
    dhT = torch.randn(S, Hv, dk, dv, generator=g)
    return dout, dhT


def _run_and_check(gdr, c, dout, dhT, read, reverse, what, units=None):
    d = lambda t: None if t is None else t.cuda()
    got = gdr.chunk_bwd(d(c.q), d(c.k), d(c.v), d(c.log_alpha), d(c.beta), d(dout), d(c.h0), d(c.cu_seqlens),
                        d(dhT), read=read, reverse=reverse)
    torch.cuda.synchronize()
    got = [t.double().cpu().numpy() for t in got]
    if units is None:
        ref = bw.grads(c.q, c.k, c.v, c.log_alpha, c.beta, c.h0, c.cu_seqlens, dout, dhT, read=read, reverse=reverse)
        for n, x, r in zip(NAMES, got, ref):
            check(x, r, "%s %s" % (what, n))
        return
    for (bi, h) in units:  # one (sequence, head) at a time, Hk = Hv
        sl = lambda t: None if t is None else t[bi:bi + 1, h:h + 1]
        ref = bw.grads(sl(c.q), sl(c.k), sl(c.v), sl(c.log_alpha), sl(c.beta), sl(c.h0), None, sl(dout), sl(dhT),
                       read=read, reverse=reverse)
        for n, x, r in zip(NAMES, got, ref):
            check(x[bi:bi + 1, h:h + 1], r, "%s %s (%d, %d)" % (what, n, bi, h))


CASES = [
    dict(B=2, T=70, Hk=2, Hv=2, dk=64, dv=64, dtype=torch.float32),
    dict(B=1, T=100, Hk=1, Hv=2, dk=128, dv=64, dtype=torch.float32),
    dict(B=1, T=65, Hk=2, Hv=4, dk=64, dv=128, dtype=torch.bfloat16),
    dict(B=2, T=45, Hk=1, Hv=1, dk=128, dv=128, dtype=torch.bfloat16),
    dict(B=1, T=40, Hk=1, Hv=1, dk=64, dv=96, dtype=torch.float32),
]


def _ids(c):
    return "B%d-T%d-Hk%d-Hv%d-dk%d-dv%d-%s" % (c["B"], c["T"], c["Hk"], c["Hv"], c["dk"], c["dv"],
                                               str(c["dtype"]).split(".")[-1])


@pytest.mark.parametrize("cfg", CASES, ids=_ids)
@pytest.mark.parametrize("regime", ["config", "slow"])
@pytest.mark.parametrize("read", ["post", "pre"])
def test_parity(gdr, cfg, regime, read):
    _say("backward %s %s %s" % (_ids(cfg), regime, read))
    c = inputs.chunk_case(**cfg, seed=3, h0_std=0.5, regime=regime)
    dout, dhT = _upstream(c, 4, cfg["B"])
    _run_and_check(gdr, c, dout, dhT, read, False, "%s %s" % (regime, read))


@pytest.mark.parametrize("reverse", [False, True])
def test_varlen_reverse(gdr, reverse):
    lengths = [0, 1, 31, 32, 33, 64, 90]
    _say("backward varlen reverse=%s" % reverse)
    c = inputs.chunk_case(Hk=1, Hv=2, dk=64, dv=64, dtype=torch.float32, seed=13, h0_std=0.5, lengths=lengths,
                          regime="slow")
    dout, dhT = _upstream(c, 14, len(lengths))
    for read in ("post", "pre"):
        _run_and_check(gdr, c, dout, dhT, read, reverse, "varlen %s" % read)


def test_no_h0_no_dhT(gdr):
    _say("backward without h0 and dhT")
    c = inputs.chunk_case(B=1, T=50, Hk=2, Hv=2, dk=64, dv=64, dtype=torch.float32, seed=23, h0_std=0.0, regime="p5")
    dout, _ = _upstream(c, 24, 1)
    _run_and_check(gdr, c, dout, None, "post", False, "no h0/dhT")


def test_full_size_sampled(gdr):
    # B4 H16 T4096 d128 bf16 (the main forward workload): two whole (sequence, head) pairs
    _say("backward full size B4 H16 T4096 d128")
    c = inputs.workload1(regime="slow")
    dout, dhT = _upstream(c, 34, 4)
    _run_and_check(gdr, c, dout, dhT, "post", False, "full", units=((0, 3), (3, 14)))


@pytest.mark.parametrize("shape", ["gqa-packed", "full"])
def test_deterministic(gdr, shape):
    # every gradient is the same bits on a second call: the column slices' and value heads' shares
    # are added in a fixed order, with no float atomics; the workspace is filled with other bytes
    # between the calls so that nothing left from the first call can carry over
    _say("backward determinism %s" % shape)
    if shape == "full":
        c = inputs.workload1(regime="slow")
        dout, dhT = _upstream(c, 44, 4)
    else:
        c = inputs.chunk_case(Hk=2, Hv=4, dk=128, dv=128, dtype=torch.bfloat16, seed=45, h0_std=0.5,
                              lengths=[100, 0, 33, 257], regime="p5")
        dout, dhT = _upstream(c, 46, 4)
    d = lambda t: None if t is None else t.cuda()
    B, Hk, T, dk = c.q.shape
    Hv, dv = c.v.shape[1], c.v.shape[3]
    S = 0 if c.cu_seqlens is None else c.cu_seqlens.numel() - 1
    need = gdr.chunk_bwd_workspace_bytes(B, T, Hk, Hv, dk, dv, S, c.q.dtype)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    args = (d(c.q), d(c.k), d(c.v), d(c.log_alpha), d(c.beta), d(dout), d(c.h0), d(c.cu_seqlens), d(dhT))
    first = gdr.chunk_bwd(*args, workspace=ws)
    ws.fill_(0x5a)
    second = gdr.chunk_bwd(*args, workspace=ws)
    torch.cuda.synchronize()
    for n, x, y in zip(NAMES, first, second):
        assert torch.equal(x, y), "%s differs between two calls" % n


EDGE = [
    dict(B=1, T=130, Hk=1, Hv=1, dk=64, dv=256, dtype=torch.bfloat16),   # the widest dv: 8 column slices
    dict(B=1, T=70, Hk=1, Hv=2, dk=128, dv=256, dtype=torch.float32),    # GQA at d_k 128, d_v 256
    dict(B=3, T=64, Hk=2, Hv=2, dk=64, dv=32, dtype=torch.bfloat16),     # one whole chunk, one slice
]


@pytest.mark.parametrize("cfg", EDGE, ids=_ids)
def test_edge_shapes(gdr, cfg):
    _say("backward edge shape %s" % _ids(cfg))
    c = inputs.chunk_case(**cfg, seed=51, h0_std=0.5, regime="slow")
    dout, dhT = _upstream(c, 52, cfg["B"])
    _run_and_check(gdr, c, dout, dhT, "post", False, "edge")


@pytest.mark.parametrize("packed", [False, True])
def test_no_tokens(gdr, packed):
    # no token at all (T = 0, or packed segments that are all empty): nothing but dh0 is written,
    # and the adjoint of h0 is dhT itself
    _say("backward with no tokens, packed=%s" % packed)
    if packed:
        c = inputs.chunk_case(Hk=1, Hv=2, dk=64, dv=64, dtype=torch.bfloat16, seed=61, h0_std=0.5, lengths=[0, 0, 0])
        S = 3
    else:
        c = inputs.chunk_case(B=2, T=0, Hk=1, Hv=2, dk=64, dv=64, dtype=torch.bfloat16, seed=61, h0_std=0.5)
        S = 2
    dout, dhT = _upstream(c, 62, S)
    d = lambda t: None if t is None else t.cuda()
    got = gdr.chunk_bwd(d(c.q), d(c.k), d(c.v), d(c.log_alpha), d(c.beta), d(dout), d(c.h0), d(c.cu_seqlens), d(dhT))
    torch.cuda.synchronize()
    for n, x in zip(NAMES[:5], got[:5]):
        assert x.numel() == 0, "%s has %d elements" % (n, x.numel())
    assert torch.equal(got[5].cpu(), dhT), "dh0 differs from dhT"
