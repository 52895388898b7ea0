"""Parity at the full workload sizes, on every unit, in every gate regime.

Each of the four benchmark-sized workloads runs once on the GPU through the C ABI, in the launch
configuration the benchmark times, and the fp64 oracle runs over the whole of it (every (sequence
or segment, head) unit; for decode every sequence at every step). The workload gates decay by
about e^-7 per token, which erases the carried state within a few tokens, so each workload is also
run with the slow-decay regimes the method's own self-test uses: log alpha = 0 (pure delta rule),
alpha ~ U(0.5, 1) and log alpha ~ -U(0, 0.05). There the initial state, the chunk-to-chunk carry
and the far off-diagonal terms of every chunk decide the result.

bf16 outputs are checked over the whole tensor, over every 64-token block of every unit and over
the rows that end a chunk; final states over the whole tensor and per unit (helpers in _parity).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_70_amd import inputs
from tests._parity import (BF16_REL, check, check_bf16_detailed, check_states, gpu_np, rel_fro,
                           segments)

pytestmark = pytest.mark.gpu

REGIMES = ["config", "zero", "p5", "slow"]


@pytest.fixture(scope="module")
def gdr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_70_amd import binding
    binding.lib()  # raises if the library is missing: there is no fallback
    return binding


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dev(case):
    d = lambda t: None if t is None else t.cuda()
    return d(case.q), d(case.k), d(case.v), d(case.log_alpha), d(case.beta), d(case.h0), d(case.cu_seqlens)


@pytest.mark.parametrize("regime", REGIMES)
def test_workload1_every_unit(gdr, regime):
    """B4 H16 T4096 d128 bf16, chunk 64, h0 ~ 0.1 N(0, 1), post-write read: all 64 units."""
    case = inputs.workload1(regime=regime)
    _say("workload1 every unit, regime=%s" % regime)
    q, k, v, la, b, h0, _ = _dev(case)
    out, hT = gdr.chunk_fwd(q, k, v, la, b, h0, None, chunk=64)
    torch.cuda.synchronize()
    o, h = gpu_np(out), gpu_np(hT)
    ro, rh = oracle.scan(case.q, case.k, case.v, case.log_alpha, case.beta, case.h0)
    segs = segments(o.shape, None)
    eo = check_bf16_detailed(o, ro, segs, "workload1 o")
    eh = check_states(h, rh, "workload1 hT")
    _say("  o: whole %.2e, worst block %.2e, chunk-last rows %.2e; hT: whole %.2e, worst unit %.2e"
         % (eo + eh))


@pytest.mark.parametrize("regime", REGIMES)
def test_workload2_every_segment(gdr, regime):
    """8 packed segments of U{512..8192} tokens, H32 d128 bf16, per-segment h0: all 256 units."""
    case = inputs.workload2(regime=regime)
    _say("workload2 every segment, regime=%s, lengths %s" % (regime, np.diff(case.cu_seqlens.numpy()).tolist()))
    q, k, v, la, b, h0, cu = _dev(case)
    out, hT = gdr.chunk_fwd(q, k, v, la, b, h0, cu, chunk=64)
    torch.cuda.synchronize()
    o, h = gpu_np(out), gpu_np(hT)
    ro, rh = oracle.scan(case.q, case.k, case.v, case.log_alpha, case.beta, case.h0, case.cu_seqlens)
    segs = segments(o.shape, case.cu_seqlens)
    eo = check_bf16_detailed(o, ro, segs, "workload2 o")
    eh = check_states(h, rh, "workload2 hT")
    _say("  o: whole %.2e, worst block %.2e, chunk-last rows %.2e; hT: whole %.2e, worst unit %.2e"
         % (eo + eh))


@pytest.mark.parametrize("regime", REGIMES)
def test_workload4_every_segment(gdr, regime):
    """4 x 4096 packed, H16 d128 bf16: forward pre-write scan plus the in-segment reversed
    pre-write scan with its own gates, summed per token (the bidirectional entry point)."""
    case = inputs.workload4(regime=regime)
    _say("workload4 every segment, regime=%s" % regime)
    q, k, v, la, b, _, cu = _dev(case)
    la_b, b_b = case.extra["log_alpha_bwd"].cuda(), case.extra["beta_bwd"].cuda()
    out, _, _ = gdr.chunk_fwd_bidir(q, k, v, la, b, la_b, b_b, None, None, cu, chunk=64, read="pre",
                                    want_state=False)
    torch.cuda.synchronize()
    o = gpu_np(out)
    rf, _ = oracle.scan(case.q, case.k, case.v, case.log_alpha, case.beta, None, case.cu_seqlens,
                        read="pre", want_state=False)
    rb, _ = oracle.scan(case.q, case.k, case.v, case.extra["log_alpha_bwd"], case.extra["beta_bwd"], None,
                        case.cu_seqlens, read="pre", reverse=True, want_state=False)
    segs = segments(o.shape, case.cu_seqlens)
    # the sum is checked on both scans' chunk grids
    e = check_bf16_detailed(o, rf + rb, segs, "workload4 o", reverse_grids=(False, True))
    _say("  o: whole %.2e, worst block %.2e, chunk-last rows %.2e" % e)


@pytest.mark.parametrize("regime", REGIMES)
def test_workload3_every_sequence(gdr, regime):
    """Decode: 256 sequences, 16 key heads -> 32 value heads, d128, fp32 state, 64 consecutive
    steps in place. Every sequence's output at every step, and every state after steps 1, 32
    and 64, against the oracle (the oracle runs the 64 tokens as one scan per (sequence, head),
    which equals 64 decode steps exactly in fp64)."""
    dc = inputs.workload3(regime=regime)
    steps, N = dc.q.shape[0], dc.q.shape[1]
    _say("workload3 every sequence, regime=%s" % regime)
    state = dc.state.cuda()
    outs, saved = [], {}
    for s in range(steps):
        args = [t[s].cuda() for t in (dc.q, dc.k, dc.v, dc.log_alpha, dc.beta)]
        o, state = gdr.decode_step(*args, state, state_out=state)
        outs.append(o)
        if s + 1 in (1, 32, 64):
            saved[s + 1] = state.clone()
    torch.cuda.synchronize()
    o_gpu = gpu_np(torch.stack(outs, dim=0))  # [steps, N, Hv, dv]
    # tokens as a scan per (sequence, head): [steps, N, H, d] -> [N, H, steps, d]
    tq = lambda t: t.permute(1, 2, 0, 3).contiguous()
    tg = lambda t: t.permute(1, 2, 0).contiguous()
    ref_o = []
    ref_state = dc.state
    span = {1: (0, 1), 32: (1, 32), 64: (32, 64)}
    for upto in (1, 32, 64):
        a, e = span[upto]
        sl = lambda t: t[a:e]
        ro, rs = oracle.scan(tq(sl(dc.q)), tq(sl(dc.k)), tq(sl(dc.v)), tg(sl(dc.log_alpha)), tg(sl(dc.beta)),
                             ref_state)
        ref_o.append(ro)
        ref_state = rs
        g = gpu_np(saved[upto])
        eh = check_states(g, rs, "decode state after step %d" % upto)
        _say("  state after step %d: whole %.2e, worst head %.2e" % ((upto,) + eh))
    ro = np.concatenate(ref_o, axis=2).transpose(2, 0, 1, 3)  # [steps, N, Hv, dv]
    worst_step, worst_vec = 0.0, 0.0
    for s in range(steps):
        worst_step = max(worst_step, check(o_gpu[s], ro[s], torch.bfloat16, "decode o step %d" % (s + 1)))
    # each (step, sequence, head) output vector on its own
    num = np.sqrt(np.sum((o_gpu - ro) ** 2, axis=-1))
    den = np.sqrt(np.sum(ro ** 2, axis=-1))
    err = num / np.maximum(den, 1e-30)
    i = np.unravel_index(int(np.argmax(err)), err.shape)
    assert err[i] <= BF16_REL, "decode o (step, seq, head) %s rel err %.3e" % (i, err[i])
    worst_vec = float(err[i])
    _say("  o: worst step %.2e, worst (step, sequence, head) vector %.2e" % (worst_step, worst_vec))
    assert rel_fro(o_gpu, ro) <= BF16_REL
