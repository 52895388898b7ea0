"""Parity of the HIP library (called through its C ABI) with the fp64 CPU oracle.

Tolerances: fp32 inputs, max abs error <= 2e-4; bf16 inputs (fp32 gates and state),
relative Frobenius error <= 2e-2, each measured over the whole compared tensor in fp64.
The oracle consumes the very same (rounded) input bytes, upcast exactly to fp64.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_70_amd import inputs

pytestmark = pytest.mark.gpu

FP32_ABS = 2e-4
BF16_REL = 2e-2


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


def max_abs(x, ref):
    x = np.asarray(x, dtype=np.float64)
    return float(np.max(np.abs(x - ref))) if x.size else 0.0


def rel_fro(x, ref):
    x = np.asarray(x, dtype=np.float64)
    den = float(np.linalg.norm(ref))
    return float(np.linalg.norm(x - ref)) / max(den, 1e-30)


def check(x, ref, dtype, what):
    if dtype == torch.float32:
        e = max_abs(x, ref)
        assert e <= FP32_ABS, "%s: max abs err %.3e > %.1e" % (what, e, FP32_ABS)
    else:
        e = rel_fro(x, ref)
        assert e <= BF16_REL, "%s: rel Frobenius err %.3e > %.1e" % (what, e, BF16_REL)
    return e


def to_dev(case):
    d = lambda t: None if t is None else t.cuda()
    return d(case.q), d(case.k), d(case.v), d(case.log_alpha), d(case.beta), d(case.h0), d(case.cu_seqlens)


def gpu_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


# ---------------------------------------------------------------- matrix-core layouts

def test_selftest_mfma_layouts(gdr):
    g = torch.Generator().manual_seed(0)
    a = torch.randn(16, 32, generator=g)
    b = torch.randn(32, 16, generator=g)
    d = gdr.selftest_mfma(a.cuda(), b.cuda()).cpu().double()
    ab, bb = a.bfloat16().double(), b.bfloat16().double()
    assert torch.allclose(d[0], ab @ bb, atol=1e-4), "bf16 16x16x32 layout"
    assert torch.allclose(d[1], a.double() @ b.double(), atol=1e-4), "fp32 16x16x4 layout"
    assert torch.allclose(d[2], ab[:, :16] @ bb[:16], atol=1e-4), "bf16 16x16x16 layout"


# ---------------------------------------------------------------- decode step

DECODE_CASES = [
    dict(N=3, Hk=2, Hv=4, dk=128, dv=128, dtype=torch.bfloat16, read="post"),
    dict(N=3, Hk=2, Hv=4, dk=128, dv=128, dtype=torch.float32, read="post"),
    dict(N=2, Hk=1, Hv=3, dk=64, dv=128, dtype=torch.float32, read="pre"),
    dict(N=5, Hk=4, Hv=4, dk=128, dv=64, dtype=torch.bfloat16, read="pre"),
    dict(N=1, Hk=2, Hv=2, dk=64, dv=64, dtype=torch.float32, read="post"),
]


@pytest.mark.parametrize("cfg", DECODE_CASES, ids=lambda c: "N%d-Hk%d-Hv%d-dk%d-dv%d-%s-%s" % (
    c["N"], c["Hk"], c["Hv"], c["dk"], c["dv"], str(c["dtype"]).split(".")[-1], c["read"]))
@pytest.mark.parametrize("inplace", [False, True])
def test_decode_step_parity(gdr, cfg, inplace):
    cfg = dict(cfg)
    read = cfg.pop("read")
    dc = inputs.decode_case(steps=4, seed=7, state_std=0.3, regime="p5", **cfg)
    _say("decode %s read=%s inplace=%s" % (cfg, read, inplace))
    state = dc.state.cuda()
    ref_state = dc.state.double().numpy()
    for s in range(dc.q.shape[0]):
        args = [t[s].cuda() for t in (dc.q, dc.k, dc.v, dc.log_alpha, dc.beta)]
        o, new_state = gdr.decode_step(*args, state, state_out=state if inplace else None, read=read)
        if inplace:
            assert new_state.data_ptr() == state.data_ptr()
        state = new_state
        ref_o, ref_state = oracle.decode(dc.q[s], dc.k[s], dc.v[s], dc.log_alpha[s], dc.beta[s],
                                         ref_state, read=read)
        torch.cuda.synchronize()
        check(gpu_np(o), ref_o, cfg["dtype"], "decode o step %d" % s)
        check(gpu_np(state), ref_state, torch.float32 if cfg["dtype"] == torch.float32 else torch.bfloat16,
              "decode state step %d" % s)


# ---------------------------------------------------------------- chunked forward

def run_chunk(gdr, case, chunk, read="post", reverse=False):
    q, k, v, la, b, h0, cu = to_dev(case)
    out, hT = gdr.chunk_fwd(q, k, v, la, b, h0, cu, chunk=chunk, read=read, reverse=reverse)
    torch.cuda.synchronize()
    return gpu_np(out), gpu_np(hT)


def oracle_chunk(case, read="post", reverse=False):
    return oracle.scan(case.q, case.k, case.v, case.log_alpha, case.beta, case.h0, case.cu_seqlens,
                       read=read, reverse=reverse)


def test_workload0_fp32(gdr):
    """B1 H2 T256 d64 fp32, chunk 64, zero h0, post-write read: max abs <= 2e-4."""
    case = inputs.workload0()
    o, hT = run_chunk(gdr, case, 64)
    ro, rh = oracle_chunk(case)
    e1 = check(o, ro, torch.float32, "workload0 o")
    e2 = check(hT, rh, torch.float32, "workload0 hT")
    _say("workload0: max abs o %.2e hT %.2e" % (e1, e2))


SMALL = [
    # (dtype, dk, dv, Hk, Hv, B, T, chunk)
    (torch.float32, 64, 64, 2, 2, 1, 256, 64),
    (torch.float32, 64, 64, 1, 2, 2, 300, 32),
    (torch.float32, 128, 128, 2, 2, 1, 200, 16),
    (torch.float32, 128, 96, 1, 1, 1, 77, 64),
    (torch.bfloat16, 128, 128, 2, 4, 2, 300, 64),
    (torch.bfloat16, 128, 128, 1, 2, 1, 333, 32),
    (torch.bfloat16, 64, 128, 2, 2, 1, 150, 16),
    (torch.bfloat16, 128, 64, 2, 2, 1, 129, 64),
    (torch.bfloat16, 128, 256, 1, 1, 1, 100, 64),
    (torch.bfloat16, 128, 96, 1, 1, 1, 77, 64),
    # long enough (five chunks and more) for the fast kernel's L2 touches, with one, three and
    # eight column tiles: each K/Q quarter touched by one tile, by wrapped quarter slots, or by
    # the first four tiles only
    (torch.bfloat16, 128, 32, 2, 2, 1, 333, 64),
    (torch.bfloat16, 128, 96, 1, 1, 2, 400, 64),
    (torch.bfloat16, 128, 256, 1, 2, 1, 390, 64),
]


def _small_id(c):
    return "%s-dk%d-dv%d-Hk%d-Hv%d-B%d-T%d-C%d" % ((str(c[0]).split(".")[-1],) + c[1:])


@pytest.mark.parametrize("regime", ["config", "zero", "p5", "slow"])
@pytest.mark.parametrize("read", ["post", "pre"])
@pytest.mark.parametrize("shape", SMALL, ids=_small_id)
def test_chunk_fwd_small(gdr, shape, read, regime):
    dtype, dk, dv, Hk, Hv, B, T, C = shape
    case = inputs.chunk_case(B=B, T=T, Hk=Hk, Hv=Hv, dk=dk, dv=dv, dtype=dtype, seed=11,
                             h0_std=0.1, regime=regime)
    _say("chunk %s read=%s regime=%s" % (_small_id(shape), read, regime))
    o, hT = run_chunk(gdr, case, C, read=read)
    ro, rh = oracle_chunk(case, read=read)
    check(o, ro, dtype, "o")
    check(hT, rh, dtype, "hT")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("read", ["post", "pre"])
def test_chunk_fwd_reverse_and_varlen(gdr, dtype, read):
    """Packed segments (with an empty one and ragged tails), scanned backwards."""
    lengths = [70, 0, 129, 64, 1, 200]
    case = inputs.chunk_case(Hk=2, Hv=2, dk=128, dv=128, dtype=dtype, seed=12, h0_std=0.1,
                             regime="p5", lengths=lengths)
    for rev in (False, True):
        _say("varlen %s read=%s reverse=%s" % (dtype, read, rev))
        o, hT = run_chunk(gdr, case, 64, read=read, reverse=rev)
        ro, rh = oracle_chunk(case, read=read, reverse=rev)
        check(o, ro, dtype, "varlen o")
        check(hT, rh, dtype, "varlen hT")


@pytest.mark.parametrize("nseg", [40, 128, 129, 2100])
def test_chunk_fwd_many_segments(gdr, nseg):
    """Many packed segments of mixed lengths (the fast kernel ranks up to 128 of them by
    length; beyond that it keeps their order)."""
    g = torch.Generator().manual_seed(nseg)
    hi = 200 if nseg < 100 else 4
    lengths = torch.randint(0, hi, (nseg,), generator=g).tolist()
    case = inputs.chunk_case(Hk=1, Hv=2, dk=128, dv=64, dtype=torch.bfloat16, seed=15, h0_std=0.1,
                             regime="slow", lengths=lengths)
    _say("many segments: %d, T=%d" % (nseg, case.q.shape[2]))
    o, hT = run_chunk(gdr, case, 64)
    ro, rh = oracle_chunk(case)
    check(o, ro, torch.bfloat16, "many segments o")
    check(hT, rh, torch.bfloat16, "many segments hT")


def test_chunk_sizes_agree(gdr):
    """Chunk 16, 32 and 64 give the same result up to rounding (fp32 inputs, slow decay so
    the carried state matters)."""
    case = inputs.chunk_case(B=1, T=500, Hk=2, dk=128, dv=128, dtype=torch.float32, seed=13,
                             h0_std=0.1, regime="slow")
    outs = [run_chunk(gdr, case, C) for C in (16, 32, 64)]
    for o, h in outs[1:]:
        assert max_abs(o, outs[0][0]) <= FP32_ABS and max_abs(h, outs[0][1]) <= FP32_ABS


def test_chunk_fwd_empty_and_accumulate(gdr):
    # T == 0: only hT (== h0) is written
    case = inputs.chunk_case(B=2, T=0, Hk=1, dk=64, dv=64, dtype=torch.float32, seed=14, h0_std=0.1)
    o, hT = run_chunk(gdr, case, 64)
    assert o.size == 0 and np.array_equal(hT, case.h0.numpy())
    # accumulate: out += o
    case = inputs.chunk_case(B=1, T=130, Hk=1, dk=64, dv=64, dtype=torch.float32, seed=15, h0_std=0.1)
    q, k, v, la, b, h0, cu = to_dev(case)
    base = torch.randn(1, 1, 130, 64, generator=torch.Generator().manual_seed(3))
    out = base.cuda()
    gdr.chunk_fwd(q, k, v, la, b, h0, chunk=64, read="pre", reverse=True, out=out, accumulate=True)
    torch.cuda.synchronize()
    ro, _ = oracle_chunk(case, read="pre", reverse=True)
    check(gpu_np(out), ro + base.double().numpy(), torch.float32, "accumulate")


def test_chunk_fwd_inplace_state_and_resume(gdr):
    """hT may be h0 itself; chunk_fwd(T1 || T2) == chunk_fwd(T2, h0 = hT(T1))."""
    case = inputs.chunk_case(B=2, T=256, Hk=2, dk=128, dv=128, dtype=torch.float32, seed=16,
                             h0_std=0.1, regime="slow")
    q, k, v, la, b, h0, cu = to_dev(case)
    o_full, h_full = gdr.chunk_fwd(q, k, v, la, b, h0, chunk=64)
    cut = 128
    sl = lambda t: t[:, :, :cut].contiguous()
    sr = lambda t: t[:, :, cut:].contiguous()
    state = h0.clone()
    o1, _ = gdr.chunk_fwd(sl(q), sl(k), sl(v), sl(la), sl(b), state, chunk=64, hT=state)
    o2, _ = gdr.chunk_fwd(sr(q), sr(k), sr(v), sr(la), sr(b), state, chunk=64, hT=state)
    torch.cuda.synchronize()
    assert max_abs(gpu_np(torch.cat([o1, o2], dim=2)), gpu_np(o_full)) <= FP32_ABS
    assert max_abs(gpu_np(state), gpu_np(h_full)) <= FP32_ABS


def test_decode_steps_match_chunk_fwd(gdr):
    """64 decode steps from state S == the chunked forward over those tokens with h0 = S."""
    N, Hk, Hv, d, steps = 2, 1, 2, 128, 64
    dc = inputs.decode_case(N=N, Hk=Hk, Hv=Hv, dk=d, dv=d, steps=steps, dtype=torch.float32,
                            seed=17, state_std=0.1, regime="slow")
    state = dc.state.cuda()
    outs = []
    for s in range(steps):
        o, state = gdr.decode_step(*(t[s].cuda() for t in (dc.q, dc.k, dc.v, dc.log_alpha, dc.beta)),
                                   state)
        outs.append(o)
    # [steps, N, H, d] -> [N, H, steps, d]
    q = dc.q.permute(1, 2, 0, 3).contiguous().cuda()
    k = dc.k.permute(1, 2, 0, 3).contiguous().cuda()
    v = dc.v.permute(1, 2, 0, 3).contiguous().cuda()
    la = dc.log_alpha.permute(1, 2, 0).contiguous().cuda()
    b = dc.beta.permute(1, 2, 0).contiguous().cuda()
    oc, hc = gdr.chunk_fwd(q, k, v, la, b, dc.state.cuda(), chunk=64)
    torch.cuda.synchronize()
    od = torch.stack(outs, dim=2)
    assert max_abs(gpu_np(od), gpu_np(oc)) <= FP32_ABS
    assert max_abs(gpu_np(state), gpu_np(hc)) <= FP32_ABS


def test_chunk_fwd_deterministic(gdr):
    case = inputs.workload1(T=512)
    q, k, v, la, b, h0, cu = to_dev(case)
    o1, h1 = gdr.chunk_fwd(q, k, v, la, b, h0, chunk=64)
    o2, h2 = gdr.chunk_fwd(q, k, v, la, b, h0, chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


# The full workload sizes (every unit, every gate regime, per-block and chunk-last-row checks) are
# in test_gpu_full_size.py.
