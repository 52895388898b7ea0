"""Parity of the GDN-2 kernels (``gdr_gdn2_chunk_fwd``, ``gdr_gdn2_decode_step``) with the fp64
oracle ``oracle.gdn2`` (the per-token recurrence of the "tiny_gdn/fugue.py" page's statement).

Tolerances: fp32 inputs, max abs error <= 2e-4 on outputs and final states; bf16 inputs,
relative Frobenius error <= 2e-2 per tensor (the oracle sees the same bf16-rounded inputs).
The decay regimes exercise both ways a 16-token diagonal block is computed: "page" and "weak"
keep every block on the matrix cores, "strong" sends every block to the exact path, "mixed"
puts both kinds side by side.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from gated_delta_rule_70_amd import inputs
from oracle import gdn2

pytestmark = pytest.mark.gpu

FP32_ABS = 2e-4
BF16_REL = 2e-2


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


def check(x, ref, dtype, what):
    x = np.asarray(x, dtype=np.float64)
    assert np.all(np.isfinite(x)), "%s: non-finite values" % what
    if dtype == torch.float32:
        e = float(np.max(np.abs(x - ref))) if x.size else 0.0
        assert e <= FP32_ABS, "%s: max abs err %.3e > %.1e" % (what, e, FP32_ABS)
    else:
        e = float(np.linalg.norm(x - ref)) / max(float(np.linalg.norm(ref)), 1e-30)
        assert e <= BF16_REL, "%s: rel Frobenius err %.3e > %.1e" % (what, e, BF16_REL)
    return e


def gpu_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _dev(c):
    d = lambda t: None if t is None else t.cuda()
    return [d(t) for t in (c.q, c.k, c.v, c.g, c.b, c.w, c.h0, c.cu_seqlens)]


CHUNK = [
    dict(B=2, T=200, Hk=2, Hv=2, dk=64, dv=64, dtype=torch.float32, chunk=64),
    dict(B=1, T=333, Hk=2, Hv=4, dk=128, dv=64, dtype=torch.bfloat16, chunk=64),
    dict(B=2, T=257, Hk=1, Hv=2, dk=128, dv=128, dtype=torch.bfloat16, chunk=64),
    dict(B=1, T=150, Hk=2, Hv=2, dk=64, dv=32, dtype=torch.bfloat16, chunk=32),
    dict(B=1, T=181, Hk=1, Hv=2, dk=128, dv=96, dtype=torch.float32, chunk=32),
    dict(B=1, T=96, Hk=1, Hv=1, dk=128, dv=64, dtype=torch.float32, chunk=16),
    dict(B=1, T=77, Hk=2, Hv=2, dk=64, dv=64, dtype=torch.bfloat16, chunk=16),
]


def _ids(c):
    return "B%d-T%d-Hk%d-Hv%d-dk%d-dv%d-%s-c%d" % (c["B"], c["T"], c["Hk"], c["Hv"], c["dk"], c["dv"],
                                                 str(c["dtype"]).split(".")[-1], c["chunk"])


def _run(gdr, c, chunk, read="post", reverse=False, l2norm=False, accumulate=None, fused=False, workspace=None):
    q, k, v, g, b, w, h0, cu = _dev(c)
    out = None
    if accumulate is not None:
        out = accumulate.cuda().clone()
    o, hT = gdr.gdn2_chunk_fwd(q, k, v, g, b, w, h0, cu, chunk=chunk, read=read, reverse=reverse,
                               l2norm=l2norm, out=out, accumulate=accumulate is not None, fused=fused,
                               workspace=workspace)
    torch.cuda.synchronize()
    return gpu_np(o), gpu_np(hT)


@pytest.mark.parametrize("cfg", CHUNK, ids=_ids)
@pytest.mark.parametrize("regime", ["page", "strong", "mixed"])
@pytest.mark.parametrize("read", ["post", "pre"])
def test_chunk_parity(gdr, cfg, regime, read):
    cfg = dict(cfg)
    chunk, dtype = cfg.pop("chunk"), cfg["dtype"]
    _say("gdn2 chunk %s %s %s" % (_ids(dict(cfg, chunk=chunk)), regime, read))
    c = inputs.gdn2_case(**cfg, seed=11, h0_std=0.5, regime=regime)
    o, hT = _run(gdr, c, chunk, read=read)
    ro, rh = gdn2.scan(c.q, c.k, c.v, c.g, c.b, c.w, c.h0, read=read)
    check(o, ro, dtype, "out")
    check(hT, rh, dtype, "hT")


# The one-pass kernel (no workspace) on a subset: every dtype, chunk and d_k it takes
@pytest.mark.parametrize("cfg", CHUNK, ids=_ids)
@pytest.mark.parametrize("read", ["post", "pre"])
def test_chunk_parity_fused(gdr, cfg, read):
    cfg = dict(cfg)
    chunk, dtype = cfg.pop("chunk"), cfg["dtype"]
    _say("gdn2 fused chunk %s %s" % (_ids(dict(cfg, chunk=chunk)), read))
    c = inputs.gdn2_case(**cfg, seed=13, h0_std=0.5, regime="mixed")
    o, hT = _run(gdr, c, chunk, read=read, fused=True)
    ro, rh = gdn2.scan(c.q, c.k, c.v, c.g, c.b, c.w, c.h0, read=read)
    check(o, ro, dtype, "out")
    check(hT, rh, dtype, "hT")


def test_chunk_workspace_reused(gdr):
    # one workspace for two calls, the second smaller and packed: nothing carries over
    _say("gdn2 workspace reuse")
    c1 = inputs.gdn2_case(B=2, T=150, Hk=1, Hv=2, dk=64, dv=64, dtype=torch.bfloat16, seed=71, h0_std=0.5)
    c2 = inputs.gdn2_case(B=1, Hk=1, Hv=2, dk=64, dv=64, dtype=torch.bfloat16, seed=72, h0_std=0.5,
                          lengths=[40, 0, 3], regime="strong")
    need = gdr.gdn2_chunk_fwd_workspace_bytes(2, 150, 1, 2, 64, 64, 32)
    ws = torch.full((need,), 255, dtype=torch.uint8, device="cuda")
    for c in (c1, c2):
        o, hT = _run(gdr, c, 32, workspace=ws)
        ro, rh = gdn2.scan(c.q, c.k, c.v, c.g, c.b, c.w, c.h0, c.cu_seqlens)
        check(o, ro, torch.bfloat16, "out")
        check(hT, rh, torch.bfloat16, "hT")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("fused", [False, True])
def test_chunk_varlen_reverse_accumulate(gdr, dtype, reverse, fused):
    lengths = [0, 1, 15, 16, 17, 64, 65, 130]
    _say("gdn2 varlen %s reverse=%s fused=%s" % (dtype, reverse, fused))
    c = inputs.gdn2_case(B=1, Hk=2, Hv=4, dk=64, dv=64, dtype=dtype, seed=21, h0_std=0.5, lengths=lengths,
                         regime="mixed")
    base = inputs._normal(inputs._gen(5), (1, 4, sum(lengths), 64)).to(dtype)
    for read in ("post", "pre"):
        o, hT = _run(gdr, c, 32, read=read, reverse=reverse, accumulate=base, fused=fused)
        ref_out = base.double().numpy().copy()
        _, rh = gdn2.scan(c.q, c.k, c.v, c.g, c.b, c.w, c.h0, c.cu_seqlens, read=read, reverse=reverse,
                          out=ref_out)
        check(o, ref_out, dtype, "out %s" % read)
        check(hT, rh, dtype, "hT %s" % read)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_chunk_l2norm(gdr, dtype):
    _say("gdn2 l2norm %s" % dtype)
    c = inputs.gdn2_case(B=1, T=203, Hk=2, Hv=2, dk=128, dv=64, dtype=dtype, seed=31, h0_std=0.3,
                         unit_rows=False)
    for read in ("post", "pre"):
        o, hT = _run(gdr, c, 32, read=read, l2norm=True)
        ro, rh = gdn2.scan(c.q, c.k, c.v, c.g, c.b, c.w, c.h0, read=read, l2norm=True)
        check(o, ro, dtype, "out %s" % read)
        check(hT, rh, dtype, "hT %s" % read)


def test_chunk_weak_decay_long(gdr):
    # long memory: the carried state dominates, across many chunks and a ragged tail
    _say("gdn2 weak decay T=1000")
    c = inputs.gdn2_case(B=1, T=1000, Hk=1, Hv=2, dk=128, dv=64, dtype=torch.float32, seed=41,
                         h0_std=0.5, regime="weak")
    o, hT = _run(gdr, c, 32)
    ro, rh = gdn2.scan(c.q, c.k, c.v, c.g, c.b, c.w, c.h0)
    check(o, ro, torch.float32, "out")
    check(hT, rh, torch.float32, "hT")


def test_chunk_sizes_agree(gdr):
    # the chunk size changes the result only through rounding
    _say("gdn2 chunk sizes")
    c = inputs.gdn2_case(B=1, T=160, Hk=1, Hv=1, dk=64, dv=64, dtype=torch.float32, seed=51, h0_std=0.5,
                         regime="mixed")
    ro, rh = gdn2.scan(c.q, c.k, c.v, c.g, c.b, c.w, c.h0)
    for chunk in (16, 32, 64):
        o, hT = _run(gdr, c, chunk)
        check(o, ro, torch.float32, "out c%d" % chunk)
        check(hT, rh, torch.float32, "hT c%d" % chunk)


def test_chunk_reduces_to_scalar_kernel(gdr):
    # uniform g, b = w = beta on every channel: the scalar chunk kernel's result
    _say("gdn2 vs scalar kernel")
    c = inputs.chunk_case(B=1, T=190, Hk=2, Hv=2, dk=64, dv=64, dtype=torch.float32, seed=61, h0_std=0.5)
    B, Hk, T, dk = c.q.shape
    g = c.log_alpha[..., None].expand(B, Hk, T, dk).contiguous()
    bb = c.beta[..., None].expand(B, Hk, T, dk).contiguous()
    ww = c.beta[..., None].expand(B, Hk, T, 64).contiguous()
    dev = lambda t: t.cuda()
    o2, h2 = gdr.gdn2_chunk_fwd(dev(c.q), dev(c.k), dev(c.v), dev(g), dev(bb), dev(ww), dev(c.h0), None, chunk=64)
    o1, h1 = gdr.chunk_fwd(dev(c.q), dev(c.k), dev(c.v), dev(c.log_alpha), dev(c.beta), dev(c.h0), None, chunk=64)
    torch.cuda.synchronize()
    check(gpu_np(o2), gpu_np(o1), torch.float32, "out")
    check(gpu_np(h2), gpu_np(h1), torch.float32, "hT")


def test_chunk_in_place_state_and_empty(gdr):
    _say("gdn2 in-place state, empty sequences")
    c = inputs.gdn2_case(B=2, T=70, Hk=1, Hv=2, dk=64, dv=64, dtype=torch.bfloat16, seed=71, h0_std=0.5)
    q, k, v, g, b, w, h0, _ = _dev(c)
    o, hT = gdr.gdn2_chunk_fwd(q, k, v, g, b, w, h0, None, chunk=64, hT=h0)
    torch.cuda.synchronize()
    ro, rh = gdn2.scan(c.q, c.k, c.v, c.g, c.b, c.w, c.h0)
    check(gpu_np(o), ro, torch.bfloat16, "out")
    check(gpu_np(h0), rh, torch.bfloat16, "hT in place")
    # T = 0: the final state is the initial state
    e = lambda *s, dt=torch.bfloat16: torch.zeros(*s, dtype=dt, device="cuda")
    h = torch.randn(2, 2, 64, 64, device="cuda")
    o, hT = gdr.gdn2_chunk_fwd(e(2, 1, 0, 64), e(2, 1, 0, 64), e(2, 2, 0, 64), e(2, 1, 0, 64, dt=torch.float32),
                               e(2, 1, 0, 64), e(2, 2, 0, 64), h, None, chunk=32)
    torch.cuda.synchronize()
    assert torch.equal(hT, h)


def test_chunk_full_size_sampled(gdr):
    # B4 H16 T4096 d128 bf16 (the size of the scalar kernel's main workload), chunk 64: every
    # output and state of four (sequence, head) pairs against the oracle
    _say("gdn2 full size B4 H16 T4096 d128")
    c = inputs.gdn2_case(B=4, T=4096, Hk=16, Hv=16, dk=128, dv=128, dtype=torch.bfloat16, seed=81, h0_std=0.1)
    o, hT = _run(gdr, c, 64)
    for (bi, h) in ((0, 0), (1, 7), (2, 13), (3, 15)):
        sl = lambda t: t[bi:bi + 1, h:h + 1]
        ro, rh = gdn2.scan(sl(c.q), sl(c.k), sl(c.v), sl(c.g), sl(c.b), sl(c.w), sl(c.h0))
        check(o[bi:bi + 1, h:h + 1], ro, torch.bfloat16, "out (%d, %d)" % (bi, h))
        check(hT[bi:bi + 1, h:h + 1], rh, torch.bfloat16, "hT (%d, %d)" % (bi, h))


DECODE = [
    dict(N=5, Hk=2, Hv=4, dk=128, dv=128, dtype=torch.bfloat16),
    dict(N=3, Hk=1, Hv=2, dk=64, dv=128, dtype=torch.float32),
    dict(N=4, Hk=2, Hv=2, dk=128, dv=64, dtype=torch.float32),
    dict(N=2, Hk=2, Hv=2, dk=64, dv=64, dtype=torch.bfloat16),
]


@pytest.mark.parametrize("cfg", DECODE, ids=lambda c: "N%d-Hk%d-Hv%d-dk%d-dv%d-%s" % (
    c["N"], c["Hk"], c["Hv"], c["dk"], c["dv"], str(c["dtype"]).split(".")[-1]))
@pytest.mark.parametrize("read", ["post", "pre"])
@pytest.mark.parametrize("l2norm", [False, True])
def test_decode_parity(gdr, cfg, read, l2norm):
    cfg = dict(cfg)
    N, dtype = cfg.pop("N"), cfg["dtype"]
    _say("gdn2 decode %s %s l2=%s" % (cfg, read, l2norm))
    # N sequences of one token: the case's batch rows
    c = inputs.gdn2_case(B=N, T=1, seed=91, h0_std=0.5, unit_rows=not l2norm, **cfg)
    one = lambda t: t[:, :, 0].contiguous().cuda()
    state = c.h0.cuda().clone()
    o, s_out = gdr.gdn2_decode_step(one(c.q), one(c.k), one(c.v), one(c.g), one(c.b), one(c.w), state,
                                    read=read, l2norm=l2norm)
    torch.cuda.synchronize()
    ro, rs = gdn2.decode(c.q[:, :, 0], c.k[:, :, 0], c.v[:, :, 0], c.g[:, :, 0], c.b[:, :, 0], c.w[:, :, 0],
                         c.h0, read=read, l2norm=l2norm)
    check(gpu_np(o), ro, dtype, "out")
    check(gpu_np(s_out), rs, dtype, "state")
    # in place: state_out is state_in
    o2, _ = gdr.gdn2_decode_step(one(c.q), one(c.k), one(c.v), one(c.g), one(c.b), one(c.w), state,
                                 state_out=state, read=read, l2norm=l2norm)
    torch.cuda.synchronize()
    check(gpu_np(state), rs, dtype, "state in place")
    check(gpu_np(o2), ro, dtype, "out in place")


def test_decode_steps_match_chunk(gdr):
    # 40 decode steps from h0 reproduce the chunk forward over the same 40 tokens
    _say("gdn2 decode steps vs chunk")
    c = inputs.gdn2_case(B=2, T=40, Hk=2, Hv=4, dk=128, dv=64, dtype=torch.float32, seed=95, h0_std=0.5,
                         regime="mixed")
    o_c, h_c = _run(gdr, c, 32)
    q, k, v, g, b, w, h0, _ = _dev(c)
    state = h0.clone()
    outs = []
    for t in range(40):
        s = lambda x: x[:, :, t].contiguous()
        o, state = gdr.gdn2_decode_step(s(q), s(k), s(v), s(g), s(b), s(w), state)
        outs.append(o)
    torch.cuda.synchronize()
    check(gpu_np(torch.stack(outs, dim=2)), o_c, torch.float32, "out")
    check(gpu_np(state), h_c, torch.float32, "state")


@pytest.mark.parametrize("regime", ["page", "weak", "mixed"])
def test_chunk_bench_shape_two_pass(gdr, regime):
    # the launch the benchmark times: B4 H16 T4096 d_k = d_v = 128 bf16, chunk 32, two passes
    # through a caller workspace; eight (sequence, head) units against the oracle, each output
    # checked whole, per 64-token block and on its chunk-last rows, and each final state
    from tests._parity import check_bf16_detailed, check_states, segments
    _say("gdn2 benchmark shape, chunk 32, two passes, regime=%s" % regime)
    c = inputs.gdn2_case(B=4, T=4096, Hk=16, Hv=16, dk=128, dv=128, dtype=torch.bfloat16, seed=1001,
                         h0_std=0.1, regime=regime)
    ws = torch.empty(gdr.gdn2_chunk_fwd_workspace_bytes(4, 4096, 16, 16, 128, 128, 32), dtype=torch.uint8,
                     device="cuda")
    o, hT = _run(gdr, c, 32, workspace=ws)
    for (bi, h) in ((0, 0), (0, 9), (1, 3), (1, 14), (2, 6), (2, 11), (3, 1), (3, 15)):
        sl = lambda t: t[bi:bi + 1, h:h + 1]
        ro, rh = gdn2.scan(sl(c.q), sl(c.k), sl(c.v), sl(c.g), sl(c.b), sl(c.w), sl(c.h0))
        ou = o[bi:bi + 1, h:h + 1]
        e = check_bf16_detailed(ou, ro, segments(ou.shape, None), "out (%d, %d)" % (bi, h))
        check_states(hT[bi:bi + 1, h:h + 1], rh, "hT (%d, %d)" % (bi, h))
        _say("  unit (%d, %d): whole %.2e, worst block %.2e, chunk-last rows %.2e" % ((bi, h) + e))


@pytest.mark.parametrize("read", ["post", "pre"])
def test_decode_full_size(gdr, read):
    # the decode step the benchmark times: 256 sequences, 16 key heads -> 32 value heads, d128,
    # bf16 inputs, fp32 state updated in place; every head-state and every output vector
    _say("gdn2 decode full size N256 Hk16 Hv32 d128 %s" % read)
    c = inputs.gdn2_case(B=256, T=1, Hk=16, Hv=32, dk=128, dv=128, dtype=torch.bfloat16, seed=1003, h0_std=0.1)
    one = lambda t: t[:, :, 0].contiguous()
    state = c.h0.cuda().clone()
    o, _ = gdr.gdn2_decode_step(*(one(t).cuda() for t in (c.q, c.k, c.v, c.g, c.b, c.w)), state, state_out=state,
                                read=read)
    torch.cuda.synchronize()
    ro, rs = gdn2.decode(one(c.q), one(c.k), one(c.v), one(c.g), one(c.b), one(c.w), c.h0, read=read)
    check(gpu_np(o), ro, torch.bfloat16, "out")
    check(gpu_np(state), rs, torch.bfloat16, "state")
    og, sg = gpu_np(o), gpu_np(state)
    ev = np.sqrt(((og - ro) ** 2).sum(-1)) / np.maximum(np.sqrt((ro ** 2).sum(-1)), 1e-30)
    es = np.sqrt(((sg - rs) ** 2).sum((-2, -1))) / np.maximum(np.sqrt((rs ** 2).sum((-2, -1))), 1e-30)
    assert ev.max() <= BF16_REL and es.max() <= BF16_REL, (ev.max(), es.max())
    _say("  worst output vector %.2e, worst head-state %.2e" % (ev.max(), es.max()))
