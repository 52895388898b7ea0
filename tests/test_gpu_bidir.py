"""Parity of the bidirectional entry point (gdr_chunk_fwd_bidir, through the C ABI) with the fp64
oracle: the forward scan plus the in-segment reversed scan over shared q, k, v, each with its own
gates and initial state, summed per token, as the bidirectional layer on the "tiny_gdn/fugue.py"
page combines them (`BidirectionalGatedDeltaNet2.scan` and `forward`). The oracle side is two
independent per-token scans (forward, then reverse) added in fp64.
"""
from __future__ import annotations

import ctypes
import sys

import pytest
import torch

import oracle
from oracle import prologue
from gated_delta_rule_70_amd import inputs
from tests._parity import check, gpu_np

pytestmark = pytest.mark.gpu


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


def _cases(dtype, lengths, B, T, Hk, Hv, dk, dv, seed, regime="slow"):
    """Shared q, k, v and the forward gates and h0 from one case; the reverse gates and h0 from a
    second case of the same shape drawn with another seed."""
    kw = dict(Hk=Hk, Hv=Hv, dk=dk, dv=dv, dtype=dtype, h0_std=0.1, regime=regime)
    if lengths is not None:
        kw["lengths"] = lengths
    else:
        kw.update(B=B, T=T)
    f = inputs.chunk_case(seed=seed, **kw)
    r = inputs.chunk_case(seed=seed + 1000, **kw)
    return f, r


def _oracle(f, r, read, l2norm=False, base=None):
    def fn(la, b, h0, **kw):
        if l2norm:  # unit rows first, then the plain scan
            return prologue.scan_fused(f.q, f.k, f.v, la, b, None, None, h0, f.cu_seqlens, l2norm=True, **kw)
        return oracle.scan(f.q, f.k, f.v, la, b, h0, f.cu_seqlens, **kw)

    of, hf = fn(f.log_alpha, f.beta, f.h0, read=read)
    orr, hr = fn(r.log_alpha, r.beta, r.h0, read=read, reverse=True)
    o = of + orr
    if base is not None:
        o = o + base
    return o, hf, hr


LAYOUTS = {
    "batched": dict(lengths=None, B=2, T=200),
    "packed": dict(lengths=[70, 0, 129, 64, 1, 200], B=1, T=0),
}


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("read", ["pre", "post"])
@pytest.mark.parametrize("layout", list(LAYOUTS))
def test_bidir_matches_oracle(gdr, dtype, read, layout):
    """Both scans, their final states and the sum, on batched and packed (empty segment, ragged
    tails) inputs, GQA (one key head for two value heads), slow decay so that both initial states
    and the chunk-to-chunk carry decide the result."""
    dk, dv = 128, 64
    f, r = _cases(dtype, LAYOUTS[layout]["lengths"], LAYOUTS[layout]["B"], LAYOUTS[layout]["T"], 1, 2, dk, dv,
                  seed=31)
    _say("bidir %s read=%s %s T=%d" % (dtype, read, layout, f.q.shape[2]))
    d = lambda t: None if t is None else t.cuda()
    out, hT_f, hT_r = gdr.chunk_fwd_bidir(d(f.q), d(f.k), d(f.v), d(f.log_alpha), d(f.beta), d(r.log_alpha),
                                          d(r.beta), d(f.h0), d(r.h0), d(f.cu_seqlens), chunk=64, read=read)
    torch.cuda.synchronize()
    ro, rhf, rhr = _oracle(f, r, read)
    check(gpu_np(out), ro, dtype, "bidir o")
    check(gpu_np(hT_f), rhf, dtype, "bidir hT_fwd")
    check(gpu_np(hT_r), rhr, dtype, "bidir hT_rev")


def test_bidir_equals_two_calls(gdr):
    """The entry point is the forward call followed by the reverse, accumulating call: the same
    bits as making those two calls."""
    f, r = _cases(torch.bfloat16, [300, 5, 64, 1000], 1, 0, 2, 4, 128, 128, seed=32)
    d = lambda t: None if t is None else t.cuda()
    q, k, v, cu = d(f.q), d(f.k), d(f.v), d(f.cu_seqlens)
    out, hT_f, hT_r = gdr.chunk_fwd_bidir(q, k, v, d(f.log_alpha), d(f.beta), d(r.log_alpha), d(r.beta), d(f.h0),
                                          d(r.h0), cu, chunk=64, read="pre")
    o2, h2f = gdr.chunk_fwd(q, k, v, d(f.log_alpha), d(f.beta), d(f.h0), cu, chunk=64, read="pre")
    _, h2r = gdr.chunk_fwd(q, k, v, d(r.log_alpha), d(r.beta), d(r.h0), cu, chunk=64, read="pre", reverse=True,
                           out=o2, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(hT_f, h2f) and torch.equal(hT_r, h2r)


def test_bidir_accumulate_inplace_and_l2norm(gdr):
    """GDR_ACCUMULATE adds both scans to out; each final state may be its own initial state;
    GDR_QK_L2NORM normalises q and k for both scans; chunk 32 and fp32 run the generic kernel."""
    f, r = _cases(torch.float32, None, 2, 150, 2, 2, 64, 64, seed=33)
    d = lambda t: None if t is None else t.cuda()
    base = torch.randn(tuple(f.v.shape), generator=torch.Generator().manual_seed(4))
    # unnormalised q and k, so that the in-kernel normalisation matters
    q, k = (f.q * 3.0).contiguous(), (f.k * 0.5).contiguous()
    out = base.cuda()
    h0f, h0r = d(f.h0), d(r.h0)
    hTf_out = h0f  # in place
    o, hf, hr = gdr.chunk_fwd_bidir(d(q), d(k), d(f.v), d(f.log_alpha), d(f.beta), d(r.log_alpha), d(r.beta),
                                    h0f, h0r, None, chunk=32, read="pre", out=out, accumulate=True, want_state=True,
                                    l2norm=True)
    torch.cuda.synchronize()
    f.q, f.k = q, k
    ro, rhf, rhr = _oracle(f, r, "pre", l2norm=True, base=base.double().numpy())
    check(gpu_np(o), ro, torch.float32, "bidir accumulate o")
    check(gpu_np(hf), rhf, torch.float32, "bidir hT_fwd")
    check(gpu_np(hr), rhr, torch.float32, "bidir hT_rev")
    # in place: hT_fwd written over h0_fwd through the C ABI directly
    o2 = base.cuda()
    lib = gdr.lib()
    dims = gdr.ChunkDims(2, 150, 2, 2, 64, 64, 0, gdr.GDR_F32,
                         gdr.GDR_READ_PRE | gdr.GDR_ACCUMULATE | gdr.GDR_QK_L2NORM)
    p = gdr._ptr
    tens = [d(q), d(k), d(f.v), d(f.log_alpha), d(f.beta), d(r.log_alpha), d(r.beta), hTf_out, h0r]
    st = lib.gdr_chunk_fwd_bidir(*[p(t) for t in tens], None, 32, p(o2), p(hTf_out), None,
                                 ctypes.byref(dims), gdr._stream(q.cuda()))
    assert gdr.STATUS[st] == "GDR_OK", lib.gdr_last_error()
    torch.cuda.synchronize()
    check(gpu_np(o2), ro, torch.float32, "bidir in-place o")
    check(gpu_np(hTf_out), rhf, torch.float32, "bidir in-place hT_fwd")
