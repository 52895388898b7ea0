"""Parity of the GDN-2 bidirectional entry point (gdr_gdn2_chunk_fwd_bidir, through the C ABI) with
the fp64 GDN-2 oracle: the layer on the "tiny_gdn/fugue.py" page (`BidirectionalGatedDeltaNet2`)
scans each packed segment forward and reversed in place, each direction with its own decay, erase
and write gates, and adds the two. The oracle side is two independent per-token GDN-2 scans added
in fp64. Tolerances as for the GDN-2 forward: fp32 inputs max abs 2e-4, bf16 inputs relative
Frobenius 2e-2.
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
    binding.lib()  # raises if the library is missing: there is no fallback
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


CASES = [
    # packed segments (an empty one, ragged tails), GQA, the benchmarked bf16 d128 chunk 32 two-pass form
    dict(lengths=[70, 0, 129, 64, 1, 200], B=1, T=0, Hk=1, Hv=2, dk=128, dv=128, dtype=torch.bfloat16, chunk=32,
         fused=False),
    # batched, fp32, chunk 16, the one-pass kernel (no workspace)
    dict(lengths=None, B=2, T=150, Hk=2, Hv=2, dk=64, dv=64, dtype=torch.float32, chunk=16, fused=True),
    # batched bf16 chunk 64, d_k 64, two passes
    dict(lengths=None, B=2, T=257, Hk=2, Hv=4, dk=64, dv=64, dtype=torch.bfloat16, chunk=64, fused=False),
]


def _cases(cfg, seed, regime):
    kw = dict(Hk=cfg["Hk"], Hv=cfg["Hv"], dk=cfg["dk"], dv=cfg["dv"], dtype=cfg["dtype"], h0_std=0.1, regime=regime)
    if cfg["lengths"] is not None:
        kw["lengths"] = cfg["lengths"]
    else:
        kw.update(B=cfg["B"], T=cfg["T"])
    return inputs.gdn2_case(seed=seed, **kw), inputs.gdn2_case(seed=seed + 1000, **kw)


@pytest.mark.parametrize("read", ["pre", "post"])
@pytest.mark.parametrize("regime", ["page", "weak"])
@pytest.mark.parametrize("ci", range(len(CASES)))
def test_gdn2_bidir_matches_oracle(gdr, ci, regime, read):
    cfg = CASES[ci]
    f, r = _cases(cfg, 41 + ci, regime)
    _say("gdn2 bidir case %d %s read=%s regime=%s" % (ci, cfg["dtype"], read, regime))
    d = lambda t: None if t is None else t.cuda()
    out, hf, hr = gdr.gdn2_chunk_fwd_bidir(d(f.q), d(f.k), d(f.v), (d(f.g), d(f.b), d(f.w)), (d(r.g), d(r.b), d(r.w)),
                                           d(f.h0), d(r.h0), d(f.cu_seqlens), chunk=cfg["chunk"], read=read,
                                           fused=cfg["fused"])
    torch.cuda.synchronize()
    of, rhf = gdn2.scan(f.q, f.k, f.v, f.g, f.b, f.w, f.h0, f.cu_seqlens, read=read)
    orr, rhr = gdn2.scan(f.q, f.k, f.v, r.g, r.b, r.w, r.h0, f.cu_seqlens, read=read, reverse=True)
    check(gpu_np(out), of + orr, cfg["dtype"], "gdn2 bidir o")
    check(gpu_np(hf), rhf, cfg["dtype"], "gdn2 bidir hT_fwd")
    check(gpu_np(hr), rhr, cfg["dtype"], "gdn2 bidir hT_rev")


def test_gdn2_bidir_equals_two_calls_and_accumulates(gdr):
    """The entry point is the forward call followed by the reverse, accumulating call (the same bits);
    with GDR_ACCUMULATE both scans add to out."""
    cfg = CASES[0]
    f, r = _cases(cfg, 60, "page")
    d = lambda t: None if t is None else t.cuda()
    q, k, v, cu = d(f.q), d(f.k), d(f.v), d(f.cu_seqlens)
    gf, gr = (d(f.g), d(f.b), d(f.w)), (d(r.g), d(r.b), d(r.w))
    ws = torch.empty(gdr.gdn2_chunk_fwd_workspace_bytes(1, f.q.shape[2], 1, 2, 128, 128, 32,
                                                         num_seqs=len(cfg["lengths"])), dtype=torch.uint8, device="cuda")
    out, hf, hr = gdr.gdn2_chunk_fwd_bidir(q, k, v, gf, gr, d(f.h0), d(r.h0), cu, chunk=32, read="pre", workspace=ws)
    o2, h2f = gdr.gdn2_chunk_fwd(q, k, v, *gf, d(f.h0), cu, chunk=32, read="pre", workspace=ws)
    _, h2r = gdr.gdn2_chunk_fwd(q, k, v, *gr, d(r.h0), cu, chunk=32, read="pre", reverse=True, out=o2, accumulate=True,
                                workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(hf, h2f) and torch.equal(hr, h2r)
    base = torch.randn(tuple(f.v.shape), generator=torch.Generator().manual_seed(7)).to(torch.bfloat16)
    o3 = base.cuda()
    gdr.gdn2_chunk_fwd_bidir(q, k, v, gf, gr, d(f.h0), d(r.h0), cu, chunk=32, read="pre", out=o3, accumulate=True,
                             want_state=False, workspace=ws)
    torch.cuda.synchronize()
    of, _ = gdn2.scan(f.q, f.k, f.v, f.g, f.b, f.w, f.h0, f.cu_seqlens, read="pre")
    orr, _ = gdn2.scan(f.q, f.k, f.v, r.g, r.b, r.w, r.h0, f.cu_seqlens, read="pre", reverse=True)
    check(gpu_np(o3), of + orr + base.double().numpy(), torch.bfloat16, "gdn2 bidir accumulate")
