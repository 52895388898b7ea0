"""The allocation-free GDN-2 entry point (``gdr_gdn2_chunk_fwd_noalloc``, the two-pass forward on
the library's fixed device scratch) against the entry point it varies (``gdr_gdn2_chunk_fwd`` with
a caller workspace): the same kernels, so the results must be the same bits. Two calls in a row,
the second with a smaller input than the first, so that whatever the first left in the shared
scratch must not leak into the second."""
from __future__ import annotations

import sys

import pytest
import torch

from gated_delta_rule_70_amd import inputs

pytestmark = pytest.mark.gpu


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


def _both(gdr, c, chunk, **kw):
    d = lambda t: None if t is None else t.cuda()
    q, k, v, g, b, w, h0, cu = (d(t) for t in (c.q, c.k, c.v, c.g, c.b, c.w, c.h0, c.cu_seqlens))
    B, Hk, T, dk = c.q.shape
    Hv, dv = c.v.shape[1], c.v.shape[3]
    S = B if c.cu_seqlens is None else c.cu_seqlens.numel() - 1
    need = gdr.gdn2_chunk_fwd_workspace_bytes(B, T, Hk, Hv, dk, dv, chunk, 0 if cu is None else S, c.q.dtype)
    assert 0 < need <= (64 << 20), need
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o_ref, h_ref = gdr.gdn2_chunk_fwd(q, k, v, g, b, w, h0, cu, chunk=chunk, workspace=ws, **kw)
    out = torch.empty_like(o_ref)
    hT = torch.empty_like(h_ref)
    gdr.gdn2_chunk_fwd_noalloc(q, k, v, g, b, w, h0, cu, out, hT, chunk=chunk, **kw)
    torch.cuda.synchronize()
    return out, hT, o_ref, h_ref


def test_noalloc_matches_workspace_entry_point(gdr):
    # first call: B1 H16 T4096 d128 bf16, chunk 32 (60 MB of workspace, most of the scratch)
    _say("gdn2 noalloc: B1 H16 T4096 d128 bf16 chunk 32")
    c1 = inputs.gdn2_case(B=1, T=4096, Hk=16, Hv=16, dk=128, dv=128, dtype=torch.bfloat16, seed=201, h0_std=0.1)
    out, hT, o_ref, h_ref = _both(gdr, c1, 32)
    assert torch.equal(out, o_ref) and torch.equal(hT, h_ref)
    # second call, smaller and packed, pre-write read, reversed: nothing of the first may carry over
    _say("gdn2 noalloc: packed [300, 0, 77], Hk 2 Hv 4, dk 128 dv 64, chunk 32, pre, reverse")
    c2 = inputs.gdn2_case(B=1, Hk=2, Hv=4, dk=128, dv=64, dtype=torch.bfloat16, seed=202, h0_std=0.5,
                          lengths=[300, 0, 77], regime="mixed")
    out, hT, o_ref, h_ref = _both(gdr, c2, 32, read="pre", reverse=True)
    assert torch.equal(out, o_ref) and torch.equal(hT, h_ref)
    # and an fp32 case with chunk 16 and d_k 64
    _say("gdn2 noalloc: fp32 B2 T150 Hk1 Hv2 dk64 dv64 chunk 16")
    c3 = inputs.gdn2_case(B=2, T=150, Hk=1, Hv=2, dk=64, dv=64, dtype=torch.float32, seed=203, h0_std=0.5,
                          regime="weak")
    out, hT, o_ref, h_ref = _both(gdr, c3, 16)
    assert torch.equal(out, o_ref) and torch.equal(hT, h_ref)
