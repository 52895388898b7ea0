"""The seeded generators: deterministic, right shapes, right ranges (CPU)."""
import torch

from gated_delta_rule_70_amd import inputs


def test_chunk_case_deterministic_and_shaped():
    a = inputs.chunk_case(B=2, T=70, Hk=2, Hv=4, dk=64, dv=32, dtype=torch.bfloat16, seed=5,
                          h0_std=0.1)
    b = inputs.chunk_case(B=2, T=70, Hk=2, Hv=4, dk=64, dv=32, dtype=torch.bfloat16, seed=5,
                          h0_std=0.1)
    for x, y in zip((a.q, a.k, a.v, a.log_alpha, a.beta, a.h0), (b.q, b.k, b.v, b.log_alpha, b.beta, b.h0)):
        assert torch.equal(x, y)
    assert a.q.shape == (2, 2, 70, 64) and a.v.shape == (2, 4, 70, 32)
    assert a.log_alpha.shape == (2, 4, 70) and a.h0.shape == (2, 4, 64, 32)
    assert a.q.dtype == torch.bfloat16 and a.log_alpha.dtype == torch.float32
    assert (a.log_alpha <= 0).all() and (a.beta > 0).all() and (a.beta < 1).all()
    n = a.k.float().norm(dim=-1)
    assert torch.allclose(n, torch.ones_like(n), atol=1e-2)


def test_gate_regimes():
    for regime, lo, hi in (("zero", 0.0, 0.0), ("p5", torch.log(torch.tensor(0.5)).item(), 0.0),
                           ("slow", -0.05, 0.0)):
        c = inputs.chunk_case(T=200, regime=regime, seed=1)
        assert c.log_alpha.min() >= lo - 1e-6 and c.log_alpha.max() <= hi


def test_workload_gate_scale():
    # log alpha = -a_h softplus(z), a_h in [1, 16]: per-token decay spans about [-48, 0)
    c = inputs.workload0()
    assert c.log_alpha.max() < 0 and c.log_alpha.min() > -16 * 10


def test_varlen_lengths_and_offsets():
    L = inputs.segment_lengths(8, 512, 8192, seed=1002 + 7919)
    assert len(L) == 8 and all(512 <= x <= 8192 for x in L)
    c = inputs.chunk_case(Hk=2, dk=64, dv=64, lengths=[3, 0, 5], h0_std=0.1, seed=2)
    assert c.cu_seqlens.tolist() == [0, 3, 3, 8] and c.h0.shape[0] == 3 and c.q.shape[2] == 8


def test_decode_case_shapes():
    d = inputs.decode_case(N=3, Hk=2, Hv=4, dk=64, dv=64, steps=5)
    assert d.q.shape == (5, 3, 2, 64) and d.v.shape == (5, 3, 4, 64)
    assert d.log_alpha.shape == (5, 3, 4) and d.state.shape == (3, 4, 64, 64)


def test_bidirectional_case():
    c = inputs.workload4(seg_len=64, nseg=2, H=2)
    assert c.cu_seqlens.tolist() == [0, 64, 128]
    assert not torch.equal(c.log_alpha, c.extra["log_alpha_bwd"])
