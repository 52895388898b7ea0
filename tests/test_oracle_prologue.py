"""Pins of the oracle's prologue (q/k L2 normalisation and gates from raw inputs).

The values checked here are fixed by mathematics, not recomputed with the oracle's own
formula: a 3-4-5 triangle, scale invariance, unit norms, the eps floor, softplus at points
where it has a closed form (0 -> ln 2, ln(e - 1) -> 1) and its two asymptotes, the logistic
function at ln 3 (-> 3/4), and, end to end, that the fused oracle does not see a positive
per-row rescaling of q and k and equals the plain recurrence on rows already of unit norm.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import prologue


def test_l2_normalize_hand_values():
    x = np.array([[3.0, 4.0, 0.0, 0.0], [0.0, 0.0, -5.0, 12.0]])
    y = prologue.l2_normalize(x)
    assert np.array_equal(y[0], np.array([0.6, 0.8, 0.0, 0.0]))
    np.testing.assert_allclose(y[1], np.array([0.0, 0.0, -5.0 / 13.0, 12.0 / 13.0]), rtol=0, atol=1e-16)


def test_l2_normalize_unit_norm_and_scale_invariance():
    g = np.random.default_rng(3)
    x = g.standard_normal((5, 7, 33))
    y = prologue.l2_normalize(x)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), 1.0, rtol=0, atol=1e-14)
    c = g.uniform(0.01, 100.0, size=(5, 7, 1))
    np.testing.assert_allclose(prologue.l2_normalize(c * x), y, rtol=0, atol=1e-14)
    # the direction is kept: y is a positive multiple of x
    cos = np.sum(x * y, axis=-1) / np.linalg.norm(x, axis=-1)
    np.testing.assert_allclose(cos, 1.0, rtol=0, atol=1e-14)


def test_l2_normalize_eps_floor():
    # a zero row stays zero; a row shorter than eps is divided by eps, not by its norm
    assert np.array_equal(prologue.l2_normalize(np.zeros((2, 8))), np.zeros((2, 8)))
    x = np.array([3e-8, 4e-8])
    np.testing.assert_allclose(prologue.l2_normalize(x), x / 1e-6, rtol=1e-15)


def test_softplus_closed_forms():
    assert prologue.softplus(0.0) == pytest.approx(math.log(2.0), rel=0, abs=1e-16)
    assert prologue.softplus(math.log(math.e - 1.0)) == pytest.approx(1.0, rel=0, abs=1e-15)
    # asymptotes: x + e^{-x} for large x, e^{x} for very negative x
    assert prologue.softplus(40.0) == pytest.approx(40.0 + math.exp(-40.0), rel=1e-15)
    assert prologue.softplus(-40.0) == pytest.approx(math.exp(-40.0), rel=1e-12)
    assert np.isfinite(prologue.softplus(1e4)) and prologue.softplus(1e4) == 1e4


def test_gates_closed_forms():
    # head 0: A_log = 0, a + dt_bias = 0  -> log alpha = -ln 2 (alpha = 1/2)
    # head 1: A_log = ln 3, a + dt_bias = ln(e - 1) -> log alpha = -3
    a = np.array([[0.5, math.log(math.e - 1.0) - 0.25]])
    A_log = np.array([0.0, math.log(3.0)])
    dt_bias = np.array([-0.5, 0.25])
    b = np.array([[math.log(3.0), 0.0]])
    la, beta = prologue.gates(a, b, A_log, dt_bias, head_axis=1)
    np.testing.assert_allclose(la, [[-math.log(2.0), -3.0]], rtol=0, atol=1e-15)
    np.testing.assert_allclose(beta, [[0.75, 0.5]], rtol=0, atol=1e-16)


def test_gates_head_axis():
    # [B, Hv, T] inputs: the per-head parameters follow axis 1
    a = np.zeros((2, 3, 4))
    la, _ = prologue.gates(a, a, np.log(np.array([1.0, 2.0, 4.0])), np.zeros(3), head_axis=1)
    for h, scale in enumerate((1.0, 2.0, 4.0)):
        np.testing.assert_allclose(la[:, h, :], -scale * math.log(2.0), rtol=0, atol=1e-15)


def _case(seed, B=1, Hk=2, Hv=4, T=37, dk=8, dv=6):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hk, T, dk, generator=g, dtype=torch.float64)
    k = torch.randn(B, Hk, T, dk, generator=g, dtype=torch.float64)
    v = torch.randn(B, Hv, T, dv, generator=g, dtype=torch.float64)
    a = torch.randn(B, Hv, T, generator=g, dtype=torch.float64)
    b = torch.randn(B, Hv, T, generator=g, dtype=torch.float64)
    A_log = torch.rand(Hv, generator=g, dtype=torch.float64) * 2.0
    dt_bias = torch.randn(Hv, generator=g, dtype=torch.float64)
    h0 = 0.1 * torch.randn(B, Hv, dk, dv, generator=g, dtype=torch.float64)
    return q, k, v, a, b, A_log, dt_bias, h0


@pytest.mark.parametrize("read", ["post", "pre"])
def test_fused_scan_ignores_row_scale(oracle_lib, read):
    q, k, v, a, b, A_log, dt_bias, h0 = _case(11)
    g = torch.Generator().manual_seed(12)
    sq = torch.rand(q.shape[:-1] + (1,), generator=g, dtype=torch.float64) * 50 + 0.01
    sk = torch.rand(k.shape[:-1] + (1,), generator=g, dtype=torch.float64) * 50 + 0.01
    o1, h1 = prologue.scan_fused(q, k, v, a, b, A_log, dt_bias, h0, read=read)
    o2, h2 = prologue.scan_fused(q * sq, k * sk, v, a, b, A_log, dt_bias, h0, read=read)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(h2, h1, rtol=0, atol=1e-12)
    # without the normalisation the scale does matter (the check above is not vacuous)
    o3, _ = prologue.scan_fused(q * sq, k * sk, v, a, b, A_log, dt_bias, h0, read=read, l2norm=False)
    assert np.max(np.abs(o3 - o1)) > 1e-3


def test_fused_scan_on_unit_rows_is_the_plain_scan(oracle_lib):
    q, k, v, a, b, A_log, dt_bias, h0 = _case(21)
    qn = q / q.norm(dim=-1, keepdim=True)
    kn = k / k.norm(dim=-1, keepdim=True)
    # gates written out directly from the page's compute_gates, in torch
    la = -torch.exp(A_log)[None, :, None] * torch.nn.functional.softplus(a + dt_bias[None, :, None])
    beta = torch.sigmoid(b)
    o1, h1 = prologue.scan_fused(qn, kn, v, a, b, A_log, dt_bias, h0)
    o2, h2 = oracle.scan(qn, kn, v, la, beta, h0)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(h1, h2, rtol=0, atol=1e-12)


def test_fused_decode_matches_fused_scan(oracle_lib):
    # one token: the decode step with the prologue equals a one-token scan with it
    q, k, v, a, b, A_log, dt_bias, h0 = _case(31, B=3, T=1)
    o_s, h_s = prologue.scan_fused(q, k, v, a, b, A_log, dt_bias, h0)
    o_d, h_d = prologue.decode_fused(q[:, :, 0], k[:, :, 0], v[:, :, 0], a[:, :, 0], b[:, :, 0], A_log, dt_bias, h0)
    np.testing.assert_allclose(o_d, o_s[:, :, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(h_d, h_s, rtol=0, atol=1e-12)
