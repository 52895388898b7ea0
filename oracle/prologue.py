"""The steps the pages run just before the recurrence, in plain fp64 numpy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* ``l2_normalize``: each row divided by max(||row||_2, eps), eps = 1e-6: F.normalize(x,
  dim=-1, eps=1e-6) as the "nested-learning self_modifying.py" page applies it to q and k;
  the "flashrt-structures fused_layer.py" page (use_qk_l2norm) and the "tiny_gdn/fugue.py"
  page (use_qk_l2norm_in_kernel) normalise q and k inside their cores without printing the
  formula, and this is the reading taken for them.
* ``gates``: log_alpha = -exp(A_log) * softplus(a + dt_bias), beta = sigmoid(b), per value
  head: ``compute_gates`` of SparseDeltaMemory on the "sparse-delta-memory layer.py" page
  (A = -exp(A_log), g = A * softplus(a + dt_bias), beta = sigmoid(b)).
* ``scan_fused`` / ``decode_fused``: these two steps, then the plain recurrence of the
  package (``oracle.scan`` / ``oracle.decode``) on their results.
"""
from __future__ import annotations

import numpy as np

from . import scan, decode

L2_EPS = 1e-6


def _f64(x):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def l2_normalize(x, eps: float = L2_EPS) -> np.ndarray:
    """x / max(||x||_2, eps) over the last axis, in fp64."""
    x = _f64(x)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, eps)


def softplus(x) -> np.ndarray:
    """log(1 + e^x), written so that it neither overflows nor loses the small tail."""
    x = _f64(x)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def gates(a, b, A_log, dt_bias, head_axis: int):
    """(log_alpha, beta) from the raw inputs a, b and per-head A_log, dt_bias [H];
    ``head_axis`` is the axis of a and b that indexes the value head."""
    a, b = _f64(a), _f64(b)
    shape = [1] * a.ndim
    shape[head_axis] = -1
    A = _f64(A_log).reshape(shape)
    dt = _f64(dt_bias).reshape(shape)
    log_alpha = -np.exp(A) * softplus(a + dt)
    beta = 1.0 / (1.0 + np.exp(-b))
    return log_alpha, beta


def scan_fused(q, k, v, a, b, A_log=None, dt_bias=None, h0=None, cu_seqlens=None, *,
               l2norm: bool = True, **kw):
    """``oracle.scan`` after the prologue: q, k [B, Hk, T, dk] normalised per row when
    ``l2norm``; with A_log, dt_bias given, a and b [B, Hv, T] are the raw gate inputs."""
    if l2norm:
        q, k = l2_normalize(q), l2_normalize(k)
    if A_log is not None:
        a, b = gates(a, b, A_log, dt_bias, head_axis=1)
    return scan(q, k, v, a, b, h0, cu_seqlens, **kw)


def decode_fused(q, k, v, a, b, A_log, dt_bias, state, *, l2norm: bool = True, **kw):
    """``oracle.decode`` after the prologue: q, k [N, Hk, dk]; a, b [N, Hv] raw when A_log
    is given."""
    if l2norm:
        q, k = l2_normalize(q), l2_normalize(k)
    if A_log is not None:
        a, b = gates(a, b, A_log, dt_bias, head_axis=1)
    return decode(q, k, v, a, b, state, **kw)
