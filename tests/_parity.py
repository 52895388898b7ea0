"""Comparison helpers for the GPU parity tests (test infrastructure, no GPU code).

Tolerances follow the workload statement: fp32 inputs, max abs error <= 2e-4; bf16 inputs with
an fp32 state, relative Frobenius error <= 2e-2. For bf16 outputs the relative error is taken
three ways, each against the same bound, so that a localised mistake cannot hide inside a large
tensor (one wrong token row adds only about 1/sqrt(T) to a whole-tensor norm):

* over the whole compared tensor;
* over every 64-token block of every (segment, head) unit, on the scan's chunk grid;
* over the rows that end a chunk of the scan (the rows that see the whole carried state and the
  farthest off-diagonal terms) together with each unit's final state.
"""
from __future__ import annotations

import numpy as np
import torch

FP32_ABS = 2e-4
BF16_REL = 2e-2
BLOCK = 64


def max_abs(x, ref):
    x = np.asarray(x, dtype=np.float64)
    return float(np.max(np.abs(x - ref))) if x.size else 0.0


def rel_fro(x, ref):
    x = np.asarray(x, dtype=np.float64)
    den = float(np.linalg.norm(ref))
    return float(np.linalg.norm(x - ref)) / max(den, 1e-30)


def check(x, ref, dtype, what):
    x = np.asarray(x, dtype=np.float64)
    assert np.all(np.isfinite(x)), "%s: non-finite values" % what
    if dtype == torch.float32:
        e = max_abs(x, ref)
        assert e <= FP32_ABS, "%s: max abs err %.3e > %.1e" % (what, e, FP32_ABS)
    else:
        e = rel_fro(x, ref)
        assert e <= BF16_REL, "%s: rel Frobenius err %.3e > %.1e" % (what, e, BF16_REL)
    return e


def gpu_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def segments(shape_bht, cu_seqlens):
    """(batch row, start, end) of every scanned segment of a [B, H, T, d] tensor."""
    B, _, T = shape_bht[:3]
    if cu_seqlens is None:
        return [(b, 0, T) for b in range(B)]
    cu = [int(x) for x in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
    return [(0, cu[i], cu[i + 1]) for i in range(len(cu) - 1)]


def _rows_rel(x, ref):
    """Relative Frobenius error over the last two axes ([..., rows, d]) -> array [...]."""
    num = np.sqrt(np.sum((x - ref) ** 2, axis=(-2, -1)))
    den = np.sqrt(np.sum(ref ** 2, axis=(-2, -1)))
    return num / np.maximum(den, 1e-30)


def block_errors(x, ref, segs, reverse=False, block=BLOCK):
    """Worst relative Frobenius error over the 64-token blocks of every (segment, head) unit,
    blocks taken on the scan's chunk grid (from the segment start, or from its end for a
    reversed scan). Returns (worst error, where)."""
    worst, where = 0.0, None
    for (b, s, e) in segs:
        L = e - s
        if L == 0:
            continue
        xs, rs = x[b, :, s:e], ref[b, :, s:e]
        if reverse:
            xs, rs = xs[:, ::-1], rs[:, ::-1]
        nfull = L // block
        if nfull:
            H, d = xs.shape[0], xs.shape[-1]
            xb = np.ascontiguousarray(xs[:, :nfull * block]).reshape(H, nfull, block, d)
            rb = np.ascontiguousarray(rs[:, :nfull * block]).reshape(H, nfull, block, d)
            err = _rows_rel(xb, rb)
            i = np.unravel_index(int(np.argmax(err)), err.shape)
            if err[i] > worst:
                worst, where = float(err[i]), "segment (%d, %d..%d) head %d block %d" % (b, s, e, i[0], i[1])
        if L % block:
            err = _rows_rel(xs[:, nfull * block:], rs[:, nfull * block:])
            i = int(np.argmax(err))
            if err[i] > worst:
                worst, where = float(err[i]), "segment (%d, %d..%d) head %d ragged tail" % (b, s, e, i)
    return worst, where


def chunk_last_rows(x, segs, reverse=False, block=BLOCK):
    """The rows that end a chunk of the scan, stacked: [H, rows, d]."""
    rows = []
    for (b, s, e) in segs:
        L = e - s
        if L == 0:
            continue
        pos = list(range(block - 1, L, block))
        if not pos or pos[-1] != L - 1:
            pos.append(L - 1)
        idx = [s + (L - 1 - p if reverse else p) for p in pos]
        rows.append(x[b][:, idx])
    return np.concatenate(rows, axis=1)


def check_bf16_detailed(o, ro, segs, what, reverse_grids=(False,)):
    """Whole-tensor, per-block and chunk-last-row checks of a bf16 output."""
    e_all = check(o, ro, torch.bfloat16, what)
    e_blk = 0.0
    e_last = 0.0
    for rev in reverse_grids:
        eb, where = block_errors(o, ro, segs, reverse=rev)
        assert eb <= BF16_REL, "%s: 64-token block rel err %.3e > %.1e at %s" % (what, eb, BF16_REL, where)
        e_blk = max(e_blk, eb)
        el = rel_fro(chunk_last_rows(o, segs, rev), chunk_last_rows(ro, segs, rev))
        assert el <= BF16_REL, "%s: chunk-last rows rel err %.3e > %.1e" % (what, el, BF16_REL)
        e_last = max(e_last, el)
    return e_all, e_blk, e_last


def check_states(hT, rh, what):
    """Final states of every (segment, head) unit, each against the bound on its own."""
    e_all = check(hT, rh, torch.bfloat16, what)
    num = np.sqrt(np.sum((hT - rh) ** 2, axis=(-2, -1)))
    den = np.sqrt(np.sum(rh ** 2, axis=(-2, -1)))
    err = num / np.maximum(den, 1e-30)
    i = np.unravel_index(int(np.argmax(err)), err.shape)
    assert err[i] <= BF16_REL, "%s: unit %s rel err %.3e > %.1e" % (what, i, err[i], BF16_REL)
    return e_all, float(err[i])
