"""Python binding of ``libgdr.so`` (the C ABI in include/gdr.h).

Argument marshalling only: torch tensors are checked for device, dtype, shape and
contiguity, their device pointers and the current HIP stream are handed to the C entry
points, and a non-zero status is raised as ``GdrError``. Every step of the computation
runs in the library's HIP kernels. There is no fallback: if the library is missing the
import fails with an error that says how to build it.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdr.so")

GDR_F32, GDR_BF16 = 0, 1
GDR_READ_PRE, GDR_REVERSE, GDR_ACCUMULATE, GDR_QK_L2NORM = 1, 2, 4, 8

STATUS = {0: "GDR_OK", 1: "GDR_ERR_NULL", 2: "GDR_ERR_DIMS", 3: "GDR_ERR_DTYPE", 4: "GDR_ERR_CHUNK",
          5: "GDR_ERR_ALIGN", 6: "GDR_ERR_ALIAS", 7: "GDR_ERR_UNSUPPORTED", 8: "GDR_ERR_FLAGS",
          9: "GDR_ERR_HIP"}

# every symbol include/gdr.h declares
EXPORTS = ("gdr_chunk_fwd", "gdr_chunk_fwd_bidir", "gdr_chunk_fwd_gated", "gdr_decode_step", "gdr_decode_step_gated",
           "gdr_gdn2_chunk_fwd", "gdr_gdn2_chunk_fwd_bidir", "gdr_gdn2_chunk_fwd_noalloc", "gdr_gdn2_chunk_fwd_workspace_bytes",
           "gdr_gdn2_decode_step",
           "gdr_delta_product_fwd",
           "gdr_chunk_bwd", "gdr_chunk_bwd_workspace_bytes",
           "gdr_status_string", "gdr_last_error", "gdr_abi_version", "gdr_selftest_mfma")


class GdrError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__("%s: %s" % (self.name, detail))


class ChunkDims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("Hk", ctypes.c_int64),
                ("Hv", ctypes.c_int64), ("dk", ctypes.c_int64), ("dv", ctypes.c_int64),
                ("num_seqs", ctypes.c_int64), ("dtype", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class DecodeDims(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64), ("Hk", ctypes.c_int64), ("Hv", ctypes.c_int64),
                ("dk", ctypes.c_int64), ("dv", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError("%s is missing: build it with `python -m gated_delta_rule_70_amd.build` "
                          "(there is no fallback path)" % path)
    lib = ctypes.CDLL(path)
    p, i32 = ctypes.c_void_p, ctypes.c_int32
    lib.gdr_chunk_fwd.argtypes = [p, p, p, p, p, p, p, i32, p, p, ctypes.POINTER(ChunkDims), p]
    lib.gdr_chunk_fwd.restype = ctypes.c_int
    lib.gdr_chunk_fwd_gated.argtypes = [p, p, p, p, p, p, p, p, p, i32, p, p, ctypes.POINTER(ChunkDims), p]
    lib.gdr_chunk_fwd_gated.restype = ctypes.c_int
    lib.gdr_chunk_fwd_bidir.argtypes = [p] * 10 + [i32, p, p, p, ctypes.POINTER(ChunkDims), p]
    lib.gdr_chunk_fwd_bidir.restype = ctypes.c_int
    lib.gdr_decode_step.argtypes = [p, p, p, p, p, p, p, p, ctypes.POINTER(DecodeDims), p]
    lib.gdr_decode_step.restype = ctypes.c_int
    lib.gdr_decode_step_gated.argtypes = [p, p, p, p, p, p, p, p, p, p, ctypes.POINTER(DecodeDims), p]
    lib.gdr_decode_step_gated.restype = ctypes.c_int
    lib.gdr_chunk_bwd.argtypes = [p] * 15 + [p, ctypes.c_int64, ctypes.POINTER(ChunkDims), p]
    lib.gdr_chunk_bwd.restype = ctypes.c_int
    lib.gdr_chunk_bwd_workspace_bytes.argtypes = [ctypes.POINTER(ChunkDims), i32]
    lib.gdr_chunk_bwd_workspace_bytes.restype = ctypes.c_int64
    lib.gdr_delta_product_fwd.argtypes = [p, p, p, p, p, p, p, i32, i32, p, p, ctypes.POINTER(ChunkDims), p]
    lib.gdr_delta_product_fwd.restype = ctypes.c_int
    lib.gdr_gdn2_chunk_fwd.argtypes = [p, p, p, p, p, p, p, p, i32, p, p, p, ctypes.c_int64,
                                       ctypes.POINTER(ChunkDims), p]
    lib.gdr_gdn2_chunk_fwd.restype = ctypes.c_int
    lib.gdr_gdn2_chunk_fwd_bidir.argtypes = [p] * 11 + [p, i32, p, p, p, p, ctypes.c_int64, ctypes.POINTER(ChunkDims), p]
    lib.gdr_gdn2_chunk_fwd_bidir.restype = ctypes.c_int
    lib.gdr_gdn2_chunk_fwd_noalloc.argtypes = [p, p, p, p, p, p, p, p, i32, p, p, ctypes.POINTER(ChunkDims), p]
    lib.gdr_gdn2_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.gdr_gdn2_chunk_fwd_workspace_bytes.argtypes = [ctypes.POINTER(ChunkDims), i32, i32]
    lib.gdr_gdn2_chunk_fwd_workspace_bytes.restype = ctypes.c_int64
    lib.gdr_gdn2_decode_step.argtypes = [p, p, p, p, p, p, p, p, p, ctypes.POINTER(DecodeDims), p]
    lib.gdr_gdn2_decode_step.restype = ctypes.c_int
    lib.gdr_status_string.argtypes = [ctypes.c_int]
    lib.gdr_status_string.restype = ctypes.c_char_p
    lib.gdr_last_error.argtypes = []
    lib.gdr_last_error.restype = ctypes.c_char_p
    lib.gdr_abi_version.argtypes = []
    lib.gdr_abi_version.restype = ctypes.c_int32
    lib.gdr_selftest_mfma.argtypes = [p, p, p, p]
    lib.gdr_selftest_mfma.restype = ctypes.c_int
    return lib


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = load()
    return _lib


def _check(status: int):
    if status != 0:
        raise GdrError(status, lib().gdr_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t, name, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor (got %s)" % (name, t.device))
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s (got %s)" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _dtype_code(dt):
    if dt == torch.bfloat16:
        return GDR_BF16
    if dt == torch.float32:
        return GDR_F32
    raise ValueError("q, k, v must be bfloat16 or float32 (got %s)" % dt)


def chunk_fwd(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, *, chunk: int = 64,
              read: str = "post", reverse: bool = False, out=None, accumulate: bool = False,
              hT=None, want_state: bool = True, l2norm: bool = False):
    """Chunked forward (``gdr_chunk_fwd``).

    q, k [B, Hk, T, dk]; v [B, Hv, T, dv] (bf16 or fp32, same dtype); log_alpha, beta
    [B, Hv, T] fp32; h0 [S, Hv, dk, dv] fp32 or None; cu_seqlens int32 [S+1] (device) or
    None. Returns (out [B, Hv, T, dv], hT [S, Hv, dk, dv] or None). ``out`` may be given
    (required for ``accumulate``); ``hT`` may be given (it may be ``h0`` itself).
    ``l2norm`` normalises each row of q and k in the kernel (``GDR_QK_L2NORM``).
    """
    return _chunk(q, k, v, log_alpha, beta, None, None, h0, cu_seqlens, chunk, read, reverse, out,
                  accumulate, hT, want_state, l2norm)


def chunk_fwd_gated(q, k, v, a, b, A_log, dt_bias, h0=None, cu_seqlens=None, *, chunk: int = 64,
                    read: str = "post", reverse: bool = False, out=None, accumulate: bool = False,
                    hT=None, want_state: bool = True, l2norm: bool = True):
    """Chunked forward with the gates formed in the kernel (``gdr_chunk_fwd_gated``): a, b
    [B, Hv, T] fp32 raw inputs, A_log, dt_bias [Hv] fp32; the rest as ``chunk_fwd``."""
    return _chunk(q, k, v, a, b, A_log, dt_bias, h0, cu_seqlens, chunk, read, reverse, out,
                  accumulate, hT, want_state, l2norm)


def chunk_fwd_bidir(q, k, v, log_alpha_fwd, beta_fwd, log_alpha_rev, beta_rev, h0_fwd=None, h0_rev=None,
                    cu_seqlens=None, *, chunk: int = 64, read: str = "pre", out=None, accumulate: bool = False,
                    want_state: bool = True, l2norm: bool = False):
    """Both scans of a bidirectional layer, summed per token (``gdr_chunk_fwd_bidir``): the
    forward scan and the in-segment reversed scan, each with its own gates [B, Hv, T] fp32 (indexed
    by token) and initial state [S, Hv, dk, dv] fp32 or None, the same ``read`` for both. Returns
    (out [B, Hv, T, dv], hT_fwd, hT_rev), the final states None without ``want_state``."""
    _need(q, "q")
    dev, dt = q.device, q.dtype
    code = _dtype_code(dt)
    B, Hk, T, dk = q.shape
    Hv, dv = v.shape[1], v.shape[3]
    _need(k, "k", dt, (B, Hk, T, dk), dev)
    _need(v, "v", dt, (B, Hv, T, dv), dev)
    for t, n in ((log_alpha_fwd, "log_alpha_fwd"), (beta_fwd, "beta_fwd"), (log_alpha_rev, "log_alpha_rev"),
                 (beta_rev, "beta_rev")):
        _need(t, n, torch.float32, (B, Hv, T), dev)
    S = B
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, None, dev)
        S = cu_seqlens.shape[0] - 1
    for t, n in ((h0_fwd, "h0_fwd"), (h0_rev, "h0_rev")):
        if t is not None:
            _need(t, n, torch.float32, (S, Hv, dk, dv), dev)
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs an existing out tensor")
        out = torch.empty((B, Hv, T, dv), dtype=dt, device=dev)
    else:
        _need(out, "out", dt, (B, Hv, T, dv), dev)
    hT_f = hT_r = None
    if want_state:
        hT_f = torch.empty((S, Hv, dk, dv), dtype=torch.float32, device=dev)
        hT_r = torch.empty((S, Hv, dk, dv), dtype=torch.float32, device=dev)
    if read not in ("pre", "post"):
        raise ValueError("read must be 'pre' or 'post'")
    flags = (GDR_READ_PRE if read == "pre" else 0) | (GDR_ACCUMULATE if accumulate else 0) | \
        (GDR_QK_L2NORM if l2norm else 0)
    dims = ChunkDims(B, T, Hk, Hv, dk, dv, S if cu_seqlens is not None else 0, code, flags)
    _check(lib().gdr_chunk_fwd_bidir(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha_fwd), _ptr(beta_fwd),
                                     _ptr(log_alpha_rev), _ptr(beta_rev), _ptr(h0_fwd), _ptr(h0_rev),
                                     _ptr(cu_seqlens), int(chunk), _ptr(out), _ptr(hT_f), _ptr(hT_r),
                                     ctypes.byref(dims), _stream(q)))
    return out, hT_f, hT_r


def _chunk(q, k, v, ga, gb, A_log, dt_bias, h0, cu_seqlens, chunk, read, reverse, out, accumulate,
           hT, want_state, l2norm):
    gated = A_log is not None or dt_bias is not None
    na, nb = ("a", "b") if gated else ("log_alpha", "beta")
    _need(q, "q")
    dev = q.device
    dt = q.dtype
    code = _dtype_code(dt)
    B, Hk, T, dk = q.shape
    Hv, dv = v.shape[1], v.shape[3]
    _need(k, "k", dt, (B, Hk, T, dk), dev)
    _need(v, "v", dt, (B, Hv, T, dv), dev)
    _need(ga, na, torch.float32, (B, Hv, T), dev)
    _need(gb, nb, torch.float32, (B, Hv, T), dev)
    if gated:
        _need(A_log, "A_log", torch.float32, (Hv,), dev)
        _need(dt_bias, "dt_bias", torch.float32, (Hv,), dev)
    S = B
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, None, dev)
        S = cu_seqlens.shape[0] - 1
    if h0 is not None:
        _need(h0, "h0", torch.float32, (S, Hv, dk, dv), dev)
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs an existing out tensor")
        out = torch.empty((B, Hv, T, dv), dtype=dt, device=dev)
    else:
        _need(out, "out", dt, (B, Hv, T, dv), dev)
    if hT is None and want_state:
        hT = torch.empty((S, Hv, dk, dv), dtype=torch.float32, device=dev)
    elif hT is not None:
        _need(hT, "hT", torch.float32, (S, Hv, dk, dv), dev)
    if read not in ("pre", "post"):
        raise ValueError("read must be 'pre' or 'post'")
    flags = (GDR_READ_PRE if read == "pre" else 0) | (GDR_REVERSE if reverse else 0) | \
        (GDR_ACCUMULATE if accumulate else 0) | (GDR_QK_L2NORM if l2norm else 0)
    dims = ChunkDims(B, T, Hk, Hv, dk, dv, S if cu_seqlens is not None else 0, code, flags)
    if gated:
        _check(lib().gdr_chunk_fwd_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(ga), _ptr(gb), _ptr(A_log),
                                         _ptr(dt_bias), _ptr(h0), _ptr(cu_seqlens), int(chunk), _ptr(out),
                                         _ptr(hT), ctypes.byref(dims), _stream(q)))
    else:
        _check(lib().gdr_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(ga), _ptr(gb), _ptr(h0),
                                   _ptr(cu_seqlens), int(chunk), _ptr(out), _ptr(hT),
                                   ctypes.byref(dims), _stream(q)))
    return out, hT


def decode_step(q, k, v, log_alpha, beta, state_in, state_out=None, out=None, *, read: str = "post",
                l2norm: bool = False):
    """One decode step (``gdr_decode_step``). q, k [N, Hk, dk]; v [N, Hv, dv]; log_alpha,
    beta [N, Hv] fp32; state_in [N, Hv, dk, dv] fp32. ``state_out`` defaults to a new
    tensor; pass ``state_in`` itself to update in place. Returns (out, state_out).
    ``l2norm`` normalises q and k in the kernel (``GDR_QK_L2NORM``)."""
    return _decode(q, k, v, log_alpha, beta, None, None, state_in, state_out, out, read, l2norm)


def decode_step_gated(q, k, v, a, b, A_log, dt_bias, state_in, state_out=None, out=None, *,
                      read: str = "post", l2norm: bool = True):
    """One decode step with the gates formed in the kernel (``gdr_decode_step_gated``): a, b
    [N, Hv] fp32 raw inputs, A_log, dt_bias [Hv] fp32; the rest as ``decode_step``."""
    return _decode(q, k, v, a, b, A_log, dt_bias, state_in, state_out, out, read, l2norm)


def _decode(q, k, v, ga, gb, A_log, dt_bias, state_in, state_out, out, read, l2norm):
    gated = A_log is not None or dt_bias is not None
    na, nb = ("a", "b") if gated else ("log_alpha", "beta")
    _need(q, "q")
    dev, dt = q.device, q.dtype
    code = _dtype_code(dt)
    N, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    _need(k, "k", dt, (N, Hk, dk), dev)
    _need(v, "v", dt, (N, Hv, dv), dev)
    _need(ga, na, torch.float32, (N, Hv), dev)
    _need(gb, nb, torch.float32, (N, Hv), dev)
    if gated:
        _need(A_log, "A_log", torch.float32, (Hv,), dev)
        _need(dt_bias, "dt_bias", torch.float32, (Hv,), dev)
    _need(state_in, "state_in", torch.float32, (N, Hv, dk, dv), dev)
    if state_out is None:
        state_out = torch.empty_like(state_in)
    else:
        _need(state_out, "state_out", torch.float32, (N, Hv, dk, dv), dev)
    if out is None:
        out = torch.empty((N, Hv, dv), dtype=dt, device=dev)
    else:
        _need(out, "out", dt, (N, Hv, dv), dev)
    if read not in ("pre", "post"):
        raise ValueError("read must be 'pre' or 'post'")
    flags = (GDR_READ_PRE if read == "pre" else 0) | (GDR_QK_L2NORM if l2norm else 0)
    dims = DecodeDims(N, Hk, Hv, dk, dv, code, flags)
    if gated:
        _check(lib().gdr_decode_step_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(ga), _ptr(gb), _ptr(A_log),
                                           _ptr(dt_bias), _ptr(state_in), _ptr(state_out), _ptr(out),
                                           ctypes.byref(dims), _stream(q)))
    else:
        _check(lib().gdr_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(ga), _ptr(gb), _ptr(state_in),
                                     _ptr(state_out), _ptr(out), ctypes.byref(dims), _stream(q)))
    return out, state_out


def chunk_bwd(q, k, v, log_alpha, beta, dout, h0=None, cu_seqlens=None, dhT=None, *, read: str = "post",
              reverse: bool = False, want_dh0: bool = True, workspace=None):
    """Gradients of ``chunk_fwd`` (``gdr_chunk_bwd``): the inputs as given to the forward, dout
    [B, Hv, T, dv] in their dtype, dhT [S, Hv, dk, dv] fp32 or None. Returns fp32 tensors
    (dq, dk, dv, dlog_alpha, dbeta, dh0 or None). ``workspace`` (a uint8 GPU tensor of at least
    ``chunk_bwd_workspace_bytes`` bytes) is allocated here when not given."""
    _need(q, "q")
    dev, dt = q.device, q.dtype
    code = _dtype_code(dt)
    B, Hk, T, dk = q.shape
    Hv, dv = v.shape[1], v.shape[3]
    _need(k, "k", dt, (B, Hk, T, dk), dev)
    _need(v, "v", dt, (B, Hv, T, dv), dev)
    _need(dout, "dout", dt, (B, Hv, T, dv), dev)
    _need(log_alpha, "log_alpha", torch.float32, (B, Hv, T), dev)
    _need(beta, "beta", torch.float32, (B, Hv, T), dev)
    S = B
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, None, dev)
        S = cu_seqlens.shape[0] - 1
    for name, t in (("h0", h0), ("dhT", dhT)):
        if t is not None:
            _need(t, name, torch.float32, (S, Hv, dk, dv), dev)
    if read not in ("pre", "post"):
        raise ValueError("read must be 'pre' or 'post'")
    flags = (GDR_READ_PRE if read == "pre" else 0) | (GDR_REVERSE if reverse else 0)
    dims = ChunkDims(B, T, Hk, Hv, dk, dv, S if cu_seqlens is not None else 0, code, flags)
    need = lib().gdr_chunk_bwd_workspace_bytes(ctypes.byref(dims), int(cu_seqlens is not None))
    if need < 0:
        raise ValueError("invalid sizes for the backward workspace")
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    elif workspace.numel() < need:
        raise ValueError("workspace holds %d bytes, %d needed" % (workspace.numel(), need))
    f32 = dict(dtype=torch.float32, device=dev)
    dq, dk_ = torch.empty((B, Hk, T, dk), **f32), torch.empty((B, Hk, T, dk), **f32)
    dv_ = torch.empty((B, Hv, T, dv), **f32)
    dla, dbe = torch.empty((B, Hv, T), **f32), torch.empty((B, Hv, T), **f32)
    dh0 = torch.empty((S, Hv, dk, dv), **f32) if want_dh0 else None
    _check(lib().gdr_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(h0), _ptr(cu_seqlens),
                               _ptr(dout), _ptr(dhT), _ptr(dq), _ptr(dk_), _ptr(dv_), _ptr(dla), _ptr(dbe), _ptr(dh0),
                               _ptr(workspace), ctypes.c_int64(workspace.numel()), ctypes.byref(dims), _stream(q)))
    return dq, dk_, dv_, dla, dbe, dh0


def chunk_bwd_workspace_bytes(B, T, Hk, Hv, dk, dv, num_seqs=0, dtype=torch.bfloat16) -> int:
    """Bytes of workspace ``gdr_chunk_bwd`` needs (num_seqs > 0: packed sequences)."""
    dims = ChunkDims(B, T, Hk, Hv, dk, dv, num_seqs, _dtype_code(dtype), 0)
    return int(lib().gdr_chunk_bwd_workspace_bytes(ctypes.byref(dims), int(num_seqs > 0)))


def delta_product_fwd(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, *, chunk: int = 64,
                      read: str = "pre", out=None, accumulate: bool = False, hT=None, want_state: bool = True,
                      l2norm: bool = False):
    """DeltaProduct forward (``gdr_delta_product_fwd``): q [B, Hk, T, dk]; k [B, Hk, T, n, dk];
    v [B, Hv, T, n, dv]; log_alpha [B, Hv, T] fp32; beta [B, Hv, T, n] fp32. ``read`` defaults
    to the pre-write read of the page this variant comes from. Returns (out, hT)."""
    _need(q, "q")
    dev, dt = q.device, q.dtype
    code = _dtype_code(dt)
    B, Hk, T, dk = q.shape
    n = k.shape[3]
    Hv, dv = v.shape[1], v.shape[4]
    _need(k, "k", dt, (B, Hk, T, n, dk), dev)
    _need(v, "v", dt, (B, Hv, T, n, dv), dev)
    _need(log_alpha, "log_alpha", torch.float32, (B, Hv, T), dev)
    _need(beta, "beta", torch.float32, (B, Hv, T, n), dev)
    S = B
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, None, dev)
        S = cu_seqlens.shape[0] - 1
    if h0 is not None:
        _need(h0, "h0", torch.float32, (S, Hv, dk, dv), dev)
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs an existing out tensor")
        out = torch.empty((B, Hv, T, dv), dtype=dt, device=dev)
    else:
        _need(out, "out", dt, (B, Hv, T, dv), dev)
    if hT is None and want_state:
        hT = torch.empty((S, Hv, dk, dv), dtype=torch.float32, device=dev)
    elif hT is not None:
        _need(hT, "hT", torch.float32, (S, Hv, dk, dv), dev)
    if read not in ("pre", "post"):
        raise ValueError("read must be 'pre' or 'post'")
    flags = (GDR_READ_PRE if read == "pre" else 0) | (GDR_ACCUMULATE if accumulate else 0) | \
        (GDR_QK_L2NORM if l2norm else 0)
    dims = ChunkDims(B, T, Hk, Hv, dk, dv, S if cu_seqlens is not None else 0, code, flags)
    _check(lib().gdr_delta_product_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(h0),
                                       _ptr(cu_seqlens), int(n), int(chunk), _ptr(out), _ptr(hT),
                                       ctypes.byref(dims), _stream(q)))
    return out, hT


def gdn2_chunk_fwd(q, k, v, g, b, w, h0=None, cu_seqlens=None, *, chunk: int = 64, read: str = "post",
                   reverse: bool = False, out=None, accumulate: bool = False, hT=None, want_state: bool = True,
                   l2norm: bool = False, workspace=None, fused: bool = False):
    """GDN-2 chunked forward (``gdr_gdn2_chunk_fwd``).

    q, k [B, Hk, T, dk] and v [B, Hv, T, dv] (bf16 or fp32, one dtype); g [B, Hk, T, dk] fp32 log
    decay per key channel; b [B, Hk, T, dk] erase gate and w [B, Hv, T, dv] write gate in the
    dtype of q. The rest as ``chunk_fwd``. The two-pass form runs with ``workspace`` (a uint8 GPU
    tensor of at least ``gdn2_chunk_fwd_workspace_bytes`` bytes, allocated here when not given);
    ``fused=True`` passes no workspace and runs the one-pass kernel.
    """
    _need(q, "q")
    dev, dt = q.device, q.dtype
    code = _dtype_code(dt)
    B, Hk, T, dk = q.shape
    Hv, dv = v.shape[1], v.shape[3]
    _need(k, "k", dt, (B, Hk, T, dk), dev)
    _need(v, "v", dt, (B, Hv, T, dv), dev)
    _need(g, "g", torch.float32, (B, Hk, T, dk), dev)
    _need(b, "b", dt, (B, Hk, T, dk), dev)
    _need(w, "w", dt, (B, Hv, T, dv), dev)
    S = B
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, None, dev)
        S = cu_seqlens.shape[0] - 1
    if h0 is not None:
        _need(h0, "h0", torch.float32, (S, Hv, dk, dv), dev)
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs an existing out tensor")
        out = torch.empty((B, Hv, T, dv), dtype=dt, device=dev)
    else:
        _need(out, "out", dt, (B, Hv, T, dv), dev)
    if hT is None and want_state:
        hT = torch.empty((S, Hv, dk, dv), dtype=torch.float32, device=dev)
    elif hT is not None:
        _need(hT, "hT", torch.float32, (S, Hv, dk, dv), dev)
    if read not in ("pre", "post"):
        raise ValueError("read must be 'pre' or 'post'")
    flags = (GDR_READ_PRE if read == "pre" else 0) | (GDR_REVERSE if reverse else 0) | \
        (GDR_ACCUMULATE if accumulate else 0) | (GDR_QK_L2NORM if l2norm else 0)
    dims = ChunkDims(B, T, Hk, Hv, dk, dv, S if cu_seqlens is not None else 0, code, flags)
    ws_ptr, ws_bytes = None, 0
    if not fused:
        need = lib().gdr_gdn2_chunk_fwd_workspace_bytes(ctypes.byref(dims), int(chunk), int(cu_seqlens is not None))
        if need < 0:
            raise ValueError("invalid sizes for the GDN-2 workspace")
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        _need(workspace, "workspace", torch.uint8, None, dev)
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel()
    _check(lib().gdr_gdn2_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(w), _ptr(h0),
                                    _ptr(cu_seqlens), int(chunk), _ptr(out), _ptr(hT), ws_ptr, ws_bytes,
                                    ctypes.byref(dims), _stream(q)))
    return out, hT


def gdn2_chunk_fwd_bidir(q, k, v, fwd_gates, rev_gates, h0_fwd=None, h0_rev=None, cu_seqlens=None, *,
                         chunk: int = 64, read: str = "pre", out=None, accumulate: bool = False,
                         want_state: bool = True, l2norm: bool = False, workspace=None, fused: bool = False):
    """Both GDN-2 scans of a bidirectional layer, summed per token (``gdr_gdn2_chunk_fwd_bidir``):
    ``fwd_gates`` and ``rev_gates`` are (g, b, w) triples in ``gdn2_chunk_fwd``'s layouts; the rest
    as ``chunk_fwd_bidir`` and ``gdn2_chunk_fwd`` (one workspace serves both passes). Returns
    (out, hT_fwd, hT_rev)."""
    _need(q, "q")
    dev, dt = q.device, q.dtype
    code = _dtype_code(dt)
    B, Hk, T, dk = q.shape
    Hv, dv = v.shape[1], v.shape[3]
    _need(k, "k", dt, (B, Hk, T, dk), dev)
    _need(v, "v", dt, (B, Hv, T, dv), dev)
    for name, (g, b, w) in (("fwd", fwd_gates), ("rev", rev_gates)):
        _need(g, "g_" + name, torch.float32, (B, Hk, T, dk), dev)
        _need(b, "b_" + name, dt, (B, Hk, T, dk), dev)
        _need(w, "w_" + name, dt, (B, Hv, T, dv), dev)
    S = B
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, None, dev)
        S = cu_seqlens.shape[0] - 1
    for t, n in ((h0_fwd, "h0_fwd"), (h0_rev, "h0_rev")):
        if t is not None:
            _need(t, n, torch.float32, (S, Hv, dk, dv), dev)
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs an existing out tensor")
        out = torch.empty((B, Hv, T, dv), dtype=dt, device=dev)
    else:
        _need(out, "out", dt, (B, Hv, T, dv), dev)
    hT_f = hT_r = None
    if want_state:
        hT_f = torch.empty((S, Hv, dk, dv), dtype=torch.float32, device=dev)
        hT_r = torch.empty((S, Hv, dk, dv), dtype=torch.float32, device=dev)
    if read not in ("pre", "post"):
        raise ValueError("read must be 'pre' or 'post'")
    flags = (GDR_READ_PRE if read == "pre" else 0) | (GDR_ACCUMULATE if accumulate else 0) | \
        (GDR_QK_L2NORM if l2norm else 0)
    dims = ChunkDims(B, T, Hk, Hv, dk, dv, S if cu_seqlens is not None else 0, code, flags)
    ws_ptr, ws_bytes = None, 0
    if not fused:
        need = lib().gdr_gdn2_chunk_fwd_workspace_bytes(ctypes.byref(dims), int(chunk), int(cu_seqlens is not None))
        if need < 0:
            raise ValueError("invalid sizes for the GDN-2 workspace")
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        _need(workspace, "workspace", torch.uint8, None, dev)
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel()
    (gf, bf, wf), (gr, br, wr) = fwd_gates, rev_gates
    _check(lib().gdr_gdn2_chunk_fwd_bidir(_ptr(q), _ptr(k), _ptr(v), _ptr(gf), _ptr(bf), _ptr(wf), _ptr(gr),
                                          _ptr(br), _ptr(wr), _ptr(h0_fwd), _ptr(h0_rev), _ptr(cu_seqlens), int(chunk),
                                          _ptr(out), _ptr(hT_f), _ptr(hT_r), ws_ptr, ws_bytes, ctypes.byref(dims),
                                          _stream(q)))
    return out, hT_f, hT_r


def gdn2_chunk_fwd_noalloc(q, k, v, g, b, w, h0, cu_seqlens, out, hT, *, chunk: int = 64, read: str = "post",
                           reverse: bool = False, accumulate: bool = False, l2norm: bool = False):
    """``gdr_gdn2_chunk_fwd_noalloc``: the two-pass GDN-2 forward on the library's fixed device
    scratch (no workspace, nothing allocated by the call). Arguments as ``gdn2_chunk_fwd``; ``out``
    and ``hT`` (or None for no final state) must be given, so that nothing is allocated here either."""
    _need(q, "q")
    dev, dt = q.device, q.dtype
    B, Hk, T, dk = q.shape
    Hv, dv = v.shape[1], v.shape[3]
    for name, t, tdt, shape in (("k", k, dt, (B, Hk, T, dk)), ("v", v, dt, (B, Hv, T, dv)),
                                ("g", g, torch.float32, (B, Hk, T, dk)), ("b", b, dt, (B, Hk, T, dk)),
                                ("w", w, dt, (B, Hv, T, dv)), ("out", out, dt, (B, Hv, T, dv))):
        _need(t, name, tdt, shape, dev)
    S = B
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, None, dev)
        S = cu_seqlens.shape[0] - 1
    for name, t in (("h0", h0), ("hT", hT)):
        if t is not None:
            _need(t, name, torch.float32, (S, Hv, dk, dv), dev)
    if read not in ("pre", "post"):
        raise ValueError("read must be 'pre' or 'post'")
    flags = (GDR_READ_PRE if read == "pre" else 0) | (GDR_REVERSE if reverse else 0) | \
        (GDR_ACCUMULATE if accumulate else 0) | (GDR_QK_L2NORM if l2norm else 0)
    dims = ChunkDims(B, T, Hk, Hv, dk, dv, S if cu_seqlens is not None else 0, _dtype_code(dt), flags)
    _check(lib().gdr_gdn2_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(w), _ptr(h0),
                                            _ptr(cu_seqlens), int(chunk), _ptr(out), _ptr(hT), ctypes.byref(dims),
                                            _stream(q)))
    return out, hT


def gdn2_chunk_fwd_workspace_bytes(B, T, Hk, Hv, dk, dv, chunk, num_seqs=0, dtype=torch.bfloat16) -> int:
    """Bytes of workspace the two-pass ``gdr_gdn2_chunk_fwd`` needs (num_seqs > 0: packed)."""
    dims = ChunkDims(B, T, Hk, Hv, dk, dv, num_seqs, _dtype_code(dtype), 0)
    return int(lib().gdr_gdn2_chunk_fwd_workspace_bytes(ctypes.byref(dims), int(chunk), int(num_seqs > 0)))


def gdn2_decode_step(q, k, v, g, b, w, state_in, state_out=None, out=None, *, read: str = "post",
                     l2norm: bool = False):
    """One GDN-2 decode step (``gdr_gdn2_decode_step``). q, k, b [N, Hk, dk] and v, w [N, Hv, dv]
    in one dtype; g [N, Hk, dk] fp32; state_in [N, Hv, dk, dv] fp32. Returns (out, state_out)."""
    _need(q, "q")
    dev, dt = q.device, q.dtype
    code = _dtype_code(dt)
    N, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    _need(k, "k", dt, (N, Hk, dk), dev)
    _need(b, "b", dt, (N, Hk, dk), dev)
    _need(g, "g", torch.float32, (N, Hk, dk), dev)
    _need(v, "v", dt, (N, Hv, dv), dev)
    _need(w, "w", dt, (N, Hv, dv), dev)
    _need(state_in, "state_in", torch.float32, (N, Hv, dk, dv), dev)
    if state_out is None:
        state_out = torch.empty_like(state_in)
    else:
        _need(state_out, "state_out", torch.float32, (N, Hv, dk, dv), dev)
    if out is None:
        out = torch.empty((N, Hv, dv), dtype=dt, device=dev)
    else:
        _need(out, "out", dt, (N, Hv, dv), dev)
    if read not in ("pre", "post"):
        raise ValueError("read must be 'pre' or 'post'")
    flags = (GDR_READ_PRE if read == "pre" else 0) | (GDR_QK_L2NORM if l2norm else 0)
    dims = DecodeDims(N, Hk, Hv, dk, dv, code, flags)
    _check(lib().gdr_gdn2_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(w), _ptr(state_in),
                                      _ptr(state_out), _ptr(out), ctypes.byref(dims), _stream(q)))
    return out, state_out


def selftest_mfma(a, b):
    """Diagnostic: the 16x16 product of a [16, 32] and b [32, 16] (fp32 GPU tensors) through
    the library's matrix-core operand layouts. Returns d [3, 16, 16] (see include/gdr.h)."""
    _need(a, "a", torch.float32, (16, 32))
    _need(b, "b", torch.float32, (32, 16), a.device)
    d = torch.empty((3, 16, 16), dtype=torch.float32, device=a.device)
    _check(lib().gdr_selftest_mfma(_ptr(a), _ptr(b), _ptr(d), _stream(a)))
    return d
