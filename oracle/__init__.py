"""Plain fp64 CPU oracle for the gated delta rule.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product library never does and
shares no code with it.

Two parts:

* ``scan`` / ``decode`` call ``gdr_oracle.c``: the per-token fp64 recurrence
  (see that file's header for the definition and the page passages it follows).
* ``chunked`` (module ``oracle.chunked``): the exact chunk-parallel (WY/UT) form
  written out in numpy from the "Prizma seq/delta.py" page, ``chunked_delta``;
  it is checked against the recurrence, never against the GPU.
* ``prologue`` (module ``oracle.prologue``): the steps before the recurrence (q/k
  row normalisation, gates from raw inputs) in fp64 numpy, then the recurrence.

Arrays are converted to contiguous float64 numpy before the call, so bf16 or
fp32 inputs are upcast exactly.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr_oracle.c")
_LIB = os.path.join(_HERE, "libgdr_oracle.so")

READ_PRE = 1
REVERSE = 2
ACCUMULATE = 4

_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile ``gdr_oracle.c`` into ``libgdr_oracle.so`` with gcc (plain -O2, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-fopenmp", "-shared", "-fPIC",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path):
    lib = ctypes.CDLL(path)
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.gdr_oracle_scan.argtypes = [p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i64, i64,
                                    ctypes.c_uint, p, p, ctypes.c_int]
    lib.gdr_oracle_scan.restype = ctypes.c_int
    lib.gdr_oracle_decode.argtypes = [p, p, p, p, p, p, p, p, i64, i64, i64, i64, i64,
                                      ctypes.c_uint, ctypes.c_int]
    lib.gdr_oracle_decode.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            _lib = _bind(_LIB)
    return _lib


class Variant:
    """The same ``scan`` / ``decode`` calls bound to another build of the oracle source
    (the mutation tests compile deliberately broken copies and check the pins catch them)."""

    def __init__(self, so_path):
        self._lib = _bind(so_path)

    def scan(self, *a, **kw):
        return scan(*a, _lib_override=self._lib, **kw)

    def decode(self, *a, **kw):
        return decode(*a, _lib_override=self._lib, **kw)


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor (any dtype, on CPU)
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def scan(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, *, read: str = "post",
         reverse: bool = False, out=None, want_state: bool = True, threads: int = 0,
         _lib_override=None):
    """Per-token fp64 scan.

    q, k: [B, Hk, T, dk]; v: [B, Hv, T, dv]; log_alpha, beta: [B, Hv, T];
    h0: [nseq, Hv, dk, dv] or None (zero state); cu_seqlens: nseq+1 offsets or None.
    ``out`` (float64 [B, Hv, T, dv]) turns on accumulation into it.
    Returns (o float64 [B, Hv, T, dv], hT float64 [nseq, Hv, dk, dv] or None).
    """
    lib = _lib_override or _load()
    q, k, v, la, b = (_f64(t) for t in (q, k, v, log_alpha, beta))
    B, Hk, T, dk = q.shape
    Hv, dv = v.shape[1], v.shape[3]
    assert k.shape == q.shape and v.shape == (B, Hv, T, dv)
    assert la.shape == (B, Hv, T) and b.shape == (B, Hv, T)
    cu = None
    nseq = B
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(
            cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens, dtype=np.int64))
        nseq = cu.shape[0] - 1
    h0a = _f64(h0)
    if h0a is not None:
        assert h0a.shape == (nseq, Hv, dk, dv), h0a.shape
    flags = (READ_PRE if read == "pre" else 0) | (REVERSE if reverse else 0)
    if out is not None:
        o = out
        assert o.dtype == np.float64 and o.flags["C_CONTIGUOUS"] and o.shape == (B, Hv, T, dv)
        flags |= ACCUMULATE
    else:
        o = np.zeros((B, Hv, T, dv), dtype=np.float64)
    hT = np.zeros((nseq, Hv, dk, dv), dtype=np.float64) if want_state else None
    rc = lib.gdr_oracle_scan(_ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(b), _ptr(h0a), _ptr(cu),
                             nseq, B, T, Hk, Hv, dk, dv, flags, _ptr(o), _ptr(hT), int(threads))
    if rc != 0:
        raise ValueError("gdr_oracle_scan rejected its arguments (rc=%d)" % rc)
    return o, hT


def decode(q, k, v, log_alpha, beta, state, *, read: str = "post", threads: int = 0,
           _lib_override=None):
    """One fp64 decode step. q, k: [N, Hk, dk]; v: [N, Hv, dv]; log_alpha, beta: [N, Hv];
    state: [N, Hv, dk, dv]. Returns (o [N, Hv, dv], new_state [N, Hv, dk, dv])."""
    lib = _lib_override or _load()
    q, k, v, la, b, s = (_f64(t) for t in (q, k, v, log_alpha, beta, state))
    N, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    assert s.shape == (N, Hv, dk, dv) and la.shape == (N, Hv) and b.shape == (N, Hv)
    o = np.zeros((N, Hv, dv), dtype=np.float64)
    ns = np.empty_like(s)
    rc = lib.gdr_oracle_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(b), _ptr(s), _ptr(ns),
                               _ptr(o), N, Hk, Hv, dk, dv, READ_PRE if read == "pre" else 0,
                               int(threads))
    if rc != 0:
        raise ValueError("gdr_oracle_decode rejected its arguments (rc=%d)" % rc)
    return o, ns
