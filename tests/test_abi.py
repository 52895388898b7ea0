"""The C-ABI library on the CPU: it loads, exports every symbol include/gdr.h declares, and
its host-side validation rejects bad arguments before touching the GPU (no compute here)."""
import ctypes
import os
import re

import pytest

from gated_delta_rule_70_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")

needs_lib = pytest.mark.skipif(not os.path.exists(binding.LIB_PATH),
                               reason="libgdr.so not built (run __graft_entry__.build())")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_binding_exports():
    assert _declared() == sorted(binding.EXPORTS)


@needs_lib
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(binding.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
    assert binding.load().gdr_abi_version() == 1


FAKE = 1 << 20  # a 16-byte aligned non-NULL address that is never dereferenced


def _chunk(lib, **over):
    d = dict(B=1, T=128, Hk=2, Hv=2, dk=64, dv=64, num_seqs=0, dtype=1, flags=0)
    ptr = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, la=FAKE * 4, beta=FAKE * 5, h0=None, cu=None,
               out=FAKE * 6, hT=None, chunk=64)
    for k_, v_ in over.items():
        (d if k_ in d else ptr)[k_] = v_
    dims = binding.ChunkDims(d["B"], d["T"], d["Hk"], d["Hv"], d["dk"], d["dv"], d["num_seqs"],
                             d["dtype"], d["flags"])
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    st = lib.gdr_chunk_fwd(vp(ptr["q"]), vp(ptr["k"]), vp(ptr["v"]), vp(ptr["la"]), vp(ptr["beta"]),
                           vp(ptr["h0"]), vp(ptr["cu"]), ptr["chunk"], vp(ptr["out"]), vp(ptr["hT"]),
                           ctypes.byref(dims), None)
    return binding.STATUS[st], lib.gdr_last_error().decode()


CHUNK_REJECTS = [
    (dict(chunk=48), "GDR_ERR_CHUNK", "chunk"),
    (dict(chunk=128), "GDR_ERR_CHUNK", "chunk"),
    (dict(dk=96), "GDR_ERR_UNSUPPORTED", "dk"),
    (dict(dv=48), "GDR_ERR_UNSUPPORTED", "dv"),
    (dict(dv=512), "GDR_ERR_UNSUPPORTED", "dv"),
    (dict(dtype=7), "GDR_ERR_DTYPE", "dtype"),
    (dict(flags=16), "GDR_ERR_FLAGS", "flags"),
    (dict(Hk=3, Hv=4), "GDR_ERR_DIMS", "Hv"),
    (dict(T=-1), "GDR_ERR_DIMS", "T"),
    (dict(B=2, cu=FAKE * 9, num_seqs=1), "GDR_ERR_DIMS", "cu_seqlens"),
    (dict(cu=FAKE * 9, num_seqs=0), "GDR_ERR_DIMS", "num_seqs"),
    (dict(q=None), "GDR_ERR_NULL", "q"),
    (dict(out=None), "GDR_ERR_NULL", "out"),
    (dict(la=None), "GDR_ERR_NULL", "log_alpha"),
    (dict(q=FAKE + 8), "GDR_ERR_ALIGN", "q"),
    (dict(hT=FAKE * 7 + 4), "GDR_ERR_ALIGN", "hT"),
    (dict(out=FAKE * 3 + 64), "GDR_ERR_ALIAS", "out overlaps v"),
    (dict(h0=FAKE * 16, hT=FAKE * 16 + 256), "GDR_ERR_ALIAS", "partially overlaps h0"),
    (dict(hT=FAKE), "GDR_ERR_ALIAS", "hT overlaps q"),
]


@needs_lib
@pytest.mark.parametrize("over,status,text", CHUNK_REJECTS, ids=[c[1] + ":" + c[2] for c in CHUNK_REJECTS])
def test_chunk_fwd_rejects(over, status, text):
    st, msg = _chunk(binding.load(), **over)
    assert st == status and text in msg, (st, msg)


def _bidir(lib, **over):
    d = dict(B=1, T=128, Hk=2, Hv=2, dk=64, dv=64, num_seqs=0, dtype=1, flags=1)
    ptr = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, la_f=FAKE * 4, b_f=FAKE * 5, la_r=FAKE * 10, b_r=FAKE * 11,
               h0_f=None, h0_r=None, cu=None, out=FAKE * 6, hT_f=FAKE * 12, hT_r=FAKE * 13, chunk=64)
    for k_, v_ in over.items():
        (d if k_ in d else ptr)[k_] = v_
    dims = binding.ChunkDims(d["B"], d["T"], d["Hk"], d["Hv"], d["dk"], d["dv"], d["num_seqs"],
                             d["dtype"], d["flags"])
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    st = lib.gdr_chunk_fwd_bidir(*[vp(ptr[n]) for n in ("q", "k", "v", "la_f", "b_f", "la_r", "b_r", "h0_f",
                                                        "h0_r", "cu")],
                                 ptr["chunk"], vp(ptr["out"]), vp(ptr["hT_f"]), vp(ptr["hT_r"]),
                                 ctypes.byref(dims), None)
    return binding.STATUS[st], lib.gdr_last_error().decode()


BIDIR_REJECTS = [
    (dict(flags=3), "GDR_ERR_FLAGS", "GDR_REVERSE"),
    (dict(la_f=None), "GDR_ERR_NULL", "forward scan"),
    (dict(b_r=None), "GDR_ERR_NULL", "reverse scan"),
    (dict(chunk=48), "GDR_ERR_CHUNK", "forward scan"),
    (dict(out=FAKE * 10), "GDR_ERR_ALIAS", "reverse scan: out overlaps log_alpha"),
    (dict(h0_r=FAKE * 12), "GDR_ERR_ALIAS", "hT_fwd overlaps h0_rev"),
    (dict(hT_r=FAKE * 12 + 4096), "GDR_ERR_ALIAS", "hT_fwd overlaps hT_rev"),
    (dict(hT_f=FAKE * 11), "GDR_ERR_ALIAS", "hT_fwd overlaps beta_rev"),
    (dict(hT_r=FAKE * 4), "GDR_ERR_ALIAS", "hT_rev overlaps log_alpha_fwd"),
    (dict(h0_r=FAKE * 20, hT_r=FAKE * 20 + 256), "GDR_ERR_ALIAS", "partially overlaps h0"),
]


@needs_lib
@pytest.mark.parametrize("over,status,text", BIDIR_REJECTS, ids=[c[1] + ":" + c[2] for c in BIDIR_REJECTS])
def test_chunk_fwd_bidir_rejects(over, status, text):
    st, msg = _bidir(binding.load(), **over)
    assert st == status and text in msg, (st, msg)


def _gdn2_bidir(lib, **over):
    d = dict(B=1, T=128, Hk=2, Hv=2, dk=64, dv=64, num_seqs=0, dtype=1, flags=1)
    ptr = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, g_f=FAKE * 4, b_f=FAKE * 5, w_f=FAKE * 6, g_r=FAKE * 7,
               b_r=FAKE * 8, w_r=FAKE * 9, h0_f=None, h0_r=None, cu=None, out=FAKE * 10, hT_f=FAKE * 11,
               hT_r=FAKE * 12, ws=FAKE * 32, ws_bytes=1 << 24, chunk=32)
    for k_, v_ in over.items():
        (d if k_ in d else ptr)[k_] = v_
    dims = binding.ChunkDims(d["B"], d["T"], d["Hk"], d["Hv"], d["dk"], d["dv"], d["num_seqs"],
                             d["dtype"], d["flags"])
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    st = lib.gdr_gdn2_chunk_fwd_bidir(*[vp(ptr[n]) for n in ("q", "k", "v", "g_f", "b_f", "w_f", "g_r", "b_r", "w_r",
                                                             "h0_f", "h0_r", "cu")],
                                      ptr["chunk"], vp(ptr["out"]), vp(ptr["hT_f"]), vp(ptr["hT_r"]), vp(ptr["ws"]),
                                      ptr["ws_bytes"], ctypes.byref(dims), None)
    return binding.STATUS[st], lib.gdr_last_error().decode()


GDN2_BIDIR_REJECTS = [
    (dict(flags=3), "GDR_ERR_FLAGS", "GDR_REVERSE"),
    (dict(g_f=None), "GDR_ERR_NULL", "forward scan"),
    (dict(w_r=None), "GDR_ERR_NULL", "reverse scan"),
    (dict(ws_bytes=64), "GDR_ERR_DIMS", "forward scan: workspace_bytes"),
    (dict(hT_f=FAKE * 7), "GDR_ERR_ALIAS", "hT_fwd overlaps g_rev"),
    (dict(hT_r=FAKE * 6), "GDR_ERR_ALIAS", "hT_rev overlaps w_fwd"),
    (dict(hT_r=FAKE * 11 + 4096), "GDR_ERR_ALIAS", "hT_fwd overlaps hT_rev"),
    (dict(ws=FAKE * 8 - 4096), "GDR_ERR_ALIAS", "reverse scan: workspace overlaps b"),
    (dict(ws=FAKE * 5 - 4096), "GDR_ERR_ALIAS", "forward scan: workspace overlaps b"),
]


@needs_lib
@pytest.mark.parametrize("over,status,text", GDN2_BIDIR_REJECTS, ids=[c[1] + ":" + c[2] for c in GDN2_BIDIR_REJECTS])
def test_gdn2_chunk_fwd_bidir_rejects(over, status, text):
    st, msg = _gdn2_bidir(binding.load(), **over)
    assert st == status and text in msg, (st, msg)


@needs_lib
def test_null_dims_and_status_strings():
    lib = binding.load()
    st = lib.gdr_chunk_fwd(None, None, None, None, None, None, None, 64, None, None, None, None)
    assert binding.STATUS[st] == "GDR_ERR_NULL"
    for code in range(10):
        assert lib.gdr_status_string(code)
    assert lib.gdr_status_string(0) == b"ok"


def _decode(lib, **over):
    d = dict(N=4, Hk=2, Hv=4, dk=128, dv=128, dtype=1, flags=0)
    ptr = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, la=FAKE * 4, beta=FAKE * 5, si=FAKE * 8,
               so=FAKE * 16, out=FAKE * 6)
    for k_, v_ in over.items():
        (d if k_ in d else ptr)[k_] = v_
    dims = binding.DecodeDims(d["N"], d["Hk"], d["Hv"], d["dk"], d["dv"], d["dtype"], d["flags"])
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    st = lib.gdr_decode_step(vp(ptr["q"]), vp(ptr["k"]), vp(ptr["v"]), vp(ptr["la"]), vp(ptr["beta"]),
                             vp(ptr["si"]), vp(ptr["so"]), vp(ptr["out"]), ctypes.byref(dims), None)
    return binding.STATUS[st], lib.gdr_last_error().decode()


DECODE_REJECTS = [
    (dict(dk=96), "GDR_ERR_UNSUPPORTED", "dk"),
    (dict(dv=256), "GDR_ERR_UNSUPPORTED", "dv"),
    (dict(flags=2), "GDR_ERR_FLAGS", "GDR_READ_PRE"),
    (dict(flags=16), "GDR_ERR_FLAGS", "GDR_QK_L2NORM"),
    (dict(Hk=3), "GDR_ERR_DIMS", "Hv"),
    (dict(N=-2), "GDR_ERR_DIMS", "N"),
    (dict(si=None), "GDR_ERR_NULL", "NULL"),
    (dict(so=FAKE * 16 + 8), "GDR_ERR_ALIGN", "state_out"),
    (dict(so=FAKE * 8 + 4096), "GDR_ERR_ALIAS", "partially overlaps"),
    (dict(out=FAKE * 8 + 64), "GDR_ERR_ALIAS", "out overlaps state_in"),
]


@needs_lib
@pytest.mark.parametrize("over,status,text", DECODE_REJECTS, ids=[c[1] + ":" + c[2] for c in DECODE_REJECTS])
def test_decode_rejects(over, status, text):
    st, msg = _decode(binding.load(), **over)
    assert st == status and text in msg, (st, msg)


def _chunk_gated(lib, **over):
    d = dict(B=1, T=128, Hk=2, Hv=2, dk=64, dv=64, num_seqs=0, dtype=1, flags=8)
    ptr = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, a=FAKE * 4, b=FAKE * 5, A_log=FAKE * 10,
               dt_bias=FAKE * 11, h0=None, cu=None, out=FAKE * 6, hT=None, chunk=64)
    for k_, v_ in over.items():
        (d if k_ in d else ptr)[k_] = v_
    dims = binding.ChunkDims(d["B"], d["T"], d["Hk"], d["Hv"], d["dk"], d["dv"], d["num_seqs"],
                             d["dtype"], d["flags"])
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    st = lib.gdr_chunk_fwd_gated(vp(ptr["q"]), vp(ptr["k"]), vp(ptr["v"]), vp(ptr["a"]), vp(ptr["b"]),
                                 vp(ptr["A_log"]), vp(ptr["dt_bias"]), vp(ptr["h0"]), vp(ptr["cu"]),
                                 ptr["chunk"], vp(ptr["out"]), vp(ptr["hT"]), ctypes.byref(dims), None)
    return binding.STATUS[st], lib.gdr_last_error().decode()


GATED_REJECTS = [
    (dict(A_log=None), "GDR_ERR_NULL", "A_log"),
    (dict(dt_bias=None), "GDR_ERR_NULL", "dt_bias"),
    (dict(a=None), "GDR_ERR_NULL", "a or b"),
    (dict(A_log=FAKE * 10 + 2), "GDR_ERR_ALIGN", "A_log"),
    (dict(out=FAKE * 10 - 64), "GDR_ERR_ALIAS", "out overlaps A_log"),
    (dict(flags=16), "GDR_ERR_FLAGS", "flags"),
    (dict(chunk=8), "GDR_ERR_CHUNK", "chunk"),
]


@needs_lib
@pytest.mark.parametrize("over,status,text", GATED_REJECTS, ids=[c[1] + ":" + c[2] for c in GATED_REJECTS])
def test_chunk_fwd_gated_rejects(over, status, text):
    st, msg = _chunk_gated(binding.load(), **over)
    assert st == status and text in msg, (st, msg)


@needs_lib
def test_decode_gated_rejects():
    lib = binding.load()
    dims = binding.DecodeDims(4, 2, 4, 128, 128, 1, 8)
    vp = ctypes.c_void_p
    st = lib.gdr_decode_step_gated(vp(FAKE), vp(FAKE * 2), vp(FAKE * 3), vp(FAKE * 4), vp(FAKE * 5), None,
                                   vp(FAKE * 11), vp(FAKE * 8), vp(FAKE * 16), vp(FAKE * 6), ctypes.byref(dims),
                                   None)
    assert binding.STATUS[st] == "GDR_ERR_NULL" and "A_log" in lib.gdr_last_error().decode()
    st = lib.gdr_decode_step_gated(vp(FAKE), vp(FAKE * 2), vp(FAKE * 3), vp(FAKE * 4), vp(FAKE * 5), vp(FAKE * 10),
                                   vp(FAKE * 11), vp(FAKE * 8), vp(FAKE * 16), vp(FAKE * 10 - 16),
                                   ctypes.byref(dims), None)
    assert binding.STATUS[st] == "GDR_ERR_ALIAS", lib.gdr_last_error().decode()


def _gdn2_chunk(lib, **over):
    d = dict(B=1, T=128, Hk=2, Hv=2, dk=64, dv=64, num_seqs=0, dtype=1, flags=8)
    ptr = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, g=FAKE * 4, b=FAKE * 5, w=FAKE * 7, h0=None, cu=None,
               out=FAKE * 6, hT=None, chunk=64, ws=None, ws_bytes=0)
    for k_, v_ in over.items():
        (d if k_ in d else ptr)[k_] = v_
    dims = binding.ChunkDims(d["B"], d["T"], d["Hk"], d["Hv"], d["dk"], d["dv"], d["num_seqs"],
                             d["dtype"], d["flags"])
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    st = lib.gdr_gdn2_chunk_fwd(vp(ptr["q"]), vp(ptr["k"]), vp(ptr["v"]), vp(ptr["g"]), vp(ptr["b"]),
                                vp(ptr["w"]), vp(ptr["h0"]), vp(ptr["cu"]), ptr["chunk"], vp(ptr["out"]),
                                vp(ptr["hT"]), vp(ptr["ws"]), ptr["ws_bytes"], ctypes.byref(dims), None)
    return binding.STATUS[st], lib.gdr_last_error().decode()


GDN2_REJECTS = [
    (dict(g=None), "GDR_ERR_NULL", "g"),
    (dict(w=None), "GDR_ERR_NULL", "w"),
    (dict(b=FAKE * 5 + 4), "GDR_ERR_ALIGN", "b"),
    (dict(g=FAKE * 4 + 8), "GDR_ERR_ALIGN", "g"),
    (dict(out=FAKE * 7 + 64), "GDR_ERR_ALIAS", "out overlaps w"),
    (dict(hT=FAKE * 4 + 4096), "GDR_ERR_ALIAS", "hT overlaps g"),
    (dict(dtype=0, dk=128), "GDR_ERR_CHUNK", "shared memory"),
    (dict(chunk=8), "GDR_ERR_CHUNK", "chunk"),
    (dict(flags=16), "GDR_ERR_FLAGS", "flags"),
    (dict(dv=40), "GDR_ERR_UNSUPPORTED", "dv"),
    (dict(Hk=4, Hv=2), "GDR_ERR_DIMS", "Hv"),
    # the two-pass form's workspace (this call needs 2 x 2 x 41216 bytes)
    (dict(ws=FAKE * 9, ws_bytes=1024), "GDR_ERR_DIMS", "workspace_bytes"),
    (dict(ws=FAKE * 9 + 8, ws_bytes=1 << 20), "GDR_ERR_ALIGN", "workspace"),
    (dict(ws=FAKE * 7 + 4096, ws_bytes=1 << 20), "GDR_ERR_ALIAS", "workspace overlaps w"),
]


@needs_lib
@pytest.mark.parametrize("over,status,text", GDN2_REJECTS, ids=[c[1] + ":" + c[2] for c in GDN2_REJECTS])
def test_gdn2_chunk_rejects(over, status, text):
    st, msg = _gdn2_chunk(binding.load(), **over)
    assert st == status and text in msg, (st, msg)


@needs_lib
def test_gdn2_workspace_bytes():
    lib = binding.load()
    # B4 H16 T4096 d128 bf16, chunk 32: 4 x 128 chunk slots; per slot 16 key-head blocks of
    # 2 (3 x 32 x 128 + 2 x 32 x 32) + 4 x 128 bytes
    dims = binding.ChunkDims(4, 4096, 16, 16, 128, 128, 0, 1, 0)
    want = 512 * 16 * (2 * (3 * 32 * 128 + 2 * 32 * 32) + 4 * 128)
    assert lib.gdr_gdn2_chunk_fwd_workspace_bytes(ctypes.byref(dims), 32, 0) == want
    # packed: T / chunk + num_seqs + 1 slots; fp32 doubles the element bytes; blocks per key head
    dims = binding.ChunkDims(1, 1000, 2, 4, 64, 32, 3, 0, 0)
    want = 66 * 2 * (4 * (3 * 16 * 64 + 2 * 16 * 16) + 4 * 64)
    assert lib.gdr_gdn2_chunk_fwd_workspace_bytes(ctypes.byref(dims), 16, 1) == want
    assert lib.gdr_gdn2_chunk_fwd_workspace_bytes(ctypes.byref(dims), 8, 1) == -1
    assert lib.gdr_gdn2_chunk_fwd_workspace_bytes(None, 16, 0) == -1
    # a workspace of the size asked for passes validation (no sequences: nothing is launched)
    st, msg = _gdn2_chunk(lib, B=0, ws=FAKE * 9, ws_bytes=0)
    assert st == "GDR_OK", msg


@needs_lib
def test_gdn2_fp32_d128_takes_chunk_32():
    # the same call with chunk 32 passes validation; with no sequences nothing is launched
    st, msg = _gdn2_chunk(binding.load(), dtype=0, dk=128, chunk=32, B=0)
    assert st == "GDR_OK", msg


@needs_lib
def test_gdn2_decode_rejects():
    lib = binding.load()
    vp = ctypes.c_void_p

    def call(dims, g=FAKE * 4, w=FAKE * 7, out=FAKE * 6):
        st = lib.gdr_gdn2_decode_step(vp(FAKE), vp(FAKE * 2), vp(FAKE * 3), None if g is None else vp(g),
                                      vp(FAKE * 5), vp(w), vp(FAKE * 8), vp(FAKE * 16), vp(out),
                                      ctypes.byref(dims), None)
        return binding.STATUS[st], lib.gdr_last_error().decode()

    ok = binding.DecodeDims(4, 2, 4, 128, 128, 1, 8)
    assert call(ok, g=None)[0] == "GDR_ERR_NULL"
    assert call(ok, g=FAKE * 4 + 4)[0] == "GDR_ERR_ALIGN"
    st, msg = call(ok, out=FAKE * 7 + 16)
    assert st == "GDR_ERR_ALIAS" and "out overlaps w" in msg, msg
    assert call(binding.DecodeDims(4, 2, 4, 128, 128, 1, 4))[0] == "GDR_ERR_FLAGS"
    assert call(binding.DecodeDims(4, 2, 4, 96, 128, 1, 0))[0] == "GDR_ERR_UNSUPPORTED"
    assert call(binding.DecodeDims(0, 2, 4, 128, 128, 1, 0))[0] == "GDR_OK"


@needs_lib
def test_delta_product_rejects():
    lib = binding.load()
    vp = ctypes.c_void_p

    def call(n=2, flags=0, T=128, out=FAKE * 6):
        dims = binding.ChunkDims(1, T, 2, 2, 64, 64, 0, 1, flags)
        st = lib.gdr_delta_product_fwd(vp(FAKE), vp(FAKE * 2), vp(FAKE * 3), vp(FAKE * 4), vp(FAKE * 5), None, None,
                                       n, 64, vp(out), None, ctypes.byref(dims), None)
        return binding.STATUS[st], lib.gdr_last_error().decode()

    assert call(n=0) == ("GDR_ERR_DIMS", "n_delta 0 is not in [1, 16]")
    assert call(n=17)[0] == "GDR_ERR_DIMS"
    st, msg = call(flags=2)
    assert st == "GDR_ERR_FLAGS" and "GDR_REVERSE" in msg, msg
    assert call(T=(1 << 30))[0] == "GDR_ERR_DIMS"
    # k holds n rows per token: an output placed after a one-row-per-token k still overlaps it
    st, msg = call(n=4, out=FAKE * 2 + 2 * 128 * 64 * 2 + 64)
    assert st == "GDR_ERR_ALIAS" and "out overlaps k" in msg, msg


@needs_lib
def test_backward_rejects():
    lib = binding.load()
    vp = lambda x: None if x is None else ctypes.c_void_p(x)

    def call(flags=0, dk=64, ws=FAKE * 20, ws_bytes=1 << 40, dq=FAKE * 10):
        dims = binding.ChunkDims(1, 128, 2, 2, dk, 64, 0, 1, flags)
        st = lib.gdr_chunk_bwd(vp(FAKE), vp(FAKE * 2), vp(FAKE * 3), vp(FAKE * 4), vp(FAKE * 5), None, None,
                               vp(FAKE * 6), None, vp(dq), vp(FAKE * 11), vp(FAKE * 12), vp(FAKE * 13),
                               vp(FAKE * 14), None, vp(ws), ctypes.c_int64(ws_bytes), ctypes.byref(dims), None)
        return binding.STATUS[st], lib.gdr_last_error().decode()

    assert call(flags=8)[0] == "GDR_ERR_FLAGS"
    assert call(dk=96)[0] == "GDR_ERR_UNSUPPORTED"
    st, msg = call(ws_bytes=1024)
    assert st == "GDR_ERR_DIMS" and "workspace_bytes" in msg, msg
    assert call(ws=None)[0] == "GDR_ERR_NULL"
    st, msg = call(dq=FAKE + 64)
    assert st == "GDR_ERR_ALIAS" and "dq overlaps q" in msg, msg
    dims = binding.ChunkDims(4, 4096, 16, 16, 128, 128, 0, 1, 0)
    # 16 value heads x (4 sequences x 64 chunks of 64 tokens): a record per chunk (three 64 x 64
    # operand matrices as split bf16, 4 bytes an element, and 2 x 64 gate cumsums), the entry state
    # and the exit adjoint (64 KiB each); then U and dR of every chunk (fp32 64 x 128 each)
    slots = 16 * 4 * 64
    rec = slots * (3 * 16384 + 2 * 64 * 4)
    states = 2 * slots * 128 * 128 * 4
    tokens = 2 * slots * 64 * 128 * 4
    assert lib.gdr_chunk_bwd_workspace_bytes(ctypes.byref(dims), 0) == rec + states + tokens
    # packed: slots for every 64 tokens of the total plus one per segment and one spare
    pdims = binding.ChunkDims(1, 1000, 2, 4, 64, 64, 3, 1, 0)
    pslots = 4 * (1000 // 64 + 3 + 1)
    want = pslots * (3 * 16384 + 2 * 64 * 4) + 2 * pslots * 64 * 64 * 4 + 2 * pslots * 64 * 64 * 4
    assert lib.gdr_chunk_bwd_workspace_bytes(ctypes.byref(pdims), 1) == want


@needs_lib
def test_gdn2_noalloc_rejects_beyond_its_scratch():
    # sizes whose two-pass workspace exceeds the fixed 64 MiB scratch are refused before anything
    # runs (B4 H16 T4096 d128 bf16, chunk 32, needs 239 MB); no GPU is touched on the way
    lib = binding.load()
    dims = binding.ChunkDims(4, 4096, 16, 16, 128, 128, 0, 1, 0)
    assert lib.gdr_gdn2_chunk_fwd_workspace_bytes(ctypes.byref(dims), 32, 0) > (64 << 20)
    vp = ctypes.c_void_p
    st = lib.gdr_gdn2_chunk_fwd_noalloc(vp(FAKE), vp(FAKE * 2), vp(FAKE * 3), vp(FAKE * 4), vp(FAKE * 5),
                                        vp(FAKE * 6), None, None, 32, vp(FAKE * 7), None, ctypes.byref(dims), None)
    msg = lib.gdr_last_error().decode()
    assert binding.STATUS[st] == "GDR_ERR_DIMS" and "allocation-free" in msg, msg
    assert lib.gdr_gdn2_chunk_fwd_noalloc(None, None, None, None, None, None, None, None, 32, None, None,
                                          None, None) == 1  # dims NULL: GDR_ERR_NULL
