"""Benchmark of the gated delta rule library on one MI355X.

Headline: chunked-forward tokens/s on the B4 H16 T4096 d128 bf16 workload (chunk 64,
nonzero h0, post-write read); one step is one gdr_chunk_fwd call over the whole batch.
Also reported: decode-step state GB/s (256 sequences, 16 key / 32 value heads, d128,
fp32 state, 64 consecutive in-place steps), the packed variable-length and bidirectional
workloads' tokens/s, roofline fractions, and the fp64 CPU oracle timed on this host.

All inputs are synthetic (seeded generators in gated_delta_rule_70_amd/inputs.py) and
resident in HBM before timing starts. Each workload's calls rotate over enough independent
copies of its inputs and outputs that no call finds the previous call's bytes in the 256 MB
last-level cache (--cache-warm times one copy instead; the headline reports both). Kernel
times come from HIP events recorded on the stream the kernels are launched on (torch's
current stream).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 matrix, published

METRIC = "GDR chunk-fwd tokens/s (B4 H16 T4096 d128); decode-step state GB/s"

CACHE_BYTES = 256 << 20  # MI355X last-level (Infinity) cache in front of HBM
CACHE_WARM = False       # --cache-warm: every workload on one copy of its inputs


def rotation(make, set_bytes):
    """A call that runs k independent copies of a workload in turn; `make()` builds one copy
    (its own inputs and outputs on the device) and returns its call. The other k - 1 copies
    hold at least twice the last-level cache, so a call does not find what its copy's previous
    call read or wrote there: its inputs come from HBM, as in a model where other layers run
    between two calls of a layer. With --cache-warm k is 1, and a workload whose inputs fit in
    the cache re-reads them from it. Returns (call, k)."""
    k = 1 if CACHE_WARM else 1 + max(1, -(-2 * CACHE_BYTES // max(1, int(set_bytes))))
    calls = [make() for _ in range(k)]
    pos = [0]

    def fn():
        i = pos[0]
        pos[0] = i + 1
        calls[i % k]()

    return fn, k


def chunk_bytes(B, H, T, dk, dv, es, nseq, gates=2, state=True):
    """Algorithmic HBM bytes of one chunked forward: q, k, v, out once each, the gates,
    h0 and hT."""
    tok = B * H * T
    b = tok * (2 * dk + dv) * es + tok * dv * es + tok * gates * 4
    if state:
        b += 2 * nseq * H * dk * dv * 4
    return b


def chunk_flops(B, H, T, dk, dv, C=64):
    """Algorithmic flops per token-head of the chunk form: 6*dk*dv for K H, Q H and the state
    update, C*(3*dk + 2*dv) for the triangular Gram products (K K^T, Q K^T), W/U and the
    intra-chunk read (halved for the triangles), C^2/3 for the solve."""
    per = 6 * dk * dv + C * (3 * dk + 2 * dv) + C * C / 3
    return B * H * T * per


# Matrix-core instructions the fast chunk kernel issues per workgroup and 64-token chunk (one
# workgroup per sequence-head and 32 value columns), counted from its source:
#   two chain waves, each 16 x16x32 (K H) + 16 (Q H) + 16 (state update) + 6 (P U) + 2
#   (substitution) = 56, and 6 x16x16 (substitution) -> 112 and 12;
#   diagonal prep 16 x16x32 (Gram tiles) and 36 x16x16 (inverses); off-diagonal -A 24 x16x32;
#   P tiles 40 x16x32.
# That is 192 v_mfma_f32_16x16x32_bf16 (16,384 flops) and 48 v_mfma_f32_16x16x16_bf16 (8,192
# flops); the matrix-core counters agree (SQ_INSTS_MFMA = 240 per workgroup-chunk).
FAST_MFMA32_PER_WG_CHUNK = 192
FAST_MFMA16_PER_WG_CHUNK = 48


def chunk_flops_executed(B, H, T, dv, C=64):
    """Flops the fast kernel's matrix cores execute per launch (whole triangular tiles, the
    products that build the diagonal inverses): instructions per workgroup-chunk x workgroups x
    chunks."""
    wg_chunks = B * H * (dv // 32) * ((T + C - 1) // C)
    return wg_chunks * (FAST_MFMA32_PER_WG_CHUNK * 16384 + FAST_MFMA16_PER_WG_CHUNK * 8192)


PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "gated_delta_rule_70_amd", "csrc")


def source_digest(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(summary, source, key):
    """HBM bytes per launch from a committed counter summary (FETCH_SIZE and WRITE_SIZE runs,
    scaled by a copy of known size), or None when the summary is missing or was taken on a
    different kernel source."""
    try:
        with open(os.path.join(PROFILES, summary)) as f:
            text = f.read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].split(": ", 1)
            fields[k.strip()] = v.strip().strip("`")
    try:
        if fields["kernel source sha256"] != source_digest(os.path.join(CSRC, source)):
            return None
        return float(fields[key])
    except (KeyError, ValueError, OSError):
        return None


def copy_calibration(mib=1024, reps=3):
    """A plain device-to-device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE
    counters: each launch reads and writes `mib` MiB."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_each_way": mib * (1 << 20), "launches": reps}), flush=True)


SETTLE_MS = 150.0  # untimed back-to-back calls before the warm-up, until the clock is steady


def settle(fn, stream, ms=None):
    """Untimed back-to-back calls for about `ms` of GPU time: the GPU takes tens of milliseconds
    of sustained work to reach its steady clock (with only a few warm-up calls the chunked
    forward times 10-20% slower)."""
    import torch
    ms = SETTLE_MS if ms is None else ms
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    done, n = 0.0, 1
    while done < ms:
        start.record(stream)
        for _ in range(n):
            fn()
        end.record(stream)
        torch.cuda.synchronize()
        done += start.elapsed_time(end)
        n = min(n * 2, 4096)
    return done


def timed(fn, steps, warmup, stream, settle_ms=None):
    """Per-call times in ms: a HIP event pair on the launch stream around each of `steps`
    back-to-back calls (after the clock settles and `warmup` untimed calls), the whole timed
    region bracketed by device synchronisation. Returns (median, mean of the bracket, wall s)."""
    import torch
    settle_ms = SETTLE_MS if settle_ms is None else min(settle_ms, SETTLE_MS)
    if settle_ms > 0:
        settle(fn, stream, settle_ms)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = sorted(a.elapsed_time(b) for a, b in ev)
    mean = ev[0][0].elapsed_time(ev[-1][1]) / steps
    return per[len(per) // 2], mean, wall


def measured_peaks(reps=10):
    """What this GPU reaches on plain library work, beside the published peaks: a 1 GiB
    device-to-device copy (bytes read + written per second) and a dense bf16 GEMM
    (8192 x 8192 x 8192, torch.matmul -> hipBLASLt). Medians of `reps` timed calls."""
    import torch
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    med, _, _ = timed(lambda: dst.copy_(src), reps, 3, stream, settle_ms=50.0)
    copy_gbs = 2 * n * 4 / (med / 1e3) / 1e9
    del src, dst
    m = 8192
    a = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    b = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    c = torch.empty(m, m, device=dev, dtype=torch.bfloat16)
    med, _, _ = timed(lambda: torch.matmul(a, b, out=c), reps, 3, stream, settle_ms=50.0)
    gemm_tflops = 2 * m ** 3 / (med / 1e3) / 1e12
    del a, b, c
    return {"hbm_copy_GBs": copy_gbs, "bf16_gemm_TFLOPs": gemm_tflops,
            "how": "median of %d calls: a 1 GiB device copy (read + written bytes) and an 8192^3 bf16 "
                   "torch.matmul (hipBLASLt)" % reps}


def bench_chunk(binding, inputs, steps, warmup, warm_too=False):
    import torch
    case = inputs.workload1()
    dev = torch.device("cuda:0")
    src = [t.to(dev) for t in (case.q, case.k, case.v, case.log_alpha, case.beta, case.h0)]

    def make():
        q, k, v, la, b, h0 = (t.clone() for t in src)
        out, hT = torch.empty_like(v), torch.empty_like(h0)
        return lambda: binding.chunk_fwd(q, k, v, la, b, h0, None, chunk=64, out=out, hT=hT)

    stream = torch.cuda.current_stream(dev)
    B, H, T, dk = case.q.shape
    dv = case.v.shape[-1]
    nbytes = chunk_bytes(B, H, T, dk, dv, 2, B)
    fn, sets = rotation(make, nbytes)
    ms, mean, wall = timed(fn, steps, warmup, stream)
    r = dict(ms=ms, mean_ms=mean, wall=wall, tokens=B * T, bytes=nbytes, sets=sets,
             flops=chunk_flops(B, H, T, dk, dv), flops_exec=chunk_flops_executed(B, H, T, dv),
             shape=(B, H, T, dk, dv))
    if warm_too and sets > 1:
        # the same calls on one copy: the inputs (about 205 MB read per call) stay in the
        # last-level cache between calls (not in the single-workload runs that profiles use)
        r["ms_cache_warm"], _, _ = timed(make(), steps, warmup, stream)
    return r


def bench_decode(binding, inputs, reps):
    import torch
    dc = inputs.workload3()
    dev = torch.device("cuda:0")
    steps = dc.q.shape[0]
    q, k, v, la, b = (t.to(dev) for t in (dc.q, dc.k, dc.v, dc.log_alpha, dc.beta))
    N, Hv, dk, dv = dc.state.shape
    sbytes = 2 * N * Hv * dk * dv * 4
    io = (dc.q[0].numel() * 2 + dc.v[0].numel()) * 2 + N * Hv * 2 * 4 + N * Hv * dv * 2
    # independent batches of 256 sequences, each with its own state (updated in place) and
    # outputs, take their steps in turn
    state0 = dc.state.to(dev)

    def make():
        state = state0.clone()
        out = torch.empty((steps,) + tuple(dc.v.shape[1:]), dtype=dc.v.dtype, device=dev)
        return lambda s: binding.decode_step(q[s], k[s], v[s], la[s], b[s], state, state_out=state, out=out[s])

    nb = 1 if CACHE_WARM else 1 + max(1, -(-2 * CACHE_BYTES // sbytes))
    batches = [make() for _ in range(nb)]
    del state0
    stream = torch.cuda.current_stream(dev)
    # the clock settles and one warm pass of the 64 steps runs, then `reps` timed passes of the 64
    # consecutive steps (the states keep evolving in place), an event pair around every step
    settle(lambda: batches[0](0), stream)
    for s in range(steps):
        batches[s % nb](s)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps * reps)]
    i = 0
    for r in range(reps):
        for s in range(steps):
            ev[i][0].record(stream)
            batches[i % nb](s)
            ev[i][1].record(stream)
            i += 1
    torch.cuda.synchronize()
    mean = ev[0][0].elapsed_time(ev[-1][1]) / (steps * reps)
    per = sorted(a.elapsed_time(b) for a, b in ev)
    median = per[len(per) // 2]
    return dict(ms=mean, median_ms=median, state_bytes=sbytes, io_bytes=io, tokens=N, steps=steps * reps,
                sets=nb)


def bench_varlen(binding, inputs, steps):
    import torch
    case = inputs.workload2()
    dev = torch.device("cuda:0")
    src = [t.to(dev) for t in (case.q, case.k, case.v, case.log_alpha, case.beta, case.h0)]
    cu = case.cu_seqlens.to(dev)

    def make():
        q, k, v, la, b, h0 = (t.clone() for t in src)
        out, hT = torch.empty_like(v), torch.empty_like(h0)
        return lambda: binding.chunk_fwd(q, k, v, la, b, h0, cu, chunk=64, out=out, hT=hT)

    T = case.q.shape[2]
    H, dk, dv = case.q.shape[1], case.q.shape[3], case.v.shape[3]
    nseq = case.cu_seqlens.numel() - 1
    nbytes = chunk_bytes(1, H, T, dk, dv, 2, nseq)
    fn, sets = rotation(make, nbytes)
    ms, _, _ = timed(fn, steps, 20, torch.cuda.current_stream(dev))
    return dict(ms=ms, tokens=T, bytes=nbytes, sets=sets,
                lengths=[int(x) for x in (case.cu_seqlens[1:] - case.cu_seqlens[:-1])])


def bench_fused(binding, inputs, steps):
    """The fused prologue on the workload-1 shapes: raw q/k rows (normalised in the kernel) and
    raw gate inputs a, b with per-head A_log, dt_bias (``gdr_chunk_fwd_gated`` with
    GDR_QK_L2NORM)."""
    import torch
    c = inputs.raw_case(B=4, T=4096, Hk=16, Hv=16, dk=128, dv=128, dtype=torch.bfloat16, seed=1001,
                        h0_std=0.1)
    dev = torch.device("cuda:0")
    src = [t.to(dev) for t in (c.q, c.k, c.v, c.a, c.b, c.A_log, c.dt_bias, c.h0)]

    def make():
        q, k, v, a, b, A_log, dtb, h0 = (t.clone() for t in src)
        out, hT = torch.empty_like(v), torch.empty_like(h0)
        return lambda: binding.chunk_fwd_gated(q, k, v, a, b, A_log, dtb, h0, chunk=64, out=out, hT=hT,
                                               l2norm=True)

    fn, sets = rotation(make, chunk_bytes(4, 16, 4096, 128, 128, 2, 4))
    ms, _, _ = timed(fn, steps, 20, torch.cuda.current_stream(dev))
    return dict(ms=ms, tokens=4 * 4096, sets=sets)


def bench_bidir(binding, inputs, steps):
    import torch
    case = inputs.workload4()
    dev = torch.device("cuda:0")
    src = [t.to(dev) for t in (case.q, case.k, case.v, case.log_alpha, case.beta, case.extra["log_alpha_bwd"],
                               case.extra["beta_bwd"])]
    cu = case.cu_seqlens.to(dev)

    def make():
        q, k, v, la, b, la2, b2 = (t.clone() for t in src)
        out = torch.empty_like(v)

        def fn():
            binding.chunk_fwd_bidir(q, k, v, la, b, la2, b2, None, None, cu, chunk=64, read="pre", out=out,
                                    want_state=False)

        return fn

    H, T, dk, dv = case.q.shape[1], case.q.shape[2], case.q.shape[3], case.v.shape[3]
    nbytes = chunk_bytes(1, H, T, dk, dv, 2, 0, gates=4, state=False)
    fn, sets = rotation(make, nbytes)
    ms, _, _ = timed(fn, steps, 20, torch.cuda.current_stream(dev))
    return dict(ms=ms, tokens=T, sets=sets, bytes=nbytes)


def gdn2_bytes(B, Hk, Hv, T, dk, dv, es, nseq):
    """Algorithmic HBM bytes of one GDN-2 chunked forward: q, k, b (erase gate) and the fp32
    decay g per key head; v, w (write gate) and out per value head; h0 and hT."""
    return B * Hk * T * dk * (3 * es + 4) + B * Hv * T * dv * 3 * es + 2 * nseq * Hv * dk * dv * 4


def bench_gdn2(binding, inputs, steps):
    """GDN-2 (per-key-channel decay, separate erase and write gates) on the workload-1 shapes,
    chunk 32, gates drawn as at the layer's initialisation; and its one-token decode step on the
    decode workload's shapes."""
    import torch
    dev = torch.device("cuda:0")
    c = inputs.gdn2_case(B=4, T=4096, Hk=16, Hv=16, dk=128, dv=128, dtype=torch.bfloat16, seed=1001,
                         h0_std=0.1)
    src = [t.to(dev) for t in (c.q, c.k, c.v, c.g, c.b, c.w, c.h0)]
    # one workspace for all copies: a call writes it before it reads it
    ws = torch.empty(binding.gdn2_chunk_fwd_workspace_bytes(4, 4096, 16, 16, 128, 128, 32), dtype=torch.uint8,
                     device=dev)

    def make(fused=False):
        q, k, v, g, b, w, h0 = (t.clone() for t in src)
        out, hT = torch.empty_like(v), torch.empty_like(h0)
        if fused:
            return lambda: binding.gdn2_chunk_fwd(q, k, v, g, b, w, h0, chunk=32, out=out, hT=hT, fused=True)
        return lambda: binding.gdn2_chunk_fwd(q, k, v, g, b, w, h0, chunk=32, out=out, hT=hT, workspace=ws)

    nbytes = gdn2_bytes(4, 16, 16, 4096, 128, 128, 2, 4)
    fn, sets = rotation(make, nbytes)
    ms, _, _ = timed(fn, steps, 20, torch.cuda.current_stream(dev))
    del fn
    # the one-pass kernel (no workspace) on the same inputs, for reference
    fn1, _ = rotation(lambda: make(fused=True), nbytes)
    ms1, _, _ = timed(fn1, max(3, steps // 4), 3, torch.cuda.current_stream(dev), settle_ms=20.0)
    chunk = dict(ms=ms, fused_ms=ms1, ws_bytes=ws.numel(), tokens=4 * 4096, bytes=nbytes, sets=sets)
    del fn1, src, ws
    N, Hk, Hv = 256, 16, 32
    dc = inputs.gdn2_case(B=N, T=1, Hk=Hk, Hv=Hv, dk=128, dv=128, dtype=torch.bfloat16, seed=1003, h0_std=0.1)
    one = lambda t: t[:, :, 0].contiguous().to(dev)
    dq, dk_, dv_, dg, db, dw = (one(t) for t in (dc.q, dc.k, dc.v, dc.g, dc.b, dc.w))
    state0 = dc.h0.to(dev)
    sbytes = 2 * N * Hv * 128 * 128 * 4

    def make():
        state = state0.clone()
        dout = torch.empty((N, Hv, 128), dtype=torch.bfloat16, device=dev)
        return lambda: binding.gdn2_decode_step(dq, dk_, dv_, dg, db, dw, state, state_out=state, out=dout)

    fn, _ = rotation(make, sbytes)
    del state0
    dms, _, _ = timed(fn, max(steps, 64), 20, torch.cuda.current_stream(dev))
    io = N * Hk * 128 * (3 * 2 + 4) + N * Hv * 128 * 3 * 2
    return chunk, dict(ms=dms, state_bytes=sbytes, io_bytes=io, tokens=N)


def bench_delta_product(binding, inputs, steps):
    """DeltaProduct with two sub-steps per token on the workload-1 shapes (B4 H16 T4096 d128 bf16),
    pre-write read (the page's), chunk 64 of sub-steps."""
    import torch
    dev = torch.device("cuda:0")
    c = inputs.delta_product_case(B=4, T=4096, n=2, Hk=16, Hv=16, dk=128, dv=128, dtype=torch.bfloat16,
                                  seed=1001, h0_std=0.1)
    src = [t.to(dev) for t in (c.q, c.k, c.v, c.log_alpha, c.beta, c.h0)]

    def make():
        q, k, v, la, b, h0 = (t.clone() for t in src)
        out, hT = torch.empty((4, 16, 4096, 128), dtype=torch.bfloat16, device=dev), torch.empty_like(h0)
        return lambda: binding.delta_product_fwd(q, k, v, la, b, h0, chunk=64, read="pre", out=out, hT=hT)

    tok = 4 * 16 * 4096
    nbytes = tok * 128 * 2 * (1 + 2 + 2 + 1) + tok * 4 * (1 + 2) + 2 * 4 * 16 * 128 * 128 * 4
    fn, sets = rotation(make, nbytes)
    ms, _, _ = timed(fn, steps, 20, torch.cuda.current_stream(dev))
    return dict(ms=ms, tokens=4 * 4096, bytes=nbytes, sets=sets)


def bench_backward(binding, inputs, steps):
    """Gradients of the workload-1 forward (B4 H16 T4096 d128, bf16 inputs, post-write read) with
    respect to every input, from random upstream gradients of the outputs and final state."""
    import torch
    dev = torch.device("cuda:0")
    c = inputs.workload1()
    g = torch.Generator(device="cpu").manual_seed(5)
    src = [t.to(dev) for t in (c.q, c.k, c.v, c.log_alpha, c.beta, c.h0)]
    src.append(torch.randn(tuple(c.v.shape), generator=g).to(torch.bfloat16).to(dev))
    src.append(torch.randn(tuple(c.h0.shape), generator=g).to(dev))
    # one workspace for all copies: a call writes it before it reads it
    ws = torch.empty(binding.chunk_bwd_workspace_bytes(4, 4096, 16, 16, 128, 128), dtype=torch.uint8, device=dev)

    def make():
        q, k, v, la, b, h0, dout, dhT = (t.clone() for t in src)
        return lambda: binding.chunk_bwd(q, k, v, la, b, dout, h0, None, dhT, workspace=ws)

    tok = 4 * 16 * 4096
    # inputs, dout read once; gradients written once (dq, dk, dv fp32); h0, dhT, dh0
    nbytes = tok * 128 * 2 * 4 + tok * 4 * 4 + tok * 128 * 4 * 3 + 3 * 4 * 16 * 128 * 128 * 4
    fn, sets = rotation(make, nbytes)
    ms, _, _ = timed(fn, steps, 2, torch.cuda.current_stream(dev), settle_ms=20.0)
    return dict(ms=ms, tokens=4 * 4096, bytes=nbytes, ws_bytes=ws.numel(), sets=sets)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def _f64(*ts):
    import numpy as np
    return [None if t is None else np.ascontiguousarray(t.double().numpy()) for t in ts]


def _repeat(fn, min_wall, max_reps):
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_wall or reps >= max_reps:
            return reps, dt


def cpu_baseline(inputs, min_wall=1.5, max_reps=20):
    """The fp64 oracle, as it is, on this host's cores: the whole B4 H16 T4096 d128 workload,
    repeated until at least `min_wall` seconds have passed (a bounded sample). Inputs are
    upcast before the clock starts."""
    import oracle
    case = inputs.workload1()
    threads = min(len(os.sched_getaffinity(0)), 64)
    args = _f64(case.q, case.k, case.v, case.log_alpha, case.beta, case.h0)
    reps, dt = _repeat(lambda: oracle.scan(*args, threads=threads), min_wall, max_reps)
    tokens = case.q.shape[0] * case.q.shape[2] * reps
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "the whole B4 H16 T4096 d128 workload (64 sequence-heads) %d times, fp64 "
                      "per-token recurrence, %.1f s wall on %d threads; CPU: %s"
                      % (reps, dt, threads, _cpu_model())}


def cpu_baseline_other(inputs, min_wall=1.0):
    """The same oracle beside the other workloads, each a bounded sample on the same threads:
    decode (consecutive fp64 steps over all 256 x 32 head-states, state GB/s counted with the
    fp32 state's bytes read + written; the fp64 oracle moves twice that), the packed
    variable-length workload and the bidirectional workload (both whole)."""
    import oracle
    threads = min(len(os.sched_getaffinity(0)), 64)
    res = {}
    dc = inputs.workload3(steps=16)
    q, k, v, la, b, st = _f64(dc.q, dc.k, dc.v, dc.log_alpha, dc.beta, dc.state)
    box = {"state": st, "step": 0}

    def one():
        s = box["step"] % q.shape[0]
        _, box["state"] = oracle.decode(q[s], k[s], v[s], la[s], b[s], box["state"], threads=threads)
        box["step"] += 1
    reps, dt = _repeat(one, min_wall, 64)
    N, Hv, dk, dv = dc.state.shape
    sbytes = 2 * N * Hv * dk * dv * 4
    res[inputs.WORKLOADS[3]] = {"value": sbytes * reps / dt / 1e9, "unit": "state GB/s", "cores": threads,
                                "kind": "oracle", "sample": "%d consecutive decode steps, %.1f s wall" % (reps, dt)}
    c2 = inputs.workload2()
    args = _f64(c2.q, c2.k, c2.v, c2.log_alpha, c2.beta, c2.h0)
    reps, dt = _repeat(lambda: oracle.scan(*args, c2.cu_seqlens, threads=threads), min_wall, 4)
    res[inputs.WORKLOADS[2]] = {"value": c2.q.shape[2] * reps / dt, "unit": "tokens/s", "cores": threads,
                                "kind": "oracle", "sample": "the whole packed workload %d times, %.1f s wall" % (reps, dt)}
    c4 = inputs.workload4()
    q, k, v, la, b, la2, b2 = _f64(c4.q, c4.k, c4.v, c4.log_alpha, c4.beta, c4.extra["log_alpha_bwd"],
                                   c4.extra["beta_bwd"])

    def both():
        oracle.scan(q, k, v, la, b, None, c4.cu_seqlens, read="pre", want_state=False, threads=threads)
        oracle.scan(q, k, v, la2, b2, None, c4.cu_seqlens, read="pre", reverse=True, want_state=False,
                    threads=threads)
    reps, dt = _repeat(both, min_wall, 4)
    res[inputs.WORKLOADS[4]] = {"value": c4.q.shape[2] * reps / dt, "unit": "tokens/s", "cores": threads,
                                "kind": "oracle", "sample": "both scans of the whole workload %d times, %.1f s wall" % (reps, dt)}
    return res


def bench_many_segments(binding, inputs, steps):
    """Packed input of 2048 short segments (lengths U{16..48}), H16 d128 bf16, chunk 64, per-segment
    h0: each workgroup ranks the segments by length before its first chunk."""
    import torch
    lengths = inputs.segment_lengths(2048, 16, 48, seed=4242)
    case = inputs.chunk_case(Hk=16, dk=128, dv=128, dtype=torch.bfloat16, seed=1005, h0_std=0.1, lengths=lengths)
    dev = torch.device("cuda:0")
    src = [t.to(dev) for t in (case.q, case.k, case.v, case.log_alpha, case.beta, case.h0)]
    cu = case.cu_seqlens.to(dev)

    def make():
        q, k, v, la, b, h0 = (t.clone() for t in src)
        out, hT = torch.empty_like(v), torch.empty_like(h0)
        return lambda: binding.chunk_fwd(q, k, v, la, b, h0, cu, chunk=64, out=out, hT=hT)

    T = case.q.shape[2]
    nbytes = chunk_bytes(1, 16, T, 128, 128, 2, len(lengths))
    fn, sets = rotation(make, nbytes)
    ms, _, _ = timed(fn, steps, 20, torch.cuda.current_stream(dev))
    return dict(ms=ms, tokens=T, bytes=nbytes, sets=sets)


def main():
    global SETTLE_MS, CACHE_WARM
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # untimed calls before the timed ones (after the clock-settling phase, see settle())
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured copy / GEMM peaks")
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="untimed GPU time before the warm-up of each workload (0 for counter runs)")
    ap.add_argument("--only", choices=["chunk", "decode", "gdn2", "bwd", "dp", "bidir", "all"], default="all",
                    help="gdn2, bwd, dp, bidir: only the GDN-2 workloads, the backward, DeltaProduct or the "
                         "bidirectional call (for profiling them)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling HBM byte counters)")
    ap.add_argument("--cache-warm", action="store_true",
                    help="time every workload on one copy of its inputs (calls may find them in the "
                         "last-level cache) instead of rotating over copies that do not fit there")
    args = ap.parse_args()
    SETTLE_MS = max(0.0, args.settle_ms)
    CACHE_WARM = args.cache_warm
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: every workload here runs on a single MI355X "
              "(--gpus %d is not supported)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return
    import torch
    from gated_delta_rule_70_amd import binding, inputs
    binding.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    if args.only == "bwd":
        r = bench_backward(binding, inputs, args.steps)
        print(json.dumps({"bwd_ms": r["ms"], "steps": args.steps, "workspace_bytes": r["ws_bytes"]}), flush=True)
        return
    if args.only == "bidir":
        r = bench_bidir(binding, inputs, args.steps)
        print(json.dumps({"bidir_ms": r["ms"], "bytes": r["bytes"], "steps": args.steps}), flush=True)
        return
    if args.only == "dp":
        r = bench_delta_product(binding, inputs, args.steps)
        print(json.dumps({"delta_product_ms": r["ms"], "bytes": r["bytes"], "steps": args.steps}), flush=True)
        return
    if args.only == "gdn2":
        g2, g2d = bench_gdn2(binding, inputs, args.steps)
        print(json.dumps({"gdn2_chunk_ms": g2["ms"], "gdn2_chunk_fused_ms": g2["fused_ms"],
                          "gdn2_chunk_bytes": g2["bytes"], "steps": args.steps,
                          "gdn2_decode_us": g2d["ms"] * 1e3}), flush=True)
        return
    res = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic"}
    print("[bench] chunked forward B4 H16 T4096 d128 ...", file=sys.stderr, flush=True)
    c = bench_chunk(binding, inputs, args.steps, args.warmup, warm_too=args.only == "all")
    B, H, T, dk, dv = c["shape"]
    res["value"] = c["tokens"] / (c["ms"] / 1e3)
    res["unit"] = "tokens/s"
    res["ms_per_step"] = c["ms"]
    res["config"] = {"workload": inputs.WORKLOADS[1], "B": B, "H": H, "T": T, "dk": dk, "dv": dv,
                     "chunk": 64, "read": "post", "h0": "N(0, 0.1)", "inputs": "bf16 q/k/v, fp32 gates/state"}
    gbs = c["bytes"] / (c["ms"] / 1e3) / 1e9
    tflops = c["flops"] / (c["ms"] / 1e3) / 1e12
    res["ms_per_step_mean"] = c["mean_ms"]
    res["input_sets"] = c["sets"]
    res["timing"] = ("median of per-call HIP event pairs on the launch stream over the %d timed calls "
                     "(ms_per_step_mean: the bracket of all of them / %d), after %.0f ms of untimed "
                     "calls that bring the clock to its steady state and %d warm-up calls; the calls "
                     "rotate over %d independent copies of the inputs and outputs, so each call reads "
                     "its inputs from HBM rather than from the 256 MB last-level cache"
                     % (args.steps, args.steps, SETTLE_MS, args.warmup, c["sets"]))
    if "ms_cache_warm" in c:
        res["ms_per_step_cache_warm"] = c["ms_cache_warm"]
        res["cache_warm_note"] = ("the same calls on one copy of the inputs: the ~205 MB they read fit "
                                  "in the last-level cache and are partly served from it")
    tflops_exec = c["flops_exec"] / (c["ms"] / 1e3) / 1e12
    res["roofline"] = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": gbs / HBM_PEAK_GBS,
                       "traffic": measured_traffic("chunk_fwd_fast_B4_H16_T4096_d128_hbm_traffic.md",
                                                   "chunk_fwd_fast.hip", "HBM bytes per launch"),
                       "kernel": "chunk_fwd_fast_kernel", "bytes_per_launch": c["bytes"],
                       "mfma": {"achieved": tflops, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                "frac": tflops / BF16_PEAK_TFLOPS, "flops_per_launch": c["flops"],
                                "count": "algorithmic",
                                "executed": {"achieved": tflops_exec, "frac": tflops_exec / BF16_PEAK_TFLOPS,
                                             "flops_per_launch": c["flops_exec"],
                                             "count": "executed (whole triangular tiles, the inverses' "
                                                      "products; 192 x16x32 + 48 x16x16 bf16 MFMAs per "
                                                      "workgroup-chunk)"}}}
    if not args.no_peaks:
        print("[bench] measured peaks (copy, bf16 GEMM) ...", file=sys.stderr, flush=True)
        mp = measured_peaks()
        res["roofline"]["measured_peak"] = mp
        res["roofline"]["frac_of_measured"] = gbs / mp["hbm_copy_GBs"]
        res["roofline"]["mfma"]["frac_of_measured"] = tflops / mp["bf16_gemm_TFLOPs"]
        res["roofline"]["mfma"]["executed"]["frac_of_measured"] = tflops_exec / mp["bf16_gemm_TFLOPs"]
    if args.only in ("all", "decode"):
        print("[bench] decode 64 steps N256 Hv32 d128 ...", file=sys.stderr, flush=True)
        d = bench_decode(binding, inputs, reps=2)
        sgbs = d["state_bytes"] / (d["ms"] / 1e3) / 1e9
        res["decode"] = {"metric": "decode-step state GB/s", "value": sgbs, "unit": "GB/s",
                         "us_per_step": d["ms"] * 1e3, "us_per_step_median": d["median_ms"] * 1e3,
                         "state_GBs_at_median": d["state_bytes"] / (d["median_ms"] / 1e3) / 1e9,
                         "tokens_per_s": d["tokens"] / (d["ms"] / 1e3),
                         "state_sets": d["sets"],
                         "workload": inputs.WORKLOADS[3],
                         "roofline": {"bound": "hbm", "achieved": (d["state_bytes"] + d["io_bytes"]) / (d["ms"] / 1e3) / 1e9,
                                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": (d["state_bytes"] + d["io_bytes"]) / (d["ms"] / 1e3) / 1e9 / HBM_PEAK_GBS,
                                      "kernel": "decode_kernel<bf16, 128, 128>",
                                      "traffic": measured_traffic("decode_N256_Hv32_d128_hbm_traffic.md",
                                                                  "decode.hip", "HBM bytes per step")}}
        if "measured_peak" in res["roofline"]:
            res["decode"]["roofline"]["frac_of_measured"] = (res["decode"]["roofline"]["achieved"] /
                                                            res["roofline"]["measured_peak"]["hbm_copy_GBs"])
    if args.only == "all":
        print("[bench] packed variable-length and bidirectional workloads ...", file=sys.stderr, flush=True)
        vl = bench_varlen(binding, inputs, max(3, args.steps // 4))
        ms_ = bench_many_segments(binding, inputs, max(3, args.steps // 4))
        bd = bench_bidir(binding, inputs, max(3, args.steps // 4))
        fu = bench_fused(binding, inputs, max(3, args.steps // 4))
        g2, g2d = bench_gdn2(binding, inputs, max(3, args.steps // 8))
        dpr = bench_delta_product(binding, inputs, max(3, args.steps // 4))
        bwr = bench_backward(binding, inputs, 3)
        res["other_workloads"] = {
            inputs.WORKLOADS[2]: {"tokens_per_s": vl["tokens"] / (vl["ms"] / 1e3), "ms": vl["ms"],
                                  "hbm_frac": vl["bytes"] / (vl["ms"] / 1e3) / 1e9 / HBM_PEAK_GBS,
                                  "lengths": vl["lengths"]},
            "gdr-varlen-bf16-2048seg-16..48-H16-d128-c64": {
                "tokens_per_s": ms_["tokens"] / (ms_["ms"] / 1e3), "ms": ms_["ms"],
                "hbm_frac": ms_["bytes"] / (ms_["ms"] / 1e3) / 1e9 / HBM_PEAK_GBS,
                "note": "2048 short packed segments (beyond 128 segments the kernel keeps their order)"},
            "gdr-chunk-fwd-fused-prologue-bf16-B4-H16-T4096-d128-c64": {
                "tokens_per_s": fu["tokens"] / (fu["ms"] / 1e3), "ms": fu["ms"],
                "prologue": "q/k rows normalised and gates formed from raw inputs in the kernel"},
            inputs.WORKLOADS[4]: {"tokens_per_s": bd["tokens"] / (bd["ms"] / 1e3), "ms": bd["ms"],
                                  "hbm_frac": bd["bytes"] / (bd["ms"] / 1e3) / 1e9 / HBM_PEAK_GBS,
                                  "entry": "gdr_chunk_fwd_bidir: the forward scan, then the reverse scan "
                                           "accumulating into out (two launches of the chunk kernel)",
                                  "bytes_note": "hbm_frac on the bytes of one read of q, k, v and both gate "
                                                "sets and one write of out"},
            "gdn2-chunk-fwd-bf16-B4-H16-T4096-d128-c32": {
                "tokens_per_s": g2["tokens"] / (g2["ms"] / 1e3), "ms": g2["ms"],
                "one_pass_ms": g2["fused_ms"], "workspace_bytes": g2["ws_bytes"],
                "roofline": {"bound": "hbm", "achieved": g2["bytes"] / (g2["ms"] / 1e3) / 1e9, "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": g2["bytes"] / (g2["ms"] / 1e3) / 1e9 / HBM_PEAK_GBS,
                             "bytes_per_launch": g2["bytes"],
                             "kernel": "gdn2_prep_kernel + gdn2_chain_kernel <bf16, 32, 128> (one call)",
                             "traffic": measured_traffic("gdn2_chunk_B4_H16_T4096_d128_hbm_traffic.md",
                                                         "gdn2_fwd.hip", "HBM bytes per call")}},
            "delta-product-n2-pre-bf16-B4-H16-T4096-d128-c64": {
                "tokens_per_s": dpr["tokens"] / (dpr["ms"] / 1e3), "ms": dpr["ms"],
                "hbm_frac": dpr["bytes"] / (dpr["ms"] / 1e3) / 1e9 / HBM_PEAK_GBS,
                "kernel": "chunk_fwd_fast_kernel<false> over 2 sub-steps per token"},
            "gdr-backward-bf16-B4-H16-T4096-d128": {
                "tokens_per_s": bwr["tokens"] / (bwr["ms"] / 1e3), "ms": bwr["ms"],
                "hbm_frac": bwr["bytes"] / (bwr["ms"] / 1e3) / 1e9 / HBM_PEAK_GBS,
                "workspace_bytes": bwr["ws_bytes"],
                "kernel": "bwd_prep_kernel + bwd_sweep_kernel + bwd_grad_kernel <bf16, 128>",
                "note": "chunk-form adjoint over 64-token chunks: chunk-parallel prep, forward and adjoint "
                        "state sweeps in one launch, chunk-parallel gradients; products as split-bf16 "
                        "matrix-core products"},
            "gdn2-decode-bf16-N256-Hk16-Hv32-d128": {
                "state_GB_per_s": g2d["state_bytes"] / (g2d["ms"] / 1e3) / 1e9, "us_per_step": g2d["ms"] * 1e3,
                "roofline": {"bound": "hbm",
                             "achieved": (g2d["state_bytes"] + g2d["io_bytes"]) / (g2d["ms"] / 1e3) / 1e9,
                             "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": (g2d["state_bytes"] + g2d["io_bytes"]) / (g2d["ms"] / 1e3) / 1e9 / HBM_PEAK_GBS,
                             "kernel": "gdn2_decode_kernel<bf16, 128, 128>"}},
        }
    if not args.no_cpu:
        print("[bench] CPU oracle baseline ...", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(inputs)
        if args.only == "all":
            res["cpu_baseline_other"] = cpu_baseline_other(inputs)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
