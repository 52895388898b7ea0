"""Benchmark of the gated delta rule library on one MI355X.

Headline: chunked-forward tokens/s on the B4 H16 T4096 d128 bf16 workload (chunk 64,
nonzero h0, post-write read); one step is one gdr_chunk_fwd call over the whole batch.
Also reported: decode-step state GB/s (256 sequences, 16 key / 32 value heads, d128,
fp32 state, 64 consecutive in-place steps), the packed variable-length and bidirectional
workloads' tokens/s, roofline fractions, and the fp64 CPU oracle timed on this host.

All inputs are synthetic (seeded generators in gated_delta_rule_70_amd/inputs.py) and
resident in HBM before timing starts. Kernel times come from HIP events recorded on the
stream the kernels are launched on (torch's current stream).
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


def timed(fn, steps, warmup, stream):
    """Mean time per call in ms: HIP events on the launch stream around `steps` back-to-back
    calls (after `warmup` untimed ones), bracketed by device synchronisation."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / steps, wall


def bench_chunk(binding, inputs, steps, warmup):
    import torch
    case = inputs.workload1()
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in (case.q, case.k, case.v))
    la, b, h0 = case.log_alpha.to(dev), case.beta.to(dev), case.h0.to(dev)
    out = torch.empty_like(v)
    hT = torch.empty_like(h0)
    stream = torch.cuda.current_stream(dev)
    fn = lambda: binding.chunk_fwd(q, k, v, la, b, h0, None, chunk=64, out=out, hT=hT)
    ms, wall = timed(fn, steps, warmup, stream)
    B, H, T, dk = case.q.shape
    dv = case.v.shape[-1]
    return dict(ms=ms, wall=wall, tokens=B * T, bytes=chunk_bytes(B, H, T, dk, dv, 2, B),
                flops=chunk_flops(B, H, T, dk, dv), shape=(B, H, T, dk, dv))


def bench_decode(binding, inputs, reps):
    import torch
    dc = inputs.workload3()
    dev = torch.device("cuda:0")
    steps = dc.q.shape[0]
    q, k, v, la, b = (t.to(dev) for t in (dc.q, dc.k, dc.v, dc.log_alpha, dc.beta))
    state = dc.state.to(dev)
    out = torch.empty((steps,) + tuple(dc.v.shape[1:]), dtype=dc.v.dtype, device=dev)
    stream = torch.cuda.current_stream(dev)
    # one warm pass of the 64 steps, then `reps` timed passes (state keeps evolving in place)
    for s in range(steps):
        binding.decode_step(q[s], k[s], v[s], la[s], b[s], state, state_out=state, out=out[s])
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for r in range(reps):
        for s in range(steps):
            binding.decode_step(q[s], k[s], v[s], la[s], b[s], state, state_out=state, out=out[s])
    end.record(stream)
    torch.cuda.synchronize()
    mean = start.elapsed_time(end) / (steps * reps)
    N, Hv, dk, dv = dc.state.shape
    sbytes = 2 * N * Hv * dk * dv * 4
    io = (dc.q[0].numel() * 2 + dc.v[0].numel()) * 2 + N * Hv * 2 * 4 + N * Hv * dv * 2
    return dict(ms=mean, state_bytes=sbytes, io_bytes=io, tokens=N, steps=steps * reps)


def bench_varlen(binding, inputs, steps):
    import torch
    case = inputs.workload2()
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in (case.q, case.k, case.v))
    la, b, h0, cu = case.log_alpha.to(dev), case.beta.to(dev), case.h0.to(dev), case.cu_seqlens.to(dev)
    out, hT = torch.empty_like(v), torch.empty_like(h0)
    fn = lambda: binding.chunk_fwd(q, k, v, la, b, h0, cu, chunk=64, out=out, hT=hT)
    ms, _ = timed(fn, steps, 200, torch.cuda.current_stream(dev))
    T = case.q.shape[2]
    H, dk, dv = case.q.shape[1], case.q.shape[3], case.v.shape[3]
    nseq = case.cu_seqlens.numel() - 1
    return dict(ms=ms, tokens=T, bytes=chunk_bytes(1, H, T, dk, dv, 2, nseq),
                lengths=[int(x) for x in (case.cu_seqlens[1:] - case.cu_seqlens[:-1])])


def bench_fused(binding, inputs, steps):
    """The fused prologue on the workload-1 shapes: raw q/k rows (normalised in the kernel) and
    raw gate inputs a, b with per-head A_log, dt_bias (``gdr_chunk_fwd_gated`` with
    GDR_QK_L2NORM)."""
    import torch
    c = inputs.raw_case(B=4, T=4096, Hk=16, Hv=16, dk=128, dv=128, dtype=torch.bfloat16, seed=1001,
                        h0_std=0.1)
    dev = torch.device("cuda:0")
    q, k, v, a, b, A_log, dtb, h0 = (t.to(dev) for t in (c.q, c.k, c.v, c.a, c.b, c.A_log, c.dt_bias, c.h0))
    out, hT = torch.empty_like(v), torch.empty_like(h0)
    fn = lambda: binding.chunk_fwd_gated(q, k, v, a, b, A_log, dtb, h0, chunk=64, out=out, hT=hT, l2norm=True)
    ms, _ = timed(fn, steps, 300, torch.cuda.current_stream(dev))
    return dict(ms=ms, tokens=4 * 4096)


def bench_bidir(binding, inputs, steps):
    import torch
    case = inputs.workload4()
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in (case.q, case.k, case.v))
    la, b, cu = case.log_alpha.to(dev), case.beta.to(dev), case.cu_seqlens.to(dev)
    la2, b2 = case.extra["log_alpha_bwd"].to(dev), case.extra["beta_bwd"].to(dev)
    out = torch.empty_like(v)

    def fn():
        binding.chunk_fwd(q, k, v, la, b, None, cu, chunk=64, read="pre", out=out, want_state=False)
        binding.chunk_fwd(q, k, v, la2, b2, None, cu, chunk=64, read="pre", reverse=True, out=out,
                          accumulate=True, want_state=False)

    ms, _ = timed(fn, steps, 200, torch.cuda.current_stream(dev))
    return dict(ms=ms, tokens=case.q.shape[2])


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
    q, k, v, g, b, w, h0 = (t.to(dev) for t in (c.q, c.k, c.v, c.g, c.b, c.w, c.h0))
    out, hT = torch.empty_like(v), torch.empty_like(h0)
    ws = torch.empty(binding.gdn2_chunk_fwd_workspace_bytes(4, 4096, 16, 16, 128, 128, 32), dtype=torch.uint8,
                     device=dev)
    fn = lambda: binding.gdn2_chunk_fwd(q, k, v, g, b, w, h0, chunk=32, out=out, hT=hT, workspace=ws)
    ms, _ = timed(fn, steps, 50, torch.cuda.current_stream(dev))
    # the one-pass kernel (no workspace) on the same inputs, for reference
    fn1 = lambda: binding.gdn2_chunk_fwd(q, k, v, g, b, w, h0, chunk=32, out=out, hT=hT, fused=True)
    ms1, _ = timed(fn1, max(3, steps // 4), 5, torch.cuda.current_stream(dev))
    chunk = dict(ms=ms, fused_ms=ms1, ws_bytes=ws.numel(), tokens=4 * 4096,
                 bytes=gdn2_bytes(4, 16, 16, 4096, 128, 128, 2, 4))
    del q, k, v, g, b, w, h0, out, hT, ws
    N, Hk, Hv = 256, 16, 32
    dc = inputs.gdn2_case(B=N, T=1, Hk=Hk, Hv=Hv, dk=128, dv=128, dtype=torch.bfloat16, seed=1003, h0_std=0.1)
    one = lambda t: t[:, :, 0].contiguous().to(dev)
    dq, dk_, dv_, dg, db, dw = (one(t) for t in (dc.q, dc.k, dc.v, dc.g, dc.b, dc.w))
    state = dc.h0.to(dev)
    dout = torch.empty((N, Hv, 128), dtype=torch.bfloat16, device=dev)
    fn = lambda: binding.gdn2_decode_step(dq, dk_, dv_, dg, db, dw, state, state_out=state, out=dout)
    dms, _ = timed(fn, max(steps, 64), 300, torch.cuda.current_stream(dev))
    sbytes = 2 * N * Hv * 128 * 128 * 4
    io = N * Hk * 128 * (3 * 2 + 4) + N * Hv * 128 * 3 * 2
    return chunk, dict(ms=dms, state_bytes=sbytes, io_bytes=io, tokens=N)


def bench_delta_product(binding, inputs, steps):
    """DeltaProduct with two sub-steps per token on the workload-1 shapes (B4 H16 T4096 d128 bf16),
    pre-write read (the page's), chunk 64 of sub-steps."""
    import torch
    dev = torch.device("cuda:0")
    c = inputs.delta_product_case(B=4, T=4096, n=2, Hk=16, Hv=16, dk=128, dv=128, dtype=torch.bfloat16,
                                  seed=1001, h0_std=0.1)
    q, k, v, la, b, h0 = (t.to(dev) for t in (c.q, c.k, c.v, c.log_alpha, c.beta, c.h0))
    out, hT = torch.empty((4, 16, 4096, 128), dtype=torch.bfloat16, device=dev), torch.empty_like(h0)
    fn = lambda: binding.delta_product_fwd(q, k, v, la, b, h0, chunk=64, read="pre", out=out, hT=hT)
    ms, _ = timed(fn, steps, 100, torch.cuda.current_stream(dev))
    tok = 4 * 16 * 4096
    nbytes = tok * 128 * 2 * (1 + 2 + 2 + 1) + tok * 4 * (1 + 2) + 2 * 4 * 16 * 128 * 128 * 4
    return dict(ms=ms, tokens=4 * 4096, bytes=nbytes)


def bench_backward(binding, inputs, steps):
    """Gradients of the workload-1 forward (B4 H16 T4096 d128, bf16 inputs, post-write read) with
    respect to every input, from random upstream gradients of the outputs and final state."""
    import torch
    dev = torch.device("cuda:0")
    c = inputs.workload1()
    q, k, v, la, b, h0 = (t.to(dev) for t in (c.q, c.k, c.v, c.log_alpha, c.beta, c.h0))
    g = torch.Generator(device="cpu").manual_seed(5)
    dout = torch.randn(tuple(c.v.shape), generator=g).to(torch.bfloat16).to(dev)
    dhT = torch.randn(tuple(c.h0.shape), generator=g).to(dev)
    ws = torch.empty(binding.chunk_bwd_workspace_bytes(4, 4096, 16, 16, 128, 128), dtype=torch.uint8, device=dev)
    fn = lambda: binding.chunk_bwd(q, k, v, la, b, dout, h0, None, dhT, workspace=ws)
    ms, _ = timed(fn, steps, 2, torch.cuda.current_stream(dev))
    tok = 4 * 16 * 4096
    # inputs, dout read once; gradients written once (dq, dk, dv fp32); h0, dhT, dh0
    nbytes = tok * 128 * 2 * 4 + tok * 4 * 4 + tok * 128 * 4 * 3 + 3 * 4 * 16 * 128 * 128 * 4
    return dict(ms=ms, tokens=4 * 4096, bytes=nbytes, ws_bytes=ws.numel())


def cpu_baseline(inputs, min_wall=1.5, max_reps=20):
    """The fp64 oracle, as it is, on this host's cores: the whole B4 H16 T4096 d128 workload,
    repeated until at least `min_wall` seconds have passed (a bounded sample)."""
    import oracle
    case = inputs.workload1()
    threads = min(len(os.sched_getaffinity(0)), 64)
    import numpy as np
    args = [np.ascontiguousarray(t.double().numpy()) for t in
            (case.q, case.k, case.v, case.log_alpha, case.beta, case.h0)]
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.scan(*args, threads=threads)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_wall or reps >= max_reps:
            break
    tokens = case.q.shape[0] * case.q.shape[2] * reps
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "the whole B4 H16 T4096 d128 workload (64 sequence-heads) %d times, fp64 "
                      "per-token recurrence, %.1f s wall on %d threads; CPU: %s"
                      % (reps, dt, threads, cpu_model)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # untimed calls before the timed ones: the GPU takes tens of milliseconds of sustained work
    # to reach its steady clock (with 50 warmup calls, about 5 ms, the chunked forward still
    # timed 16% slower than with 300); 500 calls are about 50 ms
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", choices=["chunk", "decode", "gdn2", "bwd", "dp", "all"], default="all",
                    help="gdn2, bwd, dp: only the GDN-2 workloads, the backward or DeltaProduct (for "
                         "profiling them)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling HBM byte counters)")
    args = ap.parse_args()
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
    c = bench_chunk(binding, inputs, args.steps, args.warmup)
    B, H, T, dk, dv = c["shape"]
    res["value"] = c["tokens"] / (c["ms"] / 1e3)
    res["unit"] = "tokens/s"
    res["ms_per_step"] = c["ms"]
    res["config"] = {"workload": inputs.WORKLOADS[1], "B": B, "H": H, "T": T, "dk": dk, "dv": dv,
                     "chunk": 64, "read": "post", "h0": "N(0, 0.1)", "inputs": "bf16 q/k/v, fp32 gates/state"}
    gbs = c["bytes"] / (c["ms"] / 1e3) / 1e9
    tflops = c["flops"] / (c["ms"] / 1e3) / 1e12
    res["roofline"] = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": gbs / HBM_PEAK_GBS,
                       "traffic": measured_traffic("chunk_fwd_fast_B4_H16_T4096_d128_hbm_traffic.md",
                                                   "chunk_fwd_fast.hip", "HBM bytes per launch"),
                       "kernel": "chunk_fwd_fast_kernel", "bytes_per_launch": c["bytes"],
                       "mfma": {"achieved": tflops, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                "frac": tflops / BF16_PEAK_TFLOPS, "flops_per_launch": c["flops"]}}
    if args.only in ("all", "decode"):
        print("[bench] decode 64 steps N256 Hv32 d128 ...", file=sys.stderr, flush=True)
        d = bench_decode(binding, inputs, reps=2)
        sgbs = d["state_bytes"] / (d["ms"] / 1e3) / 1e9
        res["decode"] = {"metric": "decode-step state GB/s", "value": sgbs, "unit": "GB/s",
                         "us_per_step": d["ms"] * 1e3,
                         "tokens_per_s": d["tokens"] / (d["ms"] / 1e3),
                         "workload": inputs.WORKLOADS[3],
                         "roofline": {"bound": "hbm", "achieved": (d["state_bytes"] + d["io_bytes"]) / (d["ms"] / 1e3) / 1e9,
                                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": (d["state_bytes"] + d["io_bytes"]) / (d["ms"] / 1e3) / 1e9 / HBM_PEAK_GBS,
                                      "kernel": "decode_kernel<bf16, 128, 128>",
                                      "traffic": measured_traffic("decode_N256_Hv32_d128_hbm_traffic.md",
                                                                  "decode.hip", "HBM bytes per step")}}
    if args.only == "all":
        print("[bench] packed variable-length and bidirectional workloads ...", file=sys.stderr, flush=True)
        vl = bench_varlen(binding, inputs, max(3, args.steps // 4))
        bd = bench_bidir(binding, inputs, max(3, args.steps // 4))
        fu = bench_fused(binding, inputs, max(3, args.steps // 4))
        g2, g2d = bench_gdn2(binding, inputs, max(3, args.steps // 8))
        dpr = bench_delta_product(binding, inputs, max(3, args.steps // 4))
        bwr = bench_backward(binding, inputs, 3)
        res["other_workloads"] = {
            inputs.WORKLOADS[2]: {"tokens_per_s": vl["tokens"] / (vl["ms"] / 1e3), "ms": vl["ms"],
                                  "hbm_frac": vl["bytes"] / (vl["ms"] / 1e3) / 1e9 / HBM_PEAK_GBS,
                                  "lengths": vl["lengths"]},
            "gdr-chunk-fwd-fused-prologue-bf16-B4-H16-T4096-d128-c64": {
                "tokens_per_s": fu["tokens"] / (fu["ms"] / 1e3), "ms": fu["ms"],
                "prologue": "q/k rows normalised and gates formed from raw inputs in the kernel"},
            inputs.WORKLOADS[4]: {"tokens_per_s": bd["tokens"] / (bd["ms"] / 1e3), "ms": bd["ms"],
                                  "calls": 2},
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
                "kernel": "chunk_fwd_kernel<bf16, 64, 128> over 2 sub-steps per token"},
            "gdr-backward-bf16-B4-H16-T4096-d128": {
                "tokens_per_s": bwr["tokens"] / (bwr["ms"] / 1e3), "ms": bwr["ms"],
                "hbm_frac": bwr["bytes"] / (bwr["ms"] / 1e3) / 1e9 / HBM_PEAK_GBS,
                "workspace_bytes": bwr["ws_bytes"], "kernel": "bwd_kernel<bf16, 128>",
                "note": "chunk-form adjoint (32-token chunks), one workgroup of 8 waves per sequence-head "
                        "and 32 value columns; products as split-bf16 matrix-core products"},
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
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
