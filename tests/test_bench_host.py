"""Host-side pieces of bench.py's measurement contract (no GPU): the one-GPU rule, the
algorithmic byte counts the roofline divides by, and the traffic lookup that drops a counter
summary taken on a different kernel source."""
from __future__ import annotations

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_chunk_bytes_workload_1():
    # q, k, v, out in bf16 (B4 H16 T4096, d 128), log alpha and beta in fp32, h0 and hT in fp32
    tok = 4 * 16 * 4096
    want = tok * 128 * 2 * 4 + tok * 2 * 4 + 2 * 4 * 16 * 128 * 128 * 4
    assert bench.chunk_bytes(4, 16, 4096, 128, 128, 2, 4) == want == 278921216


def test_gdn2_bytes_workload_1():
    # q, k, b bf16 and g fp32 per key head; v, w, out bf16 per value head; h0, hT fp32
    tok = 4 * 16 * 4096
    want = tok * 128 * (3 * 2 + 4) + tok * 128 * 3 * 2 + 2 * 4 * 16 * 128 * 128 * 4
    assert bench.gdn2_bytes(4, 16, 16, 4096, 128, 128, 2, 4) == want


def test_measured_traffic_checks_the_source(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("kernel text\n")
    digest = bench.source_digest(str(src))
    prof = tmp_path / "prof"
    prof.mkdir()
    (prof / "t.md").write_text("# t\n\n- HBM bytes per launch: 123456\n- kernel source sha256: `%s`\n" % digest)
    (prof / "old.md").write_text("# t\n\n- HBM bytes per launch: 999\n- kernel source sha256: `%s`\n" % ("0" * 64))
    monkeypatch.setattr(bench, "PROFILES", str(prof))
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    assert bench.measured_traffic("t.md", "k.hip", "HBM bytes per launch") == 123456.0
    assert bench.measured_traffic("old.md", "k.hip", "HBM bytes per launch") is None
    assert bench.measured_traffic("missing.md", "k.hip", "HBM bytes per launch") is None


def test_executed_mfma_count_matches_the_counter_summary():
    # 240 matrix-core instructions per workgroup-chunk (SQ_INSTS_MFMA / (256 workgroups x 64 chunks)
    # in the committed counter summary), 58 GFLOP per launch of the B4 H16 T4096 d128 workload
    assert bench.FAST_MFMA32_PER_WG_CHUNK + bench.FAST_MFMA16_PER_WG_CHUNK == 240
    ex = bench.chunk_flops_executed(4, 16, 4096, 128)
    assert abs(ex - 1.132e8 * 512) / ex < 0.01
    assert ex > bench.chunk_flops(4, 16, 4096, 128, 128)


def test_rotation_sets_leave_the_cache_behind(monkeypatch):
    """Each call's copy is revisited only after the other copies, which hold at least twice the
    256 MB last-level cache; --cache-warm times one copy."""
    made = []

    def make():
        i = len(made)
        made.append(i)
        return lambda: calls.append(i)

    calls = []
    monkeypatch.setattr(bench, "CACHE_WARM", False)
    for set_bytes in (278921216, 1 << 30, 64 << 20):
        made.clear()
        calls.clear()
        fn, k = bench.rotation(make, set_bytes)
        assert k == len(made) >= 2
        assert (k - 1) * set_bytes >= 2 * bench.CACHE_BYTES
        assert (k - 2) * set_bytes < 2 * bench.CACHE_BYTES or k == 2
        for _ in range(2 * k + 1):
            fn()
        assert calls == [i % k for i in range(2 * k + 1)]
    monkeypatch.setattr(bench, "CACHE_WARM", True)
    made.clear()
    fn, k = bench.rotation(make, 278921216)
    assert k == 1 and len(made) == 1
