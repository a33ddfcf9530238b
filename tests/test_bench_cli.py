"""Host-side checks of the benchmark's contract (no GPU): the single-GPU
refusal of --gpus N > 1 and the rule that the roofline's traffic figure is
reported only while the counter summary matches the GEMM sources."""
import os
import subprocess
import sys

from diffusion_transformer_image_mm_amd import traffic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "single GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""   # no JSON line


def _summary(path, sha, nbytes):
    path.write_text("# header\n"
                    f"kernel_source_sha256: {sha}\n"
                    "fetch_bytes_per_launch: 1\n"
                    "write_bytes_per_launch: 2\n"
                    f"traffic_bytes_per_launch: {nbytes}\n")


def test_traffic_reported_only_for_matching_sources(tmp_path, monkeypatch):
    p = tmp_path / "traffic.txt"
    monkeypatch.setattr(traffic, "SUMMARY", str(p))
    assert traffic.load_traffic() is None            # no summary
    _summary(p, traffic.source_sha256(), 123456789)
    assert traffic.load_traffic() == 123456789.0     # taken on these sources
    _summary(p, "0" * 64, 123456789)
    assert traffic.load_traffic() is None            # sources changed since
    p.write_text(f"kernel_source_sha256: {traffic.source_sha256()}\n")
    assert traffic.load_traffic() is None            # incomplete summary


def test_source_hash_covers_kernel_and_header():
    names = sorted(os.path.basename(f) for f in traffic.KERNEL_SOURCES)
    assert names == ["common.h", "k_gemm.hip"]
    assert all(os.path.isfile(f) for f in traffic.KERNEL_SOURCES)
    assert len(traffic.source_sha256()) == 64
