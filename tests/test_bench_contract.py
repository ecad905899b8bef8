"""Host-side pieces of bench.py that need no GPU: the one-GPU guard, the CPU
baseline record, and the HBM-traffic lookup that is voided when the measured
kernel's sources change."""
import hashlib
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_cpu_baseline_record():
    rec = bench.cpu_baseline(sample=4096, steps=2, gemm_mnk=(64, 48, 32))
    cores = min(16, len(os.sched_getaffinity(0)))
    assert rec["kind"] == "oracle" and rec["unit"] == "GB/s" and rec["cores"] == cores
    assert rec["value"] > 0 and f"{cores} processes x 4096 params x 2" in rec["sample"]
    assert rec["host"]["os_cpu_count"] == os.cpu_count()
    assert rec["host"]["affinity"] == len(os.sched_getaffinity(0))
    assert rec["gemm"]["shape"] == [64, 48, 32] and rec["gemm"]["gflops"] > 0


def test_traffic_lookup_follows_the_source_hash(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("kernel v1\n")
    digest = hashlib.sha256(src.read_bytes()).hexdigest()[:16]
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "apply_kernel_adamw_2pow31_hbm_bytes.md").write_text(
        f"traffic_bytes_per_launch: 123456\nsource_sha256_16: {digest}\nsources: k.hip\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic() == 123456
    src.write_text("kernel v2\n")                    # the kernel changed: the counters are void
    assert bench.measured_traffic() is None
