"""Host-side checks of bench.py's contract (no GPU needed)."""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_published_mi355x_peaks():
    # HBM3E 8 TB/s; dense matrix peaks: bf16 2.5 PFLOP/s, e4m3 5.0 PFLOP/s
    assert bench.HBM_PEAK_GBS == 8000.0
    assert bench.MFMA_PEAK_TFLOPS == 2500.0
    assert bench.FP8_PEAK_TFLOPS == 5000.0


def test_kernel_hash_covers_the_kernel_sources():
    names = sorted(os.path.basename(p) for p in bench.KERNEL_SRCS)
    assert names == ["spense_api.cpp", "spense_device.h", "spense_internal.h", "spense_kernels.hip", "spense_tile.hip"]
    h = bench.kernel_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    assert bench.kernel_hash() == h


def test_traffic_is_reported_only_for_the_sources_it_was_measured_on(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({"kernel_sha256_16": bench.kernel_hash(), "hbm_bytes_per_launch": 123.0}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.load_traffic() == 123.0
    f.write_text(json.dumps({"kernel_sha256_16": "0" * 16, "hbm_bytes_per_launch": 123.0}))
    assert bench.load_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.load_traffic() is None


class _FakeCuda:
    def __init__(self):
        self.syncs = 0

    def synchronize(self):
        self.syncs += 1


class _FakeTorch:
    def __init__(self):
        self.cuda = _FakeCuda()


def test_spin_up_runs_whole_synchronised_rounds_for_the_requested_time():
    torch = _FakeTorch()
    calls = []
    ms = bench.spin_up(torch, calls.append, seconds=0.02)
    assert ms >= 20.0
    assert len(calls) % 8 == 0 and len(calls) == 8 * torch.cuda.syncs
    assert calls == list(range(len(calls)))
