"""Host logic of bench.py, on the CPU: the one-GPU rule, the burst size, and
the rule that the counter summary's HBM bytes are used only while the kernel
sources it was taken on are unchanged."""
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""                      # no JSON line


@pytest.mark.parametrize("ms_one,steps,want", [
    (0.065, 50, 100),      # short kernel: BURST_MIN_LAUNCHES launches
    (4.5, 50, 50),         # 45 launches reach BURST_MIN_MS; --steps is larger
    (4.5, 5, 45),          # ... and larger than --steps 5
    (13.7, 5, 15),         # ceil(200 / 13.7)
    (500.0, 5, 5),         # one launch passes BURST_MIN_MS: --steps decides
    (0.0, 3, 100),         # no estimate: the launch count rule
])
def test_burst_count(ms_one, steps, want):
    assert bench.burst_count(ms_one, steps) == want


def _summary(tmp_path, name, source_hash, nbytes=123456789):
    p = tmp_path / name
    rec = {"kernel": "k", "bytes_per_launch": nbytes, "source_hash": source_hash}
    p.write_text("# a counter summary\n\ntraffic_json: " + json.dumps(rec) + "\n")
    return str(p)


def test_traffic_used_only_for_the_current_sources(tmp_path):
    h = bench.kernel_source_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    assert bench.measured_traffic(_summary(tmp_path, "same.md", h)) == 123456789
    other = format(int(h, 16) ^ 1, "016x")
    assert bench.measured_traffic(_summary(tmp_path, "other.md", other)) is None
    assert bench.measured_traffic(str(tmp_path / "missing.md")) is None
    assert bench.measured_traffic("") is None
    no_line = tmp_path / "no_line.md"
    no_line.write_text("# a summary without the record\n")
    assert bench.measured_traffic(str(no_line)) is None


def test_source_hash_covers_every_dispatching_file(tmp_path, monkeypatch):
    """A change to any of the four files changes the hash (so a stale summary
    is not used); the hash reads the files in a fixed order."""
    csrc = tmp_path / "dit_dequant_gemm_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in bench.PRODUCT_KERNEL_SOURCES:
        (csrc / f).write_bytes(f"// {f}\n".encode())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    base = bench.kernel_source_hash()
    seen = {base}
    for f in bench.PRODUCT_KERNEL_SOURCES:
        old = (csrc / f).read_bytes()
        (csrc / f).write_bytes(old + b" ")
        seen.add(bench.kernel_source_hash())
        (csrc / f).write_bytes(old)
    assert len(seen) == 1 + len(bench.PRODUCT_KERNEL_SOURCES)
    assert bench.kernel_source_hash() == base


def test_committed_traffic_summary_parses():
    """The default --traffic summary holds one record for the 256 x 192
    product at 4 bits, with bytes per launch between the algorithmic bytes
    (X, packed W and scales, Y of 4096 x 3072 x 3072) and three times them."""
    path = os.path.join(ROOT, "profiles", "dequant_gemm_attnproj3072_traffic.md")
    recs = [json.loads(l.split(":", 1)[1]) for l in open(path) if l.startswith("traffic_json:")]
    assert len(recs) == 1
    rec = recs[0]
    assert "gemm_n192_kernel<4>" in rec["kernel"]
    m, n, k = 4096, 3072, 3072
    algorithmic = m * k * 2 + n * k // 2 + n * (k // 128) * 4 + m * n * 2
    assert algorithmic <= rec["bytes_per_launch"] <= 3 * algorithmic
    assert len(rec["source_hash"]) == 16
