"""Host-side logic of bench.py (no GPU): the one-GPU guard, the expert-load summary and the rule
that a counter summary under profiles/ is used only while the kernel sources it was taken on are
unchanged."""
import os
import subprocess
import sys

import numpy as np

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_expert_histogram():
    counts = np.array([0, 5, 100, 0, 3, 12, 0, 1, 0, 40], np.int64)
    h = bench.expert_histogram(counts)
    assert h["max_rows"] == 100 and h["min_rows"] == 0
    assert h["empty"] == 4 and h["nonempty"] == 6
    assert h["max_share"] == round(100 / 161, 4)
    assert h["top8_share"] == round(161 / 161, 4)


def test_measured_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    files = bench.GEMM_SOURCES
    os.makedirs(tmp_path / "profiles")
    summary = tmp_path / "profiles" / "x.txt"

    def write(sha):
        summary.write_text("title line\n\nsource_sha256: %s\nhbm_bytes_per_dispatch: 123456789\n"
                           " indented: note\n" % sha)

    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    write(bench.source_digest(files))
    assert bench.measured_traffic("x.txt", files) == 123456789
    write("0" * 64)
    assert bench.measured_traffic("x.txt", files) is None
    assert bench.measured_traffic("missing.txt", files) is None


def test_source_digest_ignores_comments_and_layout_only():
    a = "int f(int x) {  // add one\n  return x + 1; /* a block\n   comment */ }\n"
    b = "int f(int x) {\n\n  return x + 1;   }  // another note\n"
    c = "int f(int x) { return x + 2; }"
    assert bench.source_code_text(a) == bench.source_code_text(b)
    assert bench.source_code_text(a) != bench.source_code_text(c)
