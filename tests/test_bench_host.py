"""bench.py's host logic: the byte model, launch-mode names and the one-GPU guard."""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_byte_model_at_d128():
    """Keyformer 268n + 1036 + 1048m and PyramidKV 264n + 1032 + 1040m bytes per
    cache-step at D = 128 (K read 2nD; scores read and written; Gumbel read when
    evicting; the new row; K, V, score, Gumbel and position of each moved row)."""
    n = np.array([0, 1, 511, 4096, 12288])
    m = np.array([0, 1, 7, 300, 12000])
    assert (bench.step_bytes("keyformer", n, 128, m) == 268 * n + 1036 + 1048 * m).all()
    assert (bench.step_bytes("pyramid", n, 128, m) == 264 * n + 1032 + 1040 * m).all()
    # under budget nothing is evicted and no Gumbel value is read
    assert (bench.step_bytes("keyformer", n, 128, 0, over=False) == 264 * n + 1036).all()


def test_byte_model_at_d64():
    n, m = 1000, 10
    assert bench.step_bytes("keyformer", n, 64, m) == 2 * n * 64 + 12 * n + 512 + 12 + m * 536
    assert bench.step_bytes("pyramid", n, 64, m) == 2 * n * 64 + 8 * n + 512 + 8 + m * 528


def test_launch_mode_names():
    assert bench.launch_mode(False, 1) == "per-layer_x1tok"
    assert bench.launch_mode(True, 32) == "all-layers_x32tok"


def test_missing_profile_gives_no_traffic():
    assert bench.measured_traffic("no-such-workload", "step_kernel", "per-layer_x1tok") is None


def test_source_hash_ignores_comments(tmp_path, monkeypatch):
    a = tmp_path / "a.hip"
    a.write_text("int x; // one\n/* two */ int y;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", ["a.hip"])
    h1 = bench.kernel_source_hash()
    a.write_text("int x;   // changed\n int y;\n")
    assert bench.kernel_source_hash() == h1
    a.write_text("int x; int z;\n")
    assert bench.kernel_source_hash() != h1


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
