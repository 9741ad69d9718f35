"""Host-side checks of bench.py (no GPU): the one-GPU contract and the committed HBM counter
summary that the benchmark line's roofline traffic comes from."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_committed_traffic_belongs_to_the_current_kernel():
    """The counter summary was taken on the dominant kernel's current sources, and its HBM bytes per
    launch lie within 0.5% of the algorithmic bytes (4 T: both inputs read, both gradients written)."""
    traffic = bench.traffic_from_profiles()
    assert traffic is not None, "profiles/kl_bwd_pair8192_counters.json was taken on other kernel sources"
    algorithmic = 4 * bench.T_BYTES
    assert abs(traffic - algorithmic) <= 0.005 * algorithmic, (traffic, algorithmic)


def test_source_hash_ignores_comments(tmp_path, monkeypatch):
    """Comment-only edits keep the stored counters valid; a code edit does not."""
    h0 = bench.kernel_source_hash()
    src = {p: open(os.path.join(ROOT, p)).read() for p in bench.KERNEL_SOURCES}
    for p, text in src.items():
        os.makedirs(tmp_path / os.path.dirname(p), exist_ok=True)
        (tmp_path / p).write_text(text + "\n// a comment\n\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.kernel_source_hash() == h0
    first = bench.KERNEL_SOURCES[0]
    (tmp_path / first).write_text(src[first] + "\nint vws_extra_symbol;\n")
    assert bench.kernel_source_hash() != h0
