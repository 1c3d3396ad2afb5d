"""Host logic of bench.py (CPU only): the figures it takes from the committed
counter summaries are used only while the kernel sources still hash to the
value recorded with them, and the one-GPU contract refuses more GPUs."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_committed_summaries_match_the_sources():
    # both summaries were taken on the sources in the tree
    assert bench.measured_traffic() is not None
    assert bench.walk_mfma_busy() is not None
    assert 0.0 < bench.walk_mfma_busy() < 1.0
    assert bench.measured_traffic() >= 1_000_000_000


def test_a_changed_source_voids_the_figures(tmp_path, monkeypatch):
    # a copy of the tree's sources with one byte changed hashes differently
    for rel in bench.PREFILL_SOURCES + bench.DECODE_SOURCES:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, rel), dst)
    for rel in (bench.TRAFFIC_PROFILE, bench.WALK_COUNTERS_PROFILE):
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, rel), dst)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.walk_mfma_busy() is not None and bench.measured_traffic() is not None
    with open(tmp_path / bench.PREFILL_SOURCES[0], "ab") as fh:
        fh.write(b"\n")
    assert bench.walk_mfma_busy() is None
    assert bench.measured_traffic() is not None      # the decode sources are untouched
    with open(tmp_path / bench.DECODE_SOURCES[1], "ab") as fh:
        fh.write(b"\n")
    assert bench.measured_traffic() is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode != 0
    assert "one GPU" in (r.stderr + r.stdout)
