"""Host-side checks of bench.py's contract (no GPU needed): more than one GPU
is refused with a message, and the recorded-profile lookups key on the
kernel sources."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120, cwd=ROOT)
    assert res.returncode == 2
    assert "one GPU only" in (res.stdout + res.stderr)


@pytest.mark.parametrize("sources", [bench.BWD_SOURCES, bench.SMLA_SOURCES, bench.GLA_SOURCES, bench.MERGE_SOURCES])
def test_source_hash_is_stable_and_source_specific(sources):
    h = bench.kernel_source_hash(sources)
    assert h == bench.kernel_source_hash(sources) and len(h) == 16
    assert h != bench.kernel_source_hash(sources[:-1])


def test_recorded_figures_are_keyed_by_the_source_hash(tmp_path, monkeypatch):
    """A recorded entry whose hash matches the sources is returned; one for
    other sources reads as missing (null on the bench line)."""
    h = bench.kernel_source_hash(bench.BWD_SOURCES)
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic.json").write_text(json.dumps({
        "w/now": {"source_hash": h, "bytes_per_launch": 123},
        "w/old": {"source_hash": "0" * 16, "bytes_per_launch": 456}}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda sources: h)
    assert bench.recorded_traffic("w", "now") == 123
    assert bench.recorded_traffic("w", "old") is None
    assert bench.recorded_traffic("w", "absent") is None
