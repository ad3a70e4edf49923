"""Host-side checks of bench.py (no GPU): the one-GPU guard, the number of
steps captured per graph, and the traffic lookup's source check."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.parametrize("M,steps,want", [(1024, 100, 4), (1024, 20, 4), (1024, 10, 2), (1024, 5, 1),
                                          (4096, 7, 1), (1, 5, bench.SMALL_STEPS_PER_GRAPH),
                                          (16, 100, bench.SMALL_STEPS_PER_GRAPH)])
def test_steps_per_graph(M, steps, want):
    got = bench.steps_per_graph(M, steps)
    assert got == want
    if M > 16:
        assert steps % got == 0  # exactly `steps` steps are timed


def test_traffic_summary_matches_its_sources(tmp_path, monkeypatch):
    # the committed summary is read only while the kernel sources hash to
    # the value it records; any other hash gives no traffic figure
    with open(bench.TRAFFIC_SUMMARY) as fh:
        text = fh.read()
    recorded = [ln.split(":", 1)[1].strip() for ln in text.splitlines() if ln.startswith("source_sha256:")][0]
    got = bench.read_traffic("exact_hbm_bytes_per_launch")
    if recorded == bench.kernel_source_hash():
        assert isinstance(got, int) and got > 0
    else:
        assert got is None
    stale = tmp_path / "traffic.txt"
    stale.write_text(text.replace(recorded, "0" * len(recorded)))
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(stale))
    assert bench.read_traffic("exact_hbm_bytes_per_launch") is None
