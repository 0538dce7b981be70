"""bench.py's command-line contract on the CPU: it measures one GPU and
refuses --gpus N > 1 with a message, its timed loop covers exactly the
requested steps in order, and its traffic figure is only taken from a
counter summary recorded on the current GEMV source."""

import json
import os
import subprocess
import sys

from conftest import ROOT


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single" in r.stderr


def test_traffic_summary_matches_source_or_is_ignored():
    sys.path.insert(0, ROOT)
    import bench
    traffic, note = bench.read_traffic(1)
    path = bench.TRAFFIC_SUMMARY
    if not os.path.exists(path):
        assert traffic is None
        return
    rec = [json.loads(l.split(" ", 1)[1]) for l in open(path) if l.startswith("TRAFFIC_JSON ")][0]
    if rec["gemv_source_sha"] == bench.gemv_source_sha():
        assert traffic == rec["bytes_per_launch"]
        # the weights are streamed once: counted traffic within 5% of the algorithmic bytes
        assert 0.95 < traffic / rec["algorithmic_bytes_per_launch"] < 1.05
    else:
        assert traffic is None and "changed" in note
    assert bench.read_traffic(2)[0] is None


def test_graph_plan_covers_exactly_the_steps():
    sys.path.insert(0, ROOT)
    import bench
    for first, steps, per in ((20, 200, 36), (0, 20, 36), (5, 7, 1), (0, 72, 36), (3, 1, 8)):
        plan = bench.graph_plan(first, steps, per)
        covered = [f + k for f, n in plan for k in range(n)]
        assert covered == list(range(first, first + steps))
        assert all(1 <= n <= per for _, n in plan)
    assert bench.graph_plan(0, 0, 36) == []
