"""bench.py's contract on the CPU: more than one GPU is refused with a JSON
message before any GPU work, and the counter-measured traffic of the grouped
kernel is reported only while the kernel sources hash to the ones measured."""
import json
import os
import subprocess
import sys

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, REPO)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(REPO, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    line = [l for l in r.stdout.splitlines() if l.startswith("{")][-1]
    assert "one GPU" in json.loads(line)["error"]


def _summary(tmp_path, sha, label="c3_grouped"):
    rec = {"label": label, "kernel": "k", "bytes": 123, "read_bytes": 100, "write_bytes": 23,
           "ratio_to_algorithmic": 1.0, "source_sha256": sha}
    p = tmp_path / f"traffic_{label}.md"
    p.write_text("# summary\n\ntraffic-json: " + json.dumps(rec) + "\n")
    return str(p)


def test_traffic_only_for_the_measured_sources(tmp_path):
    from weight_streaming_gemv_decode_amd import profsum
    h = profsum.source_sha256()   # of the sources' code (tests/test_profsum.py pins what it covers)
    assert bench.measured_traffic(_summary(tmp_path, h))["bytes"] == 123
    assert bench.measured_traffic(_summary(tmp_path, h, "c1")) is None          # another config
    assert bench.measured_traffic(_summary(tmp_path, h, "c1"), "c1")["bytes"] == 123
    assert bench.measured_traffic(_summary(tmp_path, "0" * 64)) is None
    assert bench.measured_traffic(str(tmp_path / "missing.md")) is None
