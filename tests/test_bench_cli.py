"""Host-side parts of bench.py: the one-GPU guard and the committed counter
summary it reads its traffic figures from (no GPU needed)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_summary_is_well_formed():
    sys.path.insert(0, ROOT)
    import bench
    d = json.load(open(bench.TRAFFIC_FILE))
    assert len(d["source_hash"]) == 16 and d["command"]
    assert d["scale"]["FETCH_SIZE"] > 0 and d["scale"]["WRITE_SIZE"] > 0
    for leg in ("gdn", "gdr2", "decode"):
        t = d["traffic"][leg]
        assert t["bytes"] > 0
