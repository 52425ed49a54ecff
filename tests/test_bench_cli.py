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


def test_counter_summary_is_well_formed():
    """The committed counter JSON: one code hash per profiled kernel, the
    copy check of the request-size byte sums (the 512 MiB copy reads and
    writes its known bytes), traffic per leg and the matrix-core figures."""
    sys.path.insert(0, ROOT)
    import bench
    d = json.load(open(bench.TRAFFIC_FILE))
    assert set(d["source_hash"]) == set(bench.KERNEL_SOURCE) and d["command"]
    assert all(len(h) == 16 for h in d["source_hash"].values())
    assert abs(d["copy_check"]["read"] - 1) < 0.01 and abs(d["copy_check"]["write"] - 1) < 0.01
    for leg in ("gdn", "gdr2", "decode"):
        t = d["traffic"][leg]
        assert t["bytes"] == t["read_bytes"] + t["write_bytes"] > 0
    for leg in ("gdn", "gdr2"):
        m = d["mfma"][leg]
        assert 0 < m["busy_frac"] < 1 and m["exec_bf16_flops"] > 0


def test_kernel_hash_ignores_comments(tmp_path):
    """A leg's counters stay valid across comment edits and lapse with any
    code edit of its source or of a file it includes."""
    sys.path.insert(0, ROOT)
    import bench
    a = tmp_path / "a.h"
    a.write_text("int x; // one\n/* two */ int y;\n")
    t1 = bench._code_text(str(a))
    a.write_text("int x; // three\n/* four\n lines */ int y;\n")
    assert bench._code_text(str(a)) == t1
    a.write_text("int x; int z;\n")
    assert bench._code_text(str(a)) != t1
