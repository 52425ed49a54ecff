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


def _write_csv(path, header, rows):
    import csv
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        w.writerows(rows)


def test_summary_finds_each_legs_timed_dispatches(tmp_path):
    """summarize() on a synthetic trace laid out as the round-end command
    makes it (--warmup 5 --steps 20): the headline kernel's first
    dispatches belong to the long-context split (25) and the headline's
    warm-up (5), the output gate's first ones to the fused-gate leg's two
    calls (5 + 10 x 20), and only the largest copies are the 512 MiB one.
    Each timed dispatch lasts 100 us more than its neighbours outside the
    timed region, so a wrong window changes the average."""
    sys.path.insert(0, ROOT)
    import bench
    W, K = 5, 20
    rows, t = [], [1000]

    def emit(name, n, us, grid=256):
        for _ in range(n):
            rows.append([name, t[0], t[0] + int(us * 1e3), grid])
            t[0] += int(us * 1e3) + 10

    gdn, gate, copy = bench.KERNELS["gdn"] + "(P)", bench.KERNELS["gate"] + "(P)", \
        bench.KERNELS["copy"]
    emit(copy, 3, 5.0, grid=512)                    # input uploads
    emit(gdn, 25, 900.0)                            # long-context split, last pass
    emit(gdn, W, 900.0)                             # headline warm-up
    emit(gdn, K, 250.0)                             # headline timed region
    emit(gdn, K, 900.0)                             # headline per-call pass
    emit(gate, W + 10 * K, 900.0)                   # fused-gate leg's two calls
    emit(gate, W, 900.0)
    emit(gate, K, 100.0)                            # gate timed region
    emit(gate, K, 900.0)
    emit(copy, W, 900.0, grid=131072)
    emit(copy, K, 200.0, grid=131072)               # copy timed region
    emit(copy, K, 900.0, grid=131072)
    tr = tmp_path / "trace"
    tr.mkdir()
    _write_csv(tr / "run_kernel_trace.csv",
               ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X"], rows)
    _write_csv(tr / "run_kernel_stats.csv", ["Name", "Calls", "AverageNs", "MinNs", "MaxNs"],
               [[gdn, 70, 1.0, 1.0, 1.0]])
    pmc = tmp_path / "pmc"
    pmc.mkdir()
    crow = []
    for i, (grid, n128) in enumerate(((512, 4), (131072, 4194304))):
        for name, v in (("TCC_EA0_RDREQ_32B_sum", 0), ("TCC_EA0_RDREQ_64B_sum", 0),
                        ("TCC_EA0_RDREQ_128B_sum", n128), ("TCC_EA0_WRREQ_sum", 2 * n128),
                        ("TCC_EA0_WRREQ_64B_sum", 2 * n128)):
            crow.append([i, grid, copy, name, v, 0, 1])
    _write_csv(pmc / "run_counter_collection.csv",
               ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value",
                "Start_Timestamp", "End_Timestamp"], crow)
    out = tmp_path / "sum.json"
    bench.summarize(str(tr), [str(pmc)], str(tmp_path / "sum.txt"), "test", timed=K,
                    warmup=W, json_out=str(out))
    d = json.load(open(out))
    assert abs(d["timed_launch_us"]["gdn"] - 250.0) < 0.01
    assert abs(d["timed_launch_us"]["gate"] - 100.0) < 0.01
    assert abs(d["timed_launch_us"]["copy"] - 200.0) < 0.01
    assert abs(d["copy_check"]["read"] - 1.0) < 1e-9 and abs(d["copy_check"]["write"] - 1.0) < 1e-9
