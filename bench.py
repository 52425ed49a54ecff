#!/usr/bin/env python3
"""Benchmark of the gated delta rule hot path on one MI355X.

One step = one chunkwise gated delta rule forward (gdr_chunk_fwd) over the
1.3B-layer workload: B=8, H=16, T=4096, d_k = d_v = 128, bf16 q/k/v, fp32
alpha/beta, zero initial state, fp32 output and final state.  Inputs are
seeded synthetic tensors resident in HBM before timing starts.  The
headline leg runs after the decode, GDN-2, long-context and bf16-o legs,
so that its launches see the steady clock rather than the ramp after idle;
its warm-up and timed calls are exactly --warmup and --steps.

The JSON line (stdout, last line) carries:
  value / unit       tokens/s of that forward: B*T tokens per call over the
                     mean call time of the timed region (per-call median
                     and minimum beside it, from a second pass)
  roofline           the chunked kernel against HBM bandwidth: the
                     algorithmic bytes of the workload (1,032 B per
                     token-head for bf16 q, k, v, o and fp32 alpha, beta,
                     plus the fp32 final state) / mean launch time; the
                     fp32-o byte count (+256 B per token-head) beside it
  mfma               the same launches against the dense bf16 MFMA peak,
                     counting 2 (3 dk dv + 5 C d) flops per token-head
  gdn_bf16_o         the same forward writing bf16 o
  decode             gdr_recurrent_step on 256 sequences x 16 heads, d=128,
                     64 consecutive steps: GB/s of state + token traffic
  gdr2               gdr2_chunk_fwd on B=4 H=16 T=4096 d=128 (bf16 gates):
                     tokens/s, HBM and MFMA fractions
  long_context       gdr_chunk_fwd on B=1 H=16 T=32768 d=128 with an initial
                     state (16 sequential chains; tokens/s, HBM and MFMA
                     fractions)
  gate_fused         gdr_chunk_fwd_gate (output gate fused on the stores)
                     against gdr_chunk_fwd + gdr_output_gate, in rounds of
                     back-to-back calls
  l2norm             the fused L2 normalisation of q, k (GDR_L2NORM_QK) on
                     the GDN and GDN-2 workloads with raw q, k: launch time
                     fused, plain (no normalisation), and a separate
                     normalise pass in PyTorch followed by the plain call
  output_gate        gdr_output_gate (RMSNorm x SiLU gate) on the B8 T4096 H16
                     d128 output: fp32 o, bf16 gate, bf16 y; GB/s of HBM
  output_gate_bwd    gdr_output_gate_bwd on the same gate: GB/s of HBM
  backward           gdr_chunk_bwd on the B8 H16 T4096 d128 workload (bf16 inputs
                     and dL/do, fp32 gradients): launch time and fp32 vector-ALU
                     fraction of its algorithmic flops
  backward2          gdr2_chunk_bwd on the B4 H16 T4096 d128 GDN-2 workload, as
                     for backward
  backward_long_context  the backward on the long-context workload, plain
                     and by gdr_chunk_bwd_split
  copy_reference     a plain 512 MiB device copy (achievable bandwidth)
  cpu_baseline       the fp64 oracle timed on the host on the same inputs:
                     the headline workload at top level, and one entry in
                     each of the decode, gdr2 and long_context legs
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 vector ALU, TFLOP/s
METRIC = "tokens/s chunkwise gated-delta fwd (H16,d128,T4K); % MFMA peak; decode GB/s"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


CSRC = os.path.join(ROOT, "gated_delta_rule_16_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bench_kernel_counters.json")
# kernel-name prefix in rocprofv3 output -> the bench leg it belongs to
KERNELS = {"gdn": "void gdr::(anonymous namespace)::chunk_bf16_kernel<128, 128, 64, float, false, "
                  "false, false>",
           "gdn_bf16o": "void gdr::(anonymous namespace)::chunk_bf16_kernel<128, 128, 64, "
                        "unsigned short, false, false, false>",
           "gdn_gate": "void gdr::(anonymous namespace)::chunk_bf16_kernel<128, 128, 64, "
                       "unsigned short, false, true, false>",
           "gdr2": "void gdr::(anonymous namespace)::gdr2_bf16_kernel<128, 128, float, false, false>",
           "decode": "void gdr::step_kernel<128, 128, unsigned short, float>",
           "gate": "void gdr::(anonymous namespace)::output_gate_kernel<128, float, unsigned short, "
                   "unsigned short>",
           "bwd": "void gdr::(anonymous namespace)::gdn_bwd_kernel<128, 128, unsigned short, "
                  "unsigned short>",
           "bwd2": "void gdr::(anonymous namespace)::chunk2_bwd_kernel<128, 128, unsigned short, "
                   "unsigned short>",
           "copy": "__amd_rocclr_copyBuffer"}


# the HIP source each profiled kernel is compiled from
KERNEL_SOURCE = {"gdn": "chunk_mfma.hip", "gdn_bf16o": "chunk_mfma.hip", "gdn_gate": "chunk_gate.hip",
                 "gdr2": "gdr2_mfma.hip", "decode": "step.hip", "gate": "epilogue.hip",
                 "bwd": "chunk_bwd.hip", "bwd2": "chunk2_bwd.hip"}


def _code_text(path):
    """A source file without its comments and blank space: edits to the
    comments do not change a kernel."""
    import re
    t = open(path).read()
    t = re.sub(r"/\*.*?\*/", " ", t, flags=re.S)
    t = re.sub(r"//[^\n]*", " ", t)
    return " ".join(t.split())


def source_hash(leg=None) -> str:
    """Hash of the code a kernel is built from (its source file and every
    file it includes, transitively; all HIP sources when leg is None):
    counter readings are only valid for the kernels they were taken on."""
    import re
    if leg is None:
        files = sorted(f for f in glob.glob(os.path.join(CSRC, "*")) if f.endswith((".hip", ".h")))
    else:
        todo, files = [os.path.join(CSRC, KERNEL_SOURCE[leg])], []
        while todo:
            f = os.path.normpath(todo.pop())
            if f in files or not os.path.exists(f):
                continue
            files.append(f)
            for inc in re.findall(r'#include "([^"]+)"', open(f).read()):
                todo.append(os.path.join(os.path.dirname(f), inc))
        files.sort()
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.relpath(f, ROOT).encode())
        h.update(_code_text(f).encode())
    return h.hexdigest()[:16]


def _csv(d, suffix):
    files = glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    return list(csv.DictReader(open(files[0])))


def _counter_means(dirs):
    """Mean per dispatch of every counter in the --pmc runs under `dirs`,
    per bench leg (kernel-name prefix in KERNELS), with each leg's mean
    dispatch duration in those runs (ns).  For the copy only the
    dispatches of the largest grid count (the 512 MiB copy; the host-to-
    device copies of the inputs use the same kernel)."""
    per, dur = {}, {}
    for d in dirs:
        rows = _csv(d, "counter_collection.csv")
        big = max((int(r["Grid_Size"]) for r in rows if r["Kernel_Name"].startswith(KERNELS["copy"])),
                  default=0)
        vals, spans = {}, {}
        for r in rows:
            for leg, prefix in KERNELS.items():
                if not r["Kernel_Name"].startswith(prefix):
                    continue
                if leg == "copy" and int(r["Grid_Size"]) != big:
                    continue
                vals.setdefault((leg, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
                spans.setdefault(leg, {})[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) -
                                                               int(r["Start_Timestamp"]))
        for (leg, name), v in vals.items():
            per.setdefault(leg, {})[name] = sum(v) / len(v)
        for leg, sp in spans.items():
            dur.setdefault(leg, {})[d] = sum(sp.values()) / len(sp)
    return per, dur


N_XCD = 8          # accelerator complex dies of an MI355X (GRBM_GUI_ACTIVE sums over them)


def summarize(trace_dir, pmc_dirs, out_txt, command, timed=20, warmup=5,
              legs_run=("decode", "gdr2", "longctx", "gdn", "gdn_bf16o", "gate_fused", "l2norm",
                        "gate", "gate_bwd", "bwd", "bwd2", "bwd_long", "copy"), json_out=None):
    """Turn rocprofv3 CSV output -- one --kernel-trace --stats run and
    several --pmc runs of the same command -- into a short text summary and
    the JSON the benchmark reads its counter figures from.

    HBM bytes: the TCC-to-memory requests summed by size,
    32 TCC_EA0_RDREQ_32B + 64 TCC_EA0_RDREQ_64B + 128 TCC_EA0_RDREQ_128B for
    reads and 64 TCC_EA0_WRREQ_64B + 32 (TCC_EA0_WRREQ - WRREQ_64B) for
    writes; the plain 512 MiB copy checks them (its known bytes over the
    reading).  FETCH_SIZE / WRITE_SIZE beside them, scaled by the copy.
    Matrix cores: executed bf16 flops = 512 SQ_INSTS_VALU_MFMA_MOPS_BF16;
    busy fraction = SQ_VALU_MFMA_BUSY_CYCLES (summed over SIMDs) /
    (GRBM_GUI_ACTIVE / 8 XCDs x 256 CUs x 4 SIMDs).  Decode:
    TCC_EA0_RDREQ_DRAM / TCC_EA0_RDREQ, the share of L2 read misses sent to
    the memory controllers."""
    stats = _csv(trace_dir, "kernel_stats.csv")
    trace = _csv(trace_dir, "kernel_trace.csv")
    per, _ = _counter_means(pmc_dirs)
    lines = ["# rocprofv3 summary", "", "Kernel source hashes (code without comments; the bench uses a "
             "leg's counters only while its hash matches):",
             "  " + ", ".join(f"{leg} {source_hash(leg)}" for leg in KERNEL_SOURCE), "",
             "Commands:"] + [f"  {c.strip()}" for c in command.split(" ;; ")] + [
             "", "Kernel trace (--kernel-trace --stats):",
             f"  {'kernel':60s} {'calls':>6s} {'avg us':>10s} {'min us':>10s} {'max us':>10s}"]
    for r in stats:
        lines.append(f"  {r['Name'][:60]:60s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.1f} "
                     f"{float(r['MinNs']) / 1e3:10.1f} {float(r['MaxNs']) / 1e3:10.1f}")
    # the same trace, per bench leg: its timed launches only.  Legs run in
    # a fixed order and some kernels serve several legs, so a leg's
    # dispatches are counted from the start of the trace: the dispatches of
    # its kernel by earlier legs are skipped, then its warm-up calls, then
    # come its timed ones (time_launches' timed region; all the rounds of
    # the fused-gate leg); the copy is the 512 MiB one (the largest grid).
    W, K = warmup, timed
    Wb, Kb = min(W, 5), min(K, 10)   # the backward legs' caps
    fused_two_calls = W + 10 * K if "gate_fused" in legs_run else 0
    # the long-context split's last pass runs the headline kernel (8 x 16
    # segment-heads of 4096 tokens) once per call, before the headline leg
    longctx_calls = min(W, 10) + 2 * min(K, 10) if "longctx" in legs_run else 0
    first = {  # leg: (index of the first timed dispatch of its kernel, timed count)
        "decode": (W, 64), "gdr2": (1 + W, K), "gdn": (longctx_calls + W, K), "gdn_bf16o": (W, K),
        "gdn_gate": (W, 10 * K), "gate": (fused_two_calls + W, K), "bwd": (Wb, Kb),
        "bwd2": (Wb, Kb), "copy": (W, K)}
    lines += ["", f"Timed launches of each leg (--warmup {W} --steps {K}; per leg the dispatches "
              "of its timed region, counted from the start of the trace; the copy's 512 MiB "
              "dispatches):",
              f"  {'leg':9s} {'kernel':50s} {'n':>4s} {'avg us':>10s} {'min us':>10s}"]
    dur_us = {}
    for leg, prefix in KERNELS.items():
        rows = [r for r in trace if r["Kernel_Name"].startswith(prefix)]
        if leg == "copy" and rows:
            gk = "Grid_Size" if "Grid_Size" in rows[0] else "Grid_Size_X"
            big = max(int(r[gk]) for r in rows)
            rows = [r for r in rows if int(r[gk]) == big]
        d = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows)
        if leg in first:
            i0, n = first[leg]
            d = d[i0:i0 + n]
        if not d:
            continue
        dur = [(e - b) / 1e3 for b, e in d]
        dur_us[leg] = sum(dur) / len(dur)
        lines.append(f"  {leg:9s} {prefix.split('::')[-1][:50]:50s} {len(dur):4d} "
                     f"{dur_us[leg]:10.1f} {min(dur):10.1f}")
    copy_bytes = 512 << 20          # the copy reads and writes 512 MiB each
    ea, traffic = {}, {}
    for leg, c in per.items():
        if all(k in c for k in ("TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum",
                                "TCC_EA0_RDREQ_128B_sum")):
            ea.setdefault(leg, {})["read"] = (32 * c["TCC_EA0_RDREQ_32B_sum"] + 64 *
                                              c["TCC_EA0_RDREQ_64B_sum"] + 128 *
                                              c["TCC_EA0_RDREQ_128B_sum"])
        if all(k in c for k in ("TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum")):
            ea.setdefault(leg, {})["write"] = (64 * c["TCC_EA0_WRREQ_64B_sum"] + 32 *
                                               (c["TCC_EA0_WRREQ_sum"] -
                                                c["TCC_EA0_WRREQ_64B_sum"]))
    for leg, e in ea.items():
        if "read" in e and "write" in e and leg != "copy":
            traffic[leg] = {"read_bytes": e["read"], "write_bytes": e["write"],
                            "bytes": e["read"] + e["write"]}
    check = {k: ea.get("copy", {}).get(k, 0) / copy_bytes for k in ("read", "write")}
    lines += ["", "HBM bytes per dispatch, from the request counts by size (the 512 MiB copy "
                  "reads as {:.4f} x and {:.4f} x its known read and write bytes):".format(
                      check["read"], check["write"])]
    for leg, e in ea.items():
        lines.append(f"  {leg:9s} read {e.get('read', 0) / 1e6:9.1f} MB   write "
                     f"{e.get('write', 0) / 1e6:9.1f} MB")
    scale = {}
    copy = per.get("copy", {})
    for name in ("FETCH_SIZE", "WRITE_SIZE"):
        if copy.get(name):
            scale[name] = copy_bytes / 1024 / copy[name]
    if scale:
        lines += ["", "FETCH_SIZE / WRITE_SIZE (KiB per dispatch as read), and scaled by the copy's "
                      f"reading (FETCH x {scale.get('FETCH_SIZE', 0):.4f}, WRITE x "
                      f"{scale.get('WRITE_SIZE', 0):.4f}):"]
        for leg, c in per.items():
            if "FETCH_SIZE" in c and "WRITE_SIZE" in c:
                lines.append(f"  {leg:9s} FETCH {c['FETCH_SIZE']:12.1f} -> "
                             f"{c['FETCH_SIZE'] * 1024 * scale['FETCH_SIZE'] / 1e6:9.1f} MB   WRITE "
                             f"{c['WRITE_SIZE']:12.1f} -> "
                             f"{c['WRITE_SIZE'] * 1024 * scale['WRITE_SIZE'] / 1e6:9.1f} MB")
    mfma = {}
    for leg, c in per.items():
        if "SQ_VALU_MFMA_BUSY_CYCLES" not in c or not c.get("GRBM_GUI_ACTIVE"):
            continue
        cyc = c["GRBM_GUI_ACTIVE"] / N_XCD
        m = {"busy_frac": c["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * 256 * 4)}
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in c:
            m["exec_bf16_flops"] = 512 * c["SQ_INSTS_VALU_MFMA_MOPS_BF16"]
            if leg in dur_us:
                m["exec_tflops"] = m["exec_bf16_flops"] / dur_us[leg] / 1e6
                m["exec_frac"] = m["exec_tflops"] / BF16_PEAK_TFLOPS
        m["raw"] = {k: v for k, v in c.items() if k.startswith(("SQ_", "GRBM_"))}
        mfma[leg] = m
    if mfma:
        lines += ["", "Matrix cores per dispatch: executed bf16 flops = 512 x "
                      "SQ_INSTS_VALU_MFMA_MOPS_BF16 (its rate over the timed launches above); "
                      "busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 256 CU x 4 SIMD), "
                      "the fraction of SIMD cycles the matrix cores were busy:"]
        for leg, m in mfma.items():
            raw = "  ".join(f"{k} {v:.4g}" for k, v in m["raw"].items())
            lines.append(f"  {leg:9s}"
                         + (f" exec {m['exec_bf16_flops'] / 1e9:8.2f} GFLOP" if "exec_bf16_flops" in m
                            else "")
                         + (f" = {m['exec_tflops']:7.1f} TFLOP/s ({m['exec_frac']:.3f} of the "
                            f"2.4 GHz peak)" if "exec_tflops" in m else "")
                         + f", busy {m['busy_frac']:.3f}")
            lines.append(f"            {raw}")
    dram = {}
    for leg, c in per.items():
        if c.get("TCC_EA0_RDREQ_sum") and "TCC_EA0_RDREQ_DRAM_sum" in c:
            dram[leg] = c["TCC_EA0_RDREQ_DRAM_sum"] / c["TCC_EA0_RDREQ_sum"]
    if dram:
        lines += ["", "L2 read misses sent to the memory controllers (TCC_EA0_RDREQ_DRAM_sum / "
                      "TCC_EA0_RDREQ_sum; the memory-side cache sits behind them, so its hits "
                      "are inside this share):"]
        for leg, f in dram.items():
            lines.append(f"  {leg:9s} {f:.4f}")
    open(out_txt, "w").write("\n".join(lines) + "\n")
    json.dump({"source_hash": {leg: source_hash(leg) for leg in KERNEL_SOURCE},
               "copy_check": check, "fetch_write_scale": scale, "traffic": traffic,
               "mfma": {k: {kk: vv for kk, vv in v.items() if kk != "raw"}
                        for k, v in mfma.items()},
               "dram_read_share": dram, "command": command,
               "timed_launch_us": dur_us},
              open(json_out or TRAFFIC_FILE, "w"), indent=1)
    print("\n".join(lines))


def _measured(key, leg):
    try:
        d = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    hashes = d.get("source_hash")
    if not isinstance(hashes, dict) or hashes.get(leg) != source_hash(leg):
        return None
    return d.get(key, {}).get(leg)


def measured_traffic(leg):
    """HBM bytes per launch from the committed counter summary, or None when
    the kernels have changed since the counters were taken."""
    t = _measured("traffic", leg)
    return None if t is None else t["bytes"]


def measured_mfma(leg):
    """Executed bf16 MFMA flops and busy fraction from the committed counter
    summary (None when the kernels have changed since)."""
    return _measured("mfma", leg)


def measured_dram(leg):
    return _measured("dram_read_share", leg)


_INPUTS = {}


def config_inputs(idx):
    """The seeded host inputs of workload `idx`, drawn once per process."""
    if idx not in _INPUTS:
        from gdr_gen import make_config
        _INPUTS[idx] = make_config(idx)
    return _INPUTS[idx]


_DEVICE = {}


def on_device(idx, *fields):
    """Fields of workload `idx` copied to cuda:0 once per process: main()
    stages every forward leg's inputs before the first timed leg, so no
    host-side generation or copy idles the GPU between the legs."""
    out = []
    for f in fields:
        if (idx, f) not in _DEVICE:
            _DEVICE[(idx, f)] = getattr(config_inputs(idx), f).to("cuda:0")
        out.append(_DEVICE[(idx, f)])
    return out


def time_launches(fn, warmup, steps):
    """The timed region: after `warmup` untimed calls, `steps` calls back to
    back between two HIP events recorded on the current stream (the stream
    the calls launch on); mean per call = elapsed / steps, and the wall time
    of the region, bracketed by synchronize.  Then `steps` more calls, each
    between its own pair of events, for the per-call minimum and median (an
    event pair per call leaves the GPU idle a few microseconds between
    launches, so these run after the timed region).  Returns seconds:
    (mean, min, median, wall)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean = start.elapsed_time(end) / steps / 1e3
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    return mean, ms[0] / 1e3, ms[len(ms) // 2] / 1e3, wall


def gdn_bytes(B, T, H, Dk, Dv, o_bytes=2, states=1):
    """Algorithmic HBM bytes of one forward call: per token-head q, k, v in
    bf16, alpha and beta in fp32 and o (bf16: 1,032 B at d = 128), plus
    each fp32 state read or written once."""
    return B * T * H * (2 * (Dk + Dk + Dv) + 8 + o_bytes * Dv) + states * 4 * B * H * Dv * Dk


def gdn_flops(B, T, H, Dk, Dv, C=64):
    """Algorithmic matrix flops of one forward call, 2 (3 dk dv + 5 C d)
    per token-head at the reference chunk C = 64 (d = (dk + dv) / 2)."""
    return B * T * H * 2 * (3 * Dk * Dv + 5 * C * (Dk + Dv) // 2)


def bench_gdn(gdr, torch, warmup, steps, out_dtype="f32"):
    inp = config_inputs(1)
    B, T, H, Dk = inp.q.shape
    Dv = inp.v.shape[-1]
    dev = torch.device("cuda:0")
    q, k, v, a, b = on_device(1, "q", "k", "v", "alpha", "beta")
    odt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    o = torch.empty((B, T, H, Dv), dtype=odt, device=dev)
    sf = torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=dev)

    def fn():
        gdr.gdr_chunk_fwd(q, k, v, a, b, None, out_dtype=odt, o=o, s_final=sf)

    mean, mn, med, wall = time_launches(fn, warmup, steps)
    return dict(inp=inp, mean=mean, min=mn, median=med, wall=wall, B=B, T=T, H=H, Dk=Dk,
                Dv=Dv, bytes=gdn_bytes(B, T, H, Dk, Dv),
                bytes_as_run=gdn_bytes(B, T, H, Dk, Dv, o_bytes=4 if out_dtype == "f32" else 2),
                flops=gdn_flops(B, T, H, Dk, Dv))


def bench_longctx(gdr, torch, warmup, steps, nseg=8):
    """The long-context workload: B1 H16 T32768 d128 with an initial state.
    Run plainly it is 16 sequential chains of 1024 chunks (few heads, so
    narrow row blocks and half the compute units idle); the split call runs
    it as nseg = 8 segments side by side (three passes plus a scan).  Both
    are timed; the bytes and flops are the workload's algorithmic ones."""
    inp = config_inputs(2)
    B, T, H, Dk = inp.q.shape
    Dv = inp.v.shape[-1]
    dev = torch.device("cuda:0")
    q, k, v, a, b, s0 = on_device(2, "q", "k", "v", "alpha", "beta", "s0")
    o = torch.empty((B, T, H, Dv), dtype=torch.float32, device=dev)
    sf = torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=dev)
    ws = torch.empty(gdr.gdr_chunk_fwd_split_workspace_size(B, T, H, Dk, Dv, q.dtype, nseg),
                     dtype=torch.uint8, device=dev)

    def plain():
        gdr.gdr_chunk_fwd(q, k, v, a, b, s0, out_dtype=torch.float32, o=o, s_final=sf)

    def split():
        gdr.gdr_chunk_fwd_split(q, k, v, a, b, s0, nseg=nseg, out_dtype=torch.float32, o=o,
                                s_final=sf, workspace=ws)

    mean, mn, med, wall = time_launches(split, warmup, steps)
    pmean, pmn, _, _ = time_launches(plain, warmup, steps)
    return dict(inp=inp, mean=mean, min=mn, median=med, plain_mean=pmean, plain_min=pmn,
                nseg=nseg, B=B, T=T, H=H, bytes=gdn_bytes(B, T, H, Dk, Dv, states=2),
                bytes_as_run=gdn_bytes(B, T, H, Dk, Dv, o_bytes=4, states=2),
                flops=gdn_flops(B, T, H, Dk, Dv))


def bench_decode(gdr, torch, warmup):
    inp = config_inputs(3)
    steps, N, H, Dk = inp.q.shape
    Dv = inp.v.shape[-1]
    dev = torch.device("cuda:0")
    S, q, k, v, a, b = on_device(3, "state0", "q", "k", "v", "alpha", "beta")
    o = torch.empty((N, H, Dv), dtype=torch.float32, device=dev)
    for s in range(warmup):
        gdr.gdr_recurrent_step(q[s], k[s], v[s], a[s], b[s], S, out_dtype=torch.float32, o=o)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for s, (e0, e1) in enumerate(evs):
        e0.record()
        gdr.gdr_recurrent_step(q[s], k[s], v[s], a[s], b[s], S, out_dtype=torch.float32, o=o)
        e1.record()
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    med = ms[len(ms) // 2] / 1e3
    nh = N * H
    # per head-step: the fp32 state read and written, q, k, v and o in bf16,
    # alpha and beta in fp32 (132,104 B at d = 128); o is written in fp32
    # here, +2 dv B per head-step
    bytes_step = nh * (2 * 4 * Dv * Dk + 2 * (2 * Dk + Dv) + 8 + 2 * Dv)
    bytes_as_run = bytes_step + nh * 2 * Dv
    return dict(inp=inp, median=med, min=ms[0] / 1e3, mean=sum(ms) / len(ms) / 1e3,
                bytes=bytes_step, bytes_as_run=bytes_as_run, N=N, H=H, steps=steps)


def bench_gdr2(gdr, torch, warmup, steps):
    inp = config_inputs(4)
    B, T, H, Dk = inp.q.shape
    Dv = inp.v.shape[-1]
    dev = torch.device("cuda:0")
    args = on_device(4, "q", "k", "v", "alpha", "erase", "write")
    o = torch.empty((B, T, H, Dv), dtype=torch.float32, device=dev)
    sf = torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=dev)

    def fn():
        gdr.gdr2_chunk_fwd(*args, None, out_dtype=torch.float32, o=o, s_final=sf)

    try:
        fn()
    except gdr.GdrError as e:
        return dict(error=str(e))
    mean, mn, med, wall = time_launches(fn, warmup, steps)
    th = B * T * H
    # algorithmic bytes: q, k, alpha, erase bf16 (d_k each), v, write, o
    # bf16 (d_v each) per token-head, plus the fp32 final state
    bytes_launch = th * 2 * (4 * Dk + 3 * Dv) + 4 * B * H * Dv * Dk
    bytes_as_run = th * (2 * (4 * Dk + 2 * Dv) + 4 * Dv) + 4 * B * H * Dv * Dk   # fp32 o
    return dict(inp=inp, mean=mean, min=mn, median=med, B=B, T=T, H=H, bytes=bytes_launch,
                bytes_as_run=bytes_as_run, flops=gdn_flops(B, T, H, Dk, Dv))


def time_interleaved(fns, warmup, rounds):
    """Median and min per-call time (us) of each callable in `fns` (a dict),
    the calls interleaved round-robin (rotating the order each round) after
    `warmup` calls of each, so that all of them see the same clocks."""
    import torch
    names = list(fns)
    for _ in range(warmup):
        for n in names:
            fns[n]()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    t = {n: [] for n in names}
    for r in range(rounds):
        for n in names[r % len(names):] + names[:r % len(names)]:
            ev[0].record()
            fns[n]()
            ev[1].record()
            torch.cuda.synchronize()
            t[n].append(ev[0].elapsed_time(ev[1]) * 1e3)
    out = {}
    for n in names:
        x = sorted(t[n])
        out[n] = {"median": x[len(x) // 2], "min": x[0]}
    return out


def time_rounds(fns, warmup, rounds, per_round=10):
    """Median and min over `rounds` of the mean call time (us) of each
    callable in `fns`: a round runs `per_round` calls of each back to back
    between two events (rotating the order each round), so all see the same
    sustained clocks and no event sits between two calls."""
    import torch
    names = list(fns)
    for _ in range(warmup):
        for n in names:
            fns[n]()
    torch.cuda.synchronize()
    t = {n: [] for n in names}
    for r in range(rounds):
        for n in names[r % len(names):] + names[:r % len(names)]:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(per_round):
                fns[n]()
            b.record()
            torch.cuda.synchronize()
            t[n].append(a.elapsed_time(b) * 1e3 / per_round)
    out = {}
    for n in names:
        x = sorted(t[n])
        out[n] = {"median": x[len(x) // 2], "min": x[0]}
    return out


def bench_l2norm(gdr, torch, warmup, steps):
    """Fused q, k normalisation against the plain call and against a
    separate normalise pass (fp32 sum of squares in PyTorch, bf16 result)
    followed by the plain call, on the GDN (B8 H16 T4096) and GDN-2 (B4 H16
    T4096) workloads with raw q, k; the three are timed interleaved."""
    from gdr_gen import make_gdn, make_gdn2
    dev = torch.device("cuda:0")
    eps = 1e-6

    def norm_pass(x):
        xf = x.float()
        return (xf * torch.rsqrt((xf * xf).sum(-1, keepdim=True) + eps)).to(x.dtype)

    res = {}
    inp = make_gdn(B=8, T=4096, H=16, Dk=128, Dv=128, dtype="bf16", seed=1001, raw_qk=True)
    q, k, v = (x.to(dev) for x in (inp.q, inp.k, inp.v))
    a, b = inp.alpha.to(dev), inp.beta.to(dev)
    o = torch.empty((8, 4096, 16, 128), dtype=torch.float32, device=dev)
    sf = torch.empty((8, 16, 128, 128), dtype=torch.float32, device=dev)
    fused = lambda: gdr.gdr_chunk_fwd(q, k, v, a, b, None, out_dtype=torch.float32, o=o,
                                      s_final=sf, l2norm_qk=True)
    plain = lambda: gdr.gdr_chunk_fwd(q, k, v, a, b, None, out_dtype=torch.float32, o=o,
                                      s_final=sf)
    sep = lambda: gdr.gdr_chunk_fwd(norm_pass(q), norm_pass(k), v, a, b, None,
                                    out_dtype=torch.float32, o=o, s_final=sf)
    t = time_interleaved({"fused": fused, "plain": plain, "separate_pass": sep}, warmup, steps)
    res["gdn"] = {f"{n}_us_median": v["median"] for n, v in t.items()}
    del q, k, v, a, b, o, sf, inp
    inp = make_gdn2(B=4, T=4096, H=16, Dk=128, Dv=128, dtype="bf16", seed=1004, raw_qk=True)
    args = [x.to(dev) for x in (inp.q, inp.k, inp.v, inp.alpha, inp.erase, inp.write)]
    o = torch.empty((4, 4096, 16, 128), dtype=torch.float32, device=dev)
    sf = torch.empty((4, 16, 128, 128), dtype=torch.float32, device=dev)
    fused = lambda: gdr.gdr2_chunk_fwd(*args, None, out_dtype=torch.float32, o=o, s_final=sf,
                                       l2norm_qk=True)
    plain = lambda: gdr.gdr2_chunk_fwd(*args, None, out_dtype=torch.float32, o=o, s_final=sf)
    sep = lambda: gdr.gdr2_chunk_fwd(norm_pass(args[0]), norm_pass(args[1]), *args[2:], None,
                                     out_dtype=torch.float32, o=o, s_final=sf)
    t = time_interleaved({"fused": fused, "plain": plain, "separate_pass": sep}, warmup, steps)
    res["gdr2"] = {f"{n}_us_median": v["median"] for n, v in t.items()}
    return res


def bench_gate(gdr, torch, warmup, steps):
    from gdr_gen import make_gate
    inp = make_gate(8 * 4096, 16, 128, "f32", "bf16", seed=450)
    dev = torch.device("cuda:0")
    o, g, w = inp.o.to(dev), inp.g.to(dev), inp.w.to(dev)
    y = torch.empty(o.shape, dtype=torch.bfloat16, device=dev)
    mean, mn, med, wall = time_launches(
        lambda: gdr.gdr_output_gate(o, g, w, 1e-6, y=y), warmup, steps)
    n = o.numel()
    return dict(mean=mean, min=mn, bytes=n * (4 + 2 + 2) + 4 * 128)


def bench_gate_bwd(gdr, torch, warmup, steps):
    """gdr_output_gate_bwd on the B8 T4096 H16 d128 gate: fp32 o, bf16 gate
    and dL/dy in, fp32 do and dg out, dw over all rows.  Algorithmic bytes:
    (4 + 2 + 2) read + (4 + 4) written per element."""
    from gdr_gen import make_gate
    inp = make_gate(8 * 4096, 16, 128, "f32", "bf16", seed=451)
    dev = torch.device("cuda:0")
    o, g, w = inp.o.to(dev), inp.g.to(dev), inp.w.to(dev)
    dy = torch.randn(o.shape, generator=torch.Generator().manual_seed(9)).to(torch.bfloat16).to(dev)
    ws = torch.empty(gdr.gdr_output_gate_bwd_workspace_size(8 * 4096, 16, 128), dtype=torch.uint8,
                     device=dev)
    mean, mn, med, wall = time_launches(
        lambda: gdr.gdr_output_gate_bwd(o, g, w, dy, 1e-6, workspace=ws), warmup, steps)
    n = o.numel()
    return dict(mean=mean, min=mn, bytes=n * (4 + 2 + 2 + 4 + 4) + 4 * 128 * 2)


def bench_gate_fused(gdr, torch, warmup, steps):
    """The forward with the output gate on the B8 H16 T4096 d128 workload
    (bf16 gate, fp32 weight, bf16 y): gdr_chunk_fwd_gate against
    gdr_chunk_fwd (fp32 o) followed by gdr_output_gate, and the plain
    forward alone, timed interleaved so that all three see the same clocks."""
    from gdr_gen import make_gate
    inp = config_inputs(1)
    B, T, H, Dk = inp.q.shape
    Dv = inp.v.shape[-1]
    dev = torch.device("cuda:0")
    q, k, v, a, b = on_device(1, "q", "k", "v", "alpha", "beta")
    gi = make_gate(B * T, H, Dv, "f32", "bf16", seed=452)
    g = gi.g.reshape(B, T, H, Dv).to(dev)
    w = gi.w.to(dev)
    o = torch.empty((B, T, H, Dv), dtype=torch.float32, device=dev)
    y = torch.empty((B, T, H, Dv), dtype=torch.bfloat16, device=dev)
    sf = torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=dev)
    ws = torch.empty(gdr.gdr_chunk_fwd_gate_workspace_size(B, T, H, Dk, Dv, q.dtype),
                     dtype=torch.uint8, device=dev)

    def two_calls():
        gdr.gdr_chunk_fwd(q, k, v, a, b, None, out_dtype=torch.float32, o=o, s_final=sf)
        gdr.gdr_output_gate(o, g, w, 1e-6, y=y)

    def fused():
        gdr.gdr_chunk_fwd_gate(q, k, v, a, b, None, g, w, 1e-6, out_dtype=torch.bfloat16, y=y,
                               s_final=sf, workspace=ws)

    def plain():
        gdr.gdr_chunk_fwd(q, k, v, a, b, None, out_dtype=torch.float32, o=o, s_final=sf)

    t = time_rounds({"fused": fused, "two_calls": two_calls, "forward_only": plain},
                    warmup, steps)
    return dict(t=t, tokens=B * T)


def bench_bwd(gdr, torch, warmup, steps):
    """gdr_chunk_bwd on B8 H16 T4096 d128 (bf16 q/k/v and dL/do, dL/dS_T
    given, zero S_0).  Algorithmic flops per token-head, chunk C = 16, as
    for bench_bwd2: 2 x (9 dk dv + 3 C dk + 3 C dv) -- nine state-sized
    products (the forward sweep's K S^T and state update, K S^T again,
    K G'^T, (lambda dO) S, (rho U) G', (beta lambda dR) S, the two terms of
    the G' update) and the chunk-sized ones."""
    from gdr_gen import make_gdn
    inp = make_gdn(B=8, T=4096, H=16, Dk=128, Dv=128, dtype="bf16", seed=1001)
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in (inp.q, inp.k, inp.v))
    a, b = inp.alpha.to(dev), inp.beta.to(dev)
    g = torch.Generator(device="cpu").manual_seed(7)
    do = torch.randn(v.shape, generator=g).to(torch.bfloat16).to(dev)
    dsf = (0.1 * torch.randn((8, 16, 128, 128), generator=g)).to(dev)
    ws = torch.empty(gdr.gdr_chunk_bwd_workspace_size(8, 4096, 16, 128, 128), dtype=torch.uint8,
                     device=dev)
    mean, mn, med, wall = time_launches(
        lambda: gdr.gdr_chunk_bwd(q, k, v, a, b, None, do, dsf, workspace=ws), warmup, steps)
    th = 8 * 4096 * 16
    C, d = 16, 128
    flops = th * 2 * (9 * d * d + 3 * C * d + 3 * C * d)
    return dict(mean=mean, min=mn, flops=flops, tokens=8 * 4096, ws=ws.numel())


def bench_bwd2(gdr, torch, warmup, steps):
    """gdr2_chunk_bwd on B4 H16 T4096 d128 (bf16 inputs and dL/do, dL/dS_T
    given, zero S_0).  Algorithmic flops per token-head, chunk C = 16:
    2 x (9 dk dv + 3 C dk + 3 C dv) -- nine state-sized products (the
    forward's E~ S^T and state update, E~ S^T again, K~ G^T, dR S, dO S,
    U G, the two terms of the G update), the decayed A and P entries and
    their four reverse sums, and the n x n-by-rows products; the exp of
    the decay tables is not counted."""
    from gdr_gen import make_gdn2
    inp = make_gdn2(B=4, T=4096, H=16, Dk=128, Dv=128, dtype="bf16", seed=1004)
    dev = torch.device("cuda:0")
    xs = [x.to(dev) for x in (inp.q, inp.k, inp.v, inp.alpha, inp.erase, inp.write)]
    g = torch.Generator(device="cpu").manual_seed(8)
    do = torch.randn(xs[2].shape, generator=g).to(torch.bfloat16).to(dev)
    dsf = (0.1 * torch.randn((4, 16, 128, 128), generator=g)).to(dev)
    ws = torch.empty(gdr.gdr2_chunk_bwd_workspace_size(4, 4096, 16, 128, 128), dtype=torch.uint8,
                     device=dev)
    mean, mn, med, wall = time_launches(
        lambda: gdr.gdr2_chunk_bwd(*xs, None, do, dsf, workspace=ws), warmup, steps)
    th = 4 * 4096 * 16
    C, d = 16, 128
    flops = th * 2 * (9 * d * d + 3 * C * d + 3 * C * d)
    return dict(mean=mean, min=mn, flops=flops, tokens=4 * 4096, ws=ws.numel())


def bench_bwd_long(gdr, torch, warmup, steps, nseg=4):
    """The backward on the long-context workload (B1 H16 T32768 d128, bf16
    inputs and dL/do, initial state, dL/dS_T given): the plain call (64
    workgroups) and the split call with nseg segments side by side."""
    inp = config_inputs(2)
    dev = torch.device("cuda:0")
    args = [x.to(dev) for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta, inp.s0)]
    B, T, H, Dk = inp.q.shape
    Dv = inp.v.shape[-1]
    g = torch.Generator(device="cpu").manual_seed(10)
    do = torch.randn((B, T, H, Dv), generator=g).to(torch.bfloat16).to(dev)
    dsf = (0.1 * torch.randn((B, H, Dv, Dk), generator=g)).to(dev)
    wsp = torch.empty(gdr.gdr_chunk_bwd_workspace_size(B, T, H, Dk, Dv), dtype=torch.uint8,
                      device=dev)
    wss = torch.empty(gdr.gdr_chunk_bwd_split_workspace_size(B, T, H, Dk, Dv, inp.q.dtype, nseg),
                      dtype=torch.uint8, device=dev)
    pmean, pmin, _, _ = time_launches(
        lambda: gdr.gdr_chunk_bwd(*args, do, dsf, workspace=wsp), warmup, steps)
    smean, smin, _, _ = time_launches(
        lambda: gdr.gdr_chunk_bwd_split(*args, do, dsf, nseg=nseg, workspace=wss), warmup, steps)
    del wsp, wss
    # Gated Delta Rule-2 at the same shape (alpha per channel near 1)
    from gdr_gen import make_gdn2
    inp2 = make_gdn2(B=B, T=T, H=H, Dk=Dk, Dv=Dv, dtype="bf16", seed=1006, alpha_shift=-4.0,
                     s0_std=0.02)
    a2 = [x.to(dev) for x in (inp2.q, inp2.k, inp2.v, inp2.alpha, inp2.erase, inp2.write,
                              inp2.s0)]
    o2 = torch.empty((B, T, H, Dv), dtype=torch.float32, device=dev)
    sf2 = torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=dev)
    wf = torch.empty(gdr.gdr_chunk_fwd_split_workspace_size(B, T, H, Dk, Dv, inp2.q.dtype, nseg),
                     dtype=torch.uint8, device=dev)
    fp, _, _, _ = time_launches(lambda: gdr.gdr2_chunk_fwd(*a2, out_dtype=torch.float32, o=o2,
                                                           s_final=sf2), warmup, steps)
    fs, _, _, _ = time_launches(lambda: gdr.gdr2_chunk_fwd_split(*a2, nseg=nseg,
                                                                 out_dtype=torch.float32, o=o2,
                                                                 s_final=sf2, workspace=wf),
                                warmup, steps)
    del wf
    w2p = torch.empty(gdr.gdr2_chunk_bwd_workspace_size(B, T, H, Dk, Dv), dtype=torch.uint8,
                      device=dev)
    bp, _, _, _ = time_launches(lambda: gdr.gdr2_chunk_bwd(*a2, do, dsf, workspace=w2p),
                                warmup, steps)
    del w2p
    w2s = torch.empty(gdr.gdr2_chunk_bwd_split_workspace_size(B, T, H, Dk, Dv, inp2.q.dtype,
                                                              nseg),
                      dtype=torch.uint8, device=dev)
    bs, _, _, _ = time_launches(lambda: gdr.gdr2_chunk_bwd_split(*a2, do, dsf, nseg=nseg,
                                                                 workspace=w2s), warmup, steps)
    # the same with the start states from the fp32 forward (GDR_SPLIT_FP32_STATES)
    bs32, _, _, _ = time_launches(lambda: gdr.gdr2_chunk_bwd_split(
        *a2, do, dsf, nseg=nseg, workspace=w2s, fp32_states=True), warmup, steps)
    return dict(plain=pmean, split=smean, nseg=nseg, tokens=B * T, gdr2_fwd_plain=fp,
                gdr2_fwd_split=fs, gdr2_bwd_plain=bp, gdr2_bwd_split=bs,
                gdr2_bwd_split_fp32_states=bs32)


def bench_copy(torch, warmup, steps, nbytes=512 << 20):
    """A plain device-to-device copy of known size: the achievable-bandwidth
    reference, and the kernel whose FETCH_SIZE / WRITE_SIZE counters scale
    the counter readings of the other kernels."""
    dev = torch.device("cuda:0")
    x = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    y = torch.empty_like(x)
    mean, mn, med, wall = time_launches(lambda: y.copy_(x), warmup, steps)
    return dict(mean=mean, min=mn, bytes=2 * nbytes)


def _cpu_model():
    """The host CPU as lscpu describes it: model name, family / model /
    stepping numbers and logical CPU count (/proc/cpuinfo if lscpu is
    missing)."""
    fields = {}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        for line in out.splitlines():
            if ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    except (OSError, subprocess.SubprocessError):
        pass
    if "Model name" not in fields:
        try:
            with open("/proc/cpuinfo") as f:
                for line in f:
                    if line.startswith("model name"):
                        fields["Model name"] = line.split(":", 1)[1].strip()
                        break
        except OSError:
            return None
    desc = fields.get("Model name")
    extra = ", ".join(f"{k.lower()} {fields[k]}" for k in ("CPU family", "Model", "Stepping",
                                                            "CPU(s)") if k in fields)
    return f"{desc} ({extra})" if extra else desc


def _oracle_timed(fn, threads, repeats=1):
    """Best wall time (s) of `repeats` runs of fn() with the oracle's OpenMP
    runtime on `threads` threads (restored afterwards)."""
    import oracle
    all_threads = oracle.num_threads()
    oracle.set_num_threads(threads)
    try:
        best = float("inf")
        for _ in range(repeats):
            t0 = time.perf_counter()
            fn()
            best = min(best, time.perf_counter() - t0)
    finally:
        oracle.set_num_threads(all_threads)
    return best


def cpu_baselines(inputs):
    """The fp64 oracle on the host, on the inputs the GPU legs used (their
    conversion to fp64 excluded).  Per leg: the whole workload on every
    thread of the oracle's OpenMP runtime (best of two runs), and a stated
    slice of it on one thread (one run), each scaled to the leg's unit.
    About 15 s of host time in all on a 16-thread host."""
    import numpy as np
    import oracle
    cores = oracle.num_threads()
    model = _cpu_model()
    f64 = oracle._f64
    res = {}

    def entry(unit, value, seconds, sample, one_value, one_seconds, one_sample, **extra):
        d = dict(value=value, unit=unit, cores=cores, kind="oracle", seconds=seconds,
                 sample=sample, cpu_model=model,
                 one_thread=dict(value=one_value, unit=unit, cores=1, seconds=one_seconds,
                                 sample=one_sample))
        d.update(extra)
        return d

    if "gdn" in inputs:
        inp = inputs["gdn"]
        x = [f64(t) for t in (inp.q, inp.k, inp.v, inp.alpha, inp.beta)]
        B, T, H, Dk = inp.q.shape
        full = _oracle_timed(lambda: oracle.gdn_fwd(*x, None), cores, 2)
        one = _oracle_timed(lambda: oracle.gdn_fwd(*[t[:1] for t in x], None), 1)
        res["gdn"] = entry("tokens/s", B * T / full, full,
                           f"whole B{B} H{H} T{T} d{Dk} workload, fp64 token-by-token "
                           f"recurrence, best of 2", T / one, one,
                           f"batch 0 of {B} (T{T}, {H} heads), one run")
    if "gdr2" in inputs:
        inp = inputs["gdr2"]
        x = [f64(t) for t in (inp.q, inp.k, inp.v, inp.alpha, inp.erase, inp.write)]
        B, T, H, Dk = inp.q.shape
        full = _oracle_timed(lambda: oracle.gdn2_fwd(*x, None), cores, 2)
        one = _oracle_timed(lambda: oracle.gdn2_fwd(*[t[:1] for t in x], None), 1)
        res["gdr2"] = entry("tokens/s", B * T / full, full,
                            f"whole GDN-2 B{B} H{H} T{T} d{Dk} workload, fp64, best of 2",
                            T / one, one, f"batch 0 of {B} (T{T}, {H} heads), one run")
    if "longctx" in inputs:
        inp = inputs["longctx"]
        x = [f64(t) for t in (inp.q, inp.k, inp.v, inp.alpha, inp.beta)]
        s0 = f64(inp.s0)
        B, T, H, Dk = inp.q.shape
        full = _oracle_timed(lambda: oracle.gdn_fwd(*x, s0), cores, 2)
        Ts = T // 8
        one = _oracle_timed(lambda: oracle.gdn_fwd(*[t[:, :Ts] for t in x], s0), 1)
        res["longctx"] = entry("tokens/s", B * T / full, full,
                               f"whole B{B} H{H} T{T} d{Dk} workload with its initial state "
                               f"({H} sequential chains), fp64, best of 2", B * Ts / one, one,
                               f"the first {Ts} of {T} tokens, one run")
    if "decode" in inputs:
        inp, nbytes = inputs["decode"]
        steps, N, H, Dk = inp.q.shape
        x = [f64(t) for t in (inp.q, inp.k, inp.v, inp.alpha, inp.beta)]
        S = f64(inp.state0)

        def run(n_steps, state):
            for s in range(n_steps):
                oracle.gdn_step(*[t[s] for t in x], state)

        st = S.copy()
        full = _oracle_timed(lambda: run(steps, st), cores)
        ns = 8
        st = np.ascontiguousarray(S[:N // 8])
        one = _oracle_timed(lambda: [oracle.gdn_step(*[t[s, :N // 8] for t in x], st)
                                     for s in range(ns)], 1)
        res["decode"] = entry("steps/s", steps / full, full,
                              f"all {steps} steps on N{N} H{H} d{Dk}, fp64 state, one run",
                              ns / (8 * one), one,
                              f"{ns} steps on sequences 0..{N // 8 - 1} of {N}, scaled to a "
                              f"full step (x8), one run",
                              GBps=nbytes * steps / full / 1e9,
                              one_thread_GBps=nbytes / 8 * ns / one / 1e9)
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-baseline leg")
    ap.add_argument("--only", choices=["gdn", "gdn_bf16o", "decode", "gdr2", "longctx", "gate_fused",
                                       "l2norm", "gate", "gate_bwd", "bwd", "bwd2", "bwd_long",
                                       "copy"],
                    default=None,
                    help="time one operation only (for profiling)")
    ap.add_argument("--skip", default="",
                    help="comma-separated legs not to run (the profiled command skips l2norm, "
                         "longctx and bwd_long, whose calls reuse the headline and backward "
                         "kernels' names at other shapes)")
    ap.add_argument("--summarize", nargs=2, metavar=("TRACE_DIR", "OUT"),
                    help="summarize rocprofv3 CSV output (a kernel trace in TRACE_DIR and the "
                         "--pmc runs named by --pmc-dir) into OUT and the counter JSON, then exit")
    ap.add_argument("--pmc-dir", action="append", default=[],
                    help="a rocprofv3 --pmc output folder (repeatable)")
    ap.add_argument("--command", default="",
                    help="the profiling commands (' ;; '-separated), recorded in --summarize")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize[0], args.pmc_dir, args.summarize[1], command=args.command,
                  timed=args.steps, warmup=args.warmup)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: this "
              f"library runs on a single GPU (batch and head shards would need no "
              f"communication, but no multi-GPU launcher is built)", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_16_amd as gdr
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    skip = set(x for x in args.skip.split(",") if x)

    def want(leg):
        return args.only in (None, leg) and leg not in skip

    # Stage the forward legs' inputs in HBM first.  The headline leg then
    # runs right after the decode, GDN-2, long-context and bf16-o legs (the
    # last one the same kernel with bf16 o): after idle the GPU takes ~100
    # launches of sustained load to settle its clocks, and back-to-back
    # launches from a cold start time 20-30 % slower.  Its own warm-up and
    # timed calls are exactly --warmup and --steps.
    stage = {1: ("q", "k", "v", "alpha", "beta"), 2: ("q", "k", "v", "alpha", "beta", "s0"),
             3: ("state0", "q", "k", "v", "alpha", "beta"),
             4: ("q", "k", "v", "alpha", "erase", "write")}
    legs_of = {1: ("gdn", "gdn_bf16o", "gate_fused"), 2: ("longctx",), 3: ("decode",),
               4: ("gdr2",)}
    for idx, fields in stage.items():
        if any(want(leg) for leg in legs_of[idx]):
            log(f"staging workload {idx} inputs ...")
            on_device(idx, *fields)
    torch.cuda.synchronize()
    res = {}
    if want("decode"):
        log("timing gdr_recurrent_step N256 H16 d128 x 64 steps ...")
        res["decode"] = bench_decode(gdr, torch, args.warmup)
        log(f"  median {res['decode']['median'] * 1e6:.1f} us/step")
    if want("gdr2"):
        log("timing gdr2_chunk_fwd B4 H16 T4096 d128 ...")
        res["gdr2"] = bench_gdr2(gdr, torch, args.warmup, args.steps)
    if want("longctx"):
        log("timing gdr_chunk_fwd B1 H16 T32768 d128 (long context) ...")
        res["longctx"] = bench_longctx(gdr, torch, min(args.warmup, 10), min(args.steps, 10))
    if want("gdn_bf16o"):
        log("timing gdr_chunk_fwd B8 H16 T4096 d128, bf16 o ...")
        res["gdn_bf16o"] = bench_gdn(gdr, torch, args.warmup, args.steps, out_dtype="bf16")
    if want("gdn"):
        log("timing gdr_chunk_fwd B8 H16 T4096 d128 ...")
        res["gdn"] = bench_gdn(gdr, torch, args.warmup, args.steps)
        log(f"  median {res['gdn']['median'] * 1e6:.1f} us, mean {res['gdn']['mean'] * 1e6:.1f} us")
    if want("gate_fused"):
        log("timing gdr_chunk_fwd_gate against gdr_chunk_fwd + gdr_output_gate ...")
        res["gate_fused"] = bench_gate_fused(gdr, torch, args.warmup, args.steps)
    if want("l2norm"):
        log("timing the fused q, k normalisation (GDN and GDN-2 workloads) ...")
        res["l2norm"] = bench_l2norm(gdr, torch, args.warmup, min(args.steps, 30))
    if want("gate"):
        log("timing gdr_output_gate B8 T4096 H16 d128 ...")
        res["gate"] = bench_gate(gdr, torch, args.warmup, args.steps)
    if want("gate_bwd"):
        log("timing gdr_output_gate_bwd B8 T4096 H16 d128 ...")
        res["gate_bwd"] = bench_gate_bwd(gdr, torch, args.warmup, args.steps)
    if want("bwd"):
        log("timing gdr_chunk_bwd B8 H16 T4096 d128 ...")
        res["bwd"] = bench_bwd(gdr, torch, min(args.warmup, 5), min(args.steps, 10))
    if want("bwd2"):
        log("timing gdr2_chunk_bwd B4 H16 T4096 d128 ...")
        res["bwd2"] = bench_bwd2(gdr, torch, min(args.warmup, 5), min(args.steps, 10))
    if want("bwd_long"):
        log("timing the backward on B1 H16 T32768 d128 (plain and split) ...")
        res["bwd_long"] = bench_bwd_long(gdr, torch, 1, min(args.steps, 3))
    if want("copy"):
        log("timing a 512 MiB device copy ...")
        res["copy"] = bench_copy(torch, args.warmup, args.steps)

    cpu = {}
    if not args.no_cpu:
        log("timing the fp64 oracle on the host ...")
        cin = {leg: res[leg]["inp"] for leg in ("gdn", "gdr2", "longctx") if leg in res
               and "inp" in res[leg]}
        if "decode" in res:
            cin["decode"] = (res["decode"]["inp"], res["decode"]["bytes"])
        cpu = cpu_baselines(cin)

    out = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic (seeded; shapes of a 1.3B GDN layer)"}
    if "gdn" in res:
        g = res["gdn"]
        tok = g["B"] * g["T"]
        out["value"] = tok / g["mean"]
        out["unit"] = "tokens/s"
        out["ms_per_step"] = g["wall"] / args.steps * 1e3
        gbs = g["bytes"] / g["mean"] / 1e9
        out["roofline"] = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                           "traffic": measured_traffic("gdn"),
                           "kernel": "chunk_bf16_kernel<128,128,64,float,false,false,false>",
                           "algorithmic_bytes_per_launch": g["bytes"],
                           "bytes_with_fp32_o": g["bytes_as_run"],
                           "frac_with_fp32_o": g["bytes_as_run"] / g["mean"] / 1e9 / HBM_PEAK_GBS,
                           "launch_us_mean": g["mean"] * 1e6, "launch_us_median": g["median"] * 1e6,
                           "launch_us_min": g["min"] * 1e6}
        tf = g["flops"] / g["mean"] / 1e12
        out["mfma"] = {"achieved": tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                       "frac": tf / BF16_PEAK_TFLOPS, "flops_per_launch": g["flops"],
                       "counters": measured_mfma("gdn")}
        out["config"] = {"workload": "gdr_chunk_fwd B8 H16 T4096 d128, bf16 q/k/v, "
                                     "fp32 alpha/beta/o/state, zero initial state",
                         "B": g["B"], "T": g["T"], "H": g["H"], "Dk": g["Dk"], "Dv": g["Dv"],
                         "chunk": 32, "global_batch": g["B"], "seq_len": g["T"]}
    if "gdn_bf16o" in res:
        g = res["gdn_bf16o"]
        gbs = g["bytes"] / g["mean"] / 1e9
        out["gdn_bf16_o"] = {"workload": "gdr_chunk_fwd B8 H16 T4096 d128, bf16 q/k/v/o",
                             "tokens/s": g["B"] * g["T"] / g["mean"],
                             "launch_us_mean": g["mean"] * 1e6,
                             "launch_us_median": g["median"] * 1e6,
                             "launch_us_min": g["min"] * 1e6, "GB/s": gbs,
                             "frac_hbm": gbs / HBM_PEAK_GBS,
                             "frac_mfma": g["flops"] / g["mean"] / 1e12 / BF16_PEAK_TFLOPS}
    if "decode" in res:
        d = res["decode"]
        gbs = d["bytes"] / d["median"] / 1e9
        out["decode"] = {"workload": "gdr_recurrent_step N256 H16 d128, 64 steps, fp32 o",
                         "us_per_step_median": d["median"] * 1e6,
                         "us_per_step_min": d["min"] * 1e6, "GB/s": gbs,
                         "frac_hbm": gbs / HBM_PEAK_GBS, "bytes_per_step": d["bytes"],
                         "bytes_with_fp32_o": d["bytes_as_run"],
                         "traffic": measured_traffic("decode"),
                         "dram_read_share": measured_dram("decode")}
        if "decode" in cpu:
            out["decode"]["cpu_baseline"] = cpu["decode"]
    if "gdr2" in res:
        r = res["gdr2"]
        if "error" in r:
            out["gdr2"] = {"error": r["error"]}
        else:
            gbs = r["bytes"] / r["mean"] / 1e9
            tf = r["flops"] / r["mean"] / 1e12
            out["gdr2"] = {"workload": "gdr2_chunk_fwd B4 H16 T4096 d128 bf16, fp32 o",
                           "tokens/s": r["B"] * r["T"] / r["mean"],
                           "launch_us_mean": r["mean"] * 1e6,
                           "launch_us_median": r["median"] * 1e6,
                           "launch_us_min": r["min"] * 1e6, "GB/s": gbs,
                           "frac_hbm": gbs / HBM_PEAK_GBS,
                           "algorithmic_bytes_per_launch": r["bytes"],
                           "bytes_with_fp32_o": r["bytes_as_run"],
                           "mfma": {"achieved": tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                    "frac": tf / BF16_PEAK_TFLOPS,
                                    "flops_per_launch": r["flops"],
                                    "counters": measured_mfma("gdr2")},
                           "traffic": measured_traffic("gdr2")}
            if "gdr2" in cpu:
                out["gdr2"]["cpu_baseline"] = cpu["gdr2"]
    if "longctx" in res:
        r = res["longctx"]
        gbs = r["bytes"] / r["mean"] / 1e9
        out["long_context"] = {
            "workload": "B1 H16 T32768 d128 bf16, fp32 alpha/beta/o, initial state: "
                        f"gdr_chunk_fwd_split, {r['nseg']} segments of {r['T'] // r['nseg']}",
            "tokens/s": r["B"] * r["T"] / r["mean"], "launch_us_mean": r["mean"] * 1e6,
            "launch_us_median": r["median"] * 1e6,
            "launch_us_min": r["min"] * 1e6, "GB/s": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
            "mfma_frac": r["flops"] / r["mean"] / 1e12 / BF16_PEAK_TFLOPS,
            "algorithmic_bytes_per_launch": r["bytes"], "bytes_with_fp32_o": r["bytes_as_run"],
            "plain_gdr_chunk_fwd": {"launch_us_mean": r["plain_mean"] * 1e6,
                                    "tokens/s": r["B"] * r["T"] / r["plain_mean"]}}
        if "longctx" in cpu:
            out["long_context"]["cpu_baseline"] = cpu["longctx"]
    if "gate_fused" in res:
        t = res["gate_fused"]["t"]
        tok = res["gate_fused"]["tokens"]
        out["gate_fused"] = {"workload": "B8 H16 T4096 d128 forward + output gate (bf16 gate, "
                                         "fp32 weight, bf16 y); rounds of 10 back-to-back calls "
                                         "of each, medians over rounds",
                             **{f"{n}_us_median": v["median"] for n, v in t.items()},
                             **{f"{n}_us_min": v["min"] for n, v in t.items()},
                             "fused_tokens/s": tok / t["fused"]["median"] * 1e6,
                             "two_calls_tokens/s": tok / t["two_calls"]["median"] * 1e6}
    if "l2norm" in res:
        out["l2norm"] = {"what": "launch us with raw q, k: fused GDR_L2NORM_QK, plain call "
                                 "(no normalisation), separate PyTorch normalise pass + plain call",
                         "gdn B8 H16 T4096": res["l2norm"]["gdn"],
                         "gdr2 B4 H16 T4096": res["l2norm"]["gdr2"]}
    if "gate" in res:
        r = res["gate"]
        gbs = r["bytes"] / r["mean"] / 1e9
        out["output_gate"] = {"workload": "gdr_output_gate B8 T4096 H16 d128: fp32 o, bf16 gate, "
                                          "fp32 weight, bf16 y",
                              "launch_us_mean": r["mean"] * 1e6, "GB/s": gbs,
                              "frac_hbm": gbs / HBM_PEAK_GBS, "bytes_per_launch": r["bytes"],
                              "traffic": measured_traffic("gate")}
    if "gate_bwd" in res:
        r = res["gate_bwd"]
        gbs = r["bytes"] / r["mean"] / 1e9
        out["output_gate_bwd"] = {"workload": "gdr_output_gate_bwd B8 T4096 H16 d128: fp32 o, "
                                              "bf16 gate and dL/dy, fp32 do, dg, dw",
                                  "launch_us_mean": r["mean"] * 1e6, "GB/s": gbs,
                                  "frac_hbm": gbs / HBM_PEAK_GBS, "bytes_per_launch": r["bytes"]}
    if "bwd" in res:
        r = res["bwd"]
        tf = r["flops"] / r["mean"] / 1e12
        out["backward"] = {"workload": "gdr_chunk_bwd B8 H16 T4096 d128, bf16 inputs and dL/do, "
                                       "fp32 gradients",
                           "launch_us_mean": r["mean"] * 1e6, "tokens/s": r["tokens"] / r["mean"],
                           "roofline": {"bound": "alu", "achieved": tf, "peak": FP32_PEAK_TFLOPS,
                                        "unit": "TFLOP/s", "frac": tf / FP32_PEAK_TFLOPS},
                           "flops_per_launch": r["flops"], "workspace_bytes": r["ws"],
                           "traffic": measured_traffic("bwd")}
    if "bwd2" in res:
        r = res["bwd2"]
        tf = r["flops"] / r["mean"] / 1e12
        out["backward2"] = {"workload": "gdr2_chunk_bwd B4 H16 T4096 d128, bf16 inputs and "
                                        "dL/do, fp32 gradients",
                            "launch_us_mean": r["mean"] * 1e6,
                            "tokens/s": r["tokens"] / r["mean"],
                            "roofline": {"bound": "alu", "achieved": tf,
                                         "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                                         "frac": tf / FP32_PEAK_TFLOPS},
                            "flops_per_launch": r["flops"], "workspace_bytes": r["ws"],
                            "traffic": measured_traffic("bwd2")}
    if "bwd_long" in res:
        r = res["bwd_long"]
        out["backward_long_context"] = {
            "workload": "B1 H16 T32768 d128 bf16 inputs and dL/do, initial state, dL/dS_T",
            "split_ms": r["split"] * 1e3, "plain_ms": r["plain"] * 1e3, "nseg": r["nseg"],
            "tokens/s_split": r["tokens"] / r["split"], "tokens/s_plain": r["tokens"] / r["plain"],
            "gdr2": {"fwd_plain_ms": r["gdr2_fwd_plain"] * 1e3,
                     "fwd_split_ms": r["gdr2_fwd_split"] * 1e3,
                     "bwd_plain_ms": r["gdr2_bwd_plain"] * 1e3,
                     "bwd_split_ms": r["gdr2_bwd_split"] * 1e3,
                     "bwd_split_fp32_states_ms": r["gdr2_bwd_split_fp32_states"] * 1e3}}
    if "copy" in res:
        cp = res["copy"]
        out["copy_reference"] = {"what": "torch device-to-device copy, 512 MiB read + 512 MiB "
                                         "written", "GB/s": cp["bytes"] / cp["mean"] / 1e9,
                                 "frac_hbm": cp["bytes"] / cp["mean"] / 1e9 / HBM_PEAK_GBS}
    if "gdn" in cpu:
        out["cpu_baseline"] = cpu["gdn"]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
