#!/usr/bin/env python3
"""Benchmark of the gated delta rule hot path on one MI355X.

One step = one chunkwise gated delta rule forward (gdr_chunk_fwd) over the
1.3B-layer workload: B=8, H=16, T=4096, d_k = d_v = 128, bf16 q/k/v, fp32
alpha/beta, zero initial state, fp32 output and final state.  Inputs are
seeded synthetic tensors resident in HBM before timing starts.

The JSON line (stdout, last line) carries:
  value / unit       tokens/s of that forward (B*T tokens per call)
  roofline           the chunked kernel against HBM bandwidth (its bound):
                     algorithmic bytes per launch / mean launch time
  mfma               the same launches against the dense bf16 MFMA peak,
                     counting 2 (3 dk dv + 5 C d) flops per token-head
  decode             gdr_recurrent_step on 256 sequences x 16 heads, d=128,
                     64 consecutive steps: GB/s of state + token traffic
  gdr2               gdr2_chunk_fwd on B=4 H=16 T=4096 d=128 (bf16 gates)
  long_context       gdr_chunk_fwd on B=1 H=16 T=32768 d=128 with an initial
                     state (16 sequential chains; tokens/s, HBM and MFMA
                     fractions)
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
  cpu_baseline       the fp64 oracle timed on the host on the same workload
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_counters.json")
# kernel-name prefix in rocprofv3 output -> the bench leg it belongs to
KERNELS = {"gdn": "void gdr::(anonymous namespace)::chunk_bf16_kernel<128, 128, 64, float, false>",
           "gdr2": "void gdr::(anonymous namespace)::gdr2_bf16_kernel<128, 128, float, false>",
           "decode": "void gdr::step_kernel<128, 128, unsigned short, float>",
           "gate": "void gdr::(anonymous namespace)::output_gate_kernel<128, float, unsigned short, "
                   "unsigned short>",
           "bwd": "void gdr::(anonymous namespace)::chunk2_bwd_kernel<128, 128, unsigned short, "
                  "unsigned short, true>",
           "bwd2": "void gdr::(anonymous namespace)::chunk2_bwd_kernel<128, 128, unsigned short, "
                   "unsigned short, false>",
           "copy": "__amd_rocclr_copyBuffer"}


def source_hash() -> str:
    """Hash of every HIP source and header: counter readings are only valid
    for the kernels they were taken on."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(CSRC, "*"))):
        if f.endswith((".hip", ".h")):
            h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def summarize(trace_dir, fetch_dir, write_dir, out_txt, command, timed=20):
    """Turn rocprofv3 CSV output (a --kernel-trace --stats run and two --pmc
    runs, FETCH_SIZE then WRITE_SIZE) into a short text summary and the JSON
    the benchmark reads its `traffic` figures from.  Counter KiB are scaled
    by what the same counter reads for the plain 512 MiB device copy."""
    stats = list(csv.DictReader(open(glob.glob(os.path.join(trace_dir, "*kernel_stats.csv"))[0])))
    per = {}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = list(csv.DictReader(open(glob.glob(os.path.join(d, "*counter_collection.csv"))[0])))
        for leg, prefix in KERNELS.items():
            vals = [float(r["Counter_Value"]) for r in rows
                    if r["Kernel_Name"].startswith(prefix) and r["Counter_Name"] == name]
            if vals:
                per.setdefault(leg, {})[name] = sum(vals) / len(vals)
    copy_bytes_kib = 512 * 1024   # the copy reads and writes 512 MiB each
    scale = {"FETCH_SIZE": copy_bytes_kib / per["copy"]["FETCH_SIZE"],
             "WRITE_SIZE": copy_bytes_kib / per["copy"]["WRITE_SIZE"]}
    traffic = {}
    for leg, c in per.items():
        if leg == "copy":
            continue
        rd = c["FETCH_SIZE"] * scale["FETCH_SIZE"] * 1024
        wr = c["WRITE_SIZE"] * scale["WRITE_SIZE"] * 1024
        traffic[leg] = {"read_bytes": rd, "write_bytes": wr, "bytes": rd + wr}
    lines = [f"# rocprofv3 summary (HIP sources hash {source_hash()})", "",
             "Command:", f"  {command}", "", "Kernel trace (--kernel-trace --stats):",
             f"  {'kernel':60s} {'calls':>6s} {'avg us':>10s} {'min us':>10s} {'max us':>10s}"]
    for r in stats:
        lines.append(f"  {r['Name'][:60]:60s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.1f} "
                     f"{float(r['MinNs']) / 1e3:10.1f} {float(r['MaxNs']) / 1e3:10.1f}")
    # the same trace, per bench leg: the timed launches only (the last
    # `timed` dispatches of each kernel; the warm-up launches before them
    # include the clock ramp after idle)
    trace = list(csv.DictReader(open(glob.glob(os.path.join(trace_dir, "*kernel_trace.csv"))[0])))
    lines += ["", f"Timed launches (the last {timed} dispatches of each kernel in the trace, 10 for "
              "the backward legs, as the bench times them):", f"  {'leg':8s} {'kernel':44s} {'n':>4s} {'avg us':>10s} {'min us':>10s}"]
    for leg, prefix in KERNELS.items():
        d = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in trace
                   if r["Kernel_Name"].startswith(prefix))
        if not d:
            continue
        n_timed = min(timed, 10) if leg in ("bwd", "bwd2") else timed   # legs capped at 10
        dur = [(e - b) / 1e3 for b, e in d[-n_timed:]]
        lines.append(f"  {leg:8s} {prefix[:44]:44s} {len(dur):4d} {sum(dur) / len(dur):10.1f} "
                     f"{min(dur):10.1f}")
    lines += ["", "HBM counters per dispatch (KiB as read; scale = copy's known bytes / reading):",
              f"  FETCH_SIZE scale {scale['FETCH_SIZE']:.4f}, WRITE_SIZE scale {scale['WRITE_SIZE']:.4f}"]
    for leg, c in per.items():
        t = traffic.get(leg)
        extra = "" if t is None else (f" -> read {t['read_bytes'] / 1e6:.1f} MB, write "
                                      f"{t['write_bytes'] / 1e6:.1f} MB per launch")
        lines.append(f"  {leg:7s} FETCH {c['FETCH_SIZE']:12.1f}  WRITE {c['WRITE_SIZE']:12.1f}{extra}")
    open(out_txt, "w").write("\n".join(lines) + "\n")
    json.dump({"source_hash": source_hash(), "scale": scale, "traffic": traffic,
               "command": command}, open(TRAFFIC_FILE, "w"), indent=1)
    print("\n".join(lines))


def measured_traffic(leg):
    """HBM bytes per launch from the committed counter summary, or None when
    the kernels have changed since the counters were taken."""
    try:
        d = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if d.get("source_hash") != source_hash():
        return None
    t = d.get("traffic", {}).get(leg)
    return None if t is None else t["bytes"]


def time_launches(fn, warmup, steps):
    """Mean and min per-call time (s) from HIP events on the current stream,
    plus the wall time of the `steps` calls bracketed by synchronize."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    mean = sum(ms) / len(ms) / 1e3
    return mean, ms[0] / 1e3, ms[len(ms) // 2] / 1e3, wall


def bench_gdn(gdr, torch, warmup, steps):
    from gdr_gen import make_config
    inp = make_config(1)
    B, T, H, Dk = inp.q.shape
    Dv = inp.v.shape[-1]
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in (inp.q, inp.k, inp.v))
    a, b = inp.alpha.to(dev), inp.beta.to(dev)
    o = torch.empty((B, T, H, Dv), dtype=torch.float32, device=dev)
    sf = torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=dev)

    def fn():
        gdr.gdr_chunk_fwd(q, k, v, a, b, None, out_dtype=torch.float32, o=o,
                          s_final=sf)

    mean, mn, med, wall = time_launches(fn, warmup, steps)
    th = B * T * H
    # algorithmic bytes: q, k, v bf16 + alpha, beta fp32 + o fp32 per
    # token-head, plus the fp32 final state once
    bytes_launch = th * (2 * (Dk + Dk + Dv) + 8 + 4 * Dv) + 4 * B * H * Dv * Dk
    C = 64
    flops_launch = th * 2 * (3 * Dk * Dv + 5 * C * (Dk + Dv) // 2)
    return dict(inp=inp, mean=mean, min=mn, median=med, wall=wall, B=B, T=T, H=H, Dk=Dk,
                Dv=Dv, bytes=bytes_launch, flops=flops_launch)


def bench_longctx(gdr, torch, warmup, steps, nseg=8):
    """The long-context workload: B1 H16 T32768 d128 with an initial state.
    Run plainly it is 16 sequential chains of 1024 chunks (few heads, so
    narrow row blocks and half the compute units idle); the split call runs
    it as nseg = 8 segments side by side (three passes plus a scan).  Both
    are timed; the bytes and flops are the workload's algorithmic ones."""
    from gdr_gen import make_config
    inp = make_config(2)
    B, T, H, Dk = inp.q.shape
    Dv = inp.v.shape[-1]
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in (inp.q, inp.k, inp.v))
    a, b = inp.alpha.to(dev), inp.beta.to(dev)
    s0 = inp.s0.to(dev)
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
    th = B * T * H
    bytes_launch = th * (2 * (Dk + Dk + Dv) + 8 + 4 * Dv) + 2 * 4 * B * H * Dv * Dk
    C = 64
    flops_launch = th * 2 * (3 * Dk * Dv + 5 * C * (Dk + Dv) // 2)
    return dict(mean=mean, min=mn, plain_mean=pmean, plain_min=pmn, nseg=nseg, B=B, T=T, H=H,
                bytes=bytes_launch, flops=flops_launch)


def bench_decode(gdr, torch, warmup):
    from gdr_gen import make_config
    inp = make_config(3)
    steps, N, H, Dk = inp.q.shape
    Dv = inp.v.shape[-1]
    dev = torch.device("cuda:0")
    S = inp.state0.to(dev)
    q, k, v = (x.to(dev) for x in (inp.q, inp.k, inp.v))
    a, b = inp.alpha.to(dev), inp.beta.to(dev)
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
    bytes_step = nh * (2 * 4 * Dv * Dk + 2 * (2 * Dk + Dv) + 8 + 4 * Dv)
    return dict(median=med, min=ms[0] / 1e3, mean=sum(ms) / len(ms) / 1e3, bytes=bytes_step,
                N=N, H=H, steps=steps)


def bench_gdr2(gdr, torch, warmup, steps):
    from gdr_gen import make_config
    inp = make_config(4)
    B, T, H, Dk = inp.q.shape
    Dv = inp.v.shape[-1]
    dev = torch.device("cuda:0")
    args = [x.to(dev) for x in (inp.q, inp.k, inp.v, inp.alpha, inp.erase, inp.write)]
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
    bytes_launch = th * (2 * (4 * Dk + 2 * Dv) + 4 * Dv) + 4 * B * H * Dv * Dk
    return dict(mean=mean, min=mn, median=med, B=B, T=T, H=H, bytes=bytes_launch)


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


def bench_bwd(gdr, torch, warmup, steps):
    """gdr_chunk_bwd on B8 H16 T4096 d128 (bf16 q/k/v and dL/do, dL/dS_T
    given, zero S_0).  It runs the GDN-2 backward with broadcast gates, so
    the flops are counted as for bench_bwd2: per token-head, chunk C = 16,
    2 x (9 dk dv + 3 C dk + 3 C dv)."""
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
    from gdr_gen import make_config
    inp = make_config(2)
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
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(inp, repeats=3):
    """The fp64 oracle on the whole workload (B8 H16 T4096 d128 finishes in
    about half a second on 16 host threads), best of `repeats`, on every thread the
    oracle's OpenMP runtime uses; then once more on one thread."""
    import oracle
    qq, kk, vv, aa, bb = (oracle._f64(x) for x in (inp.q, inp.k, inp.v, inp.alpha,
                                                     inp.beta))   # conversion excluded
    best = float("inf")
    for _ in range(repeats):
        t0 = time.perf_counter()
        oracle.gdn_fwd(qq, kk, vv, aa, bb, None)
        best = min(best, time.perf_counter() - t0)
    B, T, H, Dk = inp.q.shape
    tokens = B * T
    cores = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        t0 = time.perf_counter()
        oracle.gdn_fwd(qq, kk, vv, aa, bb, None)
        one = time.perf_counter() - t0
    finally:
        oracle.set_num_threads(cores)
    return dict(value=tokens / best, unit="tokens/s", cores=cores, kind="oracle",
                sample=f"whole workload B{B} H{H} T{T} d{Dk} ({tokens} tokens x {H} heads), "
                       f"fp64 token-by-token recurrence, best of {repeats}: {best:.2f} s; "
                       f"one thread, one run: {one:.2f} s",
                one_thread=dict(value=tokens / one, unit="tokens/s", seconds=one),
                cpu_model=_cpu_model())


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-baseline leg")
    ap.add_argument("--only", choices=["gdn", "decode", "gdr2", "longctx", "l2norm", "gate", "gate_bwd",
                                       "bwd", "bwd2", "bwd_long", "copy"],
                    default=None,
                    help="time one operation only (for profiling)")
    ap.add_argument("--skip", default="",
                    help="comma-separated legs not to run (the profiled command skips l2norm, "
                         "longctx and bwd_long, whose calls reuse the headline and backward "
                         "kernels' names at other shapes)")
    ap.add_argument("--summarize", nargs=4, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR", "OUT"),
                    help="summarize rocprofv3 CSV output into OUT and the traffic JSON, then exit")
    ap.add_argument("--command", default="", help="the profiling command, recorded in --summarize")
    args = ap.parse_args()
    if args.summarize:
        summarize(*args.summarize, command=args.command)
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

    res = {}
    if want("gdn"):
        log("timing gdr_chunk_fwd B8 H16 T4096 d128 ...")
        res["gdn"] = bench_gdn(gdr, torch, args.warmup, args.steps)
        log(f"  mean {res['gdn']['mean'] * 1e6:.1f} us")
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
                           "kernel": "chunk_bf16_kernel<128,128,64,float,false>",
                           "algorithmic_bytes_per_launch": g["bytes"],
                           "launch_us_mean": g["mean"] * 1e6, "launch_us_median": g["median"] * 1e6,
                           "launch_us_min": g["min"] * 1e6}
        tf = g["flops"] / g["mean"] / 1e12
        out["mfma"] = {"achieved": tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                       "frac": tf / BF16_PEAK_TFLOPS, "flops_per_launch": g["flops"]}
        out["config"] = {"workload": "gdr_chunk_fwd B8 H16 T4096 d128, bf16 q/k/v, "
                                     "fp32 alpha/beta/o/state, zero initial state",
                         "B": g["B"], "T": g["T"], "H": g["H"], "Dk": g["Dk"], "Dv": g["Dv"],
                         "chunk": 32, "global_batch": g["B"], "seq_len": g["T"]}
    if "decode" in res:
        d = res["decode"]
        gbs = d["bytes"] / d["median"] / 1e9
        out["decode"] = {"workload": "gdr_recurrent_step N256 H16 d128, 64 steps",
                         "us_per_step_median": d["median"] * 1e6,
                         "us_per_step_min": d["min"] * 1e6, "GB/s": gbs,
                         "frac_hbm": gbs / HBM_PEAK_GBS, "bytes_per_step": d["bytes"],
                         "traffic": measured_traffic("decode")}
    if "gdr2" in res:
        r = res["gdr2"]
        if "error" in r:
            out["gdr2"] = {"error": r["error"]}
        else:
            gbs = r["bytes"] / r["mean"] / 1e9
            out["gdr2"] = {"workload": "gdr2_chunk_fwd B4 H16 T4096 d128 bf16, fp32 o",
                           "tokens/s": r["B"] * r["T"] / r["mean"],
                           "launch_us_mean": r["mean"] * 1e6, "GB/s": gbs,
                           "frac_hbm": gbs / HBM_PEAK_GBS,
                           "algorithmic_bytes_per_launch": r["bytes"],
                           "traffic": measured_traffic("gdr2")}
    if "longctx" in res:
        r = res["longctx"]
        gbs = r["bytes"] / r["mean"] / 1e9
        out["long_context"] = {
            "workload": "B1 H16 T32768 d128 bf16, fp32 alpha/beta/o, initial state: "
                        f"gdr_chunk_fwd_split, {r['nseg']} segments of {r['T'] // r['nseg']}",
            "tokens/s": r["B"] * r["T"] / r["mean"], "launch_us_mean": r["mean"] * 1e6,
            "launch_us_min": r["min"] * 1e6, "GB/s": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
            "mfma_frac": r["flops"] / r["mean"] / 1e12 / BF16_PEAK_TFLOPS,
            "algorithmic_bytes_per_launch": r["bytes"],
            "plain_gdr_chunk_fwd": {"launch_us_mean": r["plain_mean"] * 1e6,
                                    "tokens/s": r["B"] * r["T"] / r["plain_mean"]}}
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
    if not args.no_cpu and "gdn" in res:
        log("timing the fp64 oracle on the host ...")
        out["cpu_baseline"] = cpu_baseline(res["gdn"]["inp"])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
