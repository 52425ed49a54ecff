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
  cpu_baseline       the fp64 oracle timed on the host on a bounded sample
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "tokens/s chunkwise gated-delta fwd (H16,d128,T4K); % MFMA peak; decode GB/s"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


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


def cpu_baseline(inp):
    """fp64 oracle on batches 0-1 of the same workload (2 x 16 heads x 4096
    tokens), all host threads the oracle's OpenMP runtime uses."""
    import oracle
    sel = [0, 1]
    q, k, v, a, b = (x[sel] for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta))
    qq, kk, vv, aa, bb = (oracle._f64(x) for x in (q, k, v, a, b))   # conversion excluded
    t0 = time.perf_counter()
    oracle.gdn_fwd(qq, kk, vv, aa, bb, None)
    dt = time.perf_counter() - t0
    tokens = len(sel) * inp.q.shape[1]
    return dict(value=tokens / dt, unit="tokens/s", cores=oracle.num_threads(),
                kind="oracle",
                sample=f"batches 0-1 of B8 H16 T4096 d128 ({tokens} tokens x 16 heads), "
                       f"fp64, {dt:.2f} s")


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-baseline leg")
    ap.add_argument("--only", choices=["gdn", "decode", "gdr2"], default=None,
                    help="time one operation only (for profiling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the path shards by batch/head with no communication; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_16_amd as gdr
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    res = {}
    if args.only in (None, "gdn"):
        log("timing gdr_chunk_fwd B8 H16 T4096 d128 ...")
        res["gdn"] = bench_gdn(gdr, torch, args.warmup, args.steps)
        log(f"  mean {res['gdn']['mean'] * 1e6:.1f} us")
    if args.only in (None, "decode"):
        log("timing gdr_recurrent_step N256 H16 d128 x 64 steps ...")
        res["decode"] = bench_decode(gdr, torch, args.warmup)
        log(f"  median {res['decode']['median'] * 1e6:.1f} us/step")
    if args.only in (None, "gdr2"):
        log("timing gdr2_chunk_fwd B4 H16 T4096 d128 ...")
        res["gdr2"] = bench_gdr2(gdr, torch, args.warmup, args.steps)

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
                           "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                           "kernel": "chunk_bf16_kernel<128,128,float>",
                           "algorithmic_bytes_per_launch": g["bytes"],
                           "launch_us_mean": g["mean"] * 1e6, "launch_us_min": g["min"] * 1e6}
        tf = g["flops"] / g["mean"] / 1e12
        out["mfma"] = {"achieved": tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                       "frac": tf / BF16_PEAK_TFLOPS, "flops_per_launch": g["flops"]}
        out["config"] = {"workload": "gdr_chunk_fwd B8 H16 T4096 d128, bf16 q/k/v, "
                                     "fp32 alpha/beta/o/state, zero initial state",
                         "B": g["B"], "T": g["T"], "H": g["H"], "Dk": g["Dk"], "Dv": g["Dv"],
                         "chunk": 64, "global_batch": g["B"], "seq_len": g["T"]}
    if "decode" in res:
        d = res["decode"]
        gbs = d["bytes"] / d["median"] / 1e9
        out["decode"] = {"workload": "gdr_recurrent_step N256 H16 d128, 64 steps",
                         "us_per_step_median": d["median"] * 1e6,
                         "us_per_step_min": d["min"] * 1e6, "GB/s": gbs,
                         "frac_hbm": gbs / HBM_PEAK_GBS, "bytes_per_step": d["bytes"]}
    if "gdr2" in res:
        r = res["gdr2"]
        if "error" in r:
            out["gdr2"] = {"error": r["error"]}
        else:
            gbs = r["bytes"] / r["mean"] / 1e9
            out["gdr2"] = {"workload": "gdr2_chunk_fwd B4 H16 T4096 d128 bf16, fp32 o",
                           "tokens/s": r["B"] * r["T"] / r["mean"],
                           "launch_us_mean": r["mean"] * 1e6, "GB/s": gbs,
                           "frac_hbm": gbs / HBM_PEAK_GBS}
    if not args.no_cpu and "gdn" in res:
        log("timing the fp64 oracle on the host ...")
        out["cpu_baseline"] = cpu_baseline(res["gdn"]["inp"])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
