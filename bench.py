"""Benchmark: SHA decode on one MI355X, OPT-66B-shaped layer by default.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one SHA decode layer call (split kernel + combine when split) over
one batch of synthetic decode state already resident in HBM.  Prints one
JSON line: effective KV bandwidth on active-head K/V bytes (the value), the
per-call time, the roofline of the decode kernel (HIP-event durations on the
launch stream), the same kernel with every head active, and the fp64 oracle
timed on the host cores.

Other modes (profiling helpers, no JSON line):
  --copy-calib   plain device-to-device copies of a known size, for scaling
                 rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import contextual_head_sparsity_amd as sha  # noqa: E402
from contextual_head_sparsity_amd import workloads as wl  # noqa: E402

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E peak, GB/s
KERNEL_SRC = os.path.join(ROOT, "contextual_head_sparsity_amd", "csrc", "sha_kernels.hip")


def kernel_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default=wl.HEADLINE, choices=list(wl.WORKLOADS))
    p.add_argument("--nsplit", type=int, default=0, help="0 = library plan")
    p.add_argument("--copies", type=int, default=0,
                   help="rotating K/V copies (0 = enough that consecutive steps share no bytes)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-dense", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--copy-calib", action="store_true")
    return p.parse_args()


def copy_calib(steps: int):
    """Device copies of 1 GiB (read 1 GiB + write 1 GiB per dispatch)."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(7)
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calib_bytes_read": n, "copy_calib_bytes_written": n,
                      "dispatches": steps}), flush=True)


def time_calls(call, steps: int, warmup: int, stream):
    """Wall time of `steps` back-to-back calls, and per-call HIP-event
    durations recorded on the launch stream."""
    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        call(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return wall / steps * 1e3, ev_ms


def cpu_baseline(w, q, k, v, idx, budget_s: float):
    """The fp64 oracle on the host cores: whole layer calls of this workload
    (every active unit, inputs copied to host memory first), repeated until
    about budget_s of CPU work has been timed."""
    from oracle import sha_units_ref
    try:
        from threadpoolctl import threadpool_info
        threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    G = w.H // w.H_kv
    idx_cpu = idx.cpu().numpy()
    rows = []
    for b in range(w.B):
        heads = [int(e) for e in idx_cpu[b]]
        units = ([(h, g) for g in heads for h in range(g * G, g * G + G)] if w.gqa
                 else [(h, h // G) for h in heads])
        rows.append((torch.stack([q[b, h, 0] for h, _ in units]).cpu(),
                     torch.stack([k[b, g] for _, g in units]).cpu(),
                     torch.stack([v[b, g] for _, g in units]).cpu()))
    spent, passes = 0.0, 0
    while spent < budget_s and passes < 100:
        t0 = time.perf_counter()
        for qs, ks, vs in rows:
            sha_units_ref(qs, ks, vs, w.scale)
        spent += time.perf_counter() - t0
        passes += 1
    per_call = spent / passes
    return {"value": round(w.active_kv_bytes / per_call / 1e9, 4), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "sample": f"{passes} full layer call(s) of {w.name} ({w.units} units, "
                      f"{w.active_kv_bytes / 1e6:.0f} MB active K/V each), fp64 numpy oracle, "
                      f"{spent:.1f} s timed, {per_call * 1e6:.0f} us per layer call"}


def load_traffic(workload: str):
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_hash():
        return None   # counters were taken on an older kernel
    return rec.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: SHA decode units are independent and this "
              "build runs on a single MI355X; --gpus must be 1.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calib:
        copy_calib(max(args.steps, 1))
        return

    w = wl.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    fn = sha.sha_decode_gqa if w.gqa else sha.sha_decode
    q, k, v, idx, o = wl.make_workload(w, dev)
    # Rotating K/V copies: consecutive steps read disjoint memory, so neither
    # the 4 MB L2 per XCD nor the 256 MB MALL can serve a step from the last.
    copies = args.copies or max(2, math.ceil(2 * 256e6 / w.active_kv_bytes))
    ks, vs = [k], [v]
    for c in range(1, copies):
        _, kc, vc = wl.make_qkv(w, dev, seed_offset=c)
        ks.append(kc)
        vs.append(vc)
    nsplit = args.nsplit or sha.plan_nsplit(w.B, w.H, w.H_kv, w.Nkv, w.d, w.top_k, w.gqa,
                                            q.dtype)
    ws_bytes = sha.workspace_bytes(w.B, w.H, w.H_kv, w.Nkv, w.d, w.top_k, w.gqa, q.dtype, nsplit)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def call(i, index=idx):
        fn(q, ks[i % copies], vs[i % copies], index, scale=w.scale, out=o, nsplit=nsplit,
           workspace=ws, stream=stream)

    ms, ev = time_calls(call, args.steps, args.warmup, stream)
    ev_avg_ms = float(np.mean(ev))
    us_call = ms * 1e3
    value = w.active_kv_bytes / (ms / 1e3) / 1e9

    dense = None
    if not args.no_dense:
        n_sel = w.H_kv if w.gqa else w.H
        dense_idx = torch.arange(n_sel, dtype=torch.int32, device=dev).repeat(w.B, 1)
        dn = sha.plan_nsplit(w.B, w.H, w.H_kv, w.Nkv, w.d, n_sel, w.gqa, q.dtype)
        dws = torch.empty(max(sha.workspace_bytes(w.B, w.H, w.H_kv, w.Nkv, w.d, n_sel, w.gqa,
                                                  q.dtype, dn), 1), dtype=torch.uint8, device=dev)
        od = torch.zeros_like(q)

        def dcall(i):
            fn(q, ks[i % copies], vs[i % copies], dense_idx, scale=w.scale, out=od, nsplit=dn,
               workspace=dws, stream=stream)

        dms, _ = time_calls(dcall, max(args.steps // 2, 5), max(args.warmup // 2, 2), stream)
        dense = {"us_per_layer": dms * 1e3, "top_k": n_sel, "nsplit": dn,
                 "kv_GBps": w.dense_kv_bytes / (dms / 1e3) / 1e9,
                 "speedup_sparse_vs_all_heads": dms / ms,
                 "ideal_speedup": n_sel / w.top_k}

    achieved = w.active_kv_bytes / (ev_avg_ms / 1e3) / 1e9
    traffic = load_traffic(w.name)
    out = {
        "metric": "SHA decode \u00b5s/layer + effective KV GB/s (% HBM peak), OPT-66B shape B=64",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "us_per_layer": round(us_call, 2),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: i.i.d. N(0,1) q/k/v (seeded, drawn on device), seeded index rows",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "H_kv": w.H_kv, "d": w.d,
                   "Nkv": w.Nkv, "top_k": w.top_k, "gqa": w.gqa, "index_sampling": w.sampling,
                   "nsplit": nsplit, "kv_copies_rotated": copies,
                   "active_kv_bytes": w.active_kv_bytes, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "sha_decode_gqa_kernel" if w.gqa else "sha_decode_mha_kernel",
                     "launch_avg_us": round(ev_avg_ms * 1e3, 2),
                     "launch_p10_us": round(float(np.percentile(ev, 10)) * 1e3, 2),
                     "launch_p90_us": round(float(np.percentile(ev, 90)) * 1e3, 2),
                     "bytes_per_launch": w.active_kv_bytes,
                     "note": ("event span covers the split kernel and the combine kernel"
                              if nsplit > 1 else "event span covers the one decode kernel")},
        "all_heads": dense,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, q, ks[0], vs[0], idx, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
