"""Benchmark: SHA decode on one MI355X, OPT-66B-shaped layer by default.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one SHA decode layer call (split kernel + combine when split) over
one batch of synthetic decode state already resident in HBM.  Prints one
JSON line: effective KV bandwidth on active-head K/V bytes (the value), the
per-call time, the roofline of the decode kernel (HIP-event durations on the
launch stream), the same kernel with every head active, the fp64 oracle
timed on the host cores, and (default workload) a density sweep over the
active heads, a per-workload block for the other layer shapes, and short
summaries of the selective MLP (OPT shapes) and the attention router (layer
shapes) (--no-extras skips those two).

Other modes (one JSON line each):
  --kv-layout L        the decode call on a strided or paged KV cache.
  --mlp NAME           the selective MLP (device union + up/down projections);
    --mlp-batch B      another batch size;  --mlp-sweep  batches 1, 2, 4, ...
  --router NAME        the attention router (device time per call in a graph;
                       --router-floor adds the same graph on tiny inputs).
  --decode-step L      an L-layer decode step (router, SHA, selective MLP).
Profiling helpers:
  --copy-calib         plain device-to-device copies of a known size, for
                       scaling rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes.
  --summarize-traffic  counter CSVs -> profiles/traffic_<workload>.json.
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
CSRC = os.path.join(ROOT, "contextual_head_sparsity_amd", "csrc")
# Sources of each decode kernel: its own file plus the shared device headers.
KERNEL_SOURCES = {False: ("sha_kernels.hip", "sha_device.h", "sha_decode.h"),
                  True: ("sha_gqa_mfma.hip", "sha_device.h", "sha_decode.h")}
# The density sweep at the OPT-66B shape: active heads out of 72 per row.
SWEEP_TOP_K = (7, 14, 22, 36, 54, 72)
METRIC = "SHA decode \u00b5s/layer + effective KV GB/s (% HBM peak), OPT-66B shape B=64"


def _code_only(text: str) -> str:
    """Source text without comments and with whitespace collapsed: the hash
    follows the code, not its documentation."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_hash(gqa: bool) -> str:
    """Hash of one decode kernel's sources (code only): counter-derived
    traffic is only reported for the kernel it was measured on."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[bool(gqa)]:
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default=wl.HEADLINE, choices=list(wl.WORKLOADS))
    p.add_argument("--nsplit", type=int, default=0, help="0 = library plan")
    p.add_argument("--kv-layout", default="contig",
                   help="contig | bnhd ([B, Nkv, H_kv, d] cache) | pagedP (pool of P-row pages)")
    p.add_argument("--copies", type=int, default=0,
                   help="rotating K/V copies (0 = enough that consecutive steps share no bytes)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-dense", action="store_true")
    p.add_argument("--no-probe", action="store_true", help="skip the read-bandwidth probe")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the selective-MLP and router summaries on the default line")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the per-workload block and the density sweep (headline only)")
    p.add_argument("--sweep-out", default=None,
                   help="also write the density sweep to this JSON file")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--copy-calib", action="store_true")
    p.add_argument("--summarize-traffic", action="store_true",
                   help="write profiles/traffic_<workload>.json from rocprofv3 --pmc CSVs")
    p.add_argument("--fetch-csv")
    p.add_argument("--write-csv")
    p.add_argument("--copy-fetch-csv")
    p.add_argument("--copy-write-csv")
    p.add_argument("--traffic-out", default=None,
                   help="where --summarize-traffic writes (default: profiles/traffic_<workload>.json)")
    p.add_argument("--grid", type=int, default=0, help="decode dispatch grid size to select")
    p.add_argument("--mlp", default=None, choices=list(wl.MLP_WORKLOADS),
                   help="measure the selective MLP on this workload instead of SHA decode")
    p.add_argument("--mlp-batch", type=int, default=0, help="override the MLP workload's B")
    p.add_argument("--mlp-sweep", action="store_true",
                   help="with --mlp: time batches 1, 2, 4, ..., B (union density sweep)")
    p.add_argument("--decode-step", type=int, default=0, metavar="L",
                   help="time an L-layer decode step (router -> SHA -> selective MLP, layer 0 "
                        "dense) as one HIP graph and call by call")
    p.add_argument("--step-mlp", default=None, choices=list(wl.MLP_WORKLOADS),
                   help="MLP shape inside the decode step (its dtype follows the workload)")
    p.add_argument("--router", default=None, choices=list(wl.WORKLOADS),
                   help="time the attention router (scores + per-row top-k) of this layer shape")
    p.add_argument("--router-onepass", action="store_true",
                   help="with --router: time the one-pass kernels (no workspace) even where "
                        "the library picks the K-split form")
    p.add_argument("--router-floor", action="store_true",
                   help="with --router: also time the same graph of calls on tiny inputs")
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
    """Time `steps` back-to-back calls twice: once bracketed only by device
    synchronisation (wall time per call, the throughput figure), once with a
    HIP event pair around every call on the launch stream (per-launch kernel
    durations for the roofline)."""
    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        call(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        starts[i].record(stream)
        call(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    ev_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return wall / steps * 1e3, ev_ms


def graph_us_per_call(call, n: int, dev, warm: int, reps: int) -> float:
    """Device time per call as a captured decode loop sees it: `call(i)` for
    i < n captured in one graph on a side stream (calls launch on the current,
    i.e. capturing, stream), replayed `warm` times untimed and `reps` times
    timed; wall time of the replays over reps * n."""
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        for i in range(3):
            call(i)
    s.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=s):
        for i in range(n):
            call(i)
    torch.cuda.synchronize()
    for _ in range(warm):
        gr.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        gr.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / (reps * n) * 1e6


def read_probe(dev, nbytes: int = 1 << 31):
    """Secondary ceiling: the best streaming-read rate of libsha_probe.so (the
    head kernel's access pattern: 1 KiB non-temporal wave loads, 8 in flight)
    over grid sizes from one to sixteen workgroups per CU, on a buffer far
    larger than the caches."""
    import ctypes
    path = os.path.join(ROOT, "contextual_head_sparsity_amd", "libsha_probe.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    L.sha_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                 ctypes.c_void_p]
    buf = torch.ones(nbytes // 2, dtype=torch.float16, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    best = (0.0, 0)
    for blocks in (256, 512, 1024, 2048, 4096):
        def call(i):
            st = L.sha_probe_read(buf.data_ptr(), nbytes, blocks, sink.data_ptr(), stream.cuda_stream)
            if st != 0:
                raise RuntimeError(f"sha_probe_read failed: {st}")
        _, ev = time_calls(call, 10, 3, stream)
        gbs = nbytes / (float(np.median(ev)) / 1e3) / 1e9
        best = max(best, (gbs, blocks))
    del buf
    return {"GBps": round(best[0], 1), "blocks": best[1], "bytes": nbytes,
            "kernel": "sha_probe_read_kernel (libsha_probe.so)"}


def rotating_kv(w, dev, k, v, copies=0):
    """K/V copies that consecutive calls rotate through, so that neither the
    4 MB L2 per XCD nor the 256 MB MALL can serve a call from the last one
    (at most 256 copies: the tiny workload stays launch-bound anyway)."""
    copies = copies or min(256, max(2, math.ceil(2 * 256e6 / w.active_kv_bytes)))
    ks, vs = [k], [v]
    for c in range(1, copies):
        _, kc, vc = wl.make_qkv(w, dev, seed_offset=c)
        ks.append(kc)
        vs.append(vc)
    return ks, vs, copies


def decode_timing(w, q, ks, vs, index, nsplit, steps, warmup, stream):
    """(wall ms per call, per-launch event ms) of back-to-back decode calls
    over the rotating K/V copies, with a workspace allocated up front."""
    fn = sha.sha_decode_gqa if w.gqa else sha.sha_decode
    top_k = index.shape[1]
    wsb = sha.workspace_bytes(w.B, w.H, w.H_kv, w.Nkv, w.d, top_k, w.gqa, q.dtype, nsplit)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=q.device)
    out = torch.zeros_like(q)
    n = len(ks)

    def call(i):
        fn(q, ks[i % n], vs[i % n], index, scale=w.scale, out=out, nsplit=nsplit, workspace=ws,
           stream=stream)

    return time_calls(call, steps, warmup, stream)


def selected_mask(w, idx_cpu):
    G = w.H // w.H_kv
    sel = torch.zeros(w.B, w.H, dtype=torch.bool)
    for b in range(w.B):
        for e in idx_cpu[b]:
            if w.gqa and 0 <= e < w.H_kv:
                sel[b, e * G:(e + 1) * G] = True
            elif not w.gqa and 0 <= e < w.H:
                sel[b, e] = True
    return sel


def output_check(w, q, k, v, idx, dev):
    """One call into a sentinel-filled output: unselected slots keep their
    bits, selected ones are finite."""
    fn = sha.sha_decode_gqa if w.gqa else sha.sha_decode
    o_chk = wl.sentinel_like(w, dev)
    fn(q, k, v, idx, scale=w.scale, out=o_chk)
    torch.cuda.synchronize()
    sel = selected_mask(w, idx.cpu().numpy()).to(dev)
    return o_chk, {"active_slots": int(sel.sum()),
                   "unselected_bits_untouched": bool(torch.equal(
                       wl.raw_bits(o_chk)[~sel], wl.raw_bits(wl.sentinel_like(w, dev))[~sel])),
                   "selected_finite": bool(torch.isfinite(o_chk[sel]).all())}


def config_entry(w, dev, steps, warmup, stream):
    """Per-workload summary: µs per layer call, effective KV GB/s and % of
    peak (wall time over back-to-back calls), roofline fraction from the
    per-launch event durations, planned split count, and the speedup over the
    same kernel with every head (group) active."""
    q, k, v, idx, _ = wl.make_workload(w, dev)
    ks, vs, copies = rotating_kv(w, dev, k, v)
    ns = sha.plan_nsplit(w.B, w.H, w.H_kv, w.Nkv, w.d, w.top_k, w.gqa, q.dtype)
    ms, ev = decode_timing(w, q, ks, vs, idx, ns, steps, warmup, stream)
    n_sel = w.H_kv if w.gqa else w.H
    dense_idx = torch.arange(n_sel, dtype=torch.int32, device=dev).repeat(w.B, 1)
    dn = sha.plan_nsplit(w.B, w.H, w.H_kv, w.Nkv, w.d, n_sel, w.gqa, q.dtype)
    dms, _ = decode_timing(w, q, ks, vs, dense_idx, dn, max(steps // 2, 5), max(warmup // 2, 2),
                           stream)
    _, check = output_check(w, q, k, v, idx, dev)
    ev_ms = float(np.mean(ev))
    gbs = w.active_kv_bytes / (ms / 1e3) / 1e9
    entry = {"B": w.B, "H": w.H, "H_kv": w.H_kv, "d": w.d, "Nkv": w.Nkv, "top_k": w.top_k,
             "gqa": w.gqa, "dtype": w.dtype, "index_sampling": w.sampling,
             "active_kv_bytes": w.active_kv_bytes, "nsplit": ns, "kv_copies_rotated": copies,
             "us_per_layer": round(ms * 1e3, 2), "kv_GBps": round(gbs, 1),
             "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
             "launch_avg_us": round(ev_ms * 1e3, 2),
             "roofline_frac": round(w.active_kv_bytes / (ev_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
             "all_heads_us": round(dms * 1e3, 2), "all_heads_nsplit": dn,
             "speedup_vs_all_heads": round(dms / ms, 3),
             "ideal_speedup": round(n_sel / w.top_k, 3), "check": check}
    if w.units < 64:
        entry["note"] = "launch-bound (a few KB per call): a parity case, not a bandwidth one"
    del q, k, v, ks, vs
    torch.cuda.empty_cache()
    return entry


def density_sweep(w, q, ks, vs, dev, steps, warmup, stream):
    """The same layer with top_k of the H heads active, for each top_k in
    SWEEP_TOP_K (index rows drawn like the workload's), against all heads
    active: speedup vs the ideal H / top_k (near-linear sparsity-to-speedup
    is the pages' claim for the attention kernel)."""
    pts = {}
    for k_act in SWEEP_TOP_K:
        wk = w.with_(top_k=k_act)
        idx = torch.from_numpy(wl.sample_index(wk)).to(dev)
        ns = sha.plan_nsplit(w.B, w.H, w.H_kv, w.Nkv, w.d, k_act, w.gqa, q.dtype)
        ms, ev = decode_timing(wk, q, ks, vs, idx, ns, steps, warmup, stream)
        pts[k_act] = (ms, float(np.mean(ev)), ns, wk.active_kv_bytes)
    t_all = pts[max(SWEEP_TOP_K)][0]
    n_sel = w.H_kv if w.gqa else w.H
    points = []
    for k_act, (ms, ev_ms, ns, nbytes) in pts.items():
        sp = t_all / ms
        points.append({"top_k": k_act, "density": round(k_act / n_sel, 4), "nsplit": ns,
                       "us_per_layer": round(ms * 1e3, 2),
                       "kv_GBps": round(nbytes / (ms / 1e3) / 1e9, 1),
                       "launch_avg_us": round(ev_ms * 1e3, 2),
                       "speedup_vs_all_heads": round(sp, 3),
                       "ideal_speedup": round(n_sel / k_act, 3),
                       "efficiency": round(sp * k_act / n_sel, 3)})
    return {"workload": w.name, "all_heads_top_k": max(SWEEP_TOP_K), "points": points}


ORACLE_TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 1e-2}   # max abs error, N(0, 1) inputs


def cpu_baseline(w, q, k, v, idx, budget_s: float, o_gpu=None):
    """The fp64 oracle on the host cores: whole layer calls of this workload
    (every active unit, inputs copied to host memory first), repeated until
    about budget_s of CPU work has been timed.  With o_gpu (the HIP path's
    output for the same inputs) the first pass's results are also compared
    with it slot by slot."""
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
    spent, passes, err = 0.0, 0, None
    while spent < budget_s and passes < 100:
        t0 = time.perf_counter()
        refs = [sha_units_ref(qs, ks, vs, w.scale) for qs, ks, vs in rows]
        spent += time.perf_counter() - t0
        if passes == 0 and o_gpu is not None:
            err = 0.0
            for b, ref in enumerate(refs):
                heads = [int(e) for e in idx_cpu[b]]
                hs = ([h for g in heads for h in range(g * G, g * G + G)] if w.gqa else heads)
                got = torch.stack([o_gpu[b, h, 0] for h in hs]).cpu().to(torch.float64).numpy()
                err = max(err, float(np.max(np.abs(got - ref))))
        passes += 1
    per_call = spent / passes
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count()
    return {"value": round(w.active_kv_bytes / per_call / 1e9, 4), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "us_per_layer": round(per_call * 1e6, 1), "os_cpu_count": os.cpu_count(),
            "affinity_cores": affinity, "blas_threads": threads,
            "sample": f"{passes} full layer call(s) of {w.name} ({w.units} units, "
                      f"{w.active_kv_bytes / 1e6:.0f} MB active K/V each), fp64 numpy oracle, "
                      f"{spent:.1f} s timed, {per_call * 1e6:.0f} us per layer call",
            "max_abs_err_vs_gpu": err, "tol": ORACLE_TOL[w.dtype],
            "within_tol": None if err is None else bool(err <= ORACLE_TOL[w.dtype])}


def traffic_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


def load_traffic(workload: str):
    path = traffic_path(workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_hash(wl.WORKLOADS[workload].gqa):
        return None   # counters were taken on an older kernel
    return rec.get("hbm_bytes_per_launch")


def _counter_rows(csv_path: str, counter: str):
    import csv
    with open(csv_path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") == counter:
                yield row


def summarize_traffic(args):
    """Turn rocprofv3 --pmc CSVs (FETCH_SIZE / WRITE_SIZE, KiB per dispatch)
    into HBM bytes per decode launch, each counter scaled by what it reads
    for a device copy of known size in the same kind of run."""
    w = wl.WORKLOADS[args.workload]
    kname = "sha_decode_gqa_mfma_kernel" if w.gqa else "sha_decode_mha_kernel"

    def avg(csv_path, counter, match, grid=None):
        vals = [float(r["Counter_Value"]) for r in _counter_rows(csv_path, counter)
                if match(r["Kernel_Name"]) and (grid is None or int(r["Grid_Size"]) == grid)]
        if not vals:
            raise SystemExit(f"no {counter} rows for the kernel in {csv_path}")
        return sum(vals) / len(vals), len(vals)

    grid = args.grid or None
    is_dec = lambda n: kname in n
    is_copy = lambda n: "copy" in n.lower() and "sha" not in n
    f_dec, nf = avg(args.fetch_csv, "FETCH_SIZE", is_dec, grid)
    w_dec, nw = avg(args.write_csv, "WRITE_SIZE", is_dec, grid)
    f_cp, _ = avg(args.copy_fetch_csv, "FETCH_SIZE", is_copy)
    w_cp, _ = avg(args.copy_write_csv, "WRITE_SIZE", is_copy)
    copy_bytes = float(1 << 30)
    fetch_scale = copy_bytes / (f_cp * 1024)
    write_scale = copy_bytes / (w_cp * 1024)
    read_b = f_dec * 1024 * fetch_scale
    write_b = w_dec * 1024 * write_scale
    rec = {"workload": w.name, "kernel": kname, "kernel_source_sha256_16": kernel_hash(w.gqa),
           "dispatches": {"fetch": nf, "write": nw},
           "fetch_size_kib_per_launch": f_dec, "write_size_kib_per_launch": w_dec,
           "copy_1GiB_fetch_kib": f_cp, "copy_1GiB_write_kib": w_cp,
           "fetch_scale": fetch_scale, "write_scale": write_scale,
           "hbm_read_bytes_per_launch": read_b, "hbm_write_bytes_per_launch": write_b,
           "hbm_bytes_per_launch": read_b + write_b,
           "algorithmic_bytes_per_launch": w.active_kv_bytes,
           "ratio_to_algorithmic": (read_b + write_b) / w.active_kv_bytes}
    with open(args.traffic_out or traffic_path(w.name), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def bench_mlp(args):
    """Selective MLP (device union + up/down projections) on one GPU: time per
    layer call and effective GB/s on the selected neurons' weight rows, over
    back-to-back calls from Python (the value) and as device time per call
    with the calls captured in a HIP graph (`graph`)."""
    w = wl.MLP_WORKLOADS[args.mlp]
    if args.mlp_batch:
        w = w.with_(B=args.mlp_batch)
    dev = torch.device("cuda:0")
    x, w1t, w2t, rows = wl.make_mlp(w, dev)
    copies = 2
    ws = [(w1t, w2t)]
    for c in range(1, copies):
        ws.append((torch.roll(w1t, c, 0).contiguous(), torch.roll(w2t, c, 0).contiguous()))
    stream = torch.cuda.current_stream(dev)
    sel = torch.empty(min(w.D, w.B * w.k_row), dtype=torch.int32, device=dev)
    n_sel = torch.empty(1, dtype=torch.int32, device=dev)
    n_max = sel.numel()
    wsb = sha.selective_mlp_workspace_bytes(w.B, w.d, w.D, n_max)
    work = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    uws = torch.empty(sha.lib().sha_mlp_union_workspace_bytes(w.D), dtype=torch.uint8, device=dev)
    sha.mlp_union(rows, w.D, sel=sel, n_sel=n_sel, workspace=uws)
    torch.cuda.synchronize()
    n = int(n_sel.item())

    def call(i):
        sha.mlp_union(rows, w.D, sel=sel, n_sel=n_sel, stream=stream, workspace=uws)
        a, b = ws[i % copies]
        sha.selective_mlp(x, a, b, sel, n_sel, n_max=n_max, out=y, workspace=work, stream=stream)

    ms, ev = time_calls(call, args.steps, args.warmup, stream)
    sel_all = torch.arange(w.D, dtype=torch.int32, device=dev)
    n_all = torch.tensor([w.D], dtype=torch.int32, device=dev)
    wsd = torch.empty(max(sha.selective_mlp_workspace_bytes(w.B, w.d, w.D, w.D), 1),
                      dtype=torch.uint8, device=dev)

    def dcall(i):
        a, b = ws[i % copies]
        sha.selective_mlp(x, a, b, sel_all, n_all, n_max=w.D, out=y, workspace=wsd, stream=stream)

    dms, _ = time_calls(dcall, args.steps, args.warmup, stream)
    # The same calls captured in a HIP graph (no launch gaps between the
    # union's and the MLP's kernels): device time per call.
    cur = lambda: torch.cuda.current_stream(dev)

    def gcall(i):
        sha.mlp_union(rows, w.D, sel=sel, n_sel=n_sel, stream=cur(), workspace=uws)
        a, b = ws[i % copies]
        sha.selective_mlp(x, a, b, sel, n_sel, n_max=n_max, out=y, workspace=work, stream=cur())

    def gdcall(i):
        a, b = ws[i % copies]
        sha.selective_mlp(x, a, b, sel_all, n_all, n_max=w.D, out=y, workspace=wsd, stream=cur())

    g_us = graph_us_per_call(gcall, 20, dev, 2, 5)
    gd_us = graph_us_per_call(gdcall, 20, dev, 2, 5)
    wbytes = n * w.weight_bytes_per_neuron
    out = {"metric": f"selective MLP \u00b5s/layer + effective weight GB/s, {w.name}",
           "value": round(wbytes / (ms / 1e3) / 1e9, 2), "unit": "GB/s",
           "us_per_layer": round(ms * 1e3, 2),
           "pct_hbm_peak": round(100 * wbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 2),
           "dtype": w.dtype, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "config": {"workload": w.name, "B": w.B, "d": w.d, "D": w.D, "k_row": w.k_row,
                      "union": n, "union_frac": round(n / w.D, 4), "weight_bytes": wbytes},
           "roofline": {"bound": "hbm", "achieved": round(wbytes / (float(np.mean(ev)) / 1e3) / 1e9, 2),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(wbytes / (float(np.mean(ev)) / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                        "launch_avg_us": round(float(np.mean(ev)) * 1e3, 2),
                        "note": "event span covers union + up + down (+ finalize) kernels"},
           "graph": {"us_per_layer": round(g_us, 2),
                     "weight_GBps": round(wbytes / (g_us / 1e6) / 1e9, 2),
                     "pct_hbm_peak": round(100 * wbytes / (g_us / 1e6) / 1e9 / HBM_PEAK_GBS, 2),
                     "all_neurons_us": round(gd_us, 2),
                     "speedup_selective_vs_all": round(gd_us / g_us, 3),
                     "note": "20 calls captured in a HIP graph, replayed: device time per call"},
           "all_neurons": {"us_per_layer": round(dms * 1e3, 2),
                           "GBps": round(w.D * w.weight_bytes_per_neuron / (dms / 1e3) / 1e9, 2),
                           "speedup_selective_vs_all": round(dms / ms, 3),
                           "ideal_speedup": round(w.D / max(n, 1), 3)}}
    return out


def bench_mlp_sweep(args):
    """Selective MLP speedup against the all-neurons call as the batch union
    grows: batches 1, 2, 4, ... up to the workload's B on one set of weights
    (x = the first B rows, each row's neurons the workload's seeded draw, so
    a smaller batch's rows are a prefix of a larger one's).  Per point: union
    size, µs per selective call (device union + MLP), µs per all-neurons call,
    speedup and its ideal D / |union|; wall time over back-to-back calls from
    Python, and device time per call with the same calls captured in a HIP
    graph (no host launch overhead)."""
    w = wl.MLP_WORKLOADS[args.mlp]
    dev = torch.device("cuda:0")
    x, w1t, w2t, rows = wl.make_mlp(w, dev)
    ws = [(w1t, w2t), (torch.roll(w1t, 1, 0).contiguous(), torch.roll(w2t, 1, 0).contiguous())]
    stream = torch.cuda.current_stream(dev)
    sel_all = torch.arange(w.D, dtype=torch.int32, device=dev)
    n_all = torch.tensor([w.D], dtype=torch.int32, device=dev)
    uws = torch.empty(sha.lib().sha_mlp_union_workspace_bytes(w.D), dtype=torch.uint8, device=dev)
    points = []
    B = 1
    while B <= w.B:
        xb = x[:B].contiguous()
        rb = rows[:B].contiguous()
        y = torch.empty_like(xb)
        sel = torch.empty(min(w.D, B * w.k_row), dtype=torch.int32, device=dev)
        n_sel = torch.empty(1, dtype=torch.int32, device=dev)
        work = torch.empty(max(sha.selective_mlp_workspace_bytes(B, w.d, w.D, sel.numel()), 1),
                           dtype=torch.uint8, device=dev)
        wsd = torch.empty(max(sha.selective_mlp_workspace_bytes(B, w.d, w.D, w.D), 1),
                          dtype=torch.uint8, device=dev)
        sha.mlp_union(rb, w.D, sel=sel, n_sel=n_sel, workspace=uws)
        torch.cuda.synchronize()
        n = int(n_sel.item())

        def call(i, st=None):
            st = st or stream
            sha.mlp_union(rb, w.D, sel=sel, n_sel=n_sel, stream=st, workspace=uws)
            a, b = ws[i % 2]
            sha.selective_mlp(xb, a, b, sel, n_sel, n_max=sel.numel(), out=y, workspace=work,
                              stream=st)

        def dcall(i, st=None):
            a, b = ws[i % 2]
            sha.selective_mlp(xb, a, b, sel_all, n_all, n_max=w.D, out=y, workspace=wsd,
                              stream=st or stream)

        ms, _ = time_calls(call, args.steps, args.warmup, stream)
        dms, _ = time_calls(dcall, args.steps, args.warmup, stream)
        # the same calls captured in a graph (launch overhead removed)
        ng = 20
        gs = graph_us_per_call(lambda i: call(i, torch.cuda.current_stream(dev)), ng, dev, 2, 5)
        gd = graph_us_per_call(lambda i: dcall(i, torch.cuda.current_stream(dev)), ng, dev, 2, 5)
        pt = {"B": B, "union": n, "union_frac": round(n / w.D, 4),
              "selective_us": round(ms * 1e3, 2), "all_neurons_us": round(dms * 1e3, 2),
              "speedup": round(dms / ms, 3), "ideal": round(w.D / max(n, 1), 3),
              "selective_GBps": round(n * w.weight_bytes_per_neuron / (ms / 1e3) / 1e9, 1),
              "graph_selective_us": round(gs, 2), "graph_all_neurons_us": round(gd, 2),
              "graph_speedup": round(gd / gs, 3)}
        points.append(pt)
        print(json.dumps(pt), flush=True)
        B *= 2
    out = {"metric": f"selective MLP speedup vs all neurons across batch unions, {w.name}",
           "dtype": w.dtype, "data": "synthetic: seeded N(0,1) x, N(0,1/d) / N(0,1/D) weights, "
                                     f"{w.k_row} uniform neurons per row",
           "config": {"workload": w.name, "d": w.d, "D": w.D, "k_row": w.k_row},
           "steps": args.steps, "warmup": args.warmup, "points": points}
    if args.sweep_out:
        with open(args.sweep_out, "w") as f:
            json.dump(out, f, indent=1)
    print(json.dumps(out), flush=True)


def bench_router(args):
    """Attention router of one layer on one GPU: scores = x W^T + b over the
    token's hidden state (d_model = H * d) and the per-row top-k written as the
    ascending index SHA reads.  The weights are read once per call; they are
    small (~1 MB), so the call is launch- and latency-bound.

    The headline figure is the device time per call as a decode loop captured
    in a HIP graph sees it (the pages measure with CUDA graphs): one graph of
    `copies` back-to-back calls, each on its own weight copy (>= 512 MB in all,
    so every call reads its weights from HBM), replayed and divided by the
    number of calls.  Also reported: the same with one weight matrix (warm
    caches), and call by call from Python (binding and launch overhead
    included; HIP events around each call), and with --router-floor the
    launch floor: the same graph of calls on tiny inputs (one launch, two
    launches, and this layer's grids with a 64-wide hidden state)."""
    w = wl.WORKLOADS[args.router]
    dev = torch.device("cuda:0")
    dt = wl.DTYPES[w.dtype]
    nh = w.H_kv if w.gqa else w.H
    dm = w.H * w.d
    g = torch.Generator(device=dev)
    g.manual_seed(4000)
    x = torch.randn(w.B, dm, generator=g, device=dev).to(dt)
    w0 = (torch.randn(nh, dm, generator=g, device=dev) / math.sqrt(dm)).to(dt)
    bias = torch.randn(nh, generator=g, device=dev)
    e = w0.element_size()
    wbytes = nh * dm * e
    copies = max(1, math.ceil((512 << 20) / wbytes))
    ws = [w0] + [w0.roll(c, 0).contiguous() for c in range(1, copies)]
    idx = torch.empty(w.B, w.top_k, dtype=torch.int32, device=dev)
    sc = torch.empty(w.B, nh, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    split = False if getattr(args, "router_onepass", False) else None
    need = sha.router_workspace_bytes(w.B, dm, nh, dt, split)
    rws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    kw = dict(bias=bias, index=idx, scores=sc, workspace=rws, split=split)

    def cold(i):
        sha.router_topk(x, ws[i % copies], w.top_k, stream=stream, **kw)

    def warm(i):
        sha.router_topk(x, w0, w.top_k, stream=stream, **kw)

    def graph_us(call, n):
        return graph_us_per_call(call, n, dev, max(args.warmup // 50, 2), max(args.steps // 50, 3))

    def captured(weights_of):
        # calls on the current (capturing) stream
        def call(i):
            sha.router_topk(x, weights_of(i), w.top_k, stream=torch.cuda.current_stream(dev),
                            **kw)
        return call

    g_cold = graph_us(captured(lambda i: ws[i % copies]), copies)
    g_warm = graph_us(captured(lambda i: w0), copies)

    def tiny(B, dm_, nh_, k):
        # the launch floor: the same graph of calls on a 64-wide hidden state
        xt = torch.randn(B, dm_, generator=g, device=dev).to(dt)
        wt = torch.randn(nh_, dm_, generator=g, device=dev).to(dt)
        it = torch.empty(B, k, dtype=torch.int32, device=dev) if k else None
        st = torch.empty(B, nh_, dtype=torch.float32, device=dev)

        tws = torch.empty(max(sha.router_workspace_bytes(B, dm_, nh_, dt, split), 1),
                          dtype=torch.uint8, device=dev)

        def call(i):
            sha.router_topk(xt, wt, k, index=it, scores=st, stream=torch.cuda.current_stream(dev),
                            workspace=tws, split=split)
        return round(graph_us(call, 2000), 2)

    floor = None
    if getattr(args, "router_floor", False):
        floor = {"scores_only_B1_d64_H8": tiny(1, 64, 8, 0),
                 "scores_topk_B1_d64_H8_k3": tiny(1, 64, 8, 3),
                 f"same_grid_d64_B{w.B}_H{nh}_k{w.top_k}": tiny(w.B, 64, nh, w.top_k),
                 "note": "graph device time per call of the same entry point on tiny inputs: "
                         "one launch, two launches, and this layer's grids with a 64-wide row"}
    ms, ev = time_calls(cold, args.steps, args.warmup, stream)
    wms, wev = time_calls(warm, args.steps, args.warmup, stream)
    nbytes = wbytes + w.B * dm * e + w.B * nh * 4 + w.B * w.top_k * 4
    out = {"metric": f"attention router µs/call (scores + per-row top-k, device time in a graph), {w.name}",
           "value": round(g_cold, 2), "unit": "us", "higher_is_better": False,
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "dtype": w.dtype,
           "data": "synthetic: seeded N(0,1) hidden states, N(0, 1/d_model) router weights, "
                   "N(0,1) bias",
           "config": {"workload": w.name, "B": w.B, "d_model": dm, "heads": nh, "top_k": w.top_k,
                      "gqa": w.gqa, "weight_bytes": wbytes, "weight_copies_rotated": copies,
                      "form": "k-split" if need > 0 else "one-pass"},
           "roofline": {"bound": "latency", "achieved": round(nbytes / (g_cold / 1e6) / 1e9, 2),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(nbytes / (g_cold / 1e6) / 1e9 / HBM_PEAK_GBS, 4),
                        "bytes_per_call": nbytes,
                        "note": "device time per call in a graph; at 8 TB/s the bytes alone "
                                f"would take {nbytes / HBM_PEAK_GBS / 1e3:.2f} us"},
           "warm_weights": {"graph_us_per_call": round(g_warm, 2)},
           **({"launch_floor": floor} if floor else {}),
           "call_by_call": {"cold_us_per_call": round(ms * 1e3, 2),
                            "cold_event_us": round(float(np.mean(ev)) * 1e3, 2),
                            "warm_us_per_call": round(wms * 1e3, 2),
                            "note": "Python binding + launch per call, HIP events around each call"}}
    return out


def to_pages(w, ks, vs, page, dev):
    """Move each K/V copy into a pool of `page`-row pages [num_pages, page, H_kv, d]
    placed in a seeded random page order; returns [num_pages, H_kv, page, d]
    views and the block table."""
    if w.Nkv % page:
        raise SystemExit(f"Nkv={w.Nkv} is not a multiple of the page size {page}")
    npg = w.Nkv // page
    perm = np.random.default_rng(w.seed).permutation(w.B * npg).astype(np.int32)
    bt = torch.from_numpy(perm).view(w.B, npg).to(dev)
    order = bt.view(-1).long()

    def pool(t):
        src = t.view(w.B, w.H_kv, npg, page, w.d).permute(0, 2, 3, 1, 4).reshape(-1, page, w.H_kv,
                                                                                   w.d)
        p = torch.empty_like(src)
        p[order] = src
        return p.permute(0, 2, 1, 3)

    return [pool(t) for t in ks], [pool(t) for t in vs], bt


def bench_step(args):
    """An L-layer decode step of the workload's attention shape: per layer the
    attention router (layer 0: every head, no router), the selective head
    attention and, with --step-mlp, the MLP union and selective MLP; timed
    as one HIP graph launch and as the same calls made one by one."""
    w = wl.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    dt = wl.DTYPES[w.dtype]
    n_layers = args.decode_step
    nh = w.H_kv if w.gqa else w.H
    router_d = w.H * w.d
    mw = None
    if args.step_mlp:
        mw = wl.MLP_WORKLOADS[args.step_mlp].with_(B=w.B, dtype=w.dtype)
    g = torch.Generator(device=dev)
    g.manual_seed(99)
    layers = []
    for l in range(n_layers):
        q, k, v, idx, o = wl.make_workload(w.with_(seed=w.seed + 10 * l), dev)
        L = dict(q=q, k=k, v=v, o=o, dense=(l == 0))
        if l > 0:
            L["router_x"] = torch.randn(w.B, router_d, generator=g, device=dev).to(dt)
            L["router_w"] = (torch.randn(nh, router_d, generator=g, device=dev)
                             / math.sqrt(router_d)).to(dt)
            L["router_scores"] = torch.empty(w.B, nh, device=dev)
            L["index"] = torch.empty(w.B, w.top_k, dtype=torch.int32, device=dev)
        if mw is not None:
            x, w1t, w2t, rows = wl.make_mlp(mw.with_(seed=mw.seed + l), dev)
            L.update(mlp_x=x, mlp_w1t=w1t, mlp_w2t=w2t, mlp_rows=rows, mlp_y=torch.empty_like(x))
        layers.append(L)
    kw = dict(gqa=w.gqa, scale=w.scale, router_d=router_d,
              mlp_d=mw.d if mw else 0, mlp_D=mw.D if mw else 0, mlp_k=mw.k_row if mw else 0)
    stream = torch.cuda.current_stream(dev)
    res = {}
    for mode in ("graph", "eager"):
        step = sha.DecodeStep(w.B, w.H, w.H_kv, w.Nkv, w.d, w.top_k, dt, layers,
                              use_graph=(mode == "graph"), **kw)
        ms, ev = time_calls(lambda i: step.run(stream), args.steps, args.warmup, stream)
        res[mode] = {"us_per_step": round(ms * 1e3, 2), "event_us_per_step":
                     round(float(np.mean(ev)) * 1e3, 2)}
        step.close()
    kv_bytes = w.active_kv_bytes * (n_layers - 1) + w.dense_kv_bytes
    out = {
        "metric": f"decode step of {n_layers} layers (router + SHA"
                  + (" + selective MLP" if mw else "") + ", layer 0 dense), \u00b5s per step",
        "value": res["graph"]["us_per_step"], "unit": "us", "higher_is_better": False,
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "dtype": w.dtype,
        "data": "synthetic: seeded N(0,1) q/k/v, router and MLP weights",
        "config": {"workload": w.name, "layers": n_layers, "mlp": args.step_mlp,
                   "router_d": router_d},
        "graph": res["graph"], "eager": res["eager"],
        "attention_kv_bytes_per_step": kv_bytes,
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.summarize_traffic:
        summarize_traffic(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: SHA decode units are independent and the "
              "library runs each layer call on a single MI355X; --gpus must be 1.",
              file=sys.stderr)
        sys.exit(2)
    if args.decode_step:
        bench_step(args)
        return
    if args.mlp and args.mlp_sweep:
        bench_mlp_sweep(args)
        return
    if args.mlp:
        print(json.dumps(bench_mlp(args)), flush=True)
        return
    if args.router:
        print(json.dumps(bench_router(args)), flush=True)
        return
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
    ks, vs, copies = rotating_kv(w, dev, k, v, args.copies)
    nsplit = args.nsplit or sha.plan_nsplit(w.B, w.H, w.H_kv, w.Nkv, w.d, w.top_k, w.gqa,
                                            q.dtype)
    layout = args.kv_layout
    page = int(layout[5:]) if layout.startswith("paged") else 0
    if page:
        ws_bytes = sha.workspace_bytes_paged(w.B, w.H, w.H_kv, w.Nkv, w.d, w.top_k, w.gqa, q.dtype,
                                             nsplit, page)
    else:
        ws_bytes = sha.workspace_bytes(w.B, w.H, w.H_kv, w.Nkv, w.d, w.top_k, w.gqa, q.dtype,
                                       nsplit)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    bt = None
    if layout == "bnhd":
        ks = [t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for t in ks]
        vs = [t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for t in vs]
    elif page:
        ks, vs, bt = to_pages(w, ks, vs, page, dev)
    elif layout != "contig":
        raise SystemExit(f"unknown --kv-layout {layout}")

    def call(i, index=idx, out=o):
        if page:
            sha.sha_decode_paged(q, ks[i % copies], vs[i % copies], bt, index, w.Nkv, gqa=w.gqa,
                                 scale=w.scale, out=out, nsplit=nsplit, workspace=ws, stream=stream)
        else:
            fn(q, ks[i % copies], vs[i % copies], index, scale=w.scale, out=out, nsplit=nsplit,
               workspace=ws, stream=stream)

    ms, ev = time_calls(call, args.steps, args.warmup, stream)
    ev_avg_ms = float(np.mean(ev))
    us_call = ms * 1e3
    value = w.active_kv_bytes / (ms / 1e3) / 1e9

    dense = None
    if not args.no_dense and not page:
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
    traffic = load_traffic(w.name) if layout == "contig" else None
    out = {
        "metric": METRIC if (w.name == wl.HEADLINE and layout == "contig") else
                  f"SHA decode \u00b5s/layer + effective KV GB/s (% HBM peak), {w.name}"
                  + ("" if layout == "contig" else f", {layout} KV cache"),
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
                   "nsplit": nsplit, "kv_copies_rotated": copies, "kv_layout": layout,
                   "active_kv_bytes": w.active_kv_bytes, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "sha_decode_gqa_mfma_kernel" if w.gqa else "sha_decode_mha_kernel",
                     "launch_avg_us": round(ev_avg_ms * 1e3, 2),
                     "launch_median_us": round(float(np.median(ev)) * 1e3, 2),
                     "launch_p10_us": round(float(np.percentile(ev, 10)) * 1e3, 2),
                     "launch_p90_us": round(float(np.percentile(ev, 90)) * 1e3, 2),
                     "bytes_per_launch": w.active_kv_bytes,
                     "note": ("event span covers the split kernel and the combine kernel"
                              if nsplit > 1 else "event span covers the one decode kernel")},
        "all_heads": dense,
    }
    # One more call, outside the timed region, into a fresh sentinel-filled
    # output on the first K/V copy: unselected slots must keep their bits and
    # selected ones must be finite (the oracle leg below also compares them).
    if page:
        o_chk = wl.sentinel_like(w, dev)
        call(0, out=o_chk)
        torch.cuda.synchronize()
        sel = selected_mask(w, idx.cpu().numpy()).to(dev)
        out["check"] = {"active_slots": int(sel.sum()),
                        "unselected_bits_untouched": bool(torch.equal(
                            wl.raw_bits(o_chk)[~sel], wl.raw_bits(wl.sentinel_like(w, dev))[~sel])),
                        "selected_finite": bool(torch.isfinite(o_chk[sel]).all())}
    else:
        o_chk, out["check"] = output_check(w, q, ks[0], vs[0], idx, dev)
    probe = read_probe(dev) if not args.no_probe else None
    out["read_probe"] = probe
    out["pct_of_read_probe"] = round(100 * value / probe["GBps"], 2) if probe else None
    if not args.no_cpu_baseline and layout == "contig":
        out["cpu_baseline"] = cpu_baseline(w, q, ks[0], vs[0], idx, args.cpu_seconds, o_gpu=o_chk)
    if not args.no_configs and layout == "contig" and w.name == wl.HEADLINE:
        # Each workload warms up for at least 20 calls: the headline's CPU leg
        # leaves the GPU idle for seconds just before.
        csteps, cwarm = args.steps, max(args.warmup, 20)
        sweep = density_sweep(w, q, ks, vs, dev, csteps, cwarm, stream)
        out["density_sweep"] = sweep
        if args.sweep_out:
            with open(args.sweep_out, "w") as f:
                json.dump(sweep, f, indent=1)
        entries = {w.name: {"us_per_layer": out["us_per_layer"],
                            "kv_GBps": out["value"], "pct_hbm_peak": out["pct_hbm_peak"],
                            "launch_avg_us": out["roofline"]["launch_avg_us"],
                            "roofline_frac": out["roofline"]["frac"], "nsplit": nsplit,
                            "all_heads_us": dense and round(dense["us_per_layer"], 2),
                            "speedup_vs_all_heads": dense and round(
                                dense["speedup_sparse_vs_all_heads"], 3),
                            "ideal_speedup": dense and round(dense["ideal_speedup"], 3),
                            "check": out["check"], "note": "the headline measurement above"}}
        del q, k, v, ks, vs, o_chk
        torch.cuda.empty_cache()
        for name, wc in wl.WORKLOADS.items():
            if name != w.name:
                entries[name] = config_entry(wc, dev, csteps, cwarm, stream)
        out["configs"] = {n: entries[n] for n in wl.WORKLOADS}
        if not args.no_extras:
            out["selective_mlp"], out["router"] = extras(args)
    print(json.dumps(out), flush=True)


def extras(args):
    """The other two kernel families of the sparse layer, summarised for the
    default line: the selective MLP at the two OPT MLP shapes (device union +
    up/down projections, µs and effective weight GB/s, speedup against all
    neurons) and the attention router at the four layer shapes (device time
    per call in a HIP graph, weights read from HBM).  The full records come
    from `--mlp NAME` and `--router NAME`."""
    mlp = {}
    for name in wl.MLP_WORKLOADS:
        if name.startswith("tiny"):
            continue
        r = bench_mlp(argparse.Namespace(mlp=name, mlp_batch=0, steps=args.steps,
                                         warmup=max(args.warmup, 10)))
        a = r["all_neurons"]
        mlp[name] = {"B": r["config"]["B"], "union_frac": r["config"]["union_frac"],
                     "us_per_layer": r["us_per_layer"], "weight_GBps": r["value"],
                     "pct_hbm_peak": r["pct_hbm_peak"], "all_neurons_us": a["us_per_layer"],
                     "speedup_vs_all_neurons": a["speedup_selective_vs_all"],
                     "ideal_speedup": a["ideal_speedup"],
                     "graph_us_per_layer": r["graph"]["us_per_layer"],
                     "graph_pct_hbm_peak": r["graph"]["pct_hbm_peak"],
                     "graph_speedup_vs_all_neurons": r["graph"]["speedup_selective_vs_all"]}
        torch.cuda.empty_cache()
    router = {}
    for name, w in wl.WORKLOADS.items():
        if name.startswith("tiny"):
            continue
        r = bench_router(argparse.Namespace(router=name, router_floor=False, steps=args.steps,
                                            warmup=max(args.warmup, 20)))
        router[name] = {"B": w.B, "heads": r["config"]["heads"], "top_k": w.top_k,
                        "graph_us_per_call": r["value"],
                        "graph_us_per_call_warm": r["warm_weights"]["graph_us_per_call"],
                        "python_us_per_call": r["call_by_call"]["cold_us_per_call"]}
        torch.cuda.empty_cache()
    return mlp, router


if __name__ == "__main__":
    main()
