#!/usr/bin/env python3
"""Benchmark of the BCQ product on one MI355X.

A step is one pass of the batch-1 hot path over one batch of synthetic input:
``bcq_gemv`` on the 4096x4096 q_proj-shaped store at p = 2, 3 and 4 (the
configuration the headline metric is quoted on).  The stores rotate over enough
distinct copies (> 512 MB) that the 256 MB Infinity Cache cannot hold them, so
every call reads its planes from HBM.

Printed: one JSON line with the headline value (GB/s of algorithmic bytes over
the timed region), a roofline object for the batch-1 kernel (per-launch HIP
event durations on the launch stream), the float64 CPU oracle timed on a
bounded sample, and secondary rows (14336x4096 at batch 1, per-request
precision, small batches, matrix-core batches) for context.

Algorithmic bytes of one call:
    p*M*K/8 (planes) + p*M*G*s (scales) + M*G*s (offsets) + b*K*s (x) + b*M*s (y)
with G = K/128 and s the element size; nothing else is counted.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "BCQ GEMV µs/call and HBM GB/s (% of peak), 4096x4096 b=1 at p=2/3/4"
HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20
ROTATE_BYTES = 2 * MALL_BYTES + (16 << 20)


def algorithmic_bytes(M: int, K: int, p: int, b: int = 1, elem: int = 2, g: int = 128) -> int:
    """Bytes a BCQ product must move: planes, scales, offsets, activations, outputs."""
    G = K // g
    return p * M * K // 8 + p * M * G * elem + M * G * elem + b * K * elem + b * M * elem


def mixed_bytes(M: int, K: int, p_req, elem: int = 2, g: int = 128) -> int:
    """Per-request precision with one shared scale table: planes and scales up to
    the largest precision are read once for the batch."""
    G = K // g
    pmax = max(p_req)
    b = len(p_req)
    return pmax * M * K // 8 + pmax * M * G * elem + M * G * elem + b * K * elem + b * M * elem


def source_sha() -> str:
    """Hash of the batch-1 kernel source (ties stored counter readings to a kernel version)."""
    path = os.path.join(ROOT, "binary_coded_precision_amd", "csrc", "gemv_lut.hip")
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def stored_traffic():
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they
    were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "gemv_lut_qproj_4096x4096_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha") != source_sha():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Rotation:
    """Distinct device copies of one store (and its x/y buffers), used round-robin."""

    def __init__(self, w, min_bytes: int, bcq, torch, with_x_rows: int = 1):
        base = bcq.Store.from_host(w.signs, w.alpha, w.zero)
        per = base.bits.numel() * 4 + sum(t.numel() * t.element_size() for t in
                                          (base.alpha[1], base.zero[1]))
        self.n = max(2, -(-min_bytes // per))
        self.stores = [base]
        for _ in range(self.n - 1):
            bits = base.bits.clone()
            a = base.alpha[1].clone()
            z = base.zero[1].clone()
            at = {p: a for p in base.alpha}
            zt = {p: z for p in base.zero}
            self.stores.append(bcq.Store(base.M, base.K, base.planes, bits, at, zt))
        x = torch.from_numpy(np.ascontiguousarray(w.x[:with_x_rows])).cuda()
        self.x = [x.clone() for _ in range(self.n)]
        self.bytes = per * self.n


def time_calls(torch, launch, n_calls: int, n_warm: int):
    """Per-launch durations (ms) from event pairs on the launch stream, plus the
    wall time of the whole region (ms)."""
    stream = torch.cuda.current_stream()
    for i in range(n_warm):
        launch(i)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_calls)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n_calls)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(n_calls):
        starts[i].record(stream)
        launch(i)
        ends[i].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    d = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    return d, t0.elapsed_time(t1)


def headline(args, bcq, torch, bcq_synth):
    w = bcq_synth.config(2)
    rot = Rotation(w, ROTATE_BYTES, bcq, torch)
    M, K = w.M, w.K
    ps = (2, 3, 4)
    ys = [torch.empty(M, dtype=torch.float16, device="cuda") for _ in range(rot.n)]
    stream = torch.cuda.current_stream()

    def step(s):
        c = s % rot.n
        for p in ps:
            bcq.bcq_gemv(rot.stores[c], p, rot.x[c][0], ys[c])

    # warmup, then the timed region: exactly K steps between two synchronisations
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for s in range(args.steps):
        step(args.warmup + s)
    e1.record(stream)
    torch.cuda.synchronize()
    region_ms = e0.elapsed_time(e1)
    step_bytes = sum(algorithmic_bytes(M, K, p) for p in ps)
    value = step_bytes * args.steps / (region_ms * 1e-3) / 1e9

    # per-launch durations for the roofline (same launches, events around each)
    per_p = {}
    all_d, all_b = [], []
    for p in ps:
        d, _ = time_calls(torch, lambda i, p=p: bcq.bcq_gemv(rot.stores[i % rot.n], p,
                                                              rot.x[i % rot.n][0],
                                                              ys[i % rot.n]),
                          args.steps, args.warmup)
        nb = algorithmic_bytes(M, K, p)
        per_p[str(p)] = {
            "us_per_call_median": round(float(np.median(d)) * 1e3, 3),
            "us_p10": round(float(np.percentile(d, 10)) * 1e3, 3),
            "us_p90": round(float(np.percentile(d, 90)) * 1e3, 3),
            "bytes": nb,
            "GBps": round(nb / (float(np.median(d)) * 1e-3) / 1e9, 1),
            "frac_of_peak": round(nb / (float(np.median(d)) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        }
        all_d.append(d)
        all_b.append(nb)
    mean_dur_s = float(np.mean(np.concatenate(all_d))) * 1e-3
    mean_bytes = float(np.mean(all_b))
    achieved = mean_bytes / mean_dur_s / 1e9
    traffic = stored_traffic()

    # warm-cache context: one store, repeated
    warm = {}
    for p in ps:
        d, _ = time_calls(torch, lambda i, p=p: bcq.bcq_gemv(rot.stores[0], p, rot.x[0][0], ys[0]),
                          args.steps, args.warmup)
        warm[str(p)] = round(float(np.median(d)) * 1e3, 3)

    out = {
        "value": round(value, 1),
        "ms_per_step": round(region_ms / args.steps, 6),
        "per_p": per_p,
        "warm_cache_us_median": warm,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "gemv_lut_kernel<half,2>",
            "bytes_per_launch_mean": mean_bytes,
            "launch_us_mean": round(mean_dur_s * 1e6, 3),
        },
        "rotation": {"copies": rot.n, "bytes": rot.bytes},
        "workload": w,
    }
    return out


def secondary(args, bcq, torch, bcq_synth):
    """Context rows: the other configurations (not the headline value)."""
    rows = {}
    n = max(20, args.steps // 4)

    # 14336x4096 at batch 1, p = 2/3/4 (the large-shape target row)
    w = bcq_synth.make(14336, 4096, 4, seed=3, name="gateup_14336x4096_b1")
    rot = Rotation(w, ROTATE_BYTES, bcq, torch)
    ys = [torch.empty(w.M, dtype=torch.float16, device="cuda") for _ in range(rot.n)]
    r = {}
    for p in (2, 3, 4):
        d, _ = time_calls(torch, lambda i, p=p: bcq.bcq_gemv(rot.stores[i % rot.n], p,
                                                              rot.x[i % rot.n][0], ys[i % rot.n]),
                          n, 10)
        nb = algorithmic_bytes(w.M, w.K, p)
        r[str(p)] = {"us": round(float(np.median(d)) * 1e3, 3),
                     "GBps": round(nb / (float(np.median(d)) * 1e-3) / 1e9, 1),
                     "frac_of_peak": round(nb / (float(np.median(d)) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    rows["gemv_14336x4096_b1"] = r
    del rot, ys

    # per-request precision, 8 requests on 4096x4096 vs the same call at uniform p = max
    w = bcq_synth.config(4)
    rot = Rotation(w, ROTATE_BYTES, bcq, torch, with_x_rows=w.b)
    Y = [torch.empty((w.b, w.M), dtype=torch.float16, device="cuda") for _ in range(rot.n)]
    pr = [int(p) for p in w.p_req]
    d_mixed, _ = time_calls(torch, lambda i: bcq.bcq_gemv_mixed_p(rot.stores[i % rot.n], pr,
                                                                 rot.x[i % rot.n], Y[i % rot.n]),
                            n, 10)
    d_uni, _ = time_calls(torch, lambda i: bcq.bcq_gemm_skinny(rot.stores[i % rot.n], max(pr),
                                                              rot.x[i % rot.n], Y[i % rot.n]),
                          n, 10)
    nb = mixed_bytes(w.M, w.K, pr)
    rows["mixed_p_4096x4096_b8"] = {
        "p_req": pr,
        "us": round(float(np.median(d_mixed)) * 1e3, 3),
        "uniform_pmax_us": round(float(np.median(d_uni)) * 1e3, 3),
        "GBps": round(nb / (float(np.median(d_mixed)) * 1e-3) / 1e9, 1),
    }
    del rot, Y

    # small batches (MLP shapes, p = 3) and matrix-core batches (p = 4)
    for (M, K), b, p in [((14336, 4096), 4, 3), ((14336, 4096), 8, 3), ((4096, 14336), 8, 3),
                         ((4096, 4096), 16, 4), ((4096, 4096), 32, 4), ((4096, 4096), 64, 4),
                         ((14336, 4096), 64, 4)]:
        w = bcq_synth.make(M, K, 4, b=b, seed=5)
        rot = Rotation(w, ROTATE_BYTES, bcq, torch, with_x_rows=b)
        Y = [torch.empty((b, M), dtype=torch.float16, device="cuda") for _ in range(rot.n)]
        wsb = bcq.bcq_workspace_bytes(rot.stores[0], b)
        ws = torch.empty(max(wsb // 4, 1), dtype=torch.float32, device="cuda")
        d, _ = time_calls(torch, lambda i: bcq.bcq_gemm_skinny(rot.stores[i % rot.n], p,
                                                              rot.x[i % rot.n], Y[i % rot.n],
                                                              workspace=ws), n, 10)
        t = float(np.median(d)) * 1e-3
        nb = algorithmic_bytes(M, K, p, b)
        row = {"us": round(t * 1e6, 3), "GBps": round(nb / t / 1e9, 1)}
        if b >= 16:
            row["mfma_util"] = round(2.0 * M * K * b / t / 2.5e15, 4)
        rows["skinny_%dx%d_b%d_p%d" % (M, K, b, p)] = row
        del rot, Y, ws
    return rows


def cpu_baseline(w, budget_s: float):
    """The float64 oracle as it stands, single-threaded, on full 4096x4096 calls."""
    import oracle

    oracle.gemv(w.signs, w.alpha, w.zero, w.x[0], 2)  # load / build outside the timing
    t0 = time.perf_counter()
    reps, nbytes = 0, 0
    while True:
        for p in (2, 3, 4):
            oracle.gemv(w.signs, w.alpha, w.zero, w.x[0], p)
            nbytes += algorithmic_bytes(w.M, w.K, p)
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "%d full steps (bcq_gemv 4096x4096 at p=2,3,4), %.1f s, float64 C loops, "
                      "1 thread" % (reps, dt)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (for HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build's path runs on a single MI355X "
              "(multi-GPU sharding is a design note, not built); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import bcq_synth
    import binary_coded_precision_amd as bcq

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    bcq.load(build_if_missing=True)

    if args.copy_calibration:
        src = torch.empty(64 << 20, dtype=torch.int32, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": src.numel() * 4, "copies": 5}))
        return

    print("[bench] headline", file=sys.stderr, flush=True)
    h = headline(args, bcq, torch, bcq_synth)
    w = h.pop("workload")
    sec = None
    if not args.no_secondary:
        print("[bench] secondary", file=sys.stderr, flush=True)
        sec = secondary(args, bcq, torch, bcq_synth)
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, args.cpu_seconds)
    line = {
        "metric": METRIC,
        "value": h["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "bcq_gemv q_proj-shaped 4096x4096, batch 1, one 4-plane store at "
                        "p=2,3,4 per step, fp16 scales/activations/outputs, fp32 accumulation, "
                        "g=128, 1% outlier channels x20",
            "M": 4096, "K": 4096, "b": 1, "p": [2, 3, 4], "planes_stored": 4,
            "rotating_copies": h["rotation"]["copies"],
            "rotating_bytes": h["rotation"]["bytes"],
        },
        "per_p": h["per_p"],
        "warm_cache_us_median": h["warm_cache_us_median"],
        "roofline": h["roofline"],
        "cpu_baseline": cpu,
        "secondary": sec,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
