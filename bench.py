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
bounded sample, and secondary rows (MLP shapes at batch 1, per-request
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


def code_hash(text: str) -> str:
    """Hash of C/HIP source with comments and whitespace removed."""
    import re

    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()[:16]


def source_sha() -> str:
    """Code hash of the batch-1 kernel source (ties stored counter readings to a
    kernel version; comment edits keep it)."""
    path = os.path.join(ROOT, "binary_coded_precision_amd", "csrc", "gemv_lut.hip")
    return code_hash(open(path, encoding="utf-8").read())


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


def capture(torch, body):
    """Capture the launches made by body() into a HIP graph (on a side stream,
    as torch requires) and return it."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        body()  # one eager pass first: nothing is allocated during capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        body()
    torch.cuda.synchronize()
    return g


def time_calls(torch, launch, n_calls: int, n_warm: int):
    """Average duration (ms) of one launch: n_calls launches (launch(i) for
    i < n_calls) are captured into a HIP graph, replayed once untimed, then
    timed by HIP events around one replay on the launch stream."""
    stream = torch.cuda.current_stream()
    for i in range(n_warm):
        launch(i)
    g = capture(torch, lambda: [launch(i) for i in range(n_calls)])
    g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / n_calls


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

    # The K timed steps are captured once into a HIP graph (step s uses copy
    # s mod n); replaying it keeps the GPU queue full, so the timed region
    # measures the kernels rather than Python's launch rate.  Warmup: W eager
    # steps, then one untimed replay (the first replay uploads the graph).
    graph = capture(torch, lambda: [step(s) for s in range(args.steps)])
    for s in range(args.warmup):
        step(s)
    graph.replay()
    torch.cuda.synchronize()
    n_steps = args.steps
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    region_ms = e0.elapsed_time(e1)
    step_bytes = sum(algorithmic_bytes(M, K, p) for p in ps)
    value = step_bytes * n_steps / (region_ms * 1e-3) / 1e9

    # per-precision launch durations (graphs of launches at one precision); the
    # roofline object reports the p = 4 kernel, the longest of the three
    per_p = {}
    dur = {}
    for p in ps:
        d = time_calls(torch, lambda i, p=p: bcq.bcq_gemv(rot.stores[i % rot.n], p,
                                                          rot.x[i % rot.n][0], ys[i % rot.n]),
                       args.steps, args.warmup)
        nb = algorithmic_bytes(M, K, p)
        dur[p] = d
        per_p[str(p)] = {
            "us_per_call": round(d * 1e3, 3),
            "bytes": nb,
            "GBps": round(nb / (d * 1e-3) / 1e9, 1),
            "frac_of_peak": round(nb / (d * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        }
    achieved = algorithmic_bytes(M, K, 4) / (dur[4] * 1e-3) / 1e9
    traffic = stored_traffic()

    out = {
        "value": round(value, 1),
        "steps_timed": n_steps,
        "ms_per_step": round(region_ms / n_steps, 6),
        "per_p": per_p,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "bcq_gemv batch-1 kernel at p=4 (4096x4096, fp16)",
            "bytes_per_launch": algorithmic_bytes(M, K, 4),
            "launch_us": round(dur[4] * 1e3, 3),
        },
        "rotation": {"copies": rot.n, "bytes": rot.bytes},
        "workload": w,
    }
    return out


def secondary(args, bcq, torch, bcq_synth):
    """Context rows: the other configurations (not the headline value)."""
    rows = {}
    n = max(20, args.steps // 4)

    # MLP shapes at batch 1, p = 2/3/4: 14336x4096 (gate/up projection, the
    # large-shape target row) and 4096x14336 (down projection, whose K exceeds
    # what one workgroup keeps resident, so its tables stream through LDS)
    for M, K, seed in ((14336, 4096, 3), (4096, 14336, 6)):
        print("[bench] secondary %dx%d b=1" % (M, K), file=sys.stderr, flush=True)
        w = bcq_synth.make(M, K, 4, seed=seed, name="mlp_%dx%d_b1" % (M, K))
        rot = Rotation(w, ROTATE_BYTES, bcq, torch)
        ys = [torch.empty(w.M, dtype=torch.float16, device="cuda") for _ in range(rot.n)]
        r = {}
        for p in (2, 3, 4):
            d = time_calls(torch, lambda i, p=p: bcq.bcq_gemv(rot.stores[i % rot.n], p,
                                                              rot.x[i % rot.n][0], ys[i % rot.n]),
                           n, 10)
            nb = algorithmic_bytes(w.M, w.K, p)
            r[str(p)] = {"us": round(d * 1e3, 3),
                         "GBps": round(nb / (d * 1e-3) / 1e9, 1),
                         "frac_of_peak": round(nb / (d * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        rows["gemv_%dx%d_b1" % (M, K)] = r
        del rot, ys

    # the MLP's gate and up projections as one gate/up store (2 x 14336 rows,
    # bcq_gemv_gate_up) with the silu(gate) * up epilogue in the same launch,
    # next to the two separate 14336x4096 products timed above (which would
    # still need the epilogue as a third kernel)
    print("[bench] secondary gate/up", file=sys.stderr, flush=True)
    Mo = 14336
    w = bcq_synth.make(2 * Mo, 4096, 4, seed=9, name="gate_up_28672x4096_b1")
    rot = Rotation(w, ROTATE_BYTES, bcq, torch)
    ys = [torch.empty(Mo, dtype=torch.float16, device="cuda") for _ in range(rot.n)]
    r = {}
    for p in (2, 3, 4):
        d = time_calls(torch, lambda i, p=p: bcq.bcq_gemv_gate_up(rot.stores[i % rot.n], p,
                                                                  rot.x[i % rot.n][0],
                                                                  ys[i % rot.n]),
                       n, 10)
        nb = algorithmic_bytes(2 * Mo, 4096, p) - Mo * 2  # Mo outputs, not 2 * Mo
        r[str(p)] = {"us": round(d * 1e3, 3),
                     "GBps": round(nb / (d * 1e-3) / 1e9, 1),
                     "two_products_us": round(2 * rows["gemv_14336x4096_b1"][str(p)]["us"], 3)}
    rows["gate_up_fused_28672x4096_b1"] = r
    del rot, ys

    # q, k and v (4096 + 1024 + 1024 rows over one 4096-wide input) as one
    # concatenated 6144-row store, next to the three separate products
    print("[bench] secondary q/k/v", file=sys.stderr, flush=True)
    r = {}
    stores = {}
    for M in (6144, 4096, 1024):
        w = bcq_synth.make(M, 4096, 4, seed=10 + M, name="qkv_%dx4096_b1" % M)
        rot = Rotation(w, ROTATE_BYTES, bcq, torch)
        ys = [torch.empty(M, dtype=torch.float16, device="cuda") for _ in range(rot.n)]
        stores[M] = {p: time_calls(torch, lambda i, p=p: bcq.bcq_gemv(rot.stores[i % rot.n], p,
                                                                     rot.x[i % rot.n][0],
                                                                     ys[i % rot.n]), n, 10)
                     for p in (2, 3, 4)}
        del rot, ys
    for p in (2, 3, 4):
        nb = algorithmic_bytes(6144, 4096, p)
        d = stores[6144][p]
        r[str(p)] = {"us": round(d * 1e3, 3), "GBps": round(nb / (d * 1e-3) / 1e9, 1),
                     "three_products_us": round((stores[4096][p] + 2 * stores[1024][p]) * 1e3, 3)}
    rows["qkv_concatenated_6144x4096_b1"] = r

    # binary low-rank correction y += sum_r alpha_r u_r (v_r . x) on a 4096x4096
    # output (BiLoCo's ranks 16..512); each timed call adds to the same y
    print("[bench] secondary low-rank", file=sys.stderr, flush=True)
    r = {}
    for R in (16, 128, 512):
        lr = bcq_synth.lowrank(4096, 4096, R, seed=R)
        u = torch.from_numpy(lr.u.view(np.int32)).cuda()
        v = torch.from_numpy(lr.v.view(np.int32)).cuda()
        a = torch.from_numpy(lr.alpha).cuda()
        xx = torch.from_numpy(lr.x).cuda()
        yy = torch.from_numpy(lr.y0).cuda()
        zz = torch.empty(R, dtype=torch.float32, device="cuda")
        d = time_calls(torch, lambda i: bcq.bcq_lowrank_correct(u, v, a, xx, yy, zz), n, 10)
        sign_bytes = 4096 * ((R + 31) // 32) * 4 + R * 4096 // 8
        r["rank_%d" % R] = {"us": round(d * 1e3, 3), "sign_bytes": sign_bytes}
    rows["lowrank_correction_4096x4096_b1"] = r

    # dense reconstruction export (bcq_dequantize) of the 4096x4096 store, the
    # route for batches past the matrix-core kernels: an HBM stream that reads
    # the planes and scales and writes M x K fp16
    print("[bench] secondary dequantize", file=sys.stderr, flush=True)
    w = bcq_synth.config(2)
    rot = Rotation(w, ROTATE_BYTES, bcq, torch)
    # distinct outputs, more of them together than the Infinity Cache holds
    nw = ROTATE_BYTES // (w.M * w.K * 2) + 1
    Wd = [torch.empty((w.M, w.K), dtype=torch.float16, device="cuda") for _ in range(nw)]
    r = {}
    for p in (2, 3, 4):
        d = time_calls(torch, lambda i, p=p: bcq.bcq_dequantize(rot.stores[i % rot.n], p,
                                                                Wd[i % nw]), n, 10)
        nb = algorithmic_bytes(w.M, w.K, p, b=0) + w.M * w.K * 2  # planes + scales read, W written
        r[str(p)] = {"us": round(d * 1e3, 3), "GBps": round(nb / (d * 1e-3) / 1e9, 1),
                     "frac_of_peak": round(nb / (d * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    rows["dequantize_4096x4096"] = r
    del rot

    # prefill through the dense route (bcq_dequantize, then fp16 F.linear on
    # hipBLASLt) against the matrix-core kernels at the largest batch they take,
    # and at a batch past it; 4096x4096, p = 4
    print("[bench] secondary prefill routes", file=sys.stderr, flush=True)
    F = torch.nn.functional
    r = {}
    for b in (256, 1024):
        w = bcq_synth.make(4096, 4096, 4, b=b, seed=7)
        rot = Rotation(w, ROTATE_BYTES, bcq, torch, with_x_rows=b)
        Y = [torch.empty((b, w.M), dtype=torch.float16, device="cuda") for _ in range(rot.n)]

        def dense(i):
            bcq.bcq_dequantize(rot.stores[i % rot.n], 4, Wd[i % nw])
            torch.mm(rot.x[i % rot.n], Wd[i % nw].t(), out=Y[i % rot.n])

        row = {"dequant_then_gemm_us": round(time_calls(torch, dense, n, 10) * 1e3, 3),
               "gemm_only_us": round(time_calls(torch, lambda i: torch.mm(
                   rot.x[i % rot.n], Wd[i % nw].t(), out=Y[i % rot.n]), n, 10) * 1e3, 3)}
        if b <= bcq.BCQ_MAX_BATCH:
            ws = bcq.new_workspace(rot.stores[0], b)
            row["bcq_matrix_cores_us"] = round(time_calls(torch, lambda i: bcq.bcq_gemm_skinny(
                rot.stores[i % rot.n], 4, rot.x[i % rot.n], Y[i % rot.n], workspace=ws), n, 10) * 1e3, 3)
            del ws
        r["b%d" % b] = row
        del rot, Y
    rows["prefill_routes_4096x4096_p4"] = r
    del Wd

    # 4096x4096 at batch 1 with one store repeated (planes served from the
    # Infinity Cache after the first call): context for the cold numbers
    w = bcq_synth.config(2)
    st = bcq.Store.from_host(w.signs, w.alpha, w.zero)
    x = torch.from_numpy(np.ascontiguousarray(w.x[0])).cuda()
    y = torch.empty(w.M, dtype=torch.float16, device="cuda")
    rows["gemv_4096x4096_b1_warm_cache_us"] = {
        str(p): round(time_calls(torch, lambda i, p=p: bcq.bcq_gemv(st, p, x, y), n, 10) * 1e3, 3)
        for p in (2, 3, 4)}
    del st, x, y

    # per-request precision, 8 requests on 4096x4096 vs the same call at uniform p = max
    w = bcq_synth.config(4)
    rot = Rotation(w, ROTATE_BYTES, bcq, torch, with_x_rows=w.b)
    Y = [torch.empty((w.b, w.M), dtype=torch.float16, device="cuda") for _ in range(rot.n)]
    pr = [int(p) for p in w.p_req]
    ws = bcq.new_workspace(rot.stores[0], w.b)
    d_mixed = time_calls(torch, lambda i: bcq.bcq_gemv_mixed_p(rot.stores[i % rot.n], pr,
                                                              rot.x[i % rot.n], Y[i % rot.n],
                                                              workspace=ws),
                         n, 10)
    d_uni = time_calls(torch, lambda i: bcq.bcq_gemm_skinny(rot.stores[i % rot.n], max(pr),
                                                           rot.x[i % rot.n], Y[i % rot.n],
                                                           workspace=ws),
                       n, 10)
    nb = mixed_bytes(w.M, w.K, pr)
    rows["mixed_p_4096x4096_b8"] = {
        "p_req": pr,
        "us": round(d_mixed * 1e3, 3),
        "uniform_pmax_us": round(d_uni * 1e3, 3),
        "GBps": round(nb / (d_mixed * 1e-3) / 1e9, 1),
    }
    del rot, Y, ws

    # small batches (MLP shapes, p = 3) and matrix-core batches (p = 4)
    for (M, K), b, p in [((4096, 4096), 2, 4), ((4096, 4096), 4, 4), ((4096, 4096), 8, 4),
                         ((14336, 4096), 4, 3), ((14336, 4096), 8, 3), ((4096, 14336), 4, 3),
                         ((4096, 14336), 8, 3),
                         ((4096, 4096), 16, 4), ((4096, 4096), 32, 4), ((4096, 4096), 64, 4),
                         ((14336, 4096), 64, 4)]:
        print("[bench] secondary %dx%d b=%d p=%d" % (M, K, b, p), file=sys.stderr, flush=True)
        w = bcq_synth.make(M, K, 4, b=b, seed=5)
        rot = Rotation(w, ROTATE_BYTES, bcq, torch, with_x_rows=b)
        Y = [torch.empty((b, M), dtype=torch.float16, device="cuda") for _ in range(rot.n)]
        ws = bcq.new_workspace(rot.stores[0], b)  # None where the call needs none
        d = time_calls(torch, lambda i: bcq.bcq_gemm_skinny(rot.stores[i % rot.n], p,
                                                           rot.x[i % rot.n], Y[i % rot.n],
                                                           workspace=ws), n, 10)
        t = d * 1e-3
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
    ap.add_argument("--counter-run", type=int, default=0, metavar="N",
                    help="only run N cold eager calls of the batch-1 kernel at each of p=2,3,4 "
                         "on the 4096x4096 store (for per-dispatch HBM counters)")
    ap.add_argument("--counter-batch", type=int, default=1, metavar="B",
                    help="with --counter-run: run bcq_gemm_skinny at batch B (p = 4) instead")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the BCQ product runs on a single MI355X "
              "(sharding across GPUs is not implemented); use --gpus 1", file=sys.stderr)
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

    if args.counter_run:
        b = args.counter_batch
        w = bcq_synth.make(4096, 4096, 4, b=b, seed=2) if b > 1 else bcq_synth.config(2)
        rot = Rotation(w, ROTATE_BYTES, bcq, torch, with_x_rows=b)
        ys = [torch.empty((b, w.M), dtype=torch.float16, device="cuda") for _ in range(rot.n)]
        ws = bcq.new_workspace(rot.stores[0], b) if b > 1 else None
        for p in ((2, 3, 4) if b == 1 else (4,)):
            for i in range(args.counter_run):
                c = i % rot.n
                if b == 1:
                    bcq.bcq_gemv(rot.stores[c], p, rot.x[c][0], ys[c][0])
                else:
                    bcq.bcq_gemm_skinny(rot.stores[c], p, rot.x[c], ys[c], workspace=ws)
        torch.cuda.synchronize()
        print(json.dumps({"counter_run_calls_per_p": args.counter_run, "batch": b,
                          "copies": rot.n}))
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
        "steps": h["steps_timed"],
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
        "roofline": h["roofline"],
        "cpu_baseline": cpu,
        "secondary": sec,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
