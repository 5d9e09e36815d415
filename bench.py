#!/usr/bin/env python3
"""Benchmark of the BCQ product on one MI355X.

A step is one pass of the batch-1 hot path over one batch of synthetic input:
``bcq_gemv`` on the 4096x4096 q_proj-shaped store at p = 2, 3 and 4 (the
configuration the headline metric is quoted on).  The stores rotate over enough
distinct copies (> 512 MB) that the 256 MB Infinity Cache cannot hold them:
every call of a timed region reads its own copy (call c of a replay uses copy
c mod n, and a per-precision replay makes at least n calls, so every copy is
cycled), and a 512 MB read-modify-write of a scratch buffer runs right before
each timed replay, so no copy is cached when timing starts.

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


class Flush:
    """A buffer of twice the Infinity Cache; flush() reads all of it with the
    probe library's streaming read, so the caches end up holding its clean
    lines and nothing of the stores (a write would leave dirty lines whose
    write-back then competes with the timed reads)."""

    def __init__(self, torch):
        import ctypes

        from binary_coded_precision_amd import build as hb

        self.torch = torch
        self.lib = ctypes.CDLL(hb.PROBE_LIB)
        self.lib.bcq_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                            ctypes.c_void_p, ctypes.c_void_p]
        self.buf = torch.ones(2 * MALL_BYTES // 4, dtype=torch.int32, device="cuda")
        self.sink = torch.zeros(2 * MALL_BYTES // (4096 * 8) + 1, dtype=torch.int32, device="cuda")

    def __call__(self):
        import ctypes

        st = ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream)
        rc = self.lib.bcq_probe_read(ctypes.c_void_p(self.buf.data_ptr()), 2 * MALL_BYTES, 8,
                                     ctypes.c_void_p(self.sink.data_ptr()), st)
        if rc != 0:
            raise RuntimeError("cache flush read failed: %d" % rc)


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


def time_calls(torch, launch, n_calls: int, n_warm: int, flush=None):
    """Average duration (ms) of one launch: n_calls launches (launch(i) for
    i < n_calls) are captured into a HIP graph, replayed once untimed, then
    (after flush(), when given) timed by HIP events around one replay on the
    launch stream."""
    stream = torch.cuda.current_stream()
    for i in range(n_warm):
        launch(i)
    g = capture(torch, lambda: [launch(i) for i in range(n_calls)])
    g.replay()
    if flush is not None:
        flush()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / n_calls


def rotating_calls(torch, rot, launch, n_calls: int, n_warm: int, flush):
    """time_calls over a rotation: launch(c) reads copy c; every copy is cycled."""
    return time_calls(torch, lambda i: launch(i % rot.n), max(n_calls, rot.n), n_warm, flush)


def headline(args, bcq, torch, bcq_synth, flush):
    w = bcq_synth.config(2)
    rot = Rotation(w, ROTATE_BYTES, bcq, torch)
    M, K = w.M, w.K
    ps = (2, 3, 4)
    ys = [torch.empty(M, dtype=torch.float16, device="cuda") for _ in range(rot.n)]
    stream = torch.cuda.current_stream()

    def step(s):
        # call k of step s reads copy (3s + k) mod n: no two calls of a step
        # share a copy, and a copy is read again only n calls later
        for k, p in enumerate(ps):
            c = (len(ps) * s + k) % rot.n
            bcq.bcq_gemv(rot.stores[c], p, rot.x[c][0], ys[c])

    # The K timed steps are captured once into a HIP graph; replaying it keeps
    # the GPU queue full, so the timed region measures the kernels rather than
    # Python's launch rate.  Warmup: W eager steps, then one untimed replay
    # (the first replay uploads the graph), then the cache flush.
    graph = capture(torch, lambda: [step(s) for s in range(args.steps)])
    for s in range(args.warmup):
        step(s)
    graph.replay()
    flush()
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
        d = rotating_calls(torch, rot, lambda c, p=p: bcq.bcq_gemv(rot.stores[c], p, rot.x[c][0],
                                                                   ys[c]),
                           args.steps, args.warmup, flush)
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
        "rotation": {"copies": rot.n, "bytes": rot.bytes,
                     "headline_calls_timed": len(ps) * n_steps,
                     "per_p_calls_timed": max(args.steps, rot.n)},
        "workload": w,
    }
    return out


def floor_row(torch, flush, n):
    """Floors of one launch on this GPU, measured in the same run: an empty
    kernel, and a plain streaming read (probe kernels, not the BCQ library)
    of the 4096x4096 and 14336x4096 p = 4 call sizes, cold (distinct buffers
    over > 512 MB, flushed before the timed replay), best over grid sizes."""
    import ctypes

    from binary_coded_precision_amd import build as hb

    lib = ctypes.CDLL(hb.PROBE_LIB)
    lib.bcq_probe_empty.argtypes = [ctypes.c_void_p]
    lib.bcq_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                   ctypes.c_void_p, ctypes.c_void_p]
    st = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    row = {"empty_launch_us": round(time_calls(
        torch, lambda i: lib.bcq_probe_empty(st()), max(n, 100), 10) * 1e3, 3)}
    for nb in (algorithmic_bytes(4096, 4096, 4), algorithmic_bytes(14336, 4096, 4)):
        nb16 = -(-nb // 16) * 16
        copies = -(-ROTATE_BYTES // nb16)
        bufs = [torch.empty(nb16 // 4, dtype=torch.int32, device="cuda").fill_(c)
                for c in range(copies)]
        best = None
        sweep = {}
        for per_lane in (1, 2, 4, 8, 16):
            d = time_calls(torch, lambda i, per_lane=per_lane: lib.bcq_probe_read(
                ctypes.c_void_p(bufs[i % copies].data_ptr()), nb16, per_lane,
                ctypes.c_void_p(sink.data_ptr()), st()), max(n, copies), 10, flush)
            sweep[str(per_lane)] = round(d * 1e3, 3)
            best = d if best is None else min(best, d)
        row["read_%d_bytes" % nb] = {"us": round(best * 1e3, 3),
                                     "GBps": round(nb / (best * 1e-3) / 1e9, 1),
                                     "frac_of_peak": round(nb / (best * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                     "us_by_loads_per_lane": sweep}
        del bufs
    return row


def secondary(args, bcq, torch, bcq_synth, flush):
    """Context rows: the other configurations (not the headline value).  Rows
    over a rotation are cold like the headline; the warm-cache row and the
    low-rank correction (one buffer set) are labelled as such."""
    rows = {}
    n = max(20, args.steps // 4)
    sel = [s for s in (args.rows or "").split(",") if s]

    def want(name):
        # a row is run when a selected prefix names it (or a section holding it)
        return not sel or any(name.startswith(s) or s.startswith(name) for s in sel)

    if want("floor"):
        print("[bench] secondary floor", file=sys.stderr, flush=True)
        rows["floor"] = floor_row(torch, flush, n)

    if want('gemv_'):
        # MLP shapes at batch 1, p = 2/3/4: 14336x4096 (gate/up projection, the
        # large-shape target row) and 4096x14336 (down projection, whose K is past
        # the whole-K fp32 tables: its tables are held resident in fp16)
        for M, K, seed in ((14336, 4096, 3), (4096, 14336, 6)):
            if not want("gemv_%dx%d_b1" % (M, K)):
                continue
            print("[bench] secondary %dx%d b=1" % (M, K), file=sys.stderr, flush=True)
            w = bcq_synth.make(M, K, 4, seed=seed, name="mlp_%dx%d_b1" % (M, K))
            rot = Rotation(w, ROTATE_BYTES, bcq, torch)
            ys = [torch.empty(w.M, dtype=torch.float16, device="cuda") for _ in range(rot.n)]
            r = {}
            for p in (2, 3, 4):
                d = rotating_calls(torch, rot, lambda c, p=p: bcq.bcq_gemv(rot.stores[c], p,
                                                                           rot.x[c][0], ys[c]),
                                   n, 10, flush)
                nb = algorithmic_bytes(w.M, w.K, p)
                r[str(p)] = {"us": round(d * 1e3, 3),
                             "GBps": round(nb / (d * 1e-3) / 1e9, 1),
                             "frac_of_peak": round(nb / (d * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            rows["gemv_%dx%d_b1" % (M, K)] = r
            del rot, ys

    if want('gate_up_fused'):
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
            d = rotating_calls(torch, rot, lambda c, p=p: bcq.bcq_gemv_gate_up(rot.stores[c], p,
                                                                               rot.x[c][0], ys[c]),
                               n, 10, flush)
            nb = algorithmic_bytes(2 * Mo, 4096, p) - Mo * 2  # Mo outputs, not 2 * Mo
            r[str(p)] = {"us": round(d * 1e3, 3),
                         "GBps": round(nb / (d * 1e-3) / 1e9, 1)}
            if "gemv_14336x4096_b1" in rows:
                r[str(p)]["two_products_us"] = round(2 * rows["gemv_14336x4096_b1"][str(p)]["us"], 3)
        rows["gate_up_fused_28672x4096_b1"] = r
        del rot, ys

    if want('gate_up_batched'):
        # the same gate/up store at the MLP batches (4 and 8 requests, p = 3),
        # fused epilogue (bcq_gemm_gate_up) against the plain batched product
        # of all 28672 rows (bcq_gemm_skinny, both projections, no epilogue)
        print("[bench] secondary gate/up batched", file=sys.stderr, flush=True)
        Mo = 14336
        r = {}
        for b in (4, 8):
            w = bcq_synth.make(2 * Mo, 4096, 4, b=b, seed=9, name="gate_up_28672x4096_b%d" % b)
            rot = Rotation(w, ROTATE_BYTES, bcq, torch, with_x_rows=b)
            Yg = [torch.empty((b, Mo), dtype=torch.float16, device="cuda") for _ in range(rot.n)]
            Yp = [torch.empty((b, 2 * Mo), dtype=torch.float16, device="cuda") for _ in range(rot.n)]
            # the two calls timed alternately, best of two each (the first
            # timing after the rotation is built reads high)
            fg = lambda c: bcq.bcq_gemm_gate_up(rot.stores[c], [3] * b, rot.x[c], Yg[c])
            fp = lambda c: bcq.bcq_gemm_skinny(rot.stores[c], 3, rot.x[c], Yp[c])
            dp = dg = float("inf")
            for _ in range(2):
                dp = min(dp, rotating_calls(torch, rot, fp, n, 10, flush))
                dg = min(dg, rotating_calls(torch, rot, fg, n, 10, flush))
            nb = algorithmic_bytes(2 * Mo, 4096, 3, b) - b * Mo * 2
            r["b%d" % b] = {"us": round(dg * 1e3, 3), "GBps": round(nb / (dg * 1e-3) / 1e9, 1),
                            "product_without_epilogue_us": round(dp * 1e3, 3)}
            del rot, Yg, Yp
        rows["gate_up_batched_28672x4096_p3"] = r

    if want('qkv_concatenated'):
        # q, k and v (4096 + 1024 + 1024 rows over one 4096-wide input) as one
        # concatenated 6144-row store, next to the three separate products
        print("[bench] secondary q/k/v", file=sys.stderr, flush=True)
        r = {}
        stores = {}
        for M in (6144, 4096, 1024):
            w = bcq_synth.make(M, 4096, 4, seed=10 + M, name="qkv_%dx4096_b1" % M)
            rot = Rotation(w, ROTATE_BYTES, bcq, torch)
            ys = [torch.empty(M, dtype=torch.float16, device="cuda") for _ in range(rot.n)]
            stores[M] = {p: rotating_calls(torch, rot, lambda c, p=p: bcq.bcq_gemv(
                rot.stores[c], p, rot.x[c][0], ys[c]), n, 10, flush) for p in (2, 3, 4)}
            del rot, ys
        for p in (2, 3, 4):
            nb = algorithmic_bytes(6144, 4096, p)
            d = stores[6144][p]
            r[str(p)] = {"us": round(d * 1e3, 3), "GBps": round(nb / (d * 1e-3) / 1e9, 1),
                         "three_products_us": round((stores[4096][p] + 2 * stores[1024][p]) * 1e3, 3)}
        rows["qkv_concatenated_6144x4096_b1"] = r

    if want('lowrank_correction'):
        # binary low-rank correction y += sum_r alpha_r u_r (v_r . x) on a 4096x4096
        # output (BiLoCo's ranks 16..512); each timed call adds to the same y, so
        # its sign vectors stay cached (warm)
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
            r["rank_%d" % R] = {"us": round(d * 1e3, 3), "sign_bytes": sign_bytes, "cache": "warm"}
        rows["lowrank_correction_4096x4096_b1"] = r

    if want('gemv_lowrank'):
        # the 4096x4096 product at p = 3 with a binary low-rank correction at
        # BiLoCo's ranks, cold over a rotation (sign vectors rotated with the
        # store): bcq_gemv_lowrank (z, then the product with the correction in
        # its writeback), against the product followed by bcq_lowrank_correct
        # and against the product alone
        print("[bench] secondary product + low-rank", file=sys.stderr, flush=True)
        w = bcq_synth.config(2)
        rot = Rotation(w, ROTATE_BYTES, bcq, torch)
        ys = [torch.empty(w.M, dtype=torch.float16, device="cuda") for _ in range(rot.n)]
        r = {"product_only_us": round(rotating_calls(torch, rot, lambda c: bcq.bcq_gemv(
            rot.stores[c], 3, rot.x[c][0], ys[c]), n, 10, flush) * 1e3, 3)}
        for R in (16, 128, 512):
            lr = bcq_synth.lowrank(w.M, w.K, R, seed=R)
            u0 = torch.from_numpy(lr.u.view(np.int32)).cuda()
            v0 = torch.from_numpy(lr.v.view(np.int32)).cuda()
            u = [u0.clone() for _ in range(rot.n)]
            v = [v0.clone() for _ in range(rot.n)]
            a = torch.from_numpy(lr.alpha).cuda()
            zz = [torch.empty(R, dtype=torch.float32, device="cuda") for _ in range(rot.n)]
            fused = rotating_calls(torch, rot, lambda c: bcq.bcq_gemv_lowrank(
                rot.stores[c], 3, rot.x[c][0], u[c], v[c], a, ys[c], zz[c]), n, 10, flush)

            def separate(c):
                bcq.bcq_gemv(rot.stores[c], 3, rot.x[c][0], ys[c])
                bcq.bcq_lowrank_correct(u[c], v[c], a, rot.x[c][0], ys[c], zz[c])

            sep = rotating_calls(torch, rot, separate, n, 10, flush)
            r["rank_%d" % R] = {"fused_us": round(fused * 1e3, 3),
                                "product_then_correction_us": round(sep * 1e3, 3),
                                "sign_bytes": w.M * ((R + 31) // 32) * 4 + R * w.K // 8}
            del u, v, zz
        rows["gemv_lowrank_4096x4096_p3"] = r
        del rot, ys

    if want('dequantize'):
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
            d = rotating_calls(torch, rot, lambda c, p=p: bcq.bcq_dequantize(rot.stores[c], p,
                                                                             Wd[c % nw]),
                               n, 10, flush)
            nb = algorithmic_bytes(w.M, w.K, p, b=0) + w.M * w.K * 2  # planes + scales read, W written
            r[str(p)] = {"us": round(d * 1e3, 3), "GBps": round(nb / (d * 1e-3) / 1e9, 1),
                         "frac_of_peak": round(nb / (d * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        rows["dequantize_4096x4096"] = r
        del rot, Wd

    if want('prefill_routes'):
        # prefill through the dense route (bcq_dequantize, then fp16 F.linear on
        # hipBLASLt) against the matrix-core kernels at the largest batch they take,
        # and at a batch past it; 4096x4096, p = 4
        print("[bench] secondary prefill routes", file=sys.stderr, flush=True)
        nw = ROTATE_BYTES // (4096 * 4096 * 2) + 1
        Wd = [torch.empty((4096, 4096), dtype=torch.float16, device="cuda") for _ in range(nw)]
        r = {}
        for b in (256, 1024):
            w = bcq_synth.make(4096, 4096, 4, b=b, seed=7)
            rot = Rotation(w, ROTATE_BYTES, bcq, torch, with_x_rows=b)
            Y = [torch.empty((b, w.M), dtype=torch.float16, device="cuda") for _ in range(rot.n)]

            def dense(c):
                bcq.bcq_dequantize(rot.stores[c], 4, Wd[c % nw])
                torch.mm(rot.x[c], Wd[c % nw].t(), out=Y[c])

            row = {"dequant_then_gemm_us": round(rotating_calls(torch, rot, dense, n, 10, flush)
                                                 * 1e3, 3),
                   "gemm_only_us": round(rotating_calls(torch, rot, lambda c: torch.mm(
                       rot.x[c], Wd[c % nw].t(), out=Y[c]), n, 10, flush) * 1e3, 3)}
            if b <= bcq.BCQ_MAX_BATCH:
                ws = bcq.new_workspace(rot.stores[0], b)
                row["bcq_matrix_cores_us"] = round(rotating_calls(torch, rot, lambda c: bcq.bcq_gemm_skinny(
                    rot.stores[c], 4, rot.x[c], Y[c], workspace=ws), n, 10, flush) * 1e3, 3)
                del ws
            r["b%d" % b] = row
            del rot, Y
        rows["prefill_routes_4096x4096_p4"] = r
        del Wd

    if want('gemv_4096x4096_b1_warm_cache'):
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

    if want('mixed_p'):
        # per-request precision, 8 requests on 4096x4096 vs the same call at uniform p = max
        w = bcq_synth.config(4)
        rot = Rotation(w, ROTATE_BYTES, bcq, torch, with_x_rows=w.b)
        Y = [torch.empty((w.b, w.M), dtype=torch.float16, device="cuda") for _ in range(rot.n)]
        pr = [int(p) for p in w.p_req]
        ws = bcq.new_workspace(rot.stores[0], w.b)
        d_mixed = rotating_calls(torch, rot, lambda c: bcq.bcq_gemv_mixed_p(
            rot.stores[c], pr, rot.x[c], Y[c], workspace=ws), n, 10, flush)
        d_uni = rotating_calls(torch, rot, lambda c: bcq.bcq_gemm_skinny(
            rot.stores[c], max(pr), rot.x[c], Y[c], workspace=ws), n, 10, flush)
        nb = mixed_bytes(w.M, w.K, pr)
        rows["mixed_p_4096x4096_b8"] = {
            "p_req": pr,
            "us": round(d_mixed * 1e3, 3),
            "uniform_pmax_us": round(d_uni * 1e3, 3),
            "GBps": round(nb / (d_mixed * 1e-3) / 1e9, 1),
        }
        del rot, Y, ws

    if want('quantize'):
        # the offline quantizer on one 4096x4096 fp16 weight matrix: 20
        # refinement rounds at 2 planes, then expansion to 4 (fp16 tables)
        print("[bench] secondary quantize", file=sys.stderr, flush=True)
        W = torch.from_numpy(bcq_synth.weights(4096, 4096, seed=44)).cuda()
        bcq.bcq_quantize(W, 4, 2, 20)
        torch.cuda.synchronize()
        d = time_calls(torch, lambda i: bcq.bcq_quantize(W, 4, 2, 20), 5, 1)
        rows["quantize_4096x4096_P4_from2_20rounds"] = {
            "us": round(d * 1e3, 1), "weights_per_s": round(4096 * 4096 / (d * 1e-3), 0)}
        del W

    if want('skinny'):
        # small batches (MLP shapes, p = 3) and matrix-core batches (p = 4).  The
        # batches of 2..15 are timed on both routes (BCQ_FORCE_PATH=lut: vector-ALU
        # tables; =mfma: matrix cores); "us" is the default route's time.
        for (M, K), b, p in [((4096, 4096), 2, 4), ((4096, 4096), 4, 4), ((4096, 4096), 8, 4),
                             ((14336, 4096), 4, 3), ((14336, 4096), 8, 3), ((4096, 14336), 4, 3),
                             ((4096, 14336), 8, 3),
                             ((4096, 4096), 16, 4), ((4096, 4096), 32, 4), ((4096, 4096), 64, 4),
                             ((14336, 4096), 64, 4)]:
            if not want("skinny_%dx%d_b%d_p%d" % (M, K, b, p)):
                continue
            print("[bench] secondary %dx%d b=%d p=%d" % (M, K, b, p), file=sys.stderr, flush=True)
            w = bcq_synth.make(M, K, 4, b=b, seed=5)
            rot = Rotation(w, ROTATE_BYTES, bcq, torch, with_x_rows=b)
            Y = [torch.empty((b, M), dtype=torch.float16, device="cuda") for _ in range(rot.n)]
            nb = algorithmic_bytes(M, K, p, b)
            row = {}
            for route in ((None, "lut", "mfma") if b < 16 else (None,)):
                with force_path(route):
                    ws = bcq.new_workspace(rot.stores[0], b)  # None where the call needs none
                    d = rotating_calls(torch, rot, lambda c: bcq.bcq_gemm_skinny(
                        rot.stores[c], p, rot.x[c], Y[c], workspace=ws), n, 10, flush)
                    del ws
                t = d * 1e-3
                key = "us" if route is None else "us_" + route
                row[key] = round(t * 1e6, 3)
                if route is None:
                    row["GBps"] = round(nb / t / 1e9, 1)
                    if b >= 16:
                        row["mfma_util"] = round(2.0 * M * K * b / t / 2.5e15, 4)
            rows["skinny_%dx%d_b%d_p%d" % (M, K, b, p)] = row
            del rot, Y

    return rows


class force_path:
    """Sets BCQ_FORCE_PATH for the duration of a with-block (None: unset)."""

    def __init__(self, route):
        self.route = route

    def __enter__(self):
        self.old = os.environ.pop("BCQ_FORCE_PATH", None)
        if self.route is not None:
            os.environ["BCQ_FORCE_PATH"] = self.route

    def __exit__(self, *exc):
        os.environ.pop("BCQ_FORCE_PATH", None)
        if self.old is not None:
            os.environ["BCQ_FORCE_PATH"] = self.old


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_s: float):
    """The float64 oracle as it stands, on full 4096x4096 calls at p = 2, 3, 4:
    single-threaded, then row-partitioned over the host's cores (one thread per
    core, each calling the unchanged oracle on its rows; ctypes releases the
    interpreter lock during the call).  The headline figure is the all-core
    leg; the single-thread one is reported beside it."""
    import concurrent.futures as cf

    import oracle

    oracle.gemv(w.signs, w.alpha, w.zero, w.x[0], 2)  # load / build outside the timing

    def run(call, seconds):
        t0 = time.perf_counter()
        reps, nbytes = 0, 0
        while True:
            for p in (2, 3, 4):
                call(p)
                nbytes += algorithmic_bytes(w.M, w.K, p)
            reps += 1
            if time.perf_counter() - t0 >= seconds:
                break
        return reps, nbytes, time.perf_counter() - t0

    reps1, b1, t1 = run(lambda p: oracle.gemv(w.signs, w.alpha, w.zero, w.x[0], p), budget_s / 2)
    # at most 16 threads: the core share of one GPU's job on the measured host, whatever
    # os.cpu_count() reports
    nthreads = max(1, min(16, os.cpu_count() or 1))
    bounds = np.linspace(0, w.M, nthreads + 1).astype(int)
    parts = [(np.ascontiguousarray(w.signs[:, lo:hi]), np.ascontiguousarray(w.alpha[:, lo:hi]),
              np.ascontiguousarray(w.zero[lo:hi])) for lo, hi in zip(bounds[:-1], bounds[1:])]
    x0 = w.x[0]
    with cf.ThreadPoolExecutor(max_workers=nthreads) as ex:
        def all_cores(p):
            list(ex.map(lambda part: oracle.gemv(part[0], part[1], part[2], x0, p), parts))
        all_cores(2)
        repsn, bn, tn = run(all_cores, budget_s / 2)
    return {"value": round(bn / tn / 1e9, 4), "unit": "GB/s", "cores": nthreads, "kind": "oracle",
            "sample": "%d full steps (bcq_gemv 4096x4096 at p=2,3,4) in %.1f s, float64 C loops, "
                      "rows split over %d threads; single thread: %d steps in %.1f s = %.4f GB/s"
                      % (repsn, tn, nthreads, reps1, t1, b1 / t1 / 1e9),
            "single_thread_value": round(b1 / t1 / 1e9, 4),
            "nproc": os.cpu_count(), "cpu_model": cpu_model()}


def trace_dispatches(path: str):
    """(dispatch id, kernel name, grid, duration in us) of every kernel
    dispatch in a rocprofv3 kernel trace: a rocpd SQLite database (.db, the
    default output) or a kernel-trace CSV."""
    seq = []
    if path.endswith(".db"):
        import sqlite3

        con = sqlite3.connect(path)
        for did, name, gx, gy, start, end in con.execute(
                "select dispatch_id, name, grid_x, grid_y, start, end from kernels"):
            seq.append((int(did), name, "%dx%d" % (gx, gy), (int(end) - int(start)) * 1e-3))
        con.close()
    else:
        import csv

        rows = list(csv.DictReader(open(path, newline="")))
        grid_keys = [k for k in ("Grid_Size", "Grid_Size_X") if rows and k in rows[0]]
        for r in rows:
            grid = r[grid_keys[0]] if grid_keys else "?"
            t = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
            seq.append((int(r.get("Dispatch_Id", len(seq))), r["Kernel_Name"], grid, t))
    seq.sort()
    return seq


def trace_summary(path: str, last: int, run_index: int = 2) -> None:
    """Per-kernel duration statistics from a rocprofv3 kernel trace (see
    trace_dispatches): for each (kernel, grid) with at least 10 dispatches,
    count, mean, median, p10 and p90 in microseconds over all its dispatches,
    and over the last `last` dispatches of its `run_index`-th run (counting
    from 1) of at least `last` consecutive dispatches, else of its last such
    run, else of its longest run.  In a bench run a kernel's first timing
    makes two such runs, the eager pass with the untimed replay, then (after
    the cache flush) the timed replay: run 2 is that timed replay, and later
    rows may reuse the same kernel."""
    seq = trace_dispatches(path)

    def stats(v):
        v = np.sort(np.asarray(v))
        return {"n": int(v.size), "mean": round(float(v.mean()), 3),
                "median": round(float(np.median(v)), 3),
                "p10": round(float(np.percentile(v, 10)), 3),
                "p90": round(float(np.percentile(v, 90)), 3)}

    groups = {}
    runs = {}  # every run of consecutive dispatches of one (kernel, grid), in order
    prev, cur = None, []
    for _, name, grid, t in seq + [(None, None, None, None)]:
        k = (name, grid)
        if k != prev and prev is not None:
            runs.setdefault(prev, []).append(cur)
            cur = []
        if name is None:
            break
        groups.setdefault(k, []).append(t)
        cur.append(t)
        prev = k

    def timed_run(k):
        rs = runs.get(k, [])
        full = [r for r in rs if len(r) >= last]
        if len(full) >= run_index >= 1:
            return full[run_index - 1]
        return full[-1] if full else max(rs, key=len, default=[])

    for k, v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        if len(v) < 10:
            continue
        out = {"kernel": k[0][:160], "grid": k[1], "all": stats(v)}
        run = timed_run(k)
        if len(run) >= 10:
            out["longest_run_last"] = stats(run[-last:])
        print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--rows", default="",
                    help="comma-separated name prefixes of the secondary rows to run "
                         "(default: all), e.g. floor,gemv_,skinny_14336")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (for HBM counter calibration)")
    ap.add_argument("--counter-run", type=int, default=0, metavar="N",
                    help="only run N cold eager calls of the batch-1 kernel at each of p=2,3,4 "
                         "on the 4096x4096 store (for per-dispatch HBM counters)")
    ap.add_argument("--counter-batch", type=int, default=1, metavar="B",
                    help="with --counter-run: run bcq_gemm_skinny at batch B (p = 4) instead")
    ap.add_argument("--counter-shape", default="4096x4096", metavar="MxK",
                    help="with --counter-run: the store's shape")
    ap.add_argument("--counter-p", default="", metavar="P[,P..]",
                    help="with --counter-run: precisions (default 2,3,4 at batch 1, else 4)")
    ap.add_argument("--trace-summary", metavar="CSV",
                    help="only summarise a rocprofv3 kernel-trace CSV (no GPU needed)")
    ap.add_argument("--trace-run", type=int, default=2,
                    help="with --trace-summary: which run (from 1) of at least --trace-last "
                         "consecutive dispatches to take (default 2: a kernel's first timed "
                         "replay in a bench run)")
    ap.add_argument("--trace-last", type=int, default=58,
                    help="with --trace-summary: dispatches taken from the end of each "
                         "kernel's longest run")
    args = ap.parse_args()
    if args.trace_summary:
        trace_summary(args.trace_summary, args.trace_last, args.trace_run)
        return
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
        Mc, Kc = (int(v) for v in args.counter_shape.split("x"))
        if b == 1 and (Mc, Kc) == (4096, 4096):
            w = bcq_synth.config(2)
        else:
            w = bcq_synth.make(Mc, Kc, 4, b=b, seed=2)
        rot = Rotation(w, ROTATE_BYTES, bcq, torch, with_x_rows=b)
        ys = [torch.empty((b, w.M), dtype=torch.float16, device="cuda") for _ in range(rot.n)]
        ws = bcq.new_workspace(rot.stores[0], b) if b > 1 else None
        plist = ([int(v) for v in args.counter_p.split(",")] if args.counter_p
                 else ([2, 3, 4] if b == 1 else [4]))
        for p in plist:
            for i in range(args.counter_run):
                c = i % rot.n
                if b == 1:
                    bcq.bcq_gemv(rot.stores[c], p, rot.x[c][0], ys[c][0])
                else:
                    bcq.bcq_gemm_skinny(rot.stores[c], p, rot.x[c], ys[c], workspace=ws)
        torch.cuda.synchronize()
        print(json.dumps({"counter_run_calls_per_p": args.counter_run, "batch": b,
                          "shape": [w.M, w.K], "p": plist, "copies": rot.n,
                          "route": os.environ.get("BCQ_FORCE_PATH", "default")}))
        return

    flush = Flush(torch)
    print("[bench] headline", file=sys.stderr, flush=True)
    h = headline(args, bcq, torch, bcq_synth, flush)
    w = h.pop("workload")
    sec = None
    if not args.no_secondary:
        print("[bench] secondary", file=sys.stderr, flush=True)
        sec = secondary(args, bcq, torch, bcq_synth, flush)
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
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "bcq_gemv q_proj-shaped 4096x4096, batch 1, one 4-plane store at "
                        "p=2,3,4 per step, fp16 scales/activations/outputs, fp32 accumulation, "
                        "g=128, 1% outlier channels x20",
            "M": 4096, "K": 4096, "b": 1, "p": [2, 3, 4], "planes_stored": 4,
            "rotating_copies": h["rotation"]["copies"],
            "rotating_bytes": h["rotation"]["bytes"],
            "headline_calls_timed": h["rotation"]["headline_calls_timed"],
            "per_p_calls_timed": h["rotation"]["per_p_calls_timed"],
            "cache_flush_bytes": 2 * MALL_BYTES,
        },
        "per_p": h["per_p"],
        "roofline": h["roofline"],
        "cpu_baseline": cpu,
        "secondary": sec,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
