"""Host-side logic of bench.py: the byte accounting behind every GB/s figure, the
gate that ties stored HBM counter readings to a kernel source, and the one-GPU
contract.  No GPU needed."""

import os
import subprocess
import sys

import pytest

import bench

MiB = 1 << 20
KiB = 1 << 10


# Byte counts of a stored product at batch 1: one bit per sign per plane, one
# fp16 scale per (plane, row, group of 128) and one fp16 offset per (row, group),
# fp16 activations and outputs.
@pytest.mark.parametrize("M,K,planes,alpha,zero,x,y", [
    # 4096x4096: planes 4 / 6 / 8 MiB, scales 0.5 / 0.75 / 1 MiB, offsets 0.25 MiB
    (4096, 4096, {2: 4 * MiB, 3: 6 * MiB, 4: 8 * MiB},
     {2: MiB // 2, 3: 3 * MiB // 4, 4: MiB}, MiB // 4, 8 * KiB, 8 * KiB),
    # 14336x4096: planes 14 / 21 / 28 MiB, scales 1.75 / 2.625 / 3.5 MiB, offsets 0.875 MiB
    (14336, 4096, {2: 14 * MiB, 3: 21 * MiB, 4: 28 * MiB},
     {2: 7 * MiB // 4, 3: 21 * MiB // 8, 4: 7 * MiB // 2}, 7 * MiB // 8, 8 * KiB, 28 * KiB),
])
def test_algorithmic_bytes_counts_each_stream_once(M, K, planes, alpha, zero, x, y):
    for p in (2, 3, 4):
        assert bench.algorithmic_bytes(M, K, p) == planes[p] + alpha[p] + zero + x + y


def test_headline_step_bytes():
    # the 4096x4096 step at p = 2, 3, 4 moves 4,997,120 + 7,356,416 + 9,715,712 bytes
    assert [bench.algorithmic_bytes(4096, 4096, p) for p in (2, 3, 4)] == [
        4997120, 7356416, 9715712]


def test_batch_adds_only_activations_and_outputs():
    one = bench.algorithmic_bytes(4096, 14336, 3)
    eight = bench.algorithmic_bytes(4096, 14336, 3, b=8)
    assert eight - one == 7 * (14336 * 2 + 4096 * 2)


def test_mixed_precision_reads_planes_up_to_the_largest_once():
    p_req = [2, 3, 3, 4, 2, 4, 4, 3]
    assert bench.mixed_bytes(4096, 4096, p_req) == bench.algorithmic_bytes(4096, 4096, 4, b=8)
    assert bench.mixed_bytes(4096, 4096, [2, 2]) == bench.algorithmic_bytes(4096, 4096, 2, b=2)


def test_stored_traffic_only_for_the_source_it_was_taken_on(monkeypatch):
    path = os.path.join(bench.ROOT, "profiles", "gemv_lut_qproj_4096x4096_traffic.txt")
    kv = dict(line.split(":", 1) for line in open(path)
              if ":" in line and not line.startswith("#"))
    sha = kv["source_sha"].strip()
    monkeypatch.setattr(bench, "source_sha", lambda: sha)
    assert bench.stored_traffic() == float(kv["hbm_bytes_per_launch"])
    monkeypatch.setattr(bench, "source_sha", lambda: "0" * 16)
    assert bench.stored_traffic() is None


def test_source_sha_is_a_stable_hash_of_the_kernel_file():
    assert bench.source_sha() == bench.source_sha()
    assert len(bench.source_sha()) == 16 and int(bench.source_sha(), 16) >= 0


def test_code_hash_ignores_comments_and_layout_only():
    src = "int f(int a) {\n  return a + 1;  // one more\n}\n"
    assert bench.code_hash(src) == bench.code_hash("/* doc */ int f(int a) { return a + 1; }")
    assert bench.code_hash(src) != bench.code_hash("int f(int a) { return a + 2; }")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_trace_summary_statistics(tmp_path, capsys):
    """--trace-summary: per (kernel, grid) statistics over all dispatches and
    over the last N of the longest consecutive run, from a kernel-trace CSV."""
    import json

    path = tmp_path / "kernel_trace.csv"
    lines = ["Dispatch_Id,Kernel_Name,Grid_Size,Start_Timestamp,End_Timestamp"]
    d = 0
    # an interleaved stretch (runs of one), then a run of 20 of kernel A
    for i in range(12):
        for name, dur in (("A", 5000), ("B", 7000)):
            d += 1
            lines.append("%d,%s,256,%d,%d" % (d, name, 1000 * d, 1000 * d + dur))
    for i in range(20):
        d += 1
        lines.append("%d,A,256,%d,%d" % (d, 1000 * d, 1000 * d + 3000 + 100 * i))
    path.write_text("\n".join(lines) + "\n")
    bench.trace_summary(str(path), 10)
    rows = [json.loads(l) for l in capsys.readouterr().out.splitlines()]
    a = next(r for r in rows if r["kernel"] == "A")
    assert a["all"]["n"] == 32
    last = a["longest_run_last"]
    assert last["n"] == 10
    # the last ten of the run: 4.0 .. 4.9 us
    assert abs(last["median"] - 4.45) < 1e-9 and abs(last["mean"] - 4.45) < 1e-9
    b = next(r for r in rows if r["kernel"] == "B")
    assert b["all"]["n"] == 12 and b["all"]["median"] == 7.0
    assert "longest_run_last" not in b  # its longest run is one dispatch


def test_trace_summary_takes_the_requested_run(tmp_path, capsys):
    """The n-th run of at least `last` dispatches: in a bench run, the eager
    pass with the untimed replay, then the timed replay, then a later row that
    reuses the kernel."""
    import json

    path = tmp_path / "kernel_trace.csv"
    lines = ["Dispatch_Id,Kernel_Name,Grid_Size,Start_Timestamp,End_Timestamp"]
    d = 0
    for dur, n in ((9000, 20), (5000, 10), (7000, 10)):  # runs of A, split by B
        for _ in range(n):
            d += 1
            lines.append("%d,A,256,%d,%d" % (d, 1000 * d, 1000 * d + dur))
        d += 1
        lines.append("%d,B,256,%d,%d" % (d, 1000 * d, 1000 * d + 1000))
    path.write_text("\n".join(lines) + "\n")
    for run, want in ((1, 9.0), (2, 5.0), (3, 7.0), (4, 7.0)):
        bench.trace_summary(str(path), 10, run)
        rows = [json.loads(l) for l in capsys.readouterr().out.splitlines()]
        a = next(r for r in rows if r["kernel"] == "A")
        assert a["longest_run_last"]["median"] == want, run

