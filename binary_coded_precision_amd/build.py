"""Build ``libbcq.so`` (the C-ABI library) for gfx950 with hipcc, in-tree.

Objects go to ``binary_coded_precision_amd/_build/``; the shared library lands
next to this file.  ``python -m binary_coded_precision_amd.build`` rebuilds it.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libbcq.so")
SOURCES = ["bcq_api.hip", "pack.hip", "gemv_lut.hip", "gemm_mfma.hip", "lowrank.hip", "dequant.hip",
           "quantize.hip"]
# Per-file flags: the quantizer takes its sign decisions on exactly rounded
# fp64 values, so no multiply-add there is fused into one rounding.
FILE_FLAGS = {"quantize.hip": ["-ffp-contract=off"]}
# Measurement kernels of the benchmark's floor row (empty launch, plain
# streaming read): a library of their own, outside the BCQ ABI.
PROBE_LIB = os.path.join(HERE, "libbcq_probe.so")
PROBE_SOURCES = ["probe.hip"]
ARCH = "gfx950"

# Packed-fp32 VALU forms are kept out of every kernel: hipcc would otherwise
# fuse plain float code into v_pk_* fp32 instructions.
COMMON_FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the BCQ library needs ROCm's hipcc to build")
    return path


def _compile(src: str, extra) -> str:
    obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
    cmd = ([hipcc()] + COMMON_FLAGS + FILE_FLAGS.get(src, []) + list(extra) +
           ["-c", os.path.join(CSRC, src), "-o", obj])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def _link(lib: str, objs) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + list(objs)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, lib)


def build(extra_flags=(), verbose: bool = False) -> str:
    """Compile every source, link ``libbcq.so`` (and the benchmark's
    ``libbcq_probe.so``); returns the BCQ library's path."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, extra_flags), srcs)))
    _link(LIB, [objs[s] for s in SOURCES])
    _link(PROBE_LIB, [objs[s] for s in PROBE_SOURCES])
    if verbose:
        print("built", LIB, "and", PROBE_LIB)
    return LIB


# Host-side checking build: the library's host code instrumented with
# AddressSanitizer and UndefinedBehaviorSanitizer (each flag after -Xarch_host,
# so the GPU code is compiled as usual), and a driver that calls every entry
# point's argument validation (tests/host_sanitize/validate.cpp).  Used by
# tests/test_host_sanitizers.py on the CPU; nothing in it runs a kernel.
SANITIZE_DIR = os.path.join(OBJ_DIR, "host_sanitize")
SANITIZE_HOST = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                 "-Xarch_host -fno-sanitize-recover=undefined "
                 "-Xarch_host -fno-omit-frame-pointer").split()


def build_host_sanitized(driver_src: str) -> str:
    """Build the sanitized library and the validation driver; returns the
    driver's path.  Rebuilds only when a source is newer than the driver."""
    os.makedirs(SANITIZE_DIR, exist_ok=True)
    exe = os.path.join(SANITIZE_DIR, "validate")
    srcs = [os.path.join(CSRC, s) for s in SOURCES] + [driver_src]
    headers = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    headers.append(os.path.join(os.path.dirname(HERE), "include", "bcq.h"))
    if os.path.exists(exe) and all(os.path.getmtime(f) < os.path.getmtime(exe)
                                   for f in srcs + headers):
        return exe

    def comp(src):
        obj = os.path.join(SANITIZE_DIR, os.path.splitext(src)[0] + ".o")
        cmd = ([hipcc()] + COMMON_FLAGS + FILE_FLAGS.get(src, []) + SANITIZE_HOST +
               ["-c", os.path.join(CSRC, src), "-o", obj])
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(comp, SOURCES))
    lib = os.path.join(SANITIZE_DIR, "libbcq_host_sanitize.so")
    cmd = ([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC"] + SANITIZE_HOST[:4] +
           ["-o", lib] + objs)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang++")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang++"
    cmd = ([clang, "-O1", "-std=c++17", "-D__HIP_PLATFORM_AMD__",
            "-I", os.path.join(os.path.dirname(HERE), "include"), "-I", "/opt/rocm/include"] +
           SANITIZE_HOST + [driver_src, lib, "-Wl,-rpath," + SANITIZE_DIR,
                            "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("driver build failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    return exe


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
