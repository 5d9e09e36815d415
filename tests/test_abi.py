"""The C-ABI library loads, exports every symbol include/bcq.h declares, and
rejects invalid arguments on the host before any HIP call (no GPU needed:
every call below fails validation, so nothing is launched)."""

import ctypes
import os
import re

import pytest

import binary_coded_precision_amd as bcq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bcq.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bcq_[a-z_]+)\s*\(", text)))


def test_header_declares_the_expected_entry_points():
    assert declared_functions() == sorted(bcq.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = bcq.load()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5):
        s = bcq.bcq_status_string(code)
        assert s.startswith("BCQ_")
    assert "unknown" in bcq.bcq_status_string(7)


def test_packed_bytes():
    # P planes x 16-row tiles x K/8 bytes per row
    assert bcq.bcq_packed_bytes(4, 4096, 4096) == 4 * 4096 * 512
    assert bcq.bcq_packed_bytes(2, 256, 512) == 2 * 256 * 64
    assert bcq.bcq_packed_bytes(3, 17, 128) == 3 * 32 * 16  # ragged rows pad to a full tile
    assert bcq.bcq_packed_bytes(4, 14336, 4096) // 4 == 14336 * 4096 // 8  # one plane
    for bad in [(0, 16, 128), (5, 16, 128), (1, 0, 128), (1, 16, 0), (1, 16, 100), (1, 16, 96)]:
        assert bcq.bcq_packed_bytes(*bad) == 0


# ---------------------------------------------------------------- validation

FAKE = 0x100000  # aligned, never dereferenced (validation fails before any launch)


def make_store(M=64, K=256, planes=4, dtype=bcq.BCQ_F16, bits=FAKE, group=128, tables=True):
    st = bcq._Store()
    st.M, st.K, st.group_size, st.planes = M, K, group, planes
    st.bits = bits
    st.scale_dtype = dtype
    for p in range(1, 5):
        st.alpha[p] = FAKE if tables else None
        st.zero[p] = FAKE if tables else None
    return st


def gemv(st, p=2, x=FAKE, y=FAKE, xdt=bcq.BCQ_F16, ydt=bcq.BCQ_F16):
    ref = None if st is None else ctypes.byref(st)
    return bcq.load().bcq_gemv(ref, p, x, xdt, y, ydt, None)


def gate_up(st, p=2, x=FAKE, y=FAKE, xdt=bcq.BCQ_F16, ydt=bcq.BCQ_F16):
    ref = None if st is None else ctypes.byref(st)
    return bcq.load().bcq_gemv_gate_up(ref, p, x, xdt, y, ydt, None)


def dequant(st, p=2, W=FAKE, ldw=None, dt=bcq.BCQ_F16):
    ref = None if st is None else ctypes.byref(st)
    ldw = (st.K if st is not None else 256) if ldw is None else ldw
    return bcq.load().bcq_dequantize(ref, p, W, ldw, dt, None)


def lowrank(u=FAKE, v=FAKE, a=FAKE, R=16, M=64, K=256, x=FAKE, y=FAKE, dt=bcq.BCQ_F16, z=FAKE):
    return bcq.load().bcq_lowrank_correct(u, v, a, R, M, K, x, y, dt, z, None)


def gemv_lr(st, p=2, x=FAKE, u=FAKE, v=FAKE, a=FAKE, R=16, y=FAKE, z=FAKE, xdt=bcq.BCQ_F16,
            ydt=bcq.BCQ_F16):
    ref = None if st is None else ctypes.byref(st)
    return bcq.load().bcq_gemv_lowrank(ref, p, x, xdt, u, v, a, R, y, ydt, z, None)


def skinny(st, p=2, X=FAKE, b=4, ldx=None, Y=FAKE, ldy=None, dt=bcq.BCQ_F16, ws=None, wsb=0):
    ldx = st.K if ldx is None else ldx
    ldy = st.M if ldy is None else ldy
    return bcq.load().bcq_gemm_skinny(ctypes.byref(st), p, X, b, ldx, dt, Y, ldy, dt, ws, wsb,
                                      None)


def mixed(st, ps, X=FAKE, ldx=None, Y=FAKE, ldy=None, dt=bcq.BCQ_F16, ws=None, wsb=0):
    ldx = st.K if ldx is None else ldx
    ldy = st.M if ldy is None else ldy
    arr = (ctypes.c_int32 * len(ps))(*ps)
    return bcq.load().bcq_gemv_mixed_p(ctypes.byref(st), arr, X, len(ps), ldx, dt, Y, ldy, dt,
                                       ws, wsb, None)


E_ARG, E_UNS, E_ALN = bcq.BCQ_ERR_INVALID_ARG, bcq.BCQ_ERR_UNSUPPORTED, bcq.BCQ_ERR_ALIGNMENT


@pytest.mark.parametrize("case,expect", [
    (lambda: gemv(None), E_ARG),
    (lambda: gemv(make_store(bits=0)), E_ARG),
    (lambda: gemv(make_store(group=64)), E_UNS),
    (lambda: gemv(make_store(K=100)), E_ARG),
    (lambda: gemv(make_store(K=192)), E_ARG),
    (lambda: gemv(make_store(M=0)), E_ARG),
    (lambda: gemv(make_store(planes=0)), E_ARG),
    (lambda: gemv(make_store(planes=5)), E_ARG),
    (lambda: gemv(make_store(), p=0), E_ARG),
    (lambda: gemv(make_store(planes=2), p=3), E_ARG),
    (lambda: gemv(make_store(tables=False)), E_ARG),
    (lambda: gemv(make_store(), x=0), E_ARG),
    (lambda: gemv(make_store(), y=0), E_ARG),
    (lambda: gemv(make_store(bits=FAKE + 4)), E_ALN),
    (lambda: gemv(make_store(), x=FAKE + 8), E_ALN),
    (lambda: gemv(make_store(), y=FAKE + 1), E_ALN),
    (lambda: gemv(make_store(), xdt=bcq.BCQ_F32), E_UNS),
    (lambda: gemv(make_store(), ydt=bcq.BCQ_F32), E_UNS),
    (lambda: gemv(make_store(), xdt=3), E_ARG),
    (lambda: gemv(make_store(dtype=9)), E_ARG),
    (lambda: gate_up(None), E_ARG),
    (lambda: gate_up(make_store(M=24)), E_ARG),  # gate/up stores have whole 16-row tiles
    (lambda: gate_up(make_store(M=40)), E_ARG),
    (lambda: gate_up(make_store(), p=5), E_ARG),
    (lambda: gate_up(make_store(), x=0), E_ARG),
    (lambda: gate_up(make_store(), y=FAKE + 1), E_ALN),
    (lambda: gate_up(make_store(), xdt=bcq.BCQ_F32), E_UNS),
    (lambda: dequant(None), E_ARG),
    (lambda: dequant(make_store(), p=5), E_ARG),
    (lambda: dequant(make_store(), W=0), E_ARG),
    (lambda: dequant(make_store(), ldw=255), E_ARG),
    (lambda: dequant(make_store(), W=FAKE + 8), E_ALN),
    (lambda: dequant(make_store(), ldw=260), E_ALN),  # 520-byte rows
    (lambda: dequant(make_store(), dt=bcq.BCQ_F32), E_UNS),
    (lambda: lowrank(R=0), E_ARG),
    (lambda: lowrank(R=4097), E_ARG),
    (lambda: lowrank(M=0), E_ARG),
    (lambda: lowrank(K=48), E_ARG),  # K must be whole 32-column words
    (lambda: lowrank(dt=3), E_ARG),
    (lambda: lowrank(z=0), E_ARG),
    (lambda: lowrank(u=0), E_ARG),
    (lambda: lowrank(u=FAKE + 2), E_ALN),
    (lambda: lowrank(z=FAKE + 2), E_ALN),
    (lambda: lowrank(y=FAKE + 1), E_ALN),
    (lambda: lowrank(x=FAKE + 8), E_ALN),
    (lambda: gemv_lr(None), E_ARG),
    (lambda: gemv_lr(make_store(), p=5), E_ARG),
    (lambda: gemv_lr(make_store(K=192)), E_ARG),
    (lambda: gemv_lr(make_store(), R=0), E_ARG),
    (lambda: gemv_lr(make_store(), R=4097), E_ARG),
    (lambda: gemv_lr(make_store(), u=0), E_ARG),
    (lambda: gemv_lr(make_store(), v=0), E_ARG),
    (lambda: gemv_lr(make_store(), a=0), E_ARG),
    (lambda: gemv_lr(make_store(), z=0), E_ARG),
    (lambda: gemv_lr(make_store(), y=0), E_ARG),
    (lambda: gemv_lr(make_store(), xdt=bcq.BCQ_F32), E_UNS),
    (lambda: gemv_lr(make_store(), x=FAKE + 8), E_ALN),
    (lambda: gemv_lr(make_store(), y=FAKE + 1), E_ALN),
    (lambda: gemv_lr(make_store(), u=FAKE + 2), E_ALN),
    (lambda: gemv_lr(make_store(), v=FAKE + 2), E_ALN),
    (lambda: gemv_lr(make_store(), z=FAKE + 2), E_ALN),
    (lambda: gemv_lr(make_store(), a=FAKE + 1), E_ALN),
    (lambda: gemv_lr(make_store(dtype=bcq.BCQ_F32), a=FAKE + 2, xdt=bcq.BCQ_F32,
                     ydt=bcq.BCQ_F32), E_ALN),
    (lambda: skinny(make_store(), b=0), E_ARG),
    (lambda: skinny(make_store(), b=257), E_ARG),
    (lambda: skinny(make_store(), ldx=255), E_ARG),
    (lambda: skinny(make_store(), ldy=63), E_ARG),
    (lambda: skinny(make_store(), ldx=260), E_ALN),  # 260 halves = 520 B, not a multiple of 16
    (lambda: skinny(make_store(), X=FAKE + 2), E_ALN),
    (lambda: skinny(make_store(), p=5), E_ARG),
    # K split over workgroups needs a workspace: K past 4096, or more than 16
    # requests in a launch
    (lambda: skinny(make_store(M=1024, K=8192), b=16), E_ARG),
    (lambda: skinny(make_store(M=1024, K=8192), b=16, ws=FAKE, wsb=16), E_ARG),
    (lambda: skinny(make_store(M=1024, K=8192), b=3), E_ARG),  # fp16 b >= 3: matrix cores
    (lambda: skinny(make_store(M=4096, K=4096), b=32), E_ARG),
    (lambda: mixed(make_store(M=1024, K=8192), [2, 3, 4]), E_ARG),  # needs a workspace too
    (lambda: mixed(make_store(M=4096, K=4096), [2, 3, 4] * 6), E_ARG),
    (lambda: mixed(make_store(), [2, 3, 0, 4]), E_ARG),
    (lambda: mixed(make_store(), [2, 3, 5, 4]), E_ARG),
    (lambda: mixed(make_store(planes=3), [2, 3, 4]), E_ARG),
    (lambda: mixed(make_store(), []), E_ARG),
    (lambda: mixed(make_store(), [2, 3], X=0), E_ARG),
])
def test_validation_rejects_before_launch(case, expect):
    assert case() == expect


def test_null_precision_array_rejected():
    st = make_store()
    r = bcq.load().bcq_gemv_mixed_p(ctypes.byref(st), None, FAKE, 2, st.K, bcq.BCQ_F16, FAKE,
                                    st.M, bcq.BCQ_F16, None, 0, None)
    assert r == E_ARG


def test_pack_validation():
    lib = bcq.load()
    assert lib.bcq_pack_planes(None, 1, 16, 128, FAKE, None) == E_ARG
    assert lib.bcq_pack_planes(FAKE, 1, 16, 100, FAKE, None) == E_ARG
    assert lib.bcq_pack_planes(FAKE + 2, 1, 16, 128, FAKE, None) == E_ALN
    assert lib.bcq_pack_planes(FAKE, 1, 16, 128, FAKE + 4, None) == E_ALN
    assert lib.bcq_unpack_planes(FAKE, 0, 16, 128, FAKE, None) == E_ARG


def test_workspace_sizes():
    lib = bcq.load()
    ws = lambda st, b: lib.bcq_workspace_bytes(ctypes.byref(st), b)
    st = make_store(M=4096, K=4096)
    # batch 1 uses the table kernel, 2..16 requests the whole-K matrix-core
    # kernel: none of them needs a workspace
    for b in (1, 2, 3, 16):
        assert ws(st, b) == 0, b
    # from 17 requests K is split over workgroups: one fp32 partial per (K
    # slice, request, row), at most one slice per 4-group step (8 steps here)
    need32, need64 = ws(st, 32), ws(st, 64)
    assert need32 > 0 and need32 % (32 * 4096 * 4) == 0 and need32 <= 8 * 32 * 4096 * 4
    assert need64 > 0 and need64 % (64 * 4096 * 4) == 0 and need64 <= 8 * 64 * 4096 * 4
    # a call runs launches of 64 (one precision) or 32 (per-request
    # precisions) in order, reusing the workspace: the size covers the largest
    assert ws(st, 256) == max(need64, need32)
    assert ws(st, 80) == max(need64, need32)
    # up to 16 requests keep K <= 4096 within a workgroup at any row count
    # (K <= 2048 only up to 256 row tiles); past that K is split from 3 requests
    assert ws(make_store(M=1024, K=4096), 16) == 0
    assert ws(make_store(M=4096, K=2048), 16) == 0
    assert ws(make_store(M=14336, K=2048), 16) > 0
    long_k = make_store(M=1024, K=8192)
    need3, need16 = ws(long_k, 3), ws(long_k, 16)
    assert need3 > 0 and need3 % (3 * 1024 * 4) == 0
    # at most one slice per 4-group step (16 steps here)
    assert need16 > 0 and need16 % (16 * 1024 * 4) == 0 and need16 <= 16 * 16 * 1024 * 4
    f32 = make_store(M=4096, K=4096, dtype=bcq.BCQ_F32)
    assert lib.bcq_workspace_bytes(ctypes.byref(f32), 64) == 0  # fp32 uses the table path
    assert lib.bcq_workspace_bytes(None, 16) == 0


def test_noalloc_entry_point_validates_and_rejects_oversized_calls_on_the_host():
    """bcq_gemm_skinny_noalloc checks its arguments like bcq_gemm_skinny, and a
    call whose split-K partial sums exceed the library's scratch returns
    BCQ_ERR_TOO_LARGE before any HIP call."""
    lib = bcq.load()
    call = lambda st, b, ldx=None, ldy=None, X=FAKE, Y=FAKE: lib.bcq_gemm_skinny_noalloc(
        ctypes.byref(st), 4, X, b, st.K if ldx is None else ldx, bcq.BCQ_F16, Y,
        st.M if ldy is None else ldy, bcq.BCQ_F16, None)
    st = make_store(M=64, K=256)
    assert call(st, 0) == E_ARG
    assert call(st, 2, X=None) == E_ARG
    assert call(st, 2, ldx=100) == E_ARG
    big = make_store(M=36864, K=65536)
    need = lib.bcq_workspace_bytes(ctypes.byref(big), 64)
    assert need > bcq.BCQ_NOALLOC_SCRATCH_BYTES
    assert call(big, 64) == bcq.BCQ_ERR_TOO_LARGE
    assert "BCQ_ERR_TOO_LARGE" in bcq.bcq_status_string(bcq.BCQ_ERR_TOO_LARGE)


def test_quantize_validation_rejects_before_launch():
    lib = bcq.load()
    q = lambda W=FAKE, wdt=bcq.BCQ_F16, M=16, K=256, ldw=256, P=4, pl=2, it=20, s=FAKE, a=FAKE, \
        z=FAKE, odt=bcq.BCQ_F16: lib.bcq_quantize(W, wdt, M, K, ldw, P, pl, it, s, a, z, odt, None)
    assert q(W=None) == E_ARG
    assert q(s=None) == E_ARG
    assert q(wdt=bcq.BCQ_F64) == E_ARG
    assert q(odt=7) == E_ARG
    assert q(K=200, ldw=200) == E_ARG
    assert q(ldw=128) == E_ARG
    assert q(P=5) == E_ARG
    assert q(pl=0) == E_ARG
    assert q(pl=5, P=4) == E_ARG
    assert q(it=-1) == E_ARG
    assert q(W=FAKE + 1) == E_ALN
    assert q(a=FAKE + 4, odt=bcq.BCQ_F64) == E_ALN
    assert q(s=FAKE + 2) == E_ALN
