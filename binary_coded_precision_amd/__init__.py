"""Python binding of the MI355X BCQ library (``libbcq.so``, C ABI in ``include/bcq.h``).

Argument marshalling only: every step of every product runs in the library's
HIP kernels.  PyTorch supplies device memory and the current stream.  There
is no CPU fallback: if the library is missing or fails to load, every entry
point raises.

Functions carry the C names (``bcq_pack_planes``, ``bcq_gemv``,
``bcq_gemm_skinny``, ``bcq_gemv_mixed_p``, ...) and take torch tensors on the
GPU.  :class:`Store` holds a packed weight (planes + per-precision scale tables)
and the ``bcq_store`` descriptor that points at it.
"""

from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbcq.so")

BCQ_OK = 0
BCQ_ERR_INVALID_ARG = -1
BCQ_ERR_UNSUPPORTED = -2
BCQ_ERR_ALIGNMENT = -3
BCQ_ERR_HIP = -4
BCQ_ERR_TOO_LARGE = -5
BCQ_F16 = 1
BCQ_F32 = 2
BCQ_F64 = 3
BCQ_MAX_PLANES = 4
BCQ_GROUP = 128
BCQ_TILE_ROWS = 16
BCQ_MAX_BATCH = 256
BCQ_NOALLOC_SCRATCH_BYTES = 16 << 20
BCQ_LOWRANK_MAX_RANK = 4096
BCQ_LOWRANK_FUSED_MAX_RANK = 1024

# Every symbol include/bcq.h declares.
EXPORTS = (
    "bcq_packed_bytes",
    "bcq_pack_planes",
    "bcq_unpack_planes",
    "bcq_gemv",
    "bcq_gemv_gate_up",
    "bcq_gemm_gate_up",
    "bcq_gemm_skinny",
    "bcq_gemm_skinny_noalloc",
    "bcq_workspace_bytes",
    "bcq_gemv_mixed_p",
    "bcq_lowrank_correct",
    "bcq_gemv_lowrank",
    "bcq_dequantize",
    "bcq_quantize",
    "bcq_status_string",
)


class BCQError(RuntimeError):
    """A library call returned a status other than BCQ_OK."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__("%s failed: %s" % (fn, bcq_status_string(status)))


class _Store(ctypes.Structure):
    _fields_ = [
        ("M", ctypes.c_int32),
        ("K", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
        ("planes", ctypes.c_int32),
        ("bits", ctypes.c_void_p),
        ("scale_dtype", ctypes.c_int),
        ("alpha", ctypes.c_void_p * (BCQ_MAX_PLANES + 1)),
        ("zero", ctypes.c_void_p * (BCQ_MAX_PLANES + 1)),
    ]


_lib: Optional[ctypes.CDLL] = None


def load(build_if_missing: bool = True) -> ctypes.CDLL:
    """Load ``libbcq.so`` (building it first only if no built copy exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        if not build_if_missing:
            raise RuntimeError("libbcq.so is not built: run binary_coded_precision_amd.build")
        from . import build as _build

        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    st = ctypes.POINTER(_Store)
    sig = {
        "bcq_packed_bytes": (sz, [i32, i32, i32]),
        "bcq_pack_planes": (ctypes.c_int, [vp, i32, i32, i32, vp, vp]),
        "bcq_unpack_planes": (ctypes.c_int, [vp, i32, i32, i32, vp, vp]),
        "bcq_gemv": (ctypes.c_int, [st, i32, vp, ctypes.c_int, vp, ctypes.c_int, vp]),
        "bcq_gemv_gate_up": (ctypes.c_int, [st, i32, vp, ctypes.c_int, vp, ctypes.c_int, vp]),
        "bcq_gemm_gate_up": (ctypes.c_int, [st, vp, vp, i32, i32, ctypes.c_int, vp, i32,
                                            ctypes.c_int, vp]),
        "bcq_gemm_skinny": (ctypes.c_int, [st, i32, vp, i32, i32, ctypes.c_int, vp, i32,
                                           ctypes.c_int, vp, sz, vp]),
        "bcq_gemm_skinny_noalloc": (ctypes.c_int, [st, i32, vp, i32, i32, ctypes.c_int, vp, i32,
                                                   ctypes.c_int, vp]),
        "bcq_workspace_bytes": (sz, [st, i32]),
        "bcq_gemv_mixed_p": (ctypes.c_int, [st, vp, vp, i32, i32, ctypes.c_int, vp, i32,
                                            ctypes.c_int, vp, sz, vp]),
        "bcq_lowrank_correct": (ctypes.c_int, [vp, vp, vp, i32, i32, i32, vp, vp, ctypes.c_int,
                                               vp, vp]),
        "bcq_gemv_lowrank": (ctypes.c_int, [st, i32, vp, ctypes.c_int, vp, vp, vp, i32, vp,
                                            ctypes.c_int, vp, vp]),
        "bcq_dequantize": (ctypes.c_int, [st, i32, vp, i32, ctypes.c_int, vp]),
        "bcq_quantize": (ctypes.c_int, [vp, ctypes.c_int, i32, i32, i32, i32, i32, i32, vp, vp,
                                        vp, ctypes.c_int, vp]),
        "bcq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(fn: str, status: int) -> None:
    if status != BCQ_OK:
        raise BCQError(fn, status)


def _stream(stream=None):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float16:
        return BCQ_F16
    if t.dtype == torch.float32:
        return BCQ_F32
    raise TypeError("BCQ tensors must be float16 or float32, got %s" % t.dtype)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _need_vec(name: str, t, n: int) -> None:
    """t is a device tensor with unit inner stride holding at least n elements
    from its first element on."""
    if t is None:
        raise ValueError("%s is None" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if t.dim() > 1 and t.stride(-1) != 1:
        raise ValueError("%s must have unit inner stride" % name)
    if t.dim() <= 1 and t.numel() > 1 and t.stride(0) != 1:
        raise ValueError("%s must be contiguous" % name)
    if t.numel() < n:
        raise ValueError("%s holds %d elements, %d needed" % (name, t.numel(), n))


def _need_mat(name: str, t, rows: int, cols: int) -> None:
    """t is a 2-D device tensor of at least rows x cols with unit inner stride
    (rows may be padded: stride(0) is the leading dimension)."""
    if t is None or t.dim() != 2:
        raise ValueError("%s must be a 2-D tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if t.stride(1) != 1:
        raise ValueError("%s must have unit inner stride" % name)
    if t.shape[0] < rows or t.shape[1] < cols:
        raise ValueError("%s is %dx%d, at least %dx%d needed" % (name, t.shape[0], t.shape[1],
                                                                rows, cols))
    if t.shape[0] > 1 and t.stride(0) < t.shape[1]:
        raise ValueError("%s rows overlap (stride(0) < shape[1])" % name)


def _check_store_tensors(store: "Store", ps) -> None:
    """The store's buffers are as large as the descriptor says for precisions ps."""
    _need_vec("store.bits", store.bits,
              bcq_packed_bytes(store.planes, store.M, store.K) // store.bits.element_size())
    G = store.K // BCQ_GROUP
    for p in set(int(v) for v in ps):
        if 1 <= p <= store.planes and p in store.alpha and p in store.zero:
            _need_vec("store.alpha[%d]" % p, store.alpha[p], p * store.M * G)
            _need_vec("store.zero[%d]" % p, store.zero[p], store.M * G)


# ----------------------------------------------------------------------------- C names


def bcq_status_string(status: int) -> str:
    return load().bcq_status_string(int(status)).decode()


def bcq_packed_bytes(P: int, M: int, K: int) -> int:
    return int(load().bcq_packed_bytes(P, M, K))


def bcq_pack_planes(signs, P: int, M: int, K: int, packed, stream=None) -> None:
    """``signs``: int32/uint32 device tensor [P][M][K/32]; ``packed``: device tensor of
    ``bcq_packed_bytes(P, M, K)`` bytes."""
    n = bcq_packed_bytes(P, M, K)
    if n:
        _need_vec("signs", signs, P * M * (K // 32))
        _need_vec("packed", packed, n // packed.element_size())
    _check("bcq_pack_planes",
           load().bcq_pack_planes(_ptr(signs), P, M, K, _ptr(packed), _stream(stream)))


def bcq_unpack_planes(packed, P: int, M: int, K: int, signs, stream=None) -> None:
    n = bcq_packed_bytes(P, M, K)
    if n:
        _need_vec("packed", packed, n // packed.element_size())
        _need_vec("signs", signs, P * M * (K // 32))
    _check("bcq_unpack_planes",
           load().bcq_unpack_planes(_ptr(packed), P, M, K, _ptr(signs), _stream(stream)))


def bcq_gemv(store: "Store", p: int, x, y, stream=None) -> None:
    """``y[M] = product at precision p`` of the device vector ``x[K]``."""
    _need_vec("x", x, store.K)
    _need_vec("y", y, store.M)
    _check_store_tensors(store, [p])
    _check("bcq_gemv", load().bcq_gemv(store.ref(), p, _ptr(x), _dtype_code(x), _ptr(y),
                                       _dtype_code(y), _stream(stream)))


def bcq_gemv_gate_up(store: "Store", p: int, x, y, stream=None) -> None:
    """``y[M/2] = silu(gate . x) * (up . x)`` for a store whose 16-row tiles hold
    8 gate rows then the matching 8 up rows (see ``include/bcq.h``)."""
    _need_vec("x", x, store.K)
    _need_vec("y", y, store.M // 2)
    _check_store_tensors(store, [p])
    _check("bcq_gemv_gate_up", load().bcq_gemv_gate_up(store.ref(), p, _ptr(x), _dtype_code(x),
                                                       _ptr(y), _dtype_code(y),
                                                       _stream(stream)))


def bcq_gemm_gate_up(store: "Store", p_host: Sequence[int], X, Y, stream=None) -> None:
    """``Y[r][j] = silu(gate_j . X[r]) * (up_j . X[r])`` at precision ``p_host[r]``
    for a gate/up store (see :func:`bcq_gemv_gate_up`); ``Y`` is [b][>= M/2]."""
    b = X.shape[0]
    if len(p_host) != b:
        raise ValueError("p_host has %d entries for %d requests" % (len(p_host), b))
    _need_mat("X", X, b, store.K)
    _need_mat("Y", Y, b, store.M // 2)
    _check_store_tensors(store, p_host)
    ps = (ctypes.c_int32 * b)(*[int(v) for v in p_host])
    _check("bcq_gemm_gate_up",
           load().bcq_gemm_gate_up(store.ref(), ps, _ptr(X), b, X.stride(0), _dtype_code(X),
                                   _ptr(Y), Y.stride(0), _dtype_code(Y), _stream(stream)))


def bcq_lowrank_correct(u_signs, v_signs, alpha, x, y, z=None, stream=None) -> None:
    """``y[M] += sum_r alpha[r] * u[:, r] * (v[r] . x)`` in place (see ``include/bcq.h``).

    ``u_signs`` [M][ceil(R/32)] and ``v_signs`` [R][K/32] are device int32/uint32
    sign words; ``alpha`` [R], ``x`` [K] and ``y`` [M] share one dtype; ``z`` is
    an R-float device workspace (allocated through torch when None)."""
    import torch

    R, M, K = alpha.numel(), y.numel(), x.numel()
    if not (x.dtype == y.dtype == alpha.dtype):
        raise ValueError("alpha, x and y must share one dtype")
    if z is None:
        z = torch.empty(R, dtype=torch.float32, device=y.device)
    _need_vec("u_signs", u_signs, M * ((R + 31) // 32))
    _need_vec("v_signs", v_signs, R * (K // 32))
    _need_vec("z", z, R)
    _check("bcq_lowrank_correct",
           load().bcq_lowrank_correct(_ptr(u_signs), _ptr(v_signs), _ptr(alpha), R, M, K,
                                      _ptr(x), _ptr(y), _dtype_code(y), _ptr(z),
                                      _stream(stream)))


def bcq_gemv_lowrank(store: "Store", p: int, x, u_signs, v_signs, lr_alpha, y, z=None,
                     stream=None) -> None:
    """``y[M] = product at precision p of x + sum_r lr_alpha[r] * u[:, r] * (v[r] . x)``
    (see ``include/bcq.h``): the product of :func:`bcq_gemv` with the correction
    of :func:`bcq_lowrank_correct`, written once.  ``z`` is an R-float device
    workspace (allocated through torch when None)."""
    import torch

    R, M, K = lr_alpha.numel(), store.M, store.K
    if z is None:
        z = torch.empty(R, dtype=torch.float32, device=y.device)
    _need_vec("x", x, K)
    _need_vec("y", y, M)
    _need_vec("u_signs", u_signs, M * ((R + 31) // 32))
    _need_vec("v_signs", v_signs, R * (K // 32))
    _need_vec("lr_alpha", lr_alpha, R)
    _need_vec("z", z, R)
    _check_store_tensors(store, [p])
    _check("bcq_gemv_lowrank",
           load().bcq_gemv_lowrank(store.ref(), p, _ptr(x), _dtype_code(x), _ptr(u_signs),
                                   _ptr(v_signs), _ptr(lr_alpha), R, _ptr(y), _dtype_code(y),
                                   _ptr(z), _stream(stream)))


def bcq_dequantize(store: "Store", p: int, W, stream=None) -> None:
    """Dense ``W[M][K]`` (a device tensor, rows possibly padded: ``W.stride(0)``
    is the leading dimension) at precision ``p``, in the store's scale dtype."""
    _need_mat("W", W, store.M, store.K)
    _check_store_tensors(store, [p])
    _check("bcq_dequantize", load().bcq_dequantize(store.ref(), p, _ptr(W), W.stride(0),
                                                   _dtype_code(W), _stream(stream)))


def bcq_quantize(W, P: int, p_low: int = 2, iters: int = 20, out_dtype=None, stream=None):
    """Quantize the device matrix ``W`` [M][K] (fp16 or fp32, rows may be
    padded) into P sign planes and per-precision tables (see ``include/bcq.h``).

    Returns ``(signs, alpha, zero)``: ``signs`` an int32 device tensor
    [P][M][K/32] in the canonical format ``bcq_pack_planes`` takes, and dicts
    ``alpha[p]`` [p][M][K/128], ``zero[p]`` [M][K/128] for p = p_low..P, views
    of two device buffers of ``out_dtype`` (default: W's dtype)."""
    import torch

    M, K = W.shape
    _need_mat("W", W, M, K)
    out_dtype = W.dtype if out_dtype is None else out_dtype
    codes = {torch.float16: BCQ_F16, torch.float32: BCQ_F32, torch.float64: BCQ_F64}
    if out_dtype not in codes or W.dtype not in (torch.float16, torch.float32):
        raise TypeError("W must be float16/float32 and out_dtype float16/32/64")
    if K % BCQ_GROUP or not (1 <= p_low <= P <= BCQ_MAX_PLANES):
        raise ValueError("K must be a multiple of 128 and 1 <= p_low <= P <= 4")
    G = K // BCQ_GROUP
    signs = torch.empty((P, M, K // 32), dtype=torch.int32, device=W.device)
    n_alpha = sum(p for p in range(p_low, P + 1)) * M * G
    abuf = torch.empty(n_alpha, dtype=out_dtype, device=W.device)
    zbuf = torch.empty((P - p_low + 1, M, G), dtype=out_dtype, device=W.device)
    _check("bcq_quantize",
           load().bcq_quantize(_ptr(W), _dtype_code(W), M, K, W.stride(0), P, p_low, iters,
                               _ptr(signs), _ptr(abuf), _ptr(zbuf), codes[out_dtype],
                               _stream(stream)))
    alpha, zero, off = {}, {}, 0
    for p in range(p_low, P + 1):
        alpha[p] = abuf[off:off + p * M * G].view(p, M, G)
        zero[p] = zbuf[p - p_low]
        off += p * M * G
    return signs, alpha, zero


def bcq_workspace_bytes(store: "Store", b: int) -> int:
    return int(load().bcq_workspace_bytes(store.ref(), b))


def new_workspace(store: "Store", b: int):
    """A device workspace of ``bcq_workspace_bytes(store, b)`` bytes for
    ``bcq_gemm_skinny`` or ``bcq_gemv_mixed_p`` at batch b, or None when the
    call needs none.  Its
    contents need no initialisation; calls that may overlap need separate ones."""
    import torch

    n = bcq_workspace_bytes(store, b)
    if n == 0:
        return None
    return torch.empty((n + 3) // 4, dtype=torch.int32, device=store.bits.device)


def bcq_gemm_skinny(store: "Store", p: int, X, Y, workspace=None, stream=None) -> None:
    """``Y[r] = product at precision p`` of ``X[r]`` for each row r of the [b][K] tensor X.

    ``workspace=None`` allocates the workspace the call needs (through torch);
    pass one from :func:`new_workspace` to keep allocation out of a hot loop."""
    b = X.shape[0]
    _need_mat("X", X, b, store.K)
    _need_mat("Y", Y, b, store.M)
    _check_store_tensors(store, [p])
    if workspace is None:
        workspace = new_workspace(store, b)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("bcq_gemm_skinny",
           load().bcq_gemm_skinny(store.ref(), p, _ptr(X), b, X.stride(0), _dtype_code(X),
                                  _ptr(Y), Y.stride(0), _dtype_code(Y), _ptr(workspace),
                                  ws_bytes, _stream(stream)))


def bcq_gemm_skinny_noalloc(store: "Store", p: int, X, Y, stream=None) -> None:
    """:func:`bcq_gemm_skinny` with the library's own per-GPU scratch instead of a
    workspace: nothing is allocated (see ``include/bcq.h`` for the limit and
    the rule that calls sharing a GPU's scratch must not overlap)."""
    b = X.shape[0]
    _need_mat("X", X, b, store.K)
    _need_mat("Y", Y, b, store.M)
    _check_store_tensors(store, [p])
    _check("bcq_gemm_skinny_noalloc",
           load().bcq_gemm_skinny_noalloc(store.ref(), p, _ptr(X), b, X.stride(0),
                                          _dtype_code(X), _ptr(Y), Y.stride(0), _dtype_code(Y),
                                          _stream(stream)))


def bcq_gemv_mixed_p(store: "Store", p_host: Sequence[int], X, Y, workspace=None,
                     stream=None) -> None:
    """Request r at its own precision ``p_host[r]`` (workspace as in :func:`bcq_gemm_skinny`)."""
    b = X.shape[0]
    if len(p_host) != b:
        raise ValueError("p_host has %d entries for %d requests" % (len(p_host), b))
    _need_mat("X", X, b, store.K)
    _need_mat("Y", Y, b, store.M)
    _check_store_tensors(store, p_host)
    ps = (ctypes.c_int32 * b)(*[int(v) for v in p_host])
    if workspace is None:
        workspace = new_workspace(store, b)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("bcq_gemv_mixed_p",
           load().bcq_gemv_mixed_p(store.ref(), ps, _ptr(X), b, X.stride(0), _dtype_code(X),
                                   _ptr(Y), Y.stride(0), _dtype_code(Y), _ptr(workspace),
                                   ws_bytes, _stream(stream)))


# ----------------------------------------------------------------------------- store


class Store:
    """A packed BCQ weight on the GPU and its ``bcq_store`` descriptor.

    ``bits`` is the packed device layout; ``alpha[p]`` / ``zero[p]`` are the
    tables used at precision p (tensors, possibly the same tensor for every p).
    """

    def __init__(self, M: int, K: int, planes: int, bits, alpha: Dict[int, object],
                 zero: Dict[int, object]):
        self.M, self.K, self.planes = M, K, planes
        self.bits = bits
        self.alpha = dict(alpha)
        self.zero = dict(zero)
        dt = None
        for t in list(self.alpha.values()) + list(self.zero.values()):
            d = _dtype_code(t)
            if dt is not None and d != dt:
                raise TypeError("all scale tables must share one dtype")
            dt = d
        self.scale_dtype = dt
        st = _Store()
        st.M, st.K, st.group_size, st.planes = M, K, BCQ_GROUP, planes
        st.bits = bits.data_ptr()
        st.scale_dtype = dt
        for p in range(BCQ_MAX_PLANES + 1):
            st.alpha[p] = self.alpha[p].data_ptr() if p in self.alpha else None
            st.zero[p] = self.zero[p].data_ptr() if p in self.zero else None
        self._st = st

    def ref(self):
        return ctypes.byref(self._st)

    @classmethod
    def from_quantized(cls, signs, alpha: Dict[int, object], zero: Dict[int, object],
                       stream=None) -> "Store":
        """A store from :func:`bcq_quantize`'s outputs (device tensors): packs the
        canonical sign words; precision p reads ``alpha[p]`` / ``zero[p]``."""
        import torch

        P, M, W = signs.shape
        K = W * 32
        packed = torch.empty(bcq_packed_bytes(P, M, K) // 4, dtype=torch.int32,
                             device=signs.device)
        bcq_pack_planes(signs, P, M, K, packed, stream)
        return cls(M, K, P, packed, alpha, zero)

    @classmethod
    def from_host(cls, signs: np.ndarray, alpha: np.ndarray, zero: np.ndarray, *,
                  alpha_p: Optional[Dict[int, np.ndarray]] = None,
                  zero_p: Optional[Dict[int, np.ndarray]] = None, device="cuda",
                  stream=None) -> "Store":
        """Upload canonical host arrays and pack the planes with ``bcq_pack_planes``.

        ``signs`` uint32 [P][M][K/32]; ``alpha`` [P][M][K/128]; ``zero`` [M][K/128].
        Without ``alpha_p``/``zero_p`` every precision shares ``alpha``'s leading
        planes and ``zero``.
        """
        import torch

        import contextlib

        P, M, W = signs.shape
        K = W * 32
        nbytes = bcq_packed_bytes(P, M, K)
        if nbytes == 0:
            raise BCQError("bcq_packed_bytes", BCQ_ERR_INVALID_ARG)
        # uploads and the pack run on one stream, in that order
        ctx = torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()
        with ctx:
            dsigns = torch.from_numpy(np.ascontiguousarray(signs).view(np.int32)).to(device)
            packed = torch.empty(nbytes // 4, dtype=torch.int32, device=device)
            bcq_pack_planes(dsigns, P, M, K, packed)
            if alpha_p is None:
                a = torch.from_numpy(np.ascontiguousarray(alpha)).to(device)
                z = torch.from_numpy(np.ascontiguousarray(zero)).to(device)
                at = {p: a for p in range(1, P + 1)}
                zt = {p: z for p in range(1, P + 1)}
            else:
                at = {p: torch.from_numpy(np.ascontiguousarray(alpha_p[p])).to(device)
                      for p in alpha_p}
                zt = {p: torch.from_numpy(np.ascontiguousarray(zero_p[p])).to(device)
                      for p in zero_p}
        return cls(M, K, P, packed, at, zt)
