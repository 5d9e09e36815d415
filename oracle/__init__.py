"""Float64 CPU oracle for the BCQ product -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import or call this package.  The library and its Python
binding never do: there is no CPU fallback anywhere in the product path.

The arithmetic lives in ``bcq_oracle.c`` (plain C loops in float64, see its
header for the definitions it follows and the page passages it cites).  This
module compiles it with the host C compiler when no built copy is present and
marshals NumPy arrays to it.  Inputs are converted to float64 exactly (every
fp16 and fp32 value is a float64 value).

Parity status: every function here is pinned by ``tests/test_oracle.py``
(worked example from the BiLoCo page, dense dequantise-then-matmul, brute force
over all sign patterns, closed forms, prefix invariant, linearity; the gate/up
epilogue by silu's closed-form points and a dense per-tile reconstruction; the
low-rank correction by the BiLoCo page's worked example, closed forms and a
loop-by-loop brute force).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bcq_oracle.c")
_LIB = os.path.join(_HERE, "libbcq_oracle.so")
_lib: Optional[ctypes.CDLL] = None

__all__ = ["build", "gemv", "gemv_requests", "dequant", "sign_at"]


def build(force: bool = True) -> str:
    """Compile the oracle into ``oracle/libbcq_oracle.so`` and return its path."""
    global _lib
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(
            ["gcc", "-O2", "-std=c99", "-shared", "-fPIC", "-o", tmp, _SRC],
            check=True,
        )
        os.replace(tmp, _LIB)
        _lib = None
    return _LIB


def _load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        # BCQ_ORACLE_LIB points at a deliberately broken build of bcq_oracle.c;
        # only the mutation test sets it, to prove the pins catch such mistakes.
        path = os.environ.get("BCQ_ORACLE_LIB")
        if path is None:
            if not os.path.exists(_LIB):
                build(force=False)
            path = _LIB
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i = ctypes.c_int
        lib.bcq_oracle_gemv.argtypes = [P, i, i, i, i, i, P, P, P, P]
        lib.bcq_oracle_gemv.restype = None
        lib.bcq_oracle_dequant.argtypes = [P, i, i, i, i, i, P, P, P]
        lib.bcq_oracle_dequant.restype = None
        lib.bcq_oracle_sign_at.argtypes = [P, i, i, i, i, i]
        lib.bcq_oracle_sign_at.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _u32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.uint32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def gemv(signs, alpha, zero, x, p: int, g: int = 128) -> np.ndarray:
    """One request at precision ``p``.

    ``signs`` uint32 [P][M][ceil(K/32)]; ``alpha`` [>=p][M][G] (planes beyond p
    are ignored); ``zero`` [M][G]; ``x`` [K].  Returns float64 ``y`` [M].
    """
    signs = _u32(signs)
    P, M, _ = signs.shape
    x = _f64(x).reshape(-1)
    K = x.shape[0]
    if K % g or not (1 <= p <= P):
        raise ValueError("bad K/g or p")
    a = _f64(np.asarray(alpha)[:p])
    z = _f64(zero)
    G = K // g
    if a.shape != (p, M, G) or z.shape != (M, G):
        raise ValueError("alpha/zero shapes do not match")
    y = np.empty(M, dtype=np.float64)
    _load().bcq_oracle_gemv(_ptr(signs), P, M, K, g, p, _ptr(a), _ptr(z), _ptr(x), _ptr(y))
    return y


def gemv_requests(signs, x, p_req: Sequence[int], alpha_for, zero_for, g: int = 128) -> np.ndarray:
    """Several requests, each at its own precision.

    ``x`` [b][K]; ``p_req`` [b]; ``alpha_for(p)`` / ``zero_for(p)`` return the
    tables used at precision ``p``.  Returns float64 ``y`` [b][M].
    """
    x = np.asarray(x)
    out = [gemv(signs, alpha_for(int(p)), zero_for(int(p)), x[r], int(p), g)
           for r, p in enumerate(p_req)]
    return np.stack(out)


def silu_mul(g, u) -> np.ndarray:
    """The gated-MLP epilogue in float64: silu(g) * u with silu(g) = g / (1 + exp(-g))."""
    g = _f64(g)
    u = _f64(u)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * u


def gate_up_rows(j):
    """Store rows of the gate and up products of outputs ``j`` in a gate/up store:
    16-row tile t holds gate rows 8t..8t+7, then up rows 8t..8t+7."""
    j = np.asarray(j, dtype=np.int64)
    tile, i = j // 8, j % 8
    return 16 * tile + i, 16 * tile + 8 + i


def gemv_gate_up(signs, alpha, zero, x, p: int, g: int = 128) -> np.ndarray:
    """``y[j] = silu(gate_j . x) * (up_j . x)`` for a gate/up store of 2 * Mo rows.

    Returns float64 ``y`` [Mo] (Mo = rows of ``signs`` / 2, rows a multiple of 16).
    """
    y = gemv(signs, alpha, zero, x, p, g)
    if y.shape[0] % 16:
        raise ValueError("a gate/up store has a multiple of 16 rows")
    gr, ur = gate_up_rows(np.arange(y.shape[0] // 2))
    return silu_mul(y[gr], y[ur])


def _signs_pm1(words, n: int) -> np.ndarray:
    """{-1,+1} float64 [rows][n] from sign words (bit j mod 32 of word j/32, set = +1)."""
    w = np.ascontiguousarray(np.asarray(words).astype("<u4"))
    bits = np.unpackbits(w.view(np.uint8).reshape(w.shape[0], -1), axis=-1, bitorder="little")
    return bits[:, :n].astype(np.float64) * 2.0 - 1.0


def lowrank_correct(u_signs, v_signs, alpha, x, y0) -> np.ndarray:
    """Binary low-rank correction in float64 (BiLoCo summary, "core idea"):
    ``y0 + sum_r alpha_r u_r (v_r . x)`` with u [M][R] and v [R][K] sign words."""
    alpha = _f64(alpha).reshape(-1)
    x = _f64(x).reshape(-1)
    R, K = alpha.shape[0], x.shape[0]
    u = _signs_pm1(u_signs, R)
    v = _signs_pm1(v_signs, K)
    z = alpha * (v @ x)
    return _f64(y0).reshape(-1) + u @ z


def dequant(signs, alpha, zero, p: int, K: int, g: int = 128) -> np.ndarray:
    """Dense float64 reconstruction ``[M][K]`` at precision ``p``."""
    signs = _u32(signs)
    P, M, _ = signs.shape
    a = _f64(np.asarray(alpha)[:p])
    z = _f64(zero)
    w = np.empty((M, K), dtype=np.float64)
    _load().bcq_oracle_dequant(_ptr(signs), P, M, K, g, p, _ptr(a), _ptr(z), _ptr(w))
    return w


def sign_at(signs, i: int, m: int, k: int, K: int) -> int:
    """+1 or -1: the sign the oracle reads for plane ``i``, row ``m``, column ``k``."""
    signs = _u32(signs)
    _, M, _ = signs.shape
    return int(_load().bcq_oracle_sign_at(_ptr(signs), M, K, i, m, k))
