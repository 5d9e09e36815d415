"""Seeded synthetic inputs for the binary-coded-quantization (BCQ) product.

This module is shared by the float64 oracle's tests and by the HIP path's tests
and benchmark.  It only draws random numbers and lays them out in the canonical
host format; it holds none of the BCQ arithmetic (no sign decoding, no
reconstruction, no products).

Canonical host format (the format ``bcq_pack_planes`` consumes):

* ``signs``  uint32 ``[P][M][W]`` with ``W = ceil(K / 32)``: column ``k`` of
  plane ``i`` and row ``m`` is bit ``k % 32`` (least significant first) of word
  ``signs[i, m, k // 32]``; a set bit means the sign +1, a clear bit -1.
* ``alpha``  ``[P][M][G]`` with ``G = K / g``: the scale of plane ``i`` for row
  ``m`` and the ``g``-column group ``j``.
* ``zero``   ``[M][G]``: the per-(row, group) offset of asymmetric BCQ.
* ``x``      ``[b][K]``: one activation row per request.

The value recipe follows the workloads the AnyBCQ pages evaluate on (LLaMA-3.1-8B
layer shapes, group size 128) with synthetic distributions: signs are uniform
random words (i.i.d. fair bits), ``alpha_i = |N(0, 0.02)| * 0.5**(i-1)`` drawn
independently per (plane, row, group), ``z ~ N(0, 0.005)``, ``x ~ N(0, 1)``,
optionally with 1% of the channels scaled by 20 (outliers).  The second argument
of ``N`` is a standard deviation.  Values are drawn in float64 and rounded once,
to nearest-even, to the storage dtype.  The draw order is fixed: sign words,
alpha, z, x, outlier channels, per-request precisions.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

GROUP = 128

__all__ = [
    "GROUP",
    "Workload",
    "make",
    "config",
    "mlp_cases",
    "sweep_cases",
    "independent_tables",
]


@dataclass
class Workload:
    """One synthetic BCQ problem in canonical host layout."""

    name: str
    M: int
    K: int
    P: int
    g: int
    dtype: np.dtype
    signs: np.ndarray  # uint32 [P][M][ceil(K/32)]
    alpha: np.ndarray  # dtype [P][M][G]
    zero: np.ndarray  # dtype [M][G]
    x: np.ndarray  # dtype [b][K]
    p_req: np.ndarray  # int32 [b], precision used by each request
    outlier_channels: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))
    # Optional per-precision scale tables: alpha_p[p] is [p][M][G], zero_p[p] is [M][G].
    # When absent every precision uses the leading planes of ``alpha`` and ``zero``.
    alpha_p: Optional[Dict[int, np.ndarray]] = None
    zero_p: Optional[Dict[int, np.ndarray]] = None

    @property
    def b(self) -> int:
        return int(self.x.shape[0])

    @property
    def G(self) -> int:
        return self.K // self.g

    def alpha_for(self, p: int) -> np.ndarray:
        """Scale table ``[p][M][G]`` used at precision ``p``."""
        if self.alpha_p is not None:
            return self.alpha_p[p]
        return self.alpha[:p]

    def zero_for(self, p: int) -> np.ndarray:
        """Offset table ``[M][G]`` used at precision ``p``."""
        if self.zero_p is not None:
            return self.zero_p[p]
        return self.zero


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def make(
    M: int,
    K: int,
    P: int,
    b: int = 1,
    *,
    dtype=np.float16,
    g: int = GROUP,
    seed: int = 0,
    alpha_sigma: float = 0.02,
    z_sigma: float = 0.005,
    x_sigma: float = 1.0,
    outlier_frac: float = 0.0,
    outlier_scale: float = 20.0,
    p: Optional[int] = None,
    p_choices: Optional[Sequence[int]] = None,
    name: str = "custom",
) -> Workload:
    """Draw one workload.

    ``p`` fixes the precision of every request (default ``P``); ``p_choices``
    instead draws each request's precision uniformly from the given values.
    """
    if K % g != 0:
        raise ValueError("K must be a multiple of the group size")
    dtype = np.dtype(dtype)
    rng = _rng(seed)
    W = (K + 31) // 32
    G = K // g
    signs = rng.integers(0, 1 << 32, size=(P, M, W), dtype=np.uint64).astype(np.uint32)
    if K % 32:
        # columns beyond K do not exist; keep their bits clear
        signs[..., -1] &= np.uint32((1 << (K % 32)) - 1)
    decay = 0.5 ** np.arange(P, dtype=np.float64)
    alpha = np.abs(rng.standard_normal((P, M, G))) * alpha_sigma * decay[:, None, None]
    zero = rng.standard_normal((M, G)) * z_sigma
    x = rng.standard_normal((b, K)) * x_sigma
    n_out = int(round(outlier_frac * K))
    channels = np.sort(rng.permutation(K)[:n_out]) if n_out else np.zeros(0, np.int64)
    if n_out:
        x[:, channels] *= outlier_scale
    if p_choices is not None:
        p_req = rng.choice(np.asarray(p_choices, dtype=np.int32), size=b)
    else:
        p_req = np.full(b, P if p is None else p, dtype=np.int32)
    return Workload(
        name=name,
        M=M,
        K=K,
        P=P,
        g=g,
        dtype=dtype,
        signs=np.ascontiguousarray(signs),
        alpha=np.ascontiguousarray(alpha.astype(dtype)),
        zero=np.ascontiguousarray(zero.astype(dtype)),
        x=np.ascontiguousarray(x.astype(dtype)),
        p_req=p_req.astype(np.int32),
        outlier_channels=channels,
    )


def independent_tables(w: Workload, seed: int = 1000) -> Workload:
    """Attach independently drawn per-precision tables alpha_p[p], zero_p[p].

    AnyBCQ refits every scale when it expands precision, so the table used at
    precision p need not be a prefix of the one used at p+1.  These draws use
    the same distributions as :func:`make` and exist to prove that a caller's
    per-precision tables are the ones used.
    """
    rng = _rng(seed)
    G = w.G
    alpha_p, zero_p = {}, {}
    for p in range(1, w.P + 1):
        decay = 0.5 ** np.arange(p, dtype=np.float64)
        a = np.abs(rng.standard_normal((p, w.M, G))) * 0.02 * decay[:, None, None]
        z = rng.standard_normal((w.M, G)) * 0.005
        alpha_p[p] = np.ascontiguousarray(a.astype(w.dtype))
        zero_p[p] = np.ascontiguousarray(z.astype(w.dtype))
    w.alpha_p, w.zero_p = alpha_p, zero_p
    return w


# ---------------------------------------------------------------------------
# The five synthetic configurations (seed = configuration number).
# ---------------------------------------------------------------------------

def config(n: int, **overrides) -> Workload:
    """Configuration ``n`` (1..5) at its default shape.

    1  tiny: 256x512, b=1, P=p=2, all float32.
    2  q_proj-shaped: 4096x4096, b=1, P=4 (evaluated at p=2,3,4), float16,
       1% outlier channels x20.
    3  MLP gate/up: 14336x4096, b=1, p=3 of P=4, float16 (see :func:`mlp_cases`).
    4  mixed precision decode batch: 4096x4096, 8 requests, p_r uniform in {2,3,4}.
    5  decoder-layer sweep: q/o 4096x4096 at b=16 (see :func:`sweep_cases`).
    """
    base = dict(seed=n)
    if n == 1:
        base.update(M=256, K=512, P=2, b=1, dtype=np.float32, name="tiny_256x512_p2_f32")
    elif n == 2:
        base.update(M=4096, K=4096, P=4, b=1, dtype=np.float16, outlier_frac=0.01,
                    name="qproj_4096x4096_P4_f16")
    elif n == 3:
        base.update(M=14336, K=4096, P=4, b=1, p=3, dtype=np.float16,
                    name="mlp_gateup_14336x4096_p3_f16")
    elif n == 4:
        base.update(M=4096, K=4096, P=4, b=8, p_choices=(2, 3, 4), dtype=np.float16,
                    name="mixedp_4096x4096_b8_f16")
    elif n == 5:
        base.update(M=4096, K=4096, P=4, b=16, dtype=np.float16,
                    name="sweep_qo_4096x4096_b16_f16")
    else:
        raise ValueError("configurations are numbered 1..5")
    base.update(overrides)
    return make(**base)


MLP_SHAPES = {"gate_up": (14336, 4096), "down": (4096, 14336)}
LAYER_SHAPES = {
    "q_o": (4096, 4096),
    "k_v": (1024, 4096),
    "gate_up": (14336, 4096),
    "down": (4096, 14336),
}


def mlp_cases() -> List[dict]:
    """Configuration 3: MLP shapes at batch 1, 4, 8 and p = 3 of 4 planes."""
    return [dict(shape=s, M=M, K=K, b=b, p=3)
            for s, (M, K) in MLP_SHAPES.items() for b in (1, 4, 8)]


def sweep_cases() -> List[dict]:
    """Configuration 5: decoder-layer shapes at batch 1, 16, 32, 64 and p = 4."""
    return [dict(shape=s, M=M, K=K, b=b, p=4)
            for s, (M, K) in LAYER_SHAPES.items() for b in (1, 16, 32, 64)]


class LowRank:
    """Inputs of a binary low-rank correction y += sum_r alpha_r u_r (v_r . x)."""

    def __init__(self, u, v, alpha, x, y0):
        self.u, self.v, self.alpha, self.x, self.y0 = u, v, alpha, x, y0
        self.M, self.R = y0.shape[0], alpha.shape[0]
        self.K = x.shape[0]


def lowrank(M: int, K: int, R: int, dtype=np.float16, seed: int = 0) -> LowRank:
    """Seeded synthetic low-rank correction terms: u [M][ceil(R/32)] and
    v [R][K/32] uniformly random sign words, alpha_r = |N(0, 0.02)| / sqrt(R),
    x ~ N(0, 1) and y0 ~ N(0, 1) (the output being corrected)."""
    rng = _rng(seed)
    u = rng.integers(0, 2 ** 32, size=(M, (R + 31) // 32), dtype=np.uint64).astype(np.uint32)
    v = rng.integers(0, 2 ** 32, size=(R, K // 32), dtype=np.uint64).astype(np.uint32)
    alpha = (np.abs(rng.normal(0.0, 0.02, size=R)) / np.sqrt(R)).astype(dtype)
    x = rng.normal(0.0, 1.0, size=K).astype(dtype)
    y0 = rng.normal(0.0, 1.0, size=M).astype(dtype)
    return LowRank(u, v, alpha, x, y0)


def weights(M: int, K: int, dtype=np.float16, seed: int = 0) -> np.ndarray:
    """A seeded synthetic weight matrix [M][K] for the quantizer: heavy-tailed
    like trained LLM projection weights (no trained weights are used), each
    entry 0.02 * t_4 / sqrt(2) (Student's t with 4 degrees of freedom, scaled
    to standard deviation 0.02), drawn in float64 and rounded once to dtype."""
    rng = _rng(seed)
    return np.ascontiguousarray((0.02 / np.sqrt(2.0) * rng.standard_t(4, size=(M, K))).astype(dtype))
