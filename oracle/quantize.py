"""Float64 reference of AnyBCQ's offline progressive-precision quantizer --
TEST INFRASTRUCTURE ONLY.

Only ``tests/`` may import or call this module; the library never does.  It
shares no code with the HIP quantizer (``csrc/quantize.hip``): both follow the
steps below from the pages, written independently.

What it computes, per (row, group of g columns) of a weight matrix W
(AnyBCQ paper notes, "Method / key designs", progressive precision expansion;
"Training strategy": asymmetric BCQ, g = 128, alternating refinement at
initialisation, 20 rounds):

1. Base precision p_L, greedy initialisation.  The offset starts at the group
   mean; then plane by plane the sign of the residual becomes the plane and the
   mean absolute residual its scale, and the scaled plane leaves the residual.
2. Alternating refinement, ``iters`` rounds of: least-squares fit of all scales
   and the offset for the current planes, then the sign update -- each weight
   takes the code (one sign per plane) whose reconstructed level lies nearest
   to it.  One more least-squares fit follows the last round, so the emitted
   scales are optimal for the emitted planes.
3. Expansion p -> p + 1, for p = p_L .. P - 1: the planes found so far are
   frozen, the new plane is the sign of the residual W - W_hat_p, and the
   scales of precision p + 1 (all of them, and the offset) are refit by least
   squares.  Each precision keeps its own table.

Readings where the pages leave a step open:
  * sign(0) = +1 (a residual of exactly zero gets a +1 plane entry).
  * Greedy initialisation with an offset: the offset starts at the group mean
    and the greedy planes fit the centred weights.
  * The sign update ("BS" on the pages: a search over the 2^p levels) is the
    exact nearest level; ties go to the first code in order, code c giving
    plane i the sign +1 when bit i of c is set.
  * Least squares: the normal equations over the columns [planes..., ones]
    (scales, then offset).  A plane that is linearly dependent on the offset
    column and the earlier kept planes (decided exactly on the integer Gram
    matrix) is dropped and gets scale 0.  The kept system is solved by
    Gaussian elimination without pivoting (it is symmetric positive
    definite), in index order.
  * Every sum over a group is a pairwise (halving) sum: v[:n/2] + v[n/2:],
    repeated, over the group zero-padded to a power of two.  Any summation
    order is a correct reading; fixing this one lets a parallel kernel take
    every floating-point decision (a sign, a nearest level) on exactly the
    same values as this reference.
  * A level is built as offset + (+-alpha_1) + (+-alpha_2) + ... in plane
    order; the residual is the weight minus that level.

Parity pins: ``tests/test_quantize_oracle.py`` (the BiLoCo write-up's 3x2
greedy + joint-refit example, exact recovery of representable groups, the
least-squares normal equations and numpy's lstsq, brute-force and
binary-search nearest levels, closed forms, monotone error over rounds and
over precisions, frozen planes) and ``tests/test_quantize_mutations.py``.
"""

from __future__ import annotations

from typing import Dict, Tuple

import numpy as np

__all__ = ["tree_sum", "greedy_init", "ls_fit", "nearest_codes", "reconstruct", "quantize_groups",
           "quantize", "pack_signs"]


def tree_sum(v: np.ndarray) -> np.ndarray:
    """Pairwise sum over the last axis: halves added elementwise until one
    value is left (zero-padded to a power of two first)."""
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[-1]
    n2 = 1 << max(0, (n - 1).bit_length())
    if n2 != n:
        v = np.concatenate([v, np.zeros(v.shape[:-1] + (n2 - n,))], axis=-1)
    while v.shape[-1] > 1:
        h = v.shape[-1] // 2
        v = v[..., :h] + v[..., h:]
    return v[..., 0]


def _sign(r: np.ndarray) -> np.ndarray:
    """+1 where r >= 0 (sign(0) = +1), -1 elsewhere, as float64."""
    return np.where(r >= 0, 1.0, -1.0)


def greedy_init(w: np.ndarray, p: int, offset: bool = True) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Greedy BCQ of groups w [N][n]: returns (B [p][N][n] of +-1, alpha [p][N],
    z [N]).  With offset, z is the group mean and the planes fit w - z;
    without, z = 0."""
    w = np.asarray(w, dtype=np.float64)
    n = w.shape[-1]
    z = tree_sum(w) / n if offset else np.zeros(w.shape[0])
    r = w - z[:, None]
    B, A = [], []
    for _ in range(p):
        b = _sign(r)
        a = tree_sum(np.abs(r)) / n
        r = r - a[:, None] * b
        B.append(b)
        A.append(a)
    return np.array(B), np.array(A), z


def _gram_det(Gint, idx) -> int:
    """Exact determinant of the integer Gram submatrix on columns idx, by
    fraction-free (Bareiss) elimination in the order given.  The columns
    before the last are linearly independent, so every pivot before the last
    is positive and no row exchange is needed."""
    A = [[int(Gint[i][j]) for j in idx] for i in idx]
    n = len(A)
    prev = 1
    for k in range(n - 1):
        assert A[k][k] > 0
        for i in range(k + 1, n):
            for j in range(k + 1, n):
                A[i][j] = (A[i][j] * A[k][k] - A[i][k] * A[k][j]) // prev
        prev = A[k][k]
    return A[n - 1][n - 1]


def _kept_columns(Gint: np.ndarray, offset: bool) -> np.ndarray:
    """Which of the columns [planes..., ones] are kept: the offset column (when
    present) always, then each plane in order if it is linearly independent of
    the columns kept before it (exact integer rank test)."""
    n = Gint.shape[0]
    p = n - 1 if offset else n
    kept = [p] if offset else []
    for i in range(p):
        if _gram_det(Gint, kept + [i]) != 0:
            kept.append(i)
    mask = np.zeros(n, dtype=bool)
    mask[kept] = True
    return mask


def ls_fit(w: np.ndarray, B: np.ndarray, offset: bool = True) -> Tuple[np.ndarray, np.ndarray]:
    """Least-squares scales (and offset) for groups w [N][n] and planes B
    [p][N][n]: returns (alpha [p][N], z [N]) minimising ||w - z - sum alpha_i b_i||
    through the normal equations G theta = c, G_ij = <col_i, col_j>,
    c_i = <col_i, w>, columns [b_1..b_p, ones]."""
    w = np.asarray(w, dtype=np.float64)
    p, N, _ = B.shape
    cols = [B[i] for i in range(p)] + ([np.ones_like(w)] if offset else [])
    n = len(cols)
    G = np.empty((n, n, N))
    c = np.empty((n, N))
    for i in range(n):
        for j in range(n):
            G[i, j] = tree_sum(cols[i] * cols[j])
        c[i] = tree_sum(cols[i] * w)
    # dropped columns: identity row and column, zero right-hand side (their
    # coefficient solves to 0 and the elimination of the others is unchanged)
    for g in range(N):
        keep = _kept_columns(np.rint(G[:, :, g]).astype(np.int64), offset)
        for i in range(n):
            if not keep[i]:
                G[i, :, g] = 0.0
                G[:, i, g] = 0.0
                G[i, i, g] = 1.0
                c[i, g] = 0.0
    # Gaussian elimination without pivoting, in index order
    for k in range(n):
        for i in range(k + 1, n):
            f = G[i, k] / G[k, k]
            for j in range(k, n):
                G[i, j] = G[i, j] - f * G[k, j]
            c[i] = c[i] - f * c[k]
    th = np.zeros((n, N))
    for k in range(n - 1, -1, -1):
        s = c[k]
        for j in range(k + 1, n):
            s = s - G[k, j] * th[j]
        th[k] = s / G[k, k]
    z = th[p] if offset else np.zeros(N)
    return th[:p], z


def reconstruct(B: np.ndarray, alpha: np.ndarray, z: np.ndarray) -> np.ndarray:
    """W_hat [N][n] = z + (+-alpha_1) + ... in plane order."""
    lv = np.repeat(np.asarray(z, np.float64)[:, None], B.shape[2], axis=1)
    for i in range(B.shape[0]):
        lv = lv + np.where(B[i] > 0, alpha[i][:, None], -alpha[i][:, None])
    return lv


def nearest_codes(w: np.ndarray, alpha: np.ndarray, z: np.ndarray) -> np.ndarray:
    """Sign update: each weight's nearest level among the 2^p codes (first code
    in order on a tie).  Returns B [p][N][n] of +-1."""
    w = np.asarray(w, dtype=np.float64)
    p, N = alpha.shape
    best_d = np.full(w.shape, np.inf)
    best_c = np.zeros(w.shape, dtype=np.int64)
    for code in range(1 << p):
        lv = np.repeat(np.asarray(z, np.float64)[:, None], w.shape[1], axis=1)
        for i in range(p):
            a = alpha[i][:, None]
            lv = lv + (a if (code >> i) & 1 else -a)
        d = np.abs(w - lv)
        better = d < best_d
        best_d = np.where(better, d, best_d)
        best_c = np.where(better, code, best_c)
    return np.array([np.where((best_c >> i) & 1, 1.0, -1.0) for i in range(p)])


def quantize_groups(w: np.ndarray, P: int, p_low: int = 2, iters: int = 20, offset: bool = True,
                    trace: list = None):
    """The whole quantizer on groups w [N][n].  Returns (B [P][N][n],
    tables {p: (alpha [p][N], z [N])} for p = p_low..P).  With a list as
    `trace`, the squared error of every group is appended after each step
    (greedy, then each least-squares fit and sign update)."""
    w = np.asarray(w, dtype=np.float64)

    def err(B, a, z):
        return tree_sum((w - reconstruct(B, a, z)) ** 2)

    B, a, z = greedy_init(w, p_low, offset)
    if trace is not None:
        trace.append(("greedy", err(B, a, z)))
    for _ in range(iters):
        a, z = ls_fit(w, B, offset)
        if trace is not None:
            trace.append(("ls", err(B, a, z)))
        B = nearest_codes(w, a, z)
        if trace is not None:
            trace.append(("bs", err(B, a, z)))
    a, z = ls_fit(w, B, offset)
    tables = {p_low: (a, z)}
    planes = [B[i] for i in range(p_low)]
    for p in range(p_low, P):
        r = w - reconstruct(np.array(planes), a, z)
        planes.append(_sign(r))
        a, z = ls_fit(w, np.array(planes), offset)
        tables[p + 1] = (a, z)
    return np.array(planes), tables


def pack_signs(B: np.ndarray, M: int, K: int) -> np.ndarray:
    """Planes B [P][M*G][g] (+-1, groups row-major) -> canonical uint32 sign
    words [P][M][K/32], column k at bit k mod 32 of word k/32, set = +1."""
    P = B.shape[0]
    bits = (B.reshape(P, M, K) > 0).astype(np.uint8)
    return np.packbits(bits.reshape(P, M, K // 8, 8), axis=-1, bitorder="little").reshape(
        P, M, K // 8).view("<u4").reshape(P, M, K // 32).astype(np.uint32)


def quantize(W: np.ndarray, P: int, p_low: int = 2, iters: int = 20, g: int = 128):
    """Quantize W [M][K] (K a multiple of g) into P planes.  Returns
    (signs uint32 [P][M][K/32], alpha {p: float64 [p][M][G]},
    zero {p: float64 [M][G]}) for p = p_low..P."""
    W = np.asarray(W)
    M, K = W.shape
    if K % g or not (1 <= p_low <= P <= 4):
        raise ValueError("K must be a multiple of g and 1 <= p_low <= P <= 4")
    G = K // g
    B, tables = quantize_groups(W.astype(np.float64).reshape(M * G, g), P, p_low, iters)
    alpha = {p: a.reshape(p, M, G) for p, (a, _) in tables.items()}
    zero = {p: z.reshape(M, G) for p, (_, z) in tables.items()}
    return pack_signs(B, M, K), alpha, zero
