"""Pins for the float64 oracle, each independent of the oracle's own code.

Every check here computes its expectation by a route the oracle does not take
(the pages' worked example, NumPy bit unpacking + dense matmul, sign patterns
enumerated from an integer counter, popcount closed forms, algebraic identities),
so that a dropped term, a wrong sign, a wrong index or a transposed operand in
``oracle/bcq_oracle.c`` fails at least one of them.
"""

import json
import os

import numpy as np
import pytest

import bcq_synth
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def unpack_signs(signs: np.ndarray, K: int) -> np.ndarray:
    """{-1,+1} int8 [P][M][K] from canonical words, via NumPy's own bit unpacking."""
    P, M, W = signs.shape
    bytes_le = np.ascontiguousarray(signs.astype("<u4")).view(np.uint8).reshape(P, M, W * 4)
    bits = np.unpackbits(bytes_le, axis=-1, bitorder="little")[..., :K]
    return bits.astype(np.int8) * 2 - 1


def dense_numpy(signs, alpha, zero, p, K, g=128):
    """Dequantise with NumPy broadcasting: W = sum_i alpha_i * s_i + z (per group)."""
    s = unpack_signs(signs, K)[:p].astype(np.float64)
    a = np.repeat(np.asarray(alpha, np.float64)[:p], g, axis=-1)
    z = np.repeat(np.asarray(zero, np.float64), g, axis=-1)
    return (a * s).sum(axis=0) + z


def rel(a, b):
    return np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(np.asarray(b)), 1e-300)


# ---------------------------------------------------------------- worked example

def test_worked_example_add_subtract():
    """The BiLoCo page's hand-worked v.x = 3.4 (add/subtract only)."""
    ex = json.load(open(os.path.join(GOLDEN, "biloco_vx_example.json")))
    x = np.array(ex["x"])
    word = sum(1 << k for k, v in enumerate(ex["v"]) if v > 0)  # set bit = +1
    signs = np.array([[[word]]], dtype=np.uint32)
    y = oracle.gemv(signs, np.ones((1, 1, 1)), np.zeros((1, 1)), x, p=1, g=4)
    assert y.shape == (1,)
    assert abs(y[0] - ex["expected"]) < 1e-12


def test_worked_example_in_a_full_group():
    """Same example inside one 128-column group, two planes, second scale 0."""
    ex = json.load(open(os.path.join(GOLDEN, "biloco_vx_example.json")))
    K = 128
    x = np.zeros(K)
    x[:4] = ex["x"]
    signs = np.zeros((2, 1, K // 32), dtype=np.uint32)
    signs[0, 0, 0] = 0b0101
    signs[1, 0, :] = 0xFFFFFFFF
    alpha = np.array([[[1.0]], [[0.0]]])
    y = oracle.gemv(signs, alpha, np.zeros((1, 1)), x, p=2)
    assert abs(y[0] - ex["expected"]) < 1e-12


# ---------------------------------------------------------------- dense cross-check

@pytest.mark.parametrize("M,K,P,p,seed", [
    (8, 256, 4, 4, 1), (37, 384, 4, 2, 2), (5, 128, 3, 3, 3), (64, 512, 2, 1, 4), (3, 1024, 4, 3, 5),
])
def test_matches_dense_dequant_then_matmul(M, K, P, p, seed):
    w = bcq_synth.make(M, K, P, b=1, dtype=np.float16, seed=seed, outlier_frac=0.01)
    W = dense_numpy(w.signs, w.alpha, w.zero, p, K)
    y_ref = W @ w.x[0].astype(np.float64)
    y = oracle.gemv(w.signs, w.alpha, w.zero, w.x[0], p)
    assert rel(y, y_ref) < 1e-12
    Wo = oracle.dequant(w.signs, w.alpha, w.zero, p, K)
    assert np.max(np.abs(Wo - W)) < 1e-15


# ---------------------------------------------------------------- brute force

def test_brute_force_every_sign_pattern():
    """M=2, K=4, g=2, p=2: all 2**16 sign patterns, expectations built from the pattern index."""
    npat = 1 << 16
    Mrows, K, g, P = 2, 4, 2, 2
    M = npat * Mrows
    q = np.arange(npat, dtype=np.int64)
    # bit (i*8 + r*4 + k) of the pattern index is the sign of plane i, row r, column k
    sgn = np.empty((P, M, K), dtype=np.int64)
    for i in range(P):
        for r in range(Mrows):
            for k in range(K):
                sgn[i, r::Mrows, k] = ((q >> (i * 8 + r * 4 + k)) & 1) * 2 - 1
    words = np.zeros((P, M, 1), dtype=np.uint32)
    for k in range(K):
        words[..., 0] |= ((sgn[..., k] > 0).astype(np.uint32) << np.uint32(k))
    rng = np.random.default_rng(7)
    alpha = rng.standard_normal((P, M, K // g))
    zero = rng.standard_normal((M, K // g))
    x = rng.standard_normal(K)
    y = oracle.gemv(words, alpha, zero, x, p=2, g=g)
    ref = np.zeros(M)
    for k in range(K):
        j = k // g
        wk = zero[:, j] + alpha[0, :, j] * sgn[0, :, k] + alpha[1, :, j] * sgn[1, :, k]
        ref += wk * x[k]
    assert np.max(np.abs(y - ref)) < 1e-13


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("p", [1, 2, 3, 4])
def test_closed_form_all_ones_activation(p):
    """x = 1: y_m = sum_j [sum_i alpha_ijm (2*popcount - g) + g*z_mj]."""
    M, K, P, g = 16, 512, 4, 128
    w = bcq_synth.make(M, K, P, dtype=np.float32, seed=11)
    x = np.ones(K)
    y = oracle.gemv(w.signs, w.alpha, w.zero, x, p)
    G = K // g
    ref = np.zeros(M)
    for m in range(M):
        for j in range(G):
            acc = g * float(w.zero[m, j])
            for i in range(p):
                ones = sum(bin(int(wd)).count("1") for wd in w.signs[i, m, j * 4:(j + 1) * 4])
                acc += float(w.alpha[i, m, j]) * (2 * ones - g)
            ref[m] += acc
    assert np.max(np.abs(y - ref)) < 1e-12


def test_unit_vectors_recover_every_sign_bit():
    """x = e_k gives column k of the reconstruction; with scales 1, 1/2, 1/4, 1/8
    the signs can be read back greedily and must equal the stored bits."""
    M, K, P = 6, 256, 4
    w = bcq_synth.make(M, K, P, dtype=np.float32, seed=12)
    alpha = np.zeros((P, M, K // 128))
    for i in range(P):
        alpha[i] = 2.0 ** -i
    zero = np.full((M, K // 128), 0.03125)
    for k in range(K):
        x = np.zeros(K)
        x[k] = 1.0
        col = oracle.gemv(w.signs, alpha, zero, x, P) - zero[:, k // 128]
        for i in range(P):
            s = np.where(col > 0, 1, -1)
            bit = (w.signs[i, :, k // 32] >> np.uint32(k % 32)) & 1
            assert np.array_equal(s, bit.astype(int) * 2 - 1), (i, k)
            col = col - s * alpha[i, :, 0]
        assert np.max(np.abs(col)) < 1e-15


def test_special_case_all_bits_set():
    """All signs +1: y_m = sum_j (sum_i alpha + z) * S_j, S_j the group sum of x."""
    M, K, P = 4, 384, 3
    w = bcq_synth.make(M, K, P, dtype=np.float32, seed=13)
    signs = np.full_like(w.signs, 0xFFFFFFFF)
    x = w.x[0].astype(np.float64)
    S = x.reshape(-1, 128).sum(axis=1)
    ref = ((w.alpha.astype(np.float64).sum(axis=0) + w.zero) * S).sum(axis=1)
    assert rel(oracle.gemv(signs, w.alpha, w.zero, x, P), ref) < 1e-13


def test_special_case_offset_only():
    """alpha = 0, z = 1: y_m = sum_k x_k for every row (the offset sees the group sums)."""
    M, K, P = 5, 512, 2
    w = bcq_synth.make(M, K, P, dtype=np.float32, seed=14)
    x = w.x[0].astype(np.float64)
    y = oracle.gemv(w.signs, np.zeros_like(w.alpha), np.ones_like(w.zero), x, P)
    assert np.allclose(y, x.sum(), rtol=0, atol=1e-12)


def test_special_case_flipping_a_plane_negates_its_scale():
    M, K, P = 7, 256, 4
    w = bcq_synth.make(M, K, P, dtype=np.float32, seed=15)
    x = w.x[0]
    for i in range(P):
        flipped = w.signs.copy()
        flipped[i] ^= np.uint32(0xFFFFFFFF)
        neg = w.alpha.astype(np.float64).copy()
        neg[i] = -neg[i]
        a = oracle.gemv(flipped, w.alpha, w.zero, x, P)
        b = oracle.gemv(w.signs, neg, w.zero, x, P)
        assert np.max(np.abs(a - b)) < 1e-13


# ---------------------------------------------------------------- invariants

def test_prefix_invariant():
    """y_p - y_{p-1} = sum_j alpha_{p,m,j} (B_p x)_j for shared (aliased) scale tables."""
    M, K, P = 24, 512, 4
    w = bcq_synth.make(M, K, P, dtype=np.float16, seed=16, outlier_frac=0.01)
    x = w.x[0].astype(np.float64)
    s = unpack_signs(w.signs, K).astype(np.float64)
    ys = {p: oracle.gemv(w.signs, w.alpha, w.zero, x, p) for p in range(1, P + 1)}
    for p in range(2, P + 1):
        plane = (s[p - 1] * x).reshape(M, -1, 128).sum(axis=-1)  # (B_p x) per group
        term = (w.alpha[p - 1].astype(np.float64) * plane).sum(axis=1)
        assert np.max(np.abs((ys[p] - ys[p - 1]) - term)) < 1e-12 * max(1.0, np.abs(ys[p]).max())


def test_linearity():
    M, K, P = 9, 640, 4
    w = bcq_synth.make(M, K, P, b=2, dtype=np.float32, seed=17)
    x1, x2 = w.x.astype(np.float64)
    a, c = 0.75, -2.5
    lhs = oracle.gemv(w.signs, w.alpha, w.zero, a * x1 + c * x2, 3)
    rhs = a * oracle.gemv(w.signs, w.alpha, w.zero, x1, 3) + c * oracle.gemv(w.signs, w.alpha, w.zero, x2, 3)
    assert rel(lhs, rhs) < 1e-12


def test_requests_use_their_own_precision_tables():
    w = bcq_synth.independent_tables(bcq_synth.make(32, 256, 4, b=6, dtype=np.float16, seed=18,
                                                    p_choices=(1, 2, 3, 4)))
    y = oracle.gemv_requests(w.signs, w.x, w.p_req, w.alpha_for, w.zero_for)
    for r, p in enumerate(w.p_req):
        W = dense_numpy(w.signs, w.alpha_p[int(p)], w.zero_p[int(p)], int(p), w.K)
        assert rel(y[r], W @ w.x[r].astype(np.float64)) < 1e-12
        # the shared-prefix table gives a different answer, so the table choice is observable
        Wshared = dense_numpy(w.signs, w.alpha, w.zero, int(p), w.K)
        assert rel(y[r], Wshared @ w.x[r].astype(np.float64)) > 1e-3


def test_sign_encoding_lsb_first_set_bit_positive():
    signs = np.array([[[0x80000001, 0x00000002]]], dtype=np.uint32)
    K = 64
    got = [oracle.sign_at(signs, 0, 0, k, K) for k in range(K)]
    want = [-1] * K
    want[0] = want[31] = want[33] = +1
    assert got == want


def test_rejects_bad_precision():
    w = bcq_synth.make(4, 128, 2, dtype=np.float32, seed=19)
    with pytest.raises(ValueError):
        oracle.gemv(w.signs, w.alpha, w.zero, w.x[0], 0)
    with pytest.raises(ValueError):
        oracle.gemv(w.signs, w.alpha, w.zero, w.x[0], 3)


# ---------------------------------------------------------------- gated-MLP epilogue

def test_silu_mul_closed_form_points():
    """silu(g) = g / (1 + exp(-g)): 0 at 0, 3g/4 at ln 3, g/4 at -ln 3, g and 0 in the limits."""
    g = np.array([0.0, np.log(3.0), -np.log(3.0), 40.0, -40.0, 2.0])
    u = np.array([5.0, 2.0, 2.0, 0.5, 3.0, -1.0])
    got = oracle.silu_mul(g, u)
    assert got[0] == 0.0
    assert abs(got[1] - 0.75 * np.log(3.0) * 2.0) < 1e-15
    assert abs(got[2] + 0.25 * np.log(3.0) * 2.0) < 1e-15  # silu(-ln 3) = -ln3 / 4
    assert abs(got[3] - 40.0 * 0.5) < 1e-12 and abs(got[4]) < 1e-15
    assert abs(got[5] - (-2.0 / (1.0 + np.exp(-2.0)))) < 1e-15


def test_gate_up_rows_interleave():
    gr, ur = oracle.gate_up_rows(np.arange(20))
    assert list(gr[:10]) == [0, 1, 2, 3, 4, 5, 6, 7, 16, 17]
    assert list(ur[:10]) == [8, 9, 10, 11, 12, 13, 14, 15, 24, 25]
    assert sorted(np.concatenate([gr[:16], ur[:16]])) == list(range(32))


def test_gate_up_matches_dense_tile_by_tile():
    """Dense NumPy reconstruction, then each tile's gate and up rows paired by hand."""
    w = bcq_synth.make(48, 256, 3, seed=41, outlier_frac=0.01)
    x = w.x[0].astype(np.float64)
    for p in (1, 2, 3):
        yd = dense_numpy(w.signs, w.alpha, w.zero, p, w.K) @ x
        want = []
        for t in range(3):
            for i in range(8):
                gg, uu = yd[16 * t + i], yd[16 * t + 8 + i]
                want.append(gg / (1.0 + np.exp(-gg)) * uu)
        got = oracle.gemv_gate_up(w.signs, w.alpha, w.zero, x, p)
        assert got.shape == (24,)
        assert rel(got, want) < 1e-12


def test_gate_up_rejects_partial_tiles():
    w = bcq_synth.make(40, 128, 2, seed=3)
    with pytest.raises(ValueError):
        oracle.gemv_gate_up(w.signs, w.alpha, w.zero, w.x[0], 2)


# ---------------------------------------------------------------- binary low-rank correction

def test_lowrank_worked_example():
    """The BiLoCo page's v.x = 3.4 as a rank-1 correction of one output."""
    ex = json.load(open(os.path.join(GOLDEN, "biloco_vx_example.json")))
    x = np.array(ex["x"])
    vword = sum(1 << k for k, s in enumerate(ex["v"]) if s > 0)
    v = np.array([[vword]], dtype=np.uint32)
    for uword, a, y0, want in ((1, 1.0, 0.0, 3.4), (0, 1.0, 0.0, -3.4), (1, 2.0, 1.0, 7.8)):
        y = oracle.lowrank_correct(np.array([[uword]], np.uint32), v, [a], x, [y0])
        assert abs(y[0] - want) < 1e-12
    assert ex["expected"] == 3.4


def test_lowrank_closed_forms():
    w = bcq_synth.lowrank(5, 64, 7, dtype=np.float64, seed=2)
    ones_u = np.full_like(w.u, 0xFFFFFFFF)
    ones_v = np.full_like(w.v, 0xFFFFFFFF)
    zeros_v = np.zeros_like(w.v)
    sa, sx = np.sum(w.alpha), np.sum(w.x)
    y = oracle.lowrank_correct(ones_u, ones_v, w.alpha, w.x, w.y0)
    assert np.allclose(y, w.y0 + sa * sx, rtol=0, atol=1e-12)
    y = oracle.lowrank_correct(np.zeros_like(w.u), zeros_v, w.alpha, w.x, w.y0)  # (-1)(-1)
    assert np.allclose(y, w.y0 + sa * sx, rtol=0, atol=1e-12)
    y = oracle.lowrank_correct(ones_u, zeros_v, w.alpha, w.x, w.y0)
    assert np.allclose(y, w.y0 - sa * sx, rtol=0, atol=1e-12)


def test_lowrank_brute_force_loops():
    """Bit-by-bit Python loops over ranks, rows and columns."""
    w = bcq_synth.lowrank(6, 64, 37, dtype=np.float64, seed=5)
    want = []
    for m in range(w.M):
        acc = float(w.y0[m])
        for r in range(w.R):
            dot = 0.0
            for k in range(w.K):
                bit = (int(w.v[r][k // 32]) >> (k % 32)) & 1
                dot += w.x[k] if bit else -w.x[k]
            ub = (int(w.u[m][r // 32]) >> (r % 32)) & 1
            acc += float(w.alpha[r]) * (1.0 if ub else -1.0) * dot
        want.append(acc)
    got = oracle.lowrank_correct(w.u, w.v, w.alpha, w.x, w.y0)
    assert np.max(np.abs(got - np.array(want))) < 1e-12
