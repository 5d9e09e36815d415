"""Pins of the float64 quantizer reference (oracle/quantize.py) against facts
the pages and the mathematics fix, not against itself:

* the BiLoCo write-up's worked 3x2 example (greedy components, then a joint
  refit of their coefficients to zero error) -- tests/golden/biloco_greedy_3x2.json;
* exact recovery of a group that is exactly representable at precision p;
* least squares: the normal equations hold at the fit, and numpy's lstsq on the
  same columns gives the same scales; the two-column closed form;
* the sign update: every weight's code is a nearest level (brute force over
  itertools.product, and binary search over the sorted levels, the pages' "BS");
* monotonicity: the error never rises over the refinement steps, nor from
  precision p to p + 1 (AnyBCQ paper notes, progressive precision expansion:
  accuracy rises monotonically as bits are added);
* the expansion freezes earlier planes and adds sign(residual), sign(0) = +1;
* a plane that depends on the offset column gets scale 0.
"""

import bisect
import itertools
import json
import os

import numpy as np
import pytest

import bcq_synth
from oracle import quantize as q

GOLD = os.path.join(os.path.dirname(__file__), "golden", "biloco_greedy_3x2.json")


def sq_err(w, B, a, z):
    return q.tree_sum((np.asarray(w, np.float64) - q.reconstruct(B, a, z)) ** 2)


def test_biloco_3x2_greedy_then_joint_refit():
    g = json.load(open(GOLD))
    w = np.array([g["w"]], np.float64)
    B, a, z = q.greedy_init(w, 2, offset=False)
    assert np.array_equal(B[:, 0, :], np.array(g["greedy_planes"], np.float64))
    assert np.allclose(a[:, 0], g["greedy_alpha"], rtol=0, atol=1e-15)
    assert a[0, 0] == 12 / 6 and a[1, 0] == 8 / 6
    assert np.isclose(sq_err(w, B, a, z)[0], g["greedy_residual_sq"], rtol=1e-14)
    a2, z2 = q.ls_fit(w, B, offset=False)
    assert np.allclose(a2[:, 0], g["refit_alpha"], rtol=0, atol=1e-14)
    assert sq_err(w, B, a2, z2)[0] <= 1e-28


@pytest.mark.parametrize("p", [1, 2, 3, 4])
def test_exactly_representable_group_is_recovered(p):
    """w = z + sum_i alpha_i s_i with every code equally often (so the group
    mean is z) and alpha_i > sum_{j>i} alpha_j: greedy init finds it exactly,
    refinement keeps it, and every precision's error is zero."""
    alpha = [0.5, 0.1875, 0.0625, 0.015625][:p]
    z = 0.25
    codes = list(itertools.product([1.0, -1.0], repeat=p))
    rep = 128 // len(codes)
    S = np.array([c for c in codes for _ in range(rep)])  # [128][p]
    rng = np.random.default_rng(1)
    S = S[rng.permutation(128)]
    w = (z + S @ np.array(alpha))[None, :]
    B, tables = q.quantize_groups(w, p, p_low=p, iters=3)
    a, zz = tables[p]
    assert np.array_equal(B[:, 0, :], S.T)
    assert np.array_equal(a[:, 0], np.array(alpha)) and zz[0] == z
    assert sq_err(w, B, a, zz)[0] == 0.0


def random_groups(N=40, n=128, seed=3):
    W = bcq_synth.weights(N, n, seed=seed)
    return W.astype(np.float64)


@pytest.mark.parametrize("p", [1, 2, 3, 4])
def test_ls_fit_solves_normal_equations_and_matches_lstsq(p):
    w = random_groups()
    B, _, _ = q.greedy_init(w, p)
    a, z = q.ls_fit(w, B)
    for g in range(w.shape[0]):
        A = np.column_stack([B[i, g] for i in range(p)] + [np.ones(128)])
        theta = np.concatenate([a[:, g], [z[g]]])
        resid = w[g] - A @ theta
        assert np.max(np.abs(A.T @ resid)) <= 1e-12 * np.abs(A.T @ w[g]).max() + 1e-15
        ref = np.linalg.lstsq(A, w[g], rcond=None)[0]
        assert np.allclose(theta, ref, rtol=1e-10, atol=1e-14)


def test_ls_fit_two_columns_closed_form():
    """One plane and the offset: alpha = (mean over +1 - mean over -1) / 2 and
    z = (mean over +1 + mean over -1) / 2."""
    w = random_groups(N=20)
    B, _, _ = q.greedy_init(w, 1)
    a, z = q.ls_fit(w, B)
    for g in range(w.shape[0]):
        pos, neg = w[g][B[0, g] > 0], w[g][B[0, g] < 0]
        assert np.isclose(a[0, g], (pos.mean() - neg.mean()) / 2, rtol=1e-12, atol=1e-15)
        assert np.isclose(z[g], (pos.mean() + neg.mean()) / 2, rtol=1e-12, atol=1e-15)


def test_plane_dependent_on_offset_gets_zero_scale():
    """A constant group: the residual is exactly zero, the first plane is all
    +1 (sign(0) = +1) -- the offset column itself -- so it is dropped."""
    w = np.full((1, 128), 0.375)
    B, a, z = q.greedy_init(w, 1)
    assert np.all(B == 1.0)
    a2, z2 = q.ls_fit(w, B)
    assert a2[0, 0] == 0.0 and z2[0] == 0.375


@pytest.mark.parametrize("p", [1, 2, 3])
def test_nearest_codes_brute_force_and_binary_search(p):
    w = random_groups(N=12)
    rng = np.random.default_rng(p)
    a = np.abs(rng.normal(0, 0.02, size=(p, w.shape[0])))
    z = rng.normal(0, 0.005, size=w.shape[0])
    B = q.nearest_codes(w, a, z)
    got = q.reconstruct(B, a, z)
    for g in range(w.shape[0]):
        levels = sorted(z[g] + np.dot(s, a[:, g]) for s in itertools.product([1, -1], repeat=p))
        for k in range(128):
            best = min(abs(w[g, k] - L) for L in levels)
            assert abs(w[g, k] - got[g, k]) <= best * (1 + 1e-12) + 1e-18
            # binary search over the sorted levels
            i = bisect.bisect_left(levels, w[g, k])
            cand = [levels[j] for j in (i - 1, i) if 0 <= j < len(levels)]
            assert abs(w[g, k] - got[g, k]) <= min(abs(w[g, k] - c) for c in cand) * (1 + 1e-12) + 1e-18


def test_refinement_never_increases_the_error():
    w = random_groups(N=64, seed=11)
    trace = []
    q.quantize_groups(w, 2, p_low=2, iters=20, trace=trace)
    errs = [e for _, e in trace]
    for prev, cur in zip(errs, errs[1:]):
        assert np.all(cur <= prev * (1 + 1e-12) + 1e-20)
    assert np.all(errs[-1] < errs[0])  # refinement improves on the greedy start


def test_expansion_freezes_planes_adds_residual_sign_and_error_falls():
    w = random_groups(N=48, seed=5)
    B, tables = q.quantize_groups(w, 4, p_low=2, iters=20)
    B2, tables2 = q.quantize_groups(w, 2, p_low=2, iters=20)
    assert np.array_equal(B[:2], B2)  # the base planes do not move when P grows
    prev = None
    for p in (2, 3, 4):
        a, z = tables[p]
        e = sq_err(w, B[:p], a, z)
        if prev is not None:
            assert np.all(e <= prev * (1 + 1e-12) + 1e-20)
        prev = e
    for p in (2, 3):
        a, z = tables[p]
        r = w - q.reconstruct(B[:p], a, z)
        assert np.array_equal(B[p], np.where(r >= 0, 1.0, -1.0))


def test_expansion_scales_are_least_squares_for_frozen_planes():
    w = random_groups(N=16, seed=8)
    B, tables = q.quantize_groups(w, 4, p_low=2, iters=5)
    for p in (3, 4):
        a, z = tables[p]
        a2, z2 = q.ls_fit(w, B[:p])
        assert np.array_equal(a, a2) and np.array_equal(z, z2)


def test_quantize_layout_and_sign_words():
    W = bcq_synth.weights(8, 256, seed=2)
    signs, alpha, zero = q.quantize(W, 3, p_low=2, iters=2)
    assert signs.shape == (3, 8, 8) and signs.dtype == np.uint32
    assert sorted(alpha) == [2, 3] and alpha[3].shape == (3, 8, 2) and zero[2].shape == (8, 2)
    B, _ = q.quantize_groups(W.astype(np.float64).reshape(16, 128), 3, p_low=2, iters=2)
    for i in range(3):
        for m in range(8):
            for k in range(256):
                bit = (int(signs[i, m, k // 32]) >> (k % 32)) & 1
                assert bit == (B[i, m * 2 + k // 128, k % 128] > 0)


def test_tree_sum_is_pairwise():
    v = np.array([1e16, 1.0, -1e16, 1.0])
    # pairwise: (1e16 + -1e16) + (1.0 + 1.0) = 2.0; a left-to-right sum gives 1.0
    assert q.tree_sum(v) == 2.0
    assert q.tree_sum(np.arange(6.0)) == 15.0


def test_nearest_code_tie_goes_to_first_code():
    """A weight exactly between two levels takes the first code in order
    (code 0: every plane -1)."""
    w = np.zeros((1, 128))
    B = q.nearest_codes(w, np.array([[0.5]]), np.array([0.0]))
    assert np.all(B == -1.0)
