"""Each plausible mistake planted in a copy of the quantizer reference
(oracle/quantize.py) must fail at least one of its pins.  The copy is made
from the source text on the CPU; the reference itself is untouched."""

import os
import types

import numpy as np
import pytest

import test_quantize_oracle as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "quantize.py")

MUTANTS = {
    "sign_of_zero_is_minus": ("return np.where(r >= 0, 1.0, -1.0)",
                              "return np.where(r > 0, 1.0, -1.0)"),
    "greedy_scale_signed_mean": ("a = tree_sum(np.abs(r)) / n", "a = tree_sum(r) / n"),
    "greedy_without_centring": ("z = tree_sum(w) / n if offset else", "z = 0.0 * tree_sum(w) if offset else"),
    "new_plane_from_weights": ("planes.append(_sign(r))", "planes.append(_sign(w))"),
    "elimination_transposed_operand": ("G[i, j] = G[i, j] - f * G[k, j]",
                                       "G[i, j] = G[i, j] - f * G[j, k]"),
    "back_substitution_transposed": ("s = s - G[k, j] * th[j]", "s = s - G[j, k] * th[j]"),
    "dependent_plane_kept": ("if _gram_det(Gint, kept + [i]) != 0:", "if True:"),
    "ties_to_last_code": ("better = d < best_d", "better = d <= best_d"),
    "rhs_without_weights": ("c[i] = tree_sum(cols[i] * w)", "c[i] = tree_sum(cols[i] * np.abs(w))"),
    "tree_sum_drops_half": ("v = v[..., :h] + v[..., h:]", "v = v[..., :h] + v[..., :h]"),
    "expansion_from_stale_scales": ("        a, z = ls_fit(w, np.array(planes), offset)\n        tables[p + 1] = (a, z)",
                                    "        tables[p + 1] = (np.concatenate([a, np.zeros((1, a.shape[1]))]), z)\n        a, z = tables[p + 1]"),
}

PINS = [
    (pins.test_biloco_3x2_greedy_then_joint_refit, ()),
    (pins.test_exactly_representable_group_is_recovered, (2,)),
    (pins.test_exactly_representable_group_is_recovered, (3,)),
    (pins.test_ls_fit_solves_normal_equations_and_matches_lstsq, (3,)),
    (pins.test_ls_fit_two_columns_closed_form, ()),
    (pins.test_plane_dependent_on_offset_gets_zero_scale, ()),
    (pins.test_nearest_codes_brute_force_and_binary_search, (2,)),
    (pins.test_refinement_never_increases_the_error, ()),
    (pins.test_expansion_freezes_planes_adds_residual_sign_and_error_falls, ()),
    (pins.test_expansion_scales_are_least_squares_for_frozen_planes, ()),
    (pins.test_tree_sum_is_pairwise, ()),
    (pins.test_nearest_code_tie_goes_to_first_code, ()),
]


def mutant_module(old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("quantize_mutant")
    exec(compile(src.replace(old, new), SRC + " (mutant)", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_fails_a_pin(name, monkeypatch):
    mod = mutant_module(*MUTANTS[name])
    monkeypatch.setattr(pins, "q", mod)
    failed = []
    with np.errstate(all="ignore"):
        for fn, args in PINS:
            try:
                fn(*args)
            except Exception:  # an assertion, or arithmetic the mistake broke
                failed.append(fn.__name__)
    assert failed, "mutant %s passed every pin" % name


def test_unmutated_copy_passes_every_pin(monkeypatch):
    monkeypatch.setattr(pins, "q", mutant_module("import numpy as np", "import numpy as np"))
    for fn, args in PINS:
        fn(*args)
