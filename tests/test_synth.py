"""The seeded generators produce the configured shapes, dtypes and distributions."""

import numpy as np
import pytest

import bcq_synth


def test_config1_shapes_and_dtypes():
    w = bcq_synth.config(1)
    assert (w.M, w.K, w.P, w.b, w.G) == (256, 512, 2, 1, 4)
    assert w.signs.shape == (2, 256, 16) and w.signs.dtype == np.uint32
    assert w.alpha.shape == (2, 256, 4) and w.alpha.dtype == np.float32
    assert w.zero.shape == (256, 4) and w.x.shape == (1, 512)
    assert list(w.p_req) == [2]


def test_config2_outliers_and_fp16():
    w = bcq_synth.config(2)
    assert w.x.dtype == np.float16 and w.alpha.dtype == np.float16
    assert len(w.outlier_channels) == 41  # 1% of 4096, rounded
    assert len(np.unique(w.outlier_channels)) == 41
    x = w.x[0].astype(np.float64)
    mask = np.zeros(w.K, bool)
    mask[w.outlier_channels] = True
    assert 10 < np.std(x[mask]) < 40 and 0.9 < np.std(x[~mask]) < 1.1


def test_config4_request_precisions():
    w = bcq_synth.config(4)
    assert w.b == 8 and set(np.unique(w.p_req)) <= {2, 3, 4}


def test_seeded_and_reproducible():
    a = bcq_synth.make(64, 256, 4, seed=5)
    b = bcq_synth.make(64, 256, 4, seed=5)
    c = bcq_synth.make(64, 256, 4, seed=6)
    for f in ("signs", "alpha", "zero", "x"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
        assert not np.array_equal(getattr(a, f), getattr(c, f))


def test_distributions():
    w = bcq_synth.make(512, 4096, 4, dtype=np.float32, seed=3)
    bits = np.unpackbits(w.signs.view(np.uint8))
    assert abs(bits.mean() - 0.5) < 0.002
    a = w.alpha.astype(np.float64)
    assert (a >= 0).all()
    # |N(0, 0.02)| has mean 0.02*sqrt(2/pi); each plane halves it
    assert abs(a[0].mean() - 0.02 * np.sqrt(2 / np.pi)) < 3e-4
    for i in range(1, 4):
        assert abs(a[i].mean() / a[i - 1].mean() - 0.5) < 0.02
    assert abs(w.zero.std() - 0.005) < 2e-4
    assert abs(w.x.std() - 1.0) < 0.05


def test_k_not_multiple_of_32_keeps_tail_bits_clear():
    w = bcq_synth.make(3, 4, 1, g=2, seed=1)
    assert (w.signs >> np.uint32(4)).max() == 0


def test_case_lists():
    assert len(bcq_synth.mlp_cases()) == 6
    assert len(bcq_synth.sweep_cases()) == 16


def test_independent_tables_shapes():
    w = bcq_synth.independent_tables(bcq_synth.make(16, 256, 4, seed=2))
    for p in range(1, 5):
        assert w.alpha_for(p).shape == (p, 16, 2) and w.zero_for(p).shape == (16, 2)


def test_rejects_ragged_groups():
    with pytest.raises(ValueError):
        bcq_synth.make(4, 100, 2)
