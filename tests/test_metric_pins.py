"""Pins of the parity metric itself (CPU): the relative Frobenius error
||x - ref||_F / ||ref||_F that every GPU parity test gates on, its zero-
reference rule, its combination over pieces and its per-(b, h) form, checked
against hand-computed values so that a wrong denominator, a missing square
root, a spectral instead of a Frobenius norm or a mishandled zero reference
fails here.  The GPU tests' helper (tests/parity.py) is checked too."""
import math

import numpy as np
import pytest

import oracle
from tests import parity


def test_hand_values():
    # measured against the reference: x = 2 ref gives 1 (against ||x|| it would read 0.5)
    assert oracle.rel_frobenius([2.0, 0.0], [1.0, 0.0]) == 1.0
    assert oracle.rel_frobenius([1.0, 0.0], [2.0, 0.0]) == 0.5
    # [[1,2],[3,4]] against [[1,2],[3,5]]: 1 / sqrt(1 + 4 + 9 + 25)
    assert oracle.rel_frobenius([[1, 2], [3, 4]], [[1, 2], [3, 5]]) == pytest.approx(1 / math.sqrt(39), rel=1e-15)
    # Frobenius, not spectral: the difference diag(1, 1) has Frobenius norm sqrt 2 (spectral 1),
    # the reference diag(3, 4) Frobenius norm 5 (spectral 4)
    assert oracle.rel_frobenius([[4, 0], [0, 5]], [[3, 0], [0, 4]]) == pytest.approx(math.sqrt(2) / 5, rel=1e-15)
    assert oracle.rel_frobenius(np.ones((3, 4, 5)), np.ones((3, 4, 5))) == 0.0


def test_zero_reference_reports_the_absolute_error():
    assert oracle.rel_frobenius([3.0, 4.0], [0.0, 0.0]) == 5.0
    assert oracle.rel_frobenius([0.0, 0.0], [0.0, 0.0]) == 0.0
    assert oracle.rel_frobenius(np.zeros((0, 4)), np.zeros((0, 4))) == 0.0


def test_scale_invariance_and_shape_check():
    rng = np.random.default_rng(0)
    x, r = rng.standard_normal((4, 5, 6)), rng.standard_normal((4, 5, 6))
    assert oracle.rel_frobenius(8 * x, 8 * r) == pytest.approx(oracle.rel_frobenius(x, r), rel=1e-14)
    with pytest.raises(ValueError):
        oracle.rel_frobenius(np.zeros(4), np.zeros(5))


def test_pieces_combine_to_the_whole():
    rng = np.random.default_rng(1)
    x, r = rng.standard_normal((2, 7, 30, 8)), rng.standard_normal((2, 7, 30, 8))
    parts = [oracle.frobenius_parts(x[:, a:b], r[:, a:b]) for a, b in ((0, 3), (3, 4), (4, 7))]
    assert oracle.combine_rel_frobenius(parts) == pytest.approx(oracle.rel_frobenius(x, r), rel=1e-14)
    assert oracle.combine_rel_frobenius([(3.0, 0.0), (4.0, 0.0)]) == 5.0


def test_per_slice_errors():
    ref = np.ones((2, 3, 4, 4))
    x = ref.copy()
    x[1, 2] *= 1.5          # one slice off by 50 %
    x[0, 1, 0, 0] += 4.0    # one element of another off by 4 against a slice norm of 4
    per = oracle.rel_frobenius_per_slice(x, ref)
    expect = np.zeros((2, 3))
    expect[1, 2], expect[0, 1] = 0.5, 1.0
    np.testing.assert_allclose(per, expect, rtol=1e-15, atol=0)
    z = np.zeros((1, 2, 3))
    assert oracle.rel_frobenius_per_slice(z + [[[0.0], [2.0]]], z).tolist() == [[0.0, math.sqrt(12)]]


def test_gate_catches_one_wrong_row_that_the_whole_tensor_hides():
    """2 x 6 heads of 300 rows: one row 80 % wrong moves the whole-tensor
    error to about 0.8/sqrt(3600) = 0.013, under a 2e-2 tolerance, but its
    head's to about 0.8/sqrt(300) = 0.046; the per-(b, h) gate must fail."""
    rng = np.random.default_rng(2)
    ref = rng.standard_normal((2, 6, 300, 64))
    got = ref * (1 + 1e-3 * rng.standard_normal(ref.shape))
    got[1, 1, 17] = ref[1, 1, 17] * 0.2
    assert oracle.rel_frobenius(got, ref) < 0.015
    with pytest.raises(AssertionError, match="worst"):
        parity.check("planted row", got, ref, 2e-2)
    parity.check("clean", got[:, :1], ref[:, :1], 2e-2)


def test_head_groups_accumulate_like_one_comparison():
    rng = np.random.default_rng(3)
    ref = rng.standard_normal((2, 8, 50, 16))
    got = ref + 1e-4 * rng.standard_normal(ref.shape)
    acc = parity.HeadGroups("groups", 1e-3)
    for h0 in range(0, 8, 3):
        acc.add(got[:, h0:h0 + 3], ref[:, h0:h0 + 3], h0)
    assert acc.finish() == pytest.approx(oracle.rel_frobenius(got, ref), rel=1e-13)
    got[1, 6] *= 1.01
    bad = parity.HeadGroups("one head off", 1e-3)
    for h0 in range(0, 8, 3):
        bad.add(got[:, h0:h0 + 3], ref[:, h0:h0 + 3], h0)
    assert bad.worst[1] == (1, 6)
    with pytest.raises(AssertionError):
        bad.finish()
