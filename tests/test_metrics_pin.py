"""Pins of the parity figure every GPU test goes through (CPU only).

``oracle.metrics(x, ref)`` reports max_i |x_i - ref_i| / sqrt(mean_i ref_i^2)
(the tolerance reading of max-abs-error / RMS: the error's largest magnitude
over the RMS of the oracle's values), the absolute maximum error and the RMS
error.  Each case below is worked by hand; together they catch the plausible
slips: dividing by the RMS of x or of the error instead of the reference's,
a mean error in place of the maximum, a signed in place of an absolute error,
a zero RMS read as "no error", or a NaN lost in a maximum.  ``Metrics`` is the
same figure accumulated over pieces, and must agree with one call on the whole.
"""
import math

import numpy as np
import pytest

import oracle


def test_hand_worked_case():
    # errors 0, 0, 2 (x below ref at the last element); RMS(ref) = sqrt((1 + 4 + 25) / 3) = sqrt(10)
    m = oracle.metrics([1.0, 2.0, 3.0], [1.0, 2.0, 5.0])
    assert m["max_abs"] == 2.0
    assert m["rms_ref"] == pytest.approx(math.sqrt(10.0), rel=1e-15)
    assert m["max_over_rms"] == pytest.approx(2.0 / math.sqrt(10.0), rel=1e-15)
    assert m["rms_err"] == pytest.approx(math.sqrt(4.0 / 3.0), rel=1e-15)


def test_divides_by_the_reference_rms_and_takes_the_max():
    # ref = ones: RMS(ref) = 1.  x = (4, 1, 1, 1): errors (3, 0, 0, 0).
    #   max/RMS(ref) = 3;  RMS(x) = sqrt(19 / 4) and RMS(err) = 1.5 would give other figures,
    #   and a mean error would give 0.75.
    m = oracle.metrics([4.0, 1.0, 1.0, 1.0], [1.0, 1.0, 1.0, 1.0])
    assert m["max_over_rms"] == 3.0
    assert m["max_abs"] == 3.0
    assert m["rms_err"] == 1.5
    assert m["rms_ref"] == 1.0


def test_absolute_error_and_any_shape():
    # a negative error of -6 at one element of a 2 x 2 array; ref entries 3, 4, 0, 0:
    # RMS(ref) = sqrt(25 / 4) = 2.5, so the figure is 6 / 2.5 = 2.4
    x = np.array([[3.0, -2.0], [0.0, 0.0]])
    ref = np.array([[3.0, 4.0], [0.0, 0.0]])
    m = oracle.metrics(x, ref)
    assert m["max_abs"] == 6.0
    assert m["rms_ref"] == 2.5
    assert m["max_over_rms"] == pytest.approx(2.4, rel=1e-15)
    assert m["rms_err"] == 3.0  # sqrt(36 / 4)


def test_zero_reference():
    assert oracle.metrics([0.0, 0.0], [0.0, 0.0])["max_over_rms"] == 0.0
    m = oracle.metrics([0.0, 1e-30], [0.0, 0.0])
    assert m["max_over_rms"] == float("inf") and m["max_abs"] == 1e-30


def test_empty_input():
    m = oracle.metrics(np.zeros((0, 3)), np.zeros((0, 3)))
    assert m == {"max_over_rms": 0.0, "max_abs": 0.0, "rms_err": 0.0, "rms_ref": 0.0}


def test_non_finite_results_are_not_hidden():
    m = oracle.metrics([1.0, np.nan, 1.0], [1.0, 1.0, 1.0])
    assert not (m["max_over_rms"] <= 1e-4)
    m = oracle.metrics([1.0, np.inf], [1.0, 1.0])
    assert m["max_over_rms"] == float("inf")
    # a NaN in an early piece survives later finite pieces
    acc = oracle.Metrics().add([np.nan], [1.0]).add([2.0], [1.0])
    assert math.isnan(acc.result()["max_over_rms"])


def test_shape_mismatch_is_an_error():
    with pytest.raises(ValueError):
        oracle.metrics(np.zeros(3), np.zeros(4))


def test_pieces_agree_with_the_whole():
    r = np.random.default_rng(0)
    ref = r.standard_normal((7, 5, 3))
    x = ref + 1e-3 * r.standard_normal(ref.shape)
    whole = oracle.metrics(x, ref)
    acc = oracle.Metrics()
    for i in range(7):  # uneven pieces, one of them empty
        acc.add(x[i, : i % 5], ref[i, : i % 5])
        acc.add(x[i, i % 5:], ref[i, i % 5:])
    part = acc.result()
    assert part["max_abs"] == whole["max_abs"]
    for key in ("max_over_rms", "rms_err", "rms_ref"):
        assert part[key] == pytest.approx(whole[key], rel=1e-13)


def test_bf16_storage_allowance():
    """The bf16-output check allows each element the rounding of its own storage and no more:
    fp32 values rounded to nearest even bf16 pass with no further tolerance, while values
    moved two bf16 units away fail; an element's allowance does not grow with the others'."""
    from kda_testlib import assert_close_bf16_storage
    import synth

    r = np.random.default_rng(3)
    ref = (r.standard_normal(4096) * np.exp(r.uniform(-3, 3, 4096))).astype(np.float32)
    rounded = synth.f32_to_bf16_bits(ref)
    got = (rounded.astype(np.uint32) << 16).view(np.float32)
    assert_close_bf16_storage("rounded", got, ref, 0.0)
    # 2^-6 of its magnitude (two to four bf16 units in the last place) at one element
    bad = got.copy()
    i = int(np.argmax(np.abs(ref)))
    bad[i] = np.float32(ref[i] * (1 + 2.0 ** -6))
    with pytest.raises(AssertionError):
        assert_close_bf16_storage("moved", bad, ref, 1e-3)
    # a large element's allowance does not cover a small one: moving the smallest element by
    # 2^-8 of the largest fails
    bad = got.copy()
    j = int(np.argmin(np.abs(ref)))
    bad[j] = np.float32(ref[j] + 2.0 ** -8 * np.abs(ref).max())
    with pytest.raises(AssertionError):
        assert_close_bf16_storage("small", bad, ref, 1e-3)
