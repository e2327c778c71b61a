"""Pins of the oracle's 3D rotary embedding (CPU only)."""
import math

import numpy as np
import pytest

import oracle
from oracle import brute
import synth

H, DH, SECT = 3, 16, (4, 6, 6)


def _qk(n=11, seed=21):
    q = synth.normal_array((n, H * DH), seed).astype(np.float64)
    k = synth.normal_array((n, H * DH), seed + 1).astype(np.float64)
    pos = synth.uniform_ints((n, 3), 0, 40, seed + 2)
    return q, k, pos


def _scores(qr, kr):
    a = qr.reshape(-1, H, DH)
    b = kr.reshape(-1, H, DH)
    return np.einsum("ihd,jhd->hij", a, b)


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_relative_offset_invariance_per_axis(axis):
    """Shifting every position on one axis by the same amount leaves q.k unchanged."""
    q, k, pos = _qk()
    base = _scores(oracle.rope3d(q, pos, H, DH, SECT), oracle.rope3d(k, pos, H, DH, SECT))
    shifted = pos.copy()
    shifted[:, axis] += 123
    s2 = _scores(oracle.rope3d(q, shifted, H, DH, SECT), oracle.rope3d(k, shifted, H, DH, SECT))
    np.testing.assert_allclose(s2, base, rtol=0, atol=1e-10)
    # a shift of q alone changes the scores: the axis really is encoded
    s3 = _scores(oracle.rope3d(q, shifted, H, DH, SECT), oracle.rope3d(k, pos, H, DH, SECT))
    assert np.max(np.abs(s3 - base)) > 1e-3


def test_norm_preserved_and_zero_position_identity():
    q, _, pos = _qk(seed=30)
    r = oracle.rope3d(q, pos, H, DH, SECT)
    np.testing.assert_allclose(np.linalg.norm(r.reshape(-1, DH), axis=1),
                               np.linalg.norm(q.reshape(-1, DH), axis=1), rtol=1e-13)
    z = oracle.rope3d(q, np.zeros_like(pos), H, DH, SECT)
    np.testing.assert_array_equal(z, q)


def test_time_only_rows_leave_h_w_sections_untouched():
    q, _, pos = _qk(seed=31)
    pos[:, 1:] = 0
    r = oracle.rope3d(q, pos, H, DH, SECT).reshape(-1, H, DH)
    np.testing.assert_array_equal(r[:, :, SECT[0]:], q.reshape(-1, H, DH)[:, :, SECT[0]:])


def test_hand_evaluated_example():
    """Head of 8 dims split (2, 2, 4), theta = 10000, position (3, 5, 7).

    With a section of size 2 the only frequency is theta^0 = 1; with size 4 the
    second pair turns at theta^(-1/2) = 0.01.  Input pairs chosen as unit
    vectors, so each output pair is (cos, sin) of the angle, turned by 90
    degrees for an input of (0, 1).
    """
    x = np.array([[1.0, 0.0, 0.0, 1.0, 1.0, 0.0, 1.0, 0.0]])
    r = oracle.rope3d(x, [[3, 5, 7]], 1, 8, (2, 2, 4), 10000.0)[0]
    expect = [math.cos(3), math.sin(3),
              -math.sin(5), math.cos(5),
              math.cos(7), math.sin(7),
              math.cos(0.07), math.sin(0.07)]
    np.testing.assert_allclose(r, expect, rtol=0, atol=1e-14)


def test_frequencies_textbook_values():
    """theta^(-2j/s): s = 48 -> the last pair turns at 10000^(-46/48)."""
    w = oracle.rope_frequencies(48, 10000.0)
    assert w.shape == (24,)
    assert w[0] == 1.0
    assert abs(w[12] - 0.01) < 1e-16          # 10000^(-24/48)
    assert abs(w[-1] - 10000.0 ** (-46 / 48)) < 1e-18
    assert np.all(np.diff(w) < 0)


def test_brute_force_agreement():
    q, _, pos = _qk(n=6, seed=40)
    r = oracle.rope3d(q, pos, H, DH, SECT)
    rb = brute.rope(q.tolist(), pos.tolist(), H, DH, SECT)
    np.testing.assert_allclose(r, np.array(rb), rtol=0, atol=1e-12)


def test_rows_subset_matches_full():
    q, _, pos = _qk(seed=41)
    rows = [3, 0, 10]
    np.testing.assert_array_equal(oracle.rope3d(q, pos, H, DH, SECT, rows=rows),
                                  oracle.rope3d(q, pos, H, DH, SECT)[rows])


def test_rejects_bad_sections():
    q, _, pos = _qk()
    with pytest.raises(ValueError):
        oracle.rope3d(q, pos, H, DH, (5, 5, 6))
    with pytest.raises(ValueError):
        oracle.rope3d(q, pos, H, DH, (4, 4, 4))
