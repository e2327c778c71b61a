"""Pins of the oracle's FP8 (e4m3fn) quantization and FP8 projections (CPU only)."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def test_decode_known_codes():
    d = oracle.e4m3_decode
    assert d(0x00) == 0.0 and d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9
    assert d(0x08) == 2.0 ** -6            # smallest normal
    assert d(0x38) == 1.0 and d(0x39) == 1.125 and d(0x30) == 0.5
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert math.isnan(d(0x7F)) and math.isnan(d(0xFF))
    assert d(0x80) == 0.0 and math.copysign(1.0, d(0x80)) == -1.0
    pos = oracle.e4m3_table()[:0x7F]
    assert np.all(np.diff(pos) > 0)        # codes 0..0x7E increase strictly


def test_decode_table_matches_torch_float8():
    """torch's float8_e4m3fn (a library routine) decodes every code the same way."""
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_table()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    np.testing.assert_array_equal(got[~nan], ref[~nan])


def _probe_values(n=20000, seed=31):
    rng = np.random.Generator(np.random.PCG64(seed))
    tab = oracle.e4m3_table()
    fin = tab[np.isfinite(tab)]
    mids = (np.sort(np.unique(np.abs(fin)))[1:] + np.sort(np.unique(np.abs(fin)))[:-1]) / 2
    vals = np.concatenate([
        rng.standard_normal(n) * 30, rng.standard_normal(n) * 1e-3, fin, mids, -mids,
        np.nextafter(mids, 0), np.nextafter(mids, 1e9), [0.0, -0.0, 2.0 ** -10, -2.0 ** -11,
                                                          448.0, 460.0, 464.0, -463.9]])
    return vals


def test_vectorised_encoder_equals_bruteforce():
    v = _probe_values(3000)
    np.testing.assert_array_equal(oracle.e4m3_encode(v), oracle.e4m3_encode_bruteforce(v))


def test_encoder_matches_torch_within_range_and_saturates_beyond():
    v = _probe_values()
    v = v[np.abs(v) <= 464.0]
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.e4m3_encode(v.astype(np.float32)), ref)
    # beyond the last rounding midpoint: the reading saturates (torch gives NaN there)
    assert oracle.e4m3_encode([465.0, 1e6, -1e30]).tolist() == [0x7E, 0x7E, 0xFE]
    assert oracle.e4m3_encode([float("nan")]).tolist() == [0x7F]


def test_ties_go_to_the_even_code():
    enc = oracle.e4m3_encode
    assert enc([1.0625]).tolist() == [0x38]        # between 1.0 (0x38) and 1.125 (0x39)
    assert enc([1.1875]).tolist() == [0x3A]        # between 1.125 (0x39) and 1.25 (0x3A)
    assert enc([2.0 ** -10]).tolist() == [0x00]    # between 0 and the smallest subnormal
    assert enc([3 * 2.0 ** -10]).tolist() == [0x02]
    assert enc([464.0]).tolist() == [0x7E]


def test_round_trip_of_every_finite_code():
    tab = oracle.e4m3_table()
    codes = np.array([c for c in range(256) if np.isfinite(tab[c])], dtype=np.uint8)
    np.testing.assert_array_equal(oracle.e4m3_encode(tab[codes]), codes)


def test_row_quantization_properties():
    x = synth.normal_array((64, 96), 41) * np.linspace(0.01, 50, 64, dtype=np.float32)[:, None]
    x[3] = 0.0
    codes, s = oracle.quantize_rows(x)
    assert s.dtype == np.float32 and s[3] == 1.0 and (codes[3] == 0).all()
    np.testing.assert_array_equal(s[:3], (np.abs(x[:3]).max(1) / np.float32(448)).astype(np.float32))
    # each row's largest magnitude maps to +-448 (x / (amax / 448) is within an ulp of 448)
    big = np.abs(x).argmax(1)
    mags = oracle.e4m3_table()[codes[np.arange(64), big] & 0x7F]
    assert np.all((mags == 448.0) | (np.arange(64) == 3))
    # relative error of normal values at most half a mantissa step (1/16)
    dq = oracle.dequantize_rows(codes, s)
    normal = np.abs(x) / s[:, None] >= 2.0 ** -6
    rel = np.abs(dq - x)[normal] / np.abs(x)[normal]
    assert rel.max() <= 1.0 / 16 + 1e-12


def test_exactly_representable_inputs_give_an_exact_product():
    """Rows built from e4m3 values times a power of two quantize losslessly, so the FP8
    projection equals the plain product of the original matrices."""
    rng = np.random.Generator(np.random.PCG64(43))
    tab = oracle.e4m3_table()
    fin = tab[np.isfinite(tab) & (np.abs(tab) <= 448)]
    a = rng.choice(fin, size=(9, 64)) * 2.0 ** -3
    w = rng.choice(fin, size=(7, 64)) * 2.0 ** 5
    a[:, 0] = 448 * 2.0 ** -3                     # amax of every row is the top code
    w[:, 0] = -448 * 2.0 ** 5
    ac, asc = oracle.quantize_rows(a)
    wc, wsc = oracle.quantize_rows(w)
    np.testing.assert_array_equal(oracle.dequantize_rows(ac, asc), a)
    b = rng.standard_normal(7)
    np.testing.assert_allclose(oracle.linear_fp8(ac, asc, wc, wsc, b), a @ w.T + b, rtol=1e-13,
                               atol=1e-9)
