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


# ---------------------------------------------------------------------------
# FP8 block halves
# ---------------------------------------------------------------------------

def _e4m3_grid_rows(rng, shape, top):
    """Rows of e4m3 values times 2^-6 whose largest magnitude is ``top`` = 448 * 2^-6
    (so the per-row scale is exactly 2^-6 and quantization is lossless)."""
    tab = oracle.e4m3_table()
    fin = tab[np.isfinite(tab) & (np.abs(tab) <= 448)]
    a = rng.choice(fin, size=shape) * 2.0 ** -6
    a[..., 0] = top
    return a


def _half_steps(v, s):
    """Half the e4m3 spacing at each |v| / s (per-row scale s), times s: the largest
    error of a nearest rounding of an unsaturated value."""
    u = np.abs(v) / s[:, None]
    e = np.floor(np.log2(np.maximum(u, 2.0 ** -6)))
    return s[:, None] * 2.0 ** (e - 4)


def _lossless_block(seed, d=16, h=2, n=12, with_bias=True):
    """Inputs whose AdaLN output is exactly representable: unit-free modulation
    (scale row -1, so y = shift[m]) with shift rows on the e4m3 grid."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((n, d))
    table = rng.standard_normal((3, 3, d)) * 0.3
    table[:, 1, :] = -1.0
    table[:, 0, :] = _e4m3_grid_rows(rng, (3, d), 7.0)
    mod = rng.integers(0, 3, n)
    pos = rng.integers(0, 9, (n, 3))
    wq = oracle.quantize_rows(rng.standard_normal((3 * d, d)) * 0.3)
    wo = oracle.quantize_rows(rng.standard_normal((d, d)) * 0.3)
    b_qkv = rng.standard_normal(3 * d) * 0.1 if with_bias else None
    b_o = rng.standard_normal(d) * 0.1 if with_bias else None
    return x, table, mod, pos, wq, wo, b_qkv, b_o


def test_fp8_adaln_of_a_grid_shift_is_exact():
    """y = shift[m] on the e4m3 grid: the codes are the shift's own codes, the scale 2^-6."""
    x, table, mod, _, _, _, _, _ = _lossless_block(71)
    codes, s = oracle.adaln_modulate_fp8(x, mod, table)
    np.testing.assert_array_equal(s, np.full(x.shape[0], 2.0 ** -6, np.float32))
    np.testing.assert_array_equal(codes, oracle.e4m3_encode(table[mod, 0, :] * 64.0))
    np.testing.assert_array_equal(oracle.dequantize_rows(codes, s), table[mod, 0, :])


def test_fp8_adaln_codes_are_within_half_a_step_of_the_modulated_rows():
    rng = np.random.Generator(np.random.PCG64(72))
    x = rng.standard_normal((40, 64)) * 3 + 1
    table = rng.standard_normal((3, 3, 64)) * 0.2
    mod = rng.integers(0, 3, 40)
    y = oracle.adaln_modulate(x, mod, table)
    codes, s = oracle.adaln_modulate_fp8(x, mod, table)
    np.testing.assert_array_equal(s, (np.abs(y.astype(np.float32)).max(1) / np.float32(448)))
    err = np.abs(oracle.dequantize_rows(codes, s) - y)
    assert np.all(err <= _half_steps(y, s.astype(np.float64)) * (1 + 1e-6) + 1e-12)
    big = np.abs(y).argmax(1)
    assert np.all(oracle.e4m3_table()[codes[np.arange(40), big] & 0x7F] == 448.0)


@pytest.mark.parametrize("with_bias", [False, True])
def test_fp8_block_with_a_lossless_adaln_output_matches_the_plain_block(with_bias):
    """With y exactly representable, q, k, v and o equal the plain oracle's with the
    dequantized weights, and out differs from it only by the rounding of o, which is
    bounded by half an e4m3 step per element of o."""
    x, table, mod, pos, wq, wo, b_qkv, b_o = _lossless_block(73, with_bias=with_bias)
    kw = dict(n_heads=2, head_dim=8, sections=(2, 2, 4), theta=100.0)
    cu = [0, 5, 12]
    f8 = oracle.block_forward_fp8(x, mod, pos, cu, table, *wq, *wo, b_qkv=b_qkv, b_o=b_o, **kw)
    w_qkv, w_o = oracle.dequantize_rows(*wq), oracle.dequantize_rows(*wo)
    ref = oracle.block_forward(x, mod, pos, cu, table, w_qkv, w_o, b_qkv=b_qkv, b_o=b_o, **kw)
    for key in ("q", "k", "v", "o"):
        np.testing.assert_allclose(f8[key], ref[key], rtol=1e-12, atol=1e-12)
    o = ref["o"]
    s = oracle.row_scales(o).astype(np.float64)
    bound = np.abs(table[mod, 2, :]) * (_half_steps(o, s) @ np.abs(w_o).T)
    diff = np.abs(f8["out"] - ref["out"])
    assert np.all(diff <= bound * (1 + 1e-6) + 1e-12)
    assert diff.max() > 0                     # o is not on the grid: its rounding shows


def test_fp8_ffn_with_a_lossless_adaln_output_matches_the_plain_half():
    x, table, mod, _, _, _, _, _ = _lossless_block(74, d=32, n=20)
    rng = np.random.Generator(np.random.PCG64(75))
    w1 = oracle.quantize_rows(rng.standard_normal((128, 32)) * 0.3)
    w2 = oracle.quantize_rows(rng.standard_normal((32, 128)) * 0.3)
    b1, b2 = rng.standard_normal(128) * 0.1, rng.standard_normal(32) * 0.1
    f8 = oracle.ffn_forward_fp8(x, mod, table, *w1, *w2, b1=b1, b2=b2)
    W1, W2 = oracle.dequantize_rows(*w1), oracle.dequantize_rows(*w2)
    y = oracle.adaln_modulate(x, mod, table)
    h = oracle.ffn_up(y, W1, b1)
    np.testing.assert_array_equal(f8["h"], h)
    ref = oracle.ffn_forward(x, mod, table, W1, W2, b1, b2)
    s = oracle.row_scales(h).astype(np.float64)
    bound = np.abs(table[mod, 2, :]) * (_half_steps(h, s) @ np.abs(W2).T)
    diff = np.abs(f8["out"] - ref)
    assert np.all(diff <= bound * (1 + 1e-6) + 1e-12) and diff.max() > 0


def test_fp8_block_rows_subset_matches_every_row():
    x, table, mod, pos, wq, wo, b_qkv, b_o = _lossless_block(76)
    table[:, 1, :] = 0.1                      # a general (lossy) modulation
    kw = dict(n_heads=2, head_dim=8, sections=(2, 2, 4), b_qkv=b_qkv, b_o=b_o)
    full = oracle.block_forward_fp8(x, mod, pos, [0, 5, 12], table, *wq, *wo, **kw)
    rows = np.array([0, 4, 5, 11])
    part = oracle.block_forward_fp8(x, mod, pos, [0, 5, 12], table, *wq, *wo, rows=rows, **kw)
    np.testing.assert_allclose(part["out"], full["out"][rows], rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(part["o_codes"], full["o_codes"][rows])


def test_fp8_block_tiny_workload_is_close_to_the_unquantized_block():
    """The tiny workload with weights quantized per row: the branch out - x within
    rel-L2 8e-2 of the plain oracle's (four e4m3 roundings in series, each about 2.6%
    RMS), the output itself within the bf16 output tolerance."""
    wl = synth.WORKLOADS["tiny"]
    lay = oracle.pack_layout([r.grid for r in wl.requests])
    inp = synth.block_inputs(wl)
    kw = dict(n_heads=wl.n_heads, head_dim=wl.head_dim, sections=wl.sections)
    args = (inp.x, lay["modality"], lay["pos"], lay["cu_seqlens"], inp.table)
    f8 = oracle.block_forward_fp8(*args, *oracle.quantize_rows(inp.w_qkv),
                                  *oracle.quantize_rows(inp.w_o), **kw)
    ref = oracle.block_forward(*args, inp.w_qkv, inp.w_o, **kw)
    x = inp.x.astype(np.float64)
    rel = np.linalg.norm((f8["out"] - x) - (ref["out"] - x)) / np.linalg.norm(ref["out"] - x)
    assert 5e-3 < rel < 8e-2
    assert np.abs(f8["out"] - ref["out"]).max() <= 3e-2
    assert np.linalg.norm(f8["out"] - ref["out"]) <= 1e-2 * np.linalg.norm(ref["out"])


# ---------------------------------------------------------------------------
# FP8 attention: q per (token, head) row, k and v per head, exact probabilities
# ---------------------------------------------------------------------------

def _grid_rows(rng, n_rows, width, exps):
    """Rows of e4m3 grid values times 2^e (e per row), each row holding one
    +-448 * 2^e element: the row's amax / 448 is exactly 2^e, so per-row
    quantization reproduces the row bit for bit."""
    tab = oracle.e4m3_table()
    fin = tab[np.isfinite(tab)]
    vals = rng.choice(fin[np.abs(fin) <= 64.0], size=(n_rows, width))
    vals[np.arange(n_rows), rng.integers(0, width, n_rows)] = 448.0 * rng.choice([-1.0, 1.0], n_rows)
    return vals * (2.0 ** np.asarray(exps, np.float64))[:, None]


def test_quantize_tensor_scale_codes_and_zero():
    rng = np.random.Generator(np.random.PCG64(5))
    x = (rng.standard_normal((37, 19)) * 3.0).astype(np.float32)
    codes, s = oracle.quantize_tensor(x)
    amax = np.float32(np.max(np.abs(x)))
    assert s == np.float32(amax / np.float32(448.0))
    i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert codes[i] in (0x7E, 0xFE)                     # the amax lands on +-448
    dec = oracle.e4m3_table()[codes] * np.float64(s)
    err = np.abs(dec - x)
    normal = np.abs(x) / s >= 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(x[normal]) * (1 + 1e-6))
    assert np.all(err[~normal] <= 2.0 ** -10 * s * (1 + 1e-6))
    zc, zs = oracle.quantize_tensor(np.zeros((4, 4)))
    assert zs == np.float32(1.0) and not zc.any()


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_attention_of_grid_operands_is_the_plain_attention(causal):
    """Operands on the e4m3 grid with q's power-of-two scale varying per
    (token, head) row and k's, v's per (segment, head), each (segment, head)
    block holding one +-448 * scale element: quantization is lossless, so the
    FP8 attention equals the plain one.  The second segment's k and v scales
    are 3/4 of the first's: a scale over the whole pack (one per head) would
    put 0.75 m, off the e4m3 grid for most grid values m, on its codes and
    fail, as would quantizing q per head or k, v per row."""
    rng = np.random.Generator(np.random.PCG64(11))
    n, hh, dh = 40, 2, 16
    cu = [0, 17, 40]
    q = _grid_rows(rng, n * hh, dh, rng.integers(-9, -4, n * hh)).reshape(n, hh * dh)
    k = np.empty((n, hh * dh))
    v = np.empty((n, hh * dh))
    want = {"k": np.zeros((2, hh), np.float32), "v": np.zeros((2, hh), np.float32)}
    for h in range(hh):
        cols = slice(h * dh, (h + 1) * dh)
        for name, t, e in (("k", k, -7 + h), ("v", v, -6 - h)):
            for s, (a, b) in enumerate(zip(cu, cu[1:])):
                sc = 2.0 ** e * (1.0 if s == 0 else 0.75)
                blk = _grid_rows(rng, b - a, dh, np.zeros(b - a))
                blk[np.abs(blk) == 448.0] = 64.0                 # one 448 per block only
                blk[rng.integers(0, b - a), rng.integers(0, dh)] = -448.0
                t[a:b, cols] = blk * sc
                want[name][s, h] = sc
    r = oracle.attention_fp8(q, k, v, cu, hh, dh, causal=causal)
    qd, kd, vd = oracle.dequantize_attention_operands(r, hh, dh)
    np.testing.assert_array_equal(qd, q)
    np.testing.assert_array_equal(kd, k)
    np.testing.assert_array_equal(vd, v)
    ref = oracle.attention(q, k, v, cu, hh, dh, causal=causal)
    np.testing.assert_allclose(r["o"], ref, rtol=1e-12, atol=1e-15)
    assert np.array_equal(r["k_scales"], want["k"])
    assert np.array_equal(r["v_scales"], want["v"])
    # the same operands quantized with one scale per head over the whole pack
    # are not lossless: the reading per segment is what the equality checks
    whole = oracle.attention_fp8_operands(q, k, v, hh, dh)
    _, kw, vw = oracle.dequantize_attention_operands(whole, hh, dh)
    assert not (np.array_equal(kw, k) and np.array_equal(vw, v))


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_attention_with_zero_queries_averages_the_values(causal):
    """q = 0 gives every key the same weight: o is the mean of the dequantized
    v over the query's keys (its segment, or the segment's prefix when
    causal), and o_abs the mean of |v|."""
    rng = np.random.Generator(np.random.PCG64(12))
    n, hh, dh = 30, 2, 8
    cu = [0, 7, 30]
    q = np.zeros((n, hh * dh))
    k = rng.standard_normal((n, hh * dh))
    v = rng.standard_normal((n, hh * dh)) * 2.0
    r = oracle.attention_fp8(q, k, v, cu, hh, dh, causal=causal)
    _, _, vd = oracle.dequantize_attention_operands(r, hh, dh)
    for s in range(len(cu) - 1):
        for i in range(cu[s], cu[s + 1]):
            keys = slice(cu[s], i + 1 if causal else cu[s + 1])
            np.testing.assert_allclose(r["o"][i], vd[keys].mean(axis=0), rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(r["o_abs"][i], np.abs(vd[keys]).mean(axis=0), rtol=1e-12)
    assert np.all(r["q_scales"] == 1.0) and not r["q_codes"].any()


def test_fp8_attention_per_head_scaling():
    """Scaling one head's v by 8 scales that head's o by exactly 8 (its codes
    are unchanged, its scale is 8 times larger) and leaves the other heads
    bit for bit; o_abs bounds |o| (triangle inequality)."""
    rng = np.random.Generator(np.random.PCG64(13))
    n, hh, dh = 26, 3, 8
    cu = [0, 11, 26]
    q = rng.standard_normal((n, hh * dh))
    k = rng.standard_normal((n, hh * dh))
    v = rng.standard_normal((n, hh * dh))
    a = oracle.attention_fp8(q, k, v, cu, hh, dh)
    v2 = v.copy()
    v2[:, dh:2 * dh] *= 8.0
    b = oracle.attention_fp8(q, k, v2, cu, hh, dh)
    np.testing.assert_array_equal(a["v_codes"], b["v_codes"])
    assert np.array_equal(b["v_scales"][:, 1], 8 * a["v_scales"][:, 1])
    np.testing.assert_allclose(b["o"][:, dh:2 * dh], 8 * a["o"][:, dh:2 * dh], rtol=1e-12)
    np.testing.assert_array_equal(b["o"][:, :dh], a["o"][:, :dh])
    np.testing.assert_array_equal(b["o"][:, 2 * dh:], a["o"][:, 2 * dh:])
    assert np.all(np.abs(a["o"]) <= a["o_abs"] * (1 + 1e-12))


def test_fp8_attention_rows_subset_matches_every_row():
    rng = np.random.Generator(np.random.PCG64(14))
    n, hh, dh = 33, 2, 8
    cu = [0, 20, 33]
    q, k, v = (rng.standard_normal((n, hh * dh)) for _ in range(3))
    full = oracle.attention_fp8(q, k, v, cu, hh, dh, causal=True)
    rows = [0, 5, 19, 20, 32]
    part = oracle.attention_fp8(q, k, v, cu, hh, dh, causal=True, rows=rows)
    np.testing.assert_array_equal(part["o"], full["o"][rows])


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_block_with_fp8_attention_and_zero_queries_averages_v(causal):
    """With W_q = 0 (no bias) every key gets the same weight, so the FP8
    attention half's o is, per head, the mean of v's per-head dequantized codes
    over the query's keys (its segment, or the segment's prefix when causal):
    checks that the half hands its own v, the segments and the per-(segment,
    head) scale to the attention."""
    x, table, mod, pos, wq, wo, _, _ = _lossless_block(81, d=16, h=2, n=14, with_bias=False)
    codes, scales = wq
    codes = codes.copy()
    codes[:16] = 0
    kw = dict(n_heads=2, head_dim=8, sections=(2, 2, 4), theta=100.0)
    cu = [0, 6, 14]
    f8 = oracle.block_forward_fp8(x, mod, pos, cu, table, codes, scales, *wo, causal=causal,
                                  fp8_attention=True, **kw)
    assert not f8["q"].any()
    tab = oracle.e4m3_table()
    vd = np.empty_like(f8["v"])
    for a, b in zip(cu, cu[1:]):
        for h in range(2):
            cols = slice(8 * h, 8 * h + 8)
            c, s = oracle.quantize_tensor(f8["v"][a:b, cols])
            vd[a:b, cols] = tab[c] * np.float64(s)
    for a, b in zip(cu, cu[1:]):
        for i in range(a, b):
            keys = slice(a, i + 1 if causal else b)
            np.testing.assert_allclose(f8["o"][i], vd[keys].mean(axis=0), rtol=1e-12, atol=1e-14)


def test_fp8_block_with_fp8_attention_and_zero_values():
    """W_v = 0 (no qkv bias): v = 0, so the FP8 attention gives o = 0 exactly and
    the half returns x + gate[m] * b_o."""
    x, table, mod, pos, wq, wo, _, b_o = _lossless_block(82, d=16, h=2, n=12, with_bias=True)
    codes, scales = wq
    codes = codes.copy()
    codes[32:] = 0
    kw = dict(n_heads=2, head_dim=8, sections=(2, 2, 4), theta=100.0)
    f8 = oracle.block_forward_fp8(x, mod, pos, [0, 5, 12], table, codes, scales, *wo, b_o=b_o,
                                  fp8_attention=True, **kw)
    assert not f8["v"].any() and not f8["o"].any()
    np.testing.assert_allclose(f8["out"], x + table[mod, 2, :] * b_o[None, :], rtol=1e-12,
                               atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_attention_does_not_depend_on_what_else_is_packed(causal):
    """Two requests packed together get exactly the FP8 attention each gets alone,
    although the second one's keys and values are ten times larger (with one k or
    v scale per head over the whole pack, the first request's codes would follow
    the second's magnitude)."""
    rng = np.random.Generator(np.random.PCG64(15))
    hh, dh = 2, 8
    reqs = []
    for n_r, mag in ((13, 1.0), (21, 10.0)):
        q = rng.standard_normal((n_r, hh * dh))
        reqs.append((q, rng.standard_normal((n_r, hh * dh)) * mag,
                     rng.standard_normal((n_r, hh * dh)) * mag))
    pack = [np.concatenate([r[i] for r in reqs]) for i in range(3)]
    cu = [0, 13, 34]
    both = oracle.attention_fp8(*pack, cu, hh, dh, causal=causal)
    for (a, b), r in zip(zip(cu, cu[1:]), reqs):
        alone = oracle.attention_fp8(*r, [0, b - a], hh, dh, causal=causal)
        np.testing.assert_allclose(both["o"][a:b], alone["o"], rtol=1e-13, atol=1e-15)
        np.testing.assert_array_equal(both["k_codes"][a:b], alone["k_codes"])
        np.testing.assert_array_equal(both["v_codes"][a:b], alone["v_codes"])
