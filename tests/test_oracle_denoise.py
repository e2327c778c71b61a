"""Pins of the oracle's denoising step (CPU only).

The pages give the loop's structure (Rectified Flow X0, Euler with eta = 0,
separate video and audio schedules, anchor re-pinning) and the timestep and
velocity conventions, but no sigma values: the schedules here are synthetic.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import brute
import synth

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                     "denoise_conventions.json")))
C = oracle.VIDEO_LATENT_CHANNELS


def _pack(n_video=7, n_audio=5, n_text=3):
    return np.array([0] * n_video + [1] * n_audio + [2] * n_text, dtype=np.uint8)


def _path(mod, seed=71):
    n = mod.size
    x0 = synth.normal_array((n, C), seed).astype(np.float64)
    eps = synth.normal_array((n, C), seed + 1).astype(np.float64)
    return x0, eps


def _on_path(x0, eps, sigma):
    return (1.0 - sigma) * x0 + sigma * eps


def test_video_latent_width_from_the_pages():
    # 24 latent channels, 1x2x2 patch
    assert C == 96


def test_timestep_convention():
    g = GOLDEN
    assert oracle.timestep_from_sigma(g["sigma_pure_noise"]) == g["t_h3_at_pure_noise"]
    assert oracle.timestep_from_sigma(g["sigma_clean"]) == g["t_h3_at_clean"]
    s = np.linspace(0.0, 1.0, 11)
    np.testing.assert_allclose(oracle.timestep_from_sigma(oracle.timestep_from_sigma(s)), s,
                               rtol=0, atol=1e-15)
    # monotone the other way: less noise, later data-progress time
    assert np.all(np.diff(oracle.timestep_from_sigma(s)) < 0)


def test_three_step_example_lands_on_clean_latents():
    """With the straight path's own velocity eps - x0, every Euler step stays on the
    path z(sigma) = (1 - sigma) x0 + sigma eps, every X0 estimate is x0, and the
    last step (sigma_1 -> 0) returns x0."""
    mod = _pack()
    x0, eps = _path(mod)
    sv, sa = GOLDEN["example_sigma_video"], GOLDEN["example_sigma_audio"]
    assert len(sv) == GOLDEN["example_steps"] + 1 and sv[-1] == 0.0
    lat = mod != 2
    sig_row = lambda sched, i: np.where(mod == 0, sched[0][i], sched[1][i])[:, None]
    z = np.where(lat[:, None], _on_path(x0, eps, sig_row((sv, sa), 0)), x0)
    for i in range(GOLDEN["example_steps"]):
        z, est = oracle.denoise_step(z, eps - x0, mod, [[sv[i], sv[i + 1]], [sa[i], sa[i + 1]]])
        want = _on_path(x0, eps, sig_row((sv, sa), i + 1))
        np.testing.assert_allclose(z[lat], want[lat], rtol=0, atol=1e-13)
        np.testing.assert_allclose(est[lat], x0[lat], rtol=0, atol=1e-13)
    np.testing.assert_allclose(z[lat], x0[lat], rtol=0, atol=1e-13)


def test_fifty_step_loop_with_h3_velocity():
    """The production loop length with H3's reversed velocity (x0 - eps, sign -1)."""
    mod = _pack(4, 3, 2)
    x0, eps = _path(mod, seed=72)
    n = GOLDEN["production_steps"]
    sv = np.linspace(1.0, 0.0, n + 1)
    sa = np.linspace(1.0, 0.0, n + 1) ** 1.5      # a different audio schedule
    lat = mod != 2
    z = x0.copy()
    z[mod == 0] = _on_path(x0, eps, 1.0)[mod == 0]
    z[mod == 1] = _on_path(x0, eps, 1.0)[mod == 1]
    zf, x0s = oracle.denoise_loop(z, lambda zz, i: x0 - eps, mod, sv, sa,
                                  velocity_sign=GOLDEN["velocity_sign_h3"])
    assert len(x0s) == n
    np.testing.assert_allclose(zf[lat], x0[lat], rtol=0, atol=1e-12)
    np.testing.assert_array_equal(zf[~lat], z[~lat])


def test_velocity_sign_conversion_is_exact():
    mod = _pack()
    z = synth.normal_array((mod.size, C), 73).astype(np.float64)
    v = synth.normal_array((mod.size, C), 74).astype(np.float64)
    sig = [[0.8, 0.5], [0.6, 0.45]]
    a = oracle.denoise_step(z, v, mod, sig, velocity_sign=1.0)
    b = oracle.denoise_step(z, -v, mod, sig, velocity_sign=-1.0)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    with pytest.raises(ValueError):
        oracle.denoise_step(z, v, mod, sig, velocity_sign=0.5)


def test_euler_is_one_explicit_first_order_step():
    """On dz/dsigma = a z the step is exactly z (1 + a h) (not a higher-order solver),
    and n steps of h/n give z (1 + a h / n)^n, which tends to z exp(a h)."""
    mod = np.array([0, 1], dtype=np.uint8)
    z = np.array([[1.0] * 4, [2.0] * 4])
    a, s0, s1 = 0.7, 0.9, 0.3
    h = s1 - s0
    z1, _ = oracle.denoise_step(z, a * z, mod, [[s0, s1], [s0, s1]])
    np.testing.assert_allclose(z1, z * (1.0 + a * h), rtol=1e-15, atol=0)
    errs = []
    for n in (10, 20, 40):
        sched = np.linspace(s0, s1, n + 1)
        zn, _ = oracle.denoise_loop(z, lambda zz, i: a * zz, mod, sched, sched)
        np.testing.assert_allclose(zn, z * (1.0 + a * h / n) ** n, rtol=1e-13, atol=0)
        errs.append(abs(zn[0, 0] - math.exp(a * h)))
    # first order: halving the step halves the error
    assert 1.8 < errs[0] / errs[1] < 2.2 and 1.8 < errs[1] / errs[2] < 2.2


def test_dual_schedules_are_independent():
    mod = _pack()
    z = synth.normal_array((mod.size, C), 75).astype(np.float64)
    v = synth.normal_array((mod.size, C), 76).astype(np.float64)
    sig = [[0.9, 0.7], [0.4, 0.1]]
    zn, x0 = oracle.denoise_step(z, v, mod, sig)
    for i, m in enumerate(mod):
        if m == 2:
            continue
        s, s_next = sig[m]
        np.testing.assert_allclose(zn[i], z[i] + (s_next - s) * v[i], rtol=1e-15, atol=1e-15)
        np.testing.assert_allclose(x0[i], z[i] - s * v[i], rtol=1e-15, atol=1e-15)
    # relabelling video <-> audio is the same as swapping the two schedules
    swapped = np.where(mod == 2, 2, 1 - mod.astype(np.int64)).astype(np.uint8)
    zs, x0s = oracle.denoise_step(z, v, swapped, [sig[1], sig[0]])
    np.testing.assert_array_equal(zs, zn)
    np.testing.assert_array_equal(x0s, x0)


def test_anchor_rows_are_repinned_and_text_untouched():
    mod = _pack()
    n = mod.size
    z = synth.normal_array((n, C), 77).astype(np.float64)
    v = synth.normal_array((n, C), 78).astype(np.float64)
    anchor = np.zeros(n, dtype=np.uint8)
    anchor[[0, 3, 8, n - 1]] = 1             # two video, one audio, one text row
    vals = synth.normal_array((n, C), 79).astype(np.float64)
    v[anchor == 1] = np.nan                  # whatever the model predicts there
    zn, x0 = oracle.denoise_step(z, v, mod, [[0.8, 0.6], [0.8, 0.5]], anchor, vals)
    pin = (anchor == 1) & (mod != 2)
    np.testing.assert_array_equal(zn[pin], vals[pin])
    np.testing.assert_array_equal(x0[pin], vals[pin])
    np.testing.assert_array_equal(zn[mod == 2], z[mod == 2])
    assert np.isnan(x0[mod == 2]).all()
    free = ~pin & (mod != 2)
    assert np.isfinite(zn[free]).all()
    # over many steps the anchors never drift (the re-pin cannot be skipped)
    zz = z.copy()
    for _ in range(20):
        zz, _ = oracle.denoise_step(zz, np.ones_like(zz), mod, [[0.5, 0.4], [0.5, 0.4]], anchor, vals)
    np.testing.assert_array_equal(zz[pin], vals[pin])


def test_zero_step_and_linearity():
    mod = _pack()
    z = synth.normal_array((mod.size, C), 80).astype(np.float64)
    v = synth.normal_array((mod.size, C), 81).astype(np.float64)
    zn, _ = oracle.denoise_step(z, v, mod, [[0.5, 0.5], [0.3, 0.3]])
    np.testing.assert_array_equal(zn, z)
    sig = [[0.9, 0.2], [0.7, 0.65]]
    z1, _ = oracle.denoise_step(z, v, mod, sig)
    z2, _ = oracle.denoise_step(z, 2.0 * v, mod, sig)
    np.testing.assert_allclose(z2 - z, 2.0 * (z1 - z), rtol=1e-14, atol=1e-15)


def test_matches_loops():
    mod = np.array([0, 1, 2, 0, 1, 0], dtype=np.uint8)
    n, c = mod.size, 4
    z = synth.normal_array((n, c), 82).astype(np.float64)
    v = synth.normal_array((n, c), 83).astype(np.float64)
    vals = synth.normal_array((n, c), 84).astype(np.float64)
    anchor = np.array([0, 0, 1, 1, 0, 0], dtype=np.uint8)
    sig = [[0.75, 0.5], [0.6, 0.2]]
    for sign in (1.0, -1.0):
        zn, x0 = oracle.denoise_step(z, v, mod, sig, anchor, vals, velocity_sign=sign)
        bz, bx = brute.denoise_step(z.tolist(), v.tolist(), mod.tolist(), sig, anchor.tolist(),
                                    vals.tolist(), velocity_sign=sign)
        np.testing.assert_allclose(zn, np.array(bz), rtol=1e-15, atol=0)
        bx = np.array([[np.nan if e is None else e for e in r] for r in bx])
        np.testing.assert_allclose(x0, bx, rtol=1e-15, atol=0)
