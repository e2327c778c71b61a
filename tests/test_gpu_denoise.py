"""Parity of denoise_step against the float64 oracle (MI355X only).

The state and X0 are float32 outputs (rel-L2 <= 1e-5); anchor rows must equal
their anchor values bit for bit and text rows must be left untouched.  Inputs:
synth.denoise_inputs on the workloads' packed layouts, anchors on the first
video frame (t = 0) and the first 8 audio tokens of each channel of every
request, synthetic sigmas (the pages give none).
"""
import functools

import numpy as np
import pytest

import oracle
import synth
from gpu_util import check, dev, dev_f32, dev_int, host

pytestmark = pytest.mark.gpu

C = oracle.VIDEO_LATENT_CHANNELS
SENTINEL = -7.25


@pytest.fixture(scope="module")
def jav():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import joint_audio_video_amd as m
    return m


@functools.lru_cache(maxsize=4)
def _layout(name):
    wl = synth.WORKLOADS[name]
    lay = oracle.pack_layout([r.grid for r in wl.requests])
    return {"modality": np.asarray(lay["modality"], dtype=np.uint8),
            "pos": np.asarray(lay["pos"], dtype=np.int64)}


def _anchors(name):
    lay = _layout(name)
    mod, pos = lay["modality"], lay["pos"]
    a = ((mod == 0) & (pos[:, 0] == 0)) | ((mod == 1) & (pos[:, 0] < 8))
    return a.astype(np.uint8)


def _sync():
    import torch
    torch.cuda.synchronize()


def _run(jav, name, sigmas, sign=1, with_anchor=True, with_x0=True, seed=None):
    import torch
    wl = synth.WORKLOADS[name]
    inp = synth.denoise_inputs(wl, C, seed=seed)
    mod = _layout(name)["modality"]
    anchor = _anchors(name) if with_anchor else None
    z = dev_f32(inp.z)
    v = dev(inp.v * sign, wl.dtype)
    x0 = torch.full_like(z, SENTINEL) if with_x0 else None
    av = dev_f32(inp.anchor_vals) if with_anchor else None
    jav.denoise_step(z, v, dev_int(mod, torch.uint8), sigmas, x0=x0,
                     anchor=None if anchor is None else dev_int(anchor, torch.uint8),
                     anchor_vals=av, velocity_sign=sign)
    _sync()
    s = np.asarray(sigmas, dtype=np.float32).astype(np.float64)
    ref_z, ref_x0 = oracle.denoise_step(inp.z, inp.v * sign, mod, [[s[0], s[1]], [s[2], s[3]]],
                                        anchor, inp.anchor_vals, velocity_sign=sign)
    return inp, mod, anchor, z, x0, ref_z, ref_x0


@pytest.mark.parametrize("name", ["tiny", "small", "medium", "full", "varlen"])
def test_denoise_parity(jav, name):
    print(f"denoise parity {name}", flush=True)
    sig = (0.62, 0.6, 0.5, 0.47)
    inp, mod, anchor, z, x0, ref_z, ref_x0 = _run(jav, name, sig)
    gz, gx = host(z), host(x0)
    lat = mod != 2
    pin = lat & (anchor != 0)
    free = lat & ~pin
    check(gz[free], ref_z[free], "f32", f"{name} z")
    check(gx[free], ref_x0[free], "f32", f"{name} x0")
    # anchors bit-exact, text rows untouched (state and X0)
    np.testing.assert_array_equal(gz[pin], inp.anchor_vals[pin])
    np.testing.assert_array_equal(gx[pin], inp.anchor_vals[pin])
    np.testing.assert_array_equal(gz[~lat], inp.z[~lat])
    assert (gx[~lat] == SENTINEL).all()


def test_denoise_h3_sign_and_last_step(jav):
    """H3's reversed velocity with sign -1 gives the same bits as the standard one; a
    last step (sigma_next = 0) leaves z equal to X0 bit for bit."""
    import torch
    sig = (0.125, 0.0, 0.3, 0.0)
    _, mod, _, z1, x1, _, _ = _run(jav, "small", sig, sign=1)
    _, _, _, z2, x2, ref_z, ref_x0 = _run(jav, "small", sig, sign=-1)
    assert torch.equal(z1, z2) and torch.equal(x1, x2)
    lat = mod != 2
    assert torch.equal(z1[torch.from_numpy(lat).cuda()], x1[torch.from_numpy(lat).cuda()])
    check(host(z2)[lat], ref_z[lat], "f32", "last step z")


def test_denoise_three_step_example_on_the_gpu(jav):
    """The page's three-step example: with the straight path's velocity each step stays
    on (1 - s) x0 + s eps and the last returns x0 (float32 rounding only)."""
    import torch
    name = "small"
    wl = synth.WORKLOADS[name]
    mod = _layout(name)["modality"]
    x0s = synth.normal_array((wl.n_tokens, C), 901)
    eps = synth.normal_array((wl.n_tokens, C), 902)
    sv = np.array([1.0, 0.6, 0.25, 0.0], np.float32)
    sa = np.array([1.0, 0.7, 0.3, 0.0], np.float32)
    lat = mod != 2
    z = np.where(lat[:, None], eps, x0s).astype(np.float32)   # sigma = 1: pure noise
    zd = dev_f32(z)
    v = dev_f32(eps - x0s)
    md = dev_int(mod, torch.uint8)
    for i in range(3):
        jav.denoise_step(zd, v, md, (sv[i], sv[i + 1], sa[i], sa[i + 1]))
    _sync()
    got = host(zd)
    check(got[lat], x0s.astype(np.float64)[lat], "f32", "3-step x0")
    np.testing.assert_array_equal(got[~lat], z[~lat])


def test_denoise_fifty_steps_match_the_oracle_loop(jav):
    """50 steps with per-step velocities and anchors: errors stay at float32 rounding."""
    import torch
    name = "small"
    wl = synth.WORKLOADS[name]
    mod = _layout(name)["modality"]
    anchor = _anchors(name)
    inp = synth.denoise_inputs(wl, C)
    sv, sa = synth.sigma_schedule(50), synth.sigma_schedule(50, 1.5)
    vs = [synth.normal_array((wl.n_tokens, C), 1000 + i, dtype=wl.dtype) for i in range(50)]
    zd, md = dev_f32(inp.z), dev_int(mod, torch.uint8)
    ad, avd = dev_int(anchor, torch.uint8), dev_f32(inp.anchor_vals)
    for i in range(50):
        jav.denoise_step(zd, dev(vs[i], wl.dtype), md, (sv[i], sv[i + 1], sa[i], sa[i + 1]),
                         anchor=ad, anchor_vals=avd, velocity_sign=-1)
    _sync()
    ref, _ = oracle.denoise_loop(inp.z, lambda zz, i: vs[i], mod, sv.astype(np.float64),
                                 sa.astype(np.float64), anchor, inp.anchor_vals,
                                 velocity_sign=-1)
    got = host(zd)
    check(got, ref, "f32", "50 steps")
    pin = (anchor != 0) & (mod != 2)
    np.testing.assert_array_equal(got[pin], inp.anchor_vals[pin])


@pytest.mark.parametrize("channels,n", [(4, 1), (100, 333), (96, 1000)])
def test_denoise_strided_trimmed_and_without_x0(jav, channels, n):
    """ld above channels, rows past n_rows untouched, x0 omitted, odd channel groups."""
    import torch
    ld = channels + 8                          # float32 rows: 16-byte multiples
    ldv = (channels + 7) // 8 * 8 + 8          # bf16 rows: 16-byte multiples
    rows = n + 5
    mod = synth.uniform_ints((rows,), 0, 3, seed=910 + n).astype(np.uint8)
    zh = synth.normal_array((rows, ld), 911)
    vh = synth.normal_array((rows, ldv), 912, dtype="bf16")
    zd, vd = dev_f32(zh), dev(vh, "bf16")
    sig = (0.9, 0.8, 0.4, 0.1)
    jav.denoise_step(zd[:, :channels], vd[:, :channels], dev_int(mod, torch.uint8), sig, n_rows=n)
    _sync()
    got = host(zd)
    s = np.asarray(sig, np.float32).astype(np.float64)
    ref, _ = oracle.denoise_step(zh[:n, :channels], vh[:n, :channels], mod[:n],
                                 [[s[0], s[1]], [s[2], s[3]]])
    lat = mod[:n] != 2
    if lat.any():
        check(got[:n, :channels][lat], ref[lat], "f32", f"strided c={channels}")
    np.testing.assert_array_equal(got[:n, :channels][~lat], zh[:n, :channels][~lat])
    np.testing.assert_array_equal(got[:, channels:], zh[:, channels:])   # padding columns
    np.testing.assert_array_equal(got[n:], zh[n:])                       # trimmed rows
