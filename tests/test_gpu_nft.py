"""Parity of nft_loss against the float64 oracle (MI355X only).

Per-sample losses and the gradient are float32 outputs (rel-L2 <= 1e-5);
masked rows must get an exactly zero gradient and two runs must agree bit for
bit.  Inputs: synth.nft_inputs; samples are the workloads' requests (the
varlen pack gives four); the loss mask keeps video and audio rows and drops
text rows and the first and last video frame of every request (condition
frames of a first/last-frame task); beta is synthetic (the pages give none).
"""
import functools

import numpy as np
import pytest

import oracle
import synth
from gpu_util import check, dev, dev_f32, dev_int, host

pytestmark = pytest.mark.gpu

C = oracle.VIDEO_LATENT_CHANNELS
BETA = 0.5


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
    mod = np.asarray(lay["modality"], dtype=np.uint8)
    pos = np.asarray(lay["pos"], dtype=np.int64)
    t_last = {}
    for r, (a, b) in zip(wl.requests, zip(lay["cu_seqlens"], lay["cu_seqlens"][1:])):
        t_last[(a, b)] = r.t - 1
    keep = np.zeros(mod.size, dtype=np.uint8)
    for (a, b), tl in t_last.items():
        m, p = mod[a:b], pos[a:b]
        cond = (m == 0) & ((p[:, 0] == 0) | (p[:, 0] == tl))
        keep[a:b] = ((m != 2) & ~cond).astype(np.uint8)
    return list(lay["cu_seqlens"]), keep


def _run(jav, vt, vo, tg, cu, reward, keep, dtype, beta=BETA, sign=1, scale=None, ld_pad=0):
    import torch
    n = vt.shape[0]
    c = vt.shape[1]
    max_rows = max(b - a for a, b in zip(cu, cu[1:])) or 1

    def padded(a, f):
        if ld_pad == 0:
            return f(a)
        full = np.zeros((n, c + ld_pad), np.float32)
        full[:, :c] = a
        return f(full)[:, :c]

    vt_d = padded(vt, lambda a: dev(a, dtype))
    vo_d = padded(vo, lambda a: dev(a, dtype))
    tg_d = padded(tg, dev_f32)
    grad = padded(np.full((n, c), 7.0, np.float32), dev_f32)
    mask_d = None if keep is None else dev_int(keep, torch.uint8)
    out, g = jav.nft_loss(vt_d, vo_d, tg_d, dev_int(np.array(cu), torch.int32), max_rows,
                          dev_f32(reward), beta, loss_mask=mask_d, velocity_sign=sign,
                          grad_scale=scale, grad=grad)
    torch.cuda.synchronize()
    return host(out), host(g)


@pytest.mark.parametrize("name", ["tiny", "small", "full", "varlen"])
def test_nft_loss_parity(jav, name):
    print(f"nft parity {name}", flush=True)
    wl = synth.WORKLOADS[name]
    cu, keep = _layout(name)
    inp = synth.nft_inputs(wl, len(cu) - 1, C)
    out, g = _run(jav, inp.v_theta, inp.v_old, inp.v_target, cu, inp.reward, keep, wl.dtype)
    ref = oracle.nft_loss(inp.v_theta, inp.v_old, inp.v_target, cu, inp.reward, BETA, keep)
    check(out[:, 0], ref["loss"], "f32", f"{name} loss")
    check(out[:, 1], ref["mse_pos"], "f32", f"{name} mse_pos")
    check(out[:, 2], ref["mse_neg"], "f32", f"{name} mse_neg")
    check(g[keep != 0], ref["grad"][keep != 0], "f32", f"{name} grad")
    assert (g[keep == 0] == 0).all()


def test_nft_loss_h3_sign_extreme_rewards_and_determinism(jav):
    name = "small"
    wl = synth.WORKLOADS[name]
    cu, keep = _layout(name)
    inp = synth.nft_inputs(wl, 1, C, seed=77)
    for r in (0.0, 1.0):
        rew = np.array([r], np.float32)
        a = _run(jav, inp.v_theta, inp.v_old, inp.v_target, cu, rew, keep, wl.dtype)
        b = _run(jav, -inp.v_theta, -inp.v_old, inp.v_target, cu, rew, keep, wl.dtype, sign=-1)
        np.testing.assert_array_equal(a[0], b[0])
        np.testing.assert_array_equal(a[1], -b[1])
        c2 = _run(jav, inp.v_theta, inp.v_old, inp.v_target, cu, rew, keep, wl.dtype)
        np.testing.assert_array_equal(a[0], c2[0])
        np.testing.assert_array_equal(a[1], c2[1])
        ref = oracle.nft_loss(inp.v_theta, inp.v_old, inp.v_target, cu, rew, BETA, keep)
        check(a[0][:, 0], ref["loss"], "f32", f"r={r} loss")
        check(a[1], ref["grad"], "f32", f"r={r} grad")


@pytest.mark.parametrize("channels,ld_pad", [(4, 4), (100, 4), (96, 0)])
def test_nft_loss_ragged_samples_masks_and_strides(jav, channels, ld_pad):
    """Empty and fully masked samples, samples shorter and longer than a 128-row chunk,
    no mask at all, a custom grad_scale, strided rows."""
    cu = [0, 1, 1, 130, 300, 300 + 257, 600]
    n = cu[-1]
    wl = synth.WORKLOADS["small"]
    inp = synth.nft_inputs(wl, len(cu) - 1, channels, n_rows=n, seed=88)
    keep = synth.uniform_ints((n,), 0, 4, seed=89).astype(np.uint8)   # ~3/4 kept
    keep[300:557] = 0                                                  # a fully masked sample
    for mask in (keep, None):
        out, g = _run(jav, inp.v_theta, inp.v_old, inp.v_target, cu, inp.reward, mask, "bf16",
                      beta=0.3, scale=0.125, ld_pad=ld_pad)
        ref = oracle.nft_loss(inp.v_theta, inp.v_old, inp.v_target, cu, inp.reward, 0.3, mask,
                              grad_scale=0.125)
        check(out.ravel(), np.stack([ref["loss"], ref["mse_pos"], ref["mse_neg"]], 1).ravel(),
              "f32", f"ragged c={channels} mask={mask is not None}")
        check(g, ref["grad"], "f32", "ragged grad")
        assert out[1].tolist() == [0.0, 0.0, 0.0]          # empty sample
        if mask is not None:
            assert out[4].tolist() == [0.0, 0.0, 0.0]      # fully masked sample
            assert (g[mask == 0] == 0).all()
