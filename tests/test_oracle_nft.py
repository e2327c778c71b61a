"""Pins of the oracle's DiffusionNFT loss (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
import synth

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                     "nft_loss_examples.json")))
C = 8


def _batch(n=23, seed=91, cu=(0, 9, 9, 23)):
    vt = synth.normal_array((n, C), seed).astype(np.float64)
    vo = synth.normal_array((n, C), seed + 1).astype(np.float64)
    tg = synth.normal_array((n, C), seed + 2).astype(np.float64)
    return vt, vo, tg, list(cu)


def _mse(a, b):
    return float(np.mean((a - b) ** 2))


@pytest.mark.parametrize("beta", GOLDEN["example_betas"])
def test_implicit_policy_identities(beta):
    vt, vo, _, _ = _batch()
    vp, vn = oracle.implicit_policies(vt, vo, beta)
    np.testing.assert_allclose(vp + vn, 2.0 * vo, rtol=0, atol=1e-14)
    np.testing.assert_allclose(vp - vn, 2.0 * beta * (vt - vo), rtol=0, atol=1e-14)
    # the coefficients the page prints, one basis vector at a time
    one, zero = np.ones((1, 1)), np.zeros((1, 1))
    assert oracle.implicit_policies(one, zero, beta)[0][0, 0] == beta
    assert oracle.implicit_policies(zero, one, beta)[0][0, 0] == 1.0 - beta
    assert oracle.implicit_policies(one, zero, beta)[1][0, 0] == -beta
    assert oracle.implicit_policies(zero, one, beta)[1][0, 0] == 1.0 + beta


def test_extreme_rewards_keep_one_branch():
    vt, vo, tg, cu = _batch(cu=(0, 23))
    for beta in GOLDEN["example_betas"]:
        vp, vn = oracle.implicit_policies(vt, vo, beta)
        r1 = oracle.nft_loss(vt, vo, tg, cu, [1.0], beta)
        r0 = oracle.nft_loss(vt, vo, tg, cu, [0.0], beta)
        assert r1["loss"][0] == pytest.approx(_mse(vp, tg), rel=1e-14)
        assert r0["loss"][0] == pytest.approx(_mse(vn, tg), rel=1e-14)
    # r = 1, beta = 1: plain flow-matching regression of v_theta on the target
    assert oracle.nft_loss(vt, vo, tg, cu, [1.0], 1.0)["loss"][0] == pytest.approx(_mse(vt, tg),
                                                                                rel=1e-14)


def test_loss_is_linear_in_the_reward():
    vt, vo, tg, cu = _batch(cu=(0, 23))
    a = oracle.nft_loss(vt, vo, tg, cu, [0.0], 0.5)
    b = oracle.nft_loss(vt, vo, tg, cu, [1.0], 0.5)
    m = oracle.nft_loss(vt, vo, tg, cu, [0.25], 0.5)
    assert m["loss"][0] == pytest.approx(0.75 * a["loss"][0] + 0.25 * b["loss"][0], rel=1e-14)
    np.testing.assert_allclose(m["grad"], 0.75 * a["grad"] + 0.25 * b["grad"], rtol=0, atol=1e-15)


def test_frozen_copy_gives_plain_regression():
    """At the start of a round v_theta equals v_old: both branches are v_old."""
    _, vo, tg, cu = _batch(cu=(0, 23))
    for r in GOLDEN["example_rewards"]:
        out = oracle.nft_loss(vo, vo, tg, cu, [r], 0.3)
        assert out["loss"][0] == pytest.approx(_mse(vo, tg), rel=1e-14)


def test_gradient_matches_autograd_and_differences():
    vt, vo, tg, cu = _batch()
    mask = np.ones(23, dtype=np.uint8)
    mask[[0, 1, 15]] = 0
    reward, beta = [0.8, 0.4, 0.1], 0.35
    out = oracle.nft_loss(vt, vo, tg, cu, reward, beta, loss_mask=mask)
    # torch autograd through torch's own mse_loss on the masked rows (library routines)
    t = torch.tensor(vt, requires_grad=True)
    total = 0.0
    for s in range(3):
        rows = [i for i in range(cu[s], cu[s + 1]) if mask[i]]
        if not rows:
            continue
        vp = beta * t[rows] + (1 - beta) * torch.tensor(vo[rows])
        vn = (1 + beta) * torch.tensor(vo[rows]) - beta * t[rows]
        ls = (reward[s] * torch.nn.functional.mse_loss(vp, torch.tensor(tg[rows]))
              + (1 - reward[s]) * torch.nn.functional.mse_loss(vn, torch.tensor(tg[rows])))
        assert out["loss"][s] == pytest.approx(ls.item(), rel=1e-13)
        total = total + ls
    (total / 3).backward()
    np.testing.assert_allclose(out["grad"], t.grad.numpy(), rtol=1e-12, atol=1e-16)
    # central difference on one element
    i, j, h = 5, 3, 1e-6
    vp_, vm_ = vt.copy(), vt.copy()
    vp_[i, j] += h
    vm_[i, j] -= h
    fd = (np.sum(oracle.nft_loss(vp_, vo, tg, cu, reward, beta, mask)["loss"])
          - np.sum(oracle.nft_loss(vm_, vo, tg, cu, reward, beta, mask)["loss"])) / (2 * h) / 3
    assert out["grad"][i, j] == pytest.approx(fd, rel=1e-6)


def test_reward_sets_attraction_or_repulsion():
    """From v_theta = v_old, one small descent step moves v_theta toward the target
    for r = 1 and away from it for r = 0."""
    _, vo, tg, cu = _batch(cu=(0, 23))
    for r, sign in ((1.0, -1), (0.0, +1)):
        g = oracle.nft_loss(vo, vo, tg, cu, [r], 0.5)["grad"]
        stepped = vo - 0.1 * g / np.abs(g).max()
        assert np.sign(_mse(stepped, tg) - _mse(vo, tg)) == sign


def test_mask_and_h3_sign():
    vt, vo, tg, cu = _batch()
    mask = np.ones(23, dtype=np.uint8)
    mask[[2, 3, 20]] = 0
    vt_bad, vo_bad = vt.copy(), vo.copy()
    vt_bad[[2, 3, 20]] = np.nan
    vo_bad[[2, 3, 20]] = 1e30
    a = oracle.nft_loss(vt, vo, tg, cu, [0.6, 0.5, 0.2], 0.4, loss_mask=mask)
    b = oracle.nft_loss(vt_bad, vo_bad, tg, cu, [0.6, 0.5, 0.2], 0.4, loss_mask=mask)
    np.testing.assert_array_equal(a["loss"], b["loss"])
    np.testing.assert_array_equal(a["grad"], np.nan_to_num(b["grad"]))
    assert (b["grad"][[2, 3, 20]] == 0).all()
    # H3's reversed velocity: negated outputs with sign -1 give the same loss and the
    # gradient of the raw output flips
    h = oracle.nft_loss(-vt, -vo, tg, cu, [0.6, 0.5, 0.2], 0.4, loss_mask=mask, velocity_sign=-1)
    np.testing.assert_array_equal(h["loss"], a["loss"])
    np.testing.assert_array_equal(h["grad"], -a["grad"])
    # the empty middle sample has zero loss
    assert a["loss"][1] == 0.0


def test_matches_loops():
    vt, vo, tg, cu = _batch(n=7, cu=(0, 3, 7))
    mask = [1, 0, 1, 1, 1, 0, 1]
    for sign in (1.0, -1.0):
        out = oracle.nft_loss(vt, vo, tg, cu, [0.3, 0.9], 0.6, mask, sign, grad_scale=0.7)
        loss, mp, mn, grad = brute.nft_loss(vt.tolist(), vo.tolist(), tg.tolist(), cu, [0.3, 0.9],
                                            0.6, mask, sign, grad_scale=0.7)
        np.testing.assert_allclose(out["loss"], loss, rtol=1e-14)
        np.testing.assert_allclose(out["mse_pos"], mp, rtol=1e-14)
        np.testing.assert_allclose(out["mse_neg"], mn, rtol=1e-14)
        np.testing.assert_allclose(out["grad"], np.array(grad), rtol=1e-13, atol=1e-17)
