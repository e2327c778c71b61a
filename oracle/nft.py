"""Float64 DiffusionNFT loss and its gradient with respect to the policy's velocity.

Test infrastructure only (see the package docstring).

[VeRL-Omni] section 4, "算法映射：DiffusionNFT 与标量最优奖励" (implicit
positive / negative policies; scalar-reward loss; the r = 1 and r = 0 minimal
examples): the current policy v_theta and the frozen old adapter v_old give
two implicit policies,

    v_pos = beta v_theta + (1 - beta) v_old
    v_neg = (1 + beta) v_old - beta v_theta,

and a sample with scalar reward r in [0, 1] contributes

    L = r MSE(v_pos, v_target) + (1 - r) MSE(v_neg, v_target).

[H3-NFT] section "FL2VA: First-Frame Conditioning With Shared
Infrastructure": condition-frame latents are masked out of the loss, only the
generated video and audio latents are optimised.  [VeRL-Omni] section 5.1:
H3's velocity is sign-reversed, and the adapter negates it before the
flow-matching loss.

Readings (the pages leave these open):

* MSE is the mean of the squared error over the sample's loss-bearing
  elements: the rows whose loss-mask flag is set, every channel of them.
  Rows outside the mask (condition frames, text, padding) add nothing to the
  loss or its denominator and get a zero gradient.
* Samples are row ranges of a packed batch given by cu offsets, one reward
  per sample.  The batch objective is grad_scale * sum_s L_s (grad_scale
  defaults to 1 / S, the mean over samples); the gradient is taken with
  respect to the raw network output, so velocity_sign = -1 (H3's own
  convention) negates it.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def implicit_policies(v_theta, v_old, beta: float):
    """(v_pos, v_neg) from the current and the frozen velocity."""
    vt = np.asarray(v_theta, dtype=np.float64)
    vo = np.asarray(v_old, dtype=np.float64)
    return beta * vt + (1.0 - beta) * vo, (1.0 + beta) * vo - beta * vt


def nft_loss(v_theta, v_old, v_target, cu, reward, beta: float, loss_mask=None,
             velocity_sign: float = 1.0, grad_scale: Optional[float] = None) -> dict:
    """Per-sample DiffusionNFT losses and d(grad_scale * sum_s L_s) / d v_theta.

    v_theta, v_old: [N][C] network outputs (raw; multiplied by velocity_sign);
    v_target: [N][C] standard flow-matching target; cu: [S+1] row offsets;
    reward: [S]; loss_mask: [N] flags or None (every row counts).
    Returns dict(loss [S], mse_pos [S], mse_neg [S], grad [N][C]); a sample with
    no loss-bearing row has loss, mse_pos and mse_neg 0.
    """
    if velocity_sign not in (1.0, -1.0):
        raise ValueError("velocity_sign must be +1 or -1")
    vt = velocity_sign * np.asarray(v_theta, dtype=np.float64)
    vo = velocity_sign * np.asarray(v_old, dtype=np.float64)
    tgt = np.asarray(v_target, dtype=np.float64)
    n, c = vt.shape
    cu = [int(x) for x in cu]
    r = np.asarray(reward, dtype=np.float64)
    n_s = len(cu) - 1
    scale = 1.0 / n_s if grad_scale is None else float(grad_scale)
    keep = np.ones(n, dtype=bool) if loss_mask is None else np.asarray(loss_mask) != 0
    v_pos, v_neg = implicit_policies(vt, vo, beta)
    loss = np.zeros(n_s)
    mse_pos = np.zeros(n_s)
    mse_neg = np.zeros(n_s)
    grad = np.zeros((n, c))
    for s in range(n_s):
        rows = np.arange(cu[s], cu[s + 1])
        rows = rows[keep[rows]]
        if rows.size == 0:
            continue
        cnt = rows.size * c
        e_pos = v_pos[rows] - tgt[rows]
        e_neg = v_neg[rows] - tgt[rows]
        mse_pos[s] = np.sum(e_pos * e_pos) / cnt
        mse_neg[s] = np.sum(e_neg * e_neg) / cnt
        loss[s] = r[s] * mse_pos[s] + (1.0 - r[s]) * mse_neg[s]
        # dL_s/dv_theta: v_pos carries +beta v_theta, v_neg carries -beta v_theta
        g_std = (2.0 / cnt) * (r[s] * beta * e_pos - (1.0 - r[s]) * beta * e_neg)
        grad[rows] = scale * velocity_sign * g_std
    return dict(loss=loss, mse_pos=mse_pos, mse_neg=mse_neg, grad=grad)
