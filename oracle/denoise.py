"""Float64 denoising step of the joint audio-video latent state.

Test infrastructure only (see the package docstring).

[vLLM-Omni] section "4. Joint Audio-Video Denoising Execution Flow" (runtime
loop table, stages 4-7; "Key Causal Chains"; "State Evolution Example";
boundary conditions) describes one step after the DiT forward pass:

* the packed output is split by modality into a video and an audio velocity
  (stage 4), and each modality keeps its own noise schedule, sigma_video and
  sigma_audio, whose step sizes are taken separately before one joint
  write-back;
* the Rectified Flow velocity parameterisation turns the predicted velocity
  into a clean estimate X0 (stage 5);
* a deterministic Euler step (eta = 0, no fresh noise) moves each modality
  from its current sigma to its next one (stage 6);
* anchor rows (reference frames or clips) are restored to their original
  values after the update (stage 7).

[VeRL-Omni] section 5.1 fixes the two conventions: generic flow-matching
schedulers count sigma from 1 (pure noise) down to 0 (clean data), while
H3's DiT takes data-progress time t = 1 - sigma (t = 0 noise, t = 1 the
finished video) and emits a velocity whose sign is reversed; the fix maps the
timestep and negates the velocity.

Readings (the pages give no formulas for stages 5 and 6):

* Rectified Flow path z(sigma) = (1 - sigma) x0 + sigma eps, with the standard
  velocity v = dz/dsigma = eps - x0.  Then X0 = z - sigma v, and the Euler
  step from sigma to sigma' is z' = z + (sigma' - sigma) v.  H3's own velocity
  is dz/dt = x0 - eps = -v, so velocity_sign = -1 converts it.
* The state is a packed array of rows with one modality id per row, the ids
  of the block's sequence.  Video rows (id 0) use the video sigmas, audio rows
  (id 1) the audio sigmas; text rows (id 2) are conditioning, not latent
  state: they are neither advanced nor given an X0.
* An anchor row's new state and its X0 are both its original value (a known,
  clean row).  Text rows stay untouched even when flagged.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .layout import MOD_AUDIO, MOD_TEXT, MOD_VIDEO

# Latent channels of one video token: 24 VAE channels times the 1x2x2 patch
# ([H3-NFT], section "MiniMax H3 and Why It's Hard to Train").  The packed state
# gives every row this width (a reading: the pages give no audio latent width).
VIDEO_LATENT_CHANNELS = 24 * 1 * 2 * 2


def timestep_from_sigma(sigma):
    """H3's data-progress time from a scheduler's noise level: t = 1 - sigma."""
    return 1.0 - np.asarray(sigma, dtype=np.float64)


def standard_velocity(v, velocity_sign: float = 1.0) -> np.ndarray:
    """The standard velocity eps - x0; H3's own output needs velocity_sign = -1."""
    if velocity_sign not in (1.0, -1.0):
        raise ValueError("velocity_sign must be +1 or -1")
    return velocity_sign * np.asarray(v, dtype=np.float64)


def clean_estimate(z, v_std, sigma) -> np.ndarray:
    """Rectified Flow X0 from the state at noise level sigma: z - sigma v."""
    return np.asarray(z, dtype=np.float64) - sigma * np.asarray(v_std, dtype=np.float64)


def euler_step(z, v_std, sigma, sigma_next) -> np.ndarray:
    """Deterministic Euler step (eta = 0) from sigma to sigma_next."""
    return (np.asarray(z, dtype=np.float64)
            + (sigma_next - sigma) * np.asarray(v_std, dtype=np.float64))


def denoise_step(z, v, modality, sigmas, anchor=None, anchor_vals=None,
                 velocity_sign: float = 1.0) -> Tuple[np.ndarray, np.ndarray]:
    """One step of the joint loop over a packed latent state.

    z, v: [N][C] state and predicted velocity; modality: [N] ids; sigmas:
    [[sigma_video, sigma_video_next], [sigma_audio, sigma_audio_next]];
    anchor: [N] flags or None; anchor_vals: [N][C] original values (read on
    flagged rows only).  Returns (z_next, x0) in float64.  Rows that are not
    advanced (text) hold z in z_next and NaN in x0: the library leaves them
    unwritten.
    """
    z = np.asarray(z, dtype=np.float64)
    modality = np.asarray(modality)
    sig = np.asarray(sigmas, dtype=np.float64).reshape(2, 2)
    v_std = standard_velocity(v, velocity_sign)
    z_next = z.copy()
    x0 = np.full_like(z, np.nan)
    # stage 4: each modality's rows with that modality's schedule
    for m in (MOD_VIDEO, MOD_AUDIO):
        rows = modality == m
        s, s_next = sig[m]
        x0[rows] = clean_estimate(z[rows], v_std[rows], s)             # stage 5
        z_next[rows] = euler_step(z[rows], v_std[rows], s, s_next)     # stage 6
    # stage 7: re-pin anchors (latent rows only)
    if anchor is not None:
        pin = (np.asarray(anchor) != 0) & (modality != MOD_TEXT)
        a = np.asarray(anchor_vals, dtype=np.float64)
        z_next[pin] = a[pin]
        x0[pin] = a[pin]
    return z_next, x0


def denoise_loop(z, velocity_fn, modality, sigma_video, sigma_audio, anchor=None,
                 anchor_vals=None, velocity_sign: float = 1.0) -> Tuple[np.ndarray, list]:
    """Run the loop over decreasing schedules (each ending at its last value).

    velocity_fn(z, step) returns the velocity for state z; returns the final
    state and the list of X0 estimates, one per step.
    """
    sv = np.asarray(sigma_video, dtype=np.float64)
    sa = np.asarray(sigma_audio, dtype=np.float64)
    if sv.shape != sa.shape or sv.ndim != 1 or sv.size < 2:
        raise ValueError("schedules must be 1-D of one length >= 2")
    x0s = []
    for i in range(sv.size - 1):
        v = velocity_fn(z, i)
        z, x0 = denoise_step(z, v, modality, [[sv[i], sv[i + 1]], [sa[i], sa[i + 1]]],
                             anchor, anchor_vals, velocity_sign)
        x0s.append(x0)
    return z, x0s
