"""Plain CPU oracle of the denoising loop around the velocity forward (float64).

TEST INFRASTRUCTURE ONLY, like ``h3_block``: only the tests, the smoke check of
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.  It shares
no code with the HIP kernels or their host library.

The sampler is rectified-flow Euler with an exponential sigma shift
(minimax-h3-mlx README, "Layout": scheduler.py).  Video and audio run their own
shifted schedules, 12.0 and 3.0, so their timesteps only partly coincide: 77
distinct ones in a 40-step run (minimax-h3-mlx README, "AdaLN precompute").
The number of passes is the step count and a terminal zero follows the last
pass (H3-metal digest, "Sampler and DiT controls").

Reading of those statements, fixed by the 77:
  base grid    b_i = 1 - i / steps, i = 0 .. steps - 1, then the terminal 0
  shift        sigma = s b / (1 + (s - 1) b)   (the exponential shift, s = e^mu)
  Euler pass i for each modality m:
               z_m <- z_m + (sigma_m[i+1] - sigma_m[i]) * v_m(z, sigma[i])
With these, the video (12) and audio (3) schedules of 40 passes meet at exactly
three base points (b = 1; 0.5 with 0.8; 0.2 with 0.5), 80 - 3 = 77.  Text and
condition rows are not denoised.

Whole-velocity reuse (H3-metal digest, "4. Choose a speed/quality preset":
with reuse r, a 20-pass run makes 20, 11 or 8 fresh model evaluations for
r = 1, 2, 3; "Sampler and DiT controls": the first and last pass and every
requested interval are evaluated, and the skipped video and audio velocities
are extrapolated on their independent schedules).  Reading: pass i is fresh
when i % r == 0 or it is the last pass (the only forward schedule that gives
those counts and starts fresh).  A skipped pass i extrapolates each modality's
velocity linearly in that modality's own sigma from its last two fresh
velocities, taken at passes j0 < j1:

    u_m = v_m(j1) + (sigma_m[i] - sigma_m[j1]) / (sigma_m[j1] - sigma_m[j0]) * (v_m(j1) - v_m(j0))

While only one fresh velocity exists (the passes right after pass 0), the
straight line has one point and u_m = v_m(j1).
"""
from __future__ import annotations

from typing import Callable, Tuple

import numpy as np


def base_grid(steps: int) -> np.ndarray:
    """b_i = 1 - i/steps for i < steps, then 0: [steps + 1]."""
    return np.concatenate([1.0 - np.arange(steps, dtype=np.float64) / steps, [0.0]])


def shift_sigmas(b: np.ndarray, shift: float) -> np.ndarray:
    """Exponential shift s b / (1 + (s - 1) b) (identity at s = 1; keeps 0 and 1)."""
    b = np.asarray(b, np.float64)
    return shift * b / (1.0 + (shift - 1.0) * b)


def schedule(steps: int, shift: float) -> np.ndarray:
    """The sigmas of one modality, [steps + 1], from 1 down to the terminal 0."""
    return shift_sigmas(base_grid(steps), shift)


def euler(z0, sigmas, velocity: Callable[[int, np.ndarray], np.ndarray]) -> np.ndarray:
    """Euler over one schedule: z <- z + (s[i+1] - s[i]) * velocity(i, z)."""
    z = np.asarray(z0, np.float64).copy()
    for i in range(len(sigmas) - 1):
        z = z + (sigmas[i + 1] - sigmas[i]) * velocity(i, z)
    return z


def fresh_passes(steps: int, reuse: int = 1) -> np.ndarray:
    """Which of the passes evaluate the model: i % reuse == 0, and the last."""
    i = np.arange(steps)
    return (i % reuse == 0) | (i == steps - 1)


def extrapolate(sigmas, i: int, j0: int, v0, j1: int, v1) -> np.ndarray:
    """The velocity at pass i on the straight line through (sigma[j0], v0) and
    (sigma[j1], v1), sigma being one modality's schedule."""
    c = (sigmas[i] - sigmas[j1]) / (sigmas[j1] - sigmas[j0])
    return v1 + c * (v1 - v0)


def denoise(audio0, video0, sig_audio, sig_video,
            velocity_pair: Callable[[int, np.ndarray, np.ndarray], Tuple[np.ndarray, np.ndarray]],
            reuse: int = 1):
    """Joint Euler over both modalities: a fresh pass runs one velocity forward
    for (v_audio, v_video) from the current latents; a skipped one (reuse > 1)
    extrapolates each modality's last two fresh velocities in its own sigma
    (holds the only one right after pass 0); each latent steps on its own
    schedule."""
    a = np.asarray(audio0, np.float64).copy()
    v = np.asarray(video0, np.float64).copy()
    steps = len(sig_video) - 1
    fresh = fresh_passes(steps, reuse)
    hist = []          # (pass, v_audio, v_video) of the last two fresh passes
    for i in range(steps):
        if fresh[i]:
            va, vv = velocity_pair(i, a, v)
            hist = (hist + [(i, np.asarray(va, np.float64), np.asarray(vv, np.float64))])[-2:]
            ua, uv = hist[-1][1], hist[-1][2]
        elif len(hist) == 1:
            ua, uv = hist[0][1], hist[0][2]
        else:
            (j0, a0, w0), (j1, a1, w1) = hist
            ua = extrapolate(sig_audio, i, j0, a0, j1, a1)
            uv = extrapolate(sig_video, i, j0, w0, j1, w1)
        a = a + (sig_audio[i + 1] - sig_audio[i]) * ua
        v = v + (sig_video[i + 1] - sig_video[i]) * uv
    return a, v
