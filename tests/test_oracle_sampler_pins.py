"""Pins of the sampler oracle (rectified-flow Euler with exponential sigma shift).

The pages' figure fixes the schedule: 40 passes with the video shift 12.0 and
the audio shift 3.0 evaluate 77 distinct timesteps.  The Euler update is tied
to closed forms: a constant velocity telescopes to z0 - c, and the linear field
dz/dsigma = lambda z gives the product of (1 + lambda dt) exactly.
"""
import json
import os

import numpy as np
import pytest

import oracle.h3_sampler as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")


def test_distinct_timesteps_of_the_pages_40_step_run():
    g = json.load(open(GOLDEN))["sampler_shifts_40_steps"]
    sv = S.schedule(g["steps"], g["shift_video"])[:-1]      # the model evaluations
    sa = S.schedule(g["steps"], g["shift_audio"])[:-1]
    distinct = np.unique(np.round(np.concatenate([sv, sa]), 12))
    assert len(distinct) == g["distinct_timesteps"]
    # and the coincidences are the three predicted by s b/(1+(s-1)b): b = 1; 0.5 ~ 0.8; 0.2 ~ 0.5
    common = sorted(set(np.round(sv, 12)) & set(np.round(sa, 12)))
    np.testing.assert_allclose(common, [0.75, 12 / 13, 1.0], rtol=1e-12)


@pytest.mark.parametrize("steps", [1, 4, 40])
def test_schedule_shape(steps):
    b = S.base_grid(steps)
    np.testing.assert_array_equal(S.schedule(steps, 1.0), b)
    assert b[0] == 1.0 and b[-1] == 0.0 and len(b) == steps + 1
    for s in (3.0, 12.0):
        sig = S.schedule(steps, s)
        assert sig[0] == 1.0 and sig[-1] == 0.0
        assert np.all(np.diff(sig) < 0)
        assert np.all(sig >= b - 1e-15)                       # a shift above 1 holds sigma high


def test_euler_constant_velocity_telescopes():
    z0 = np.random.default_rng(0).standard_normal(7)
    c = np.random.default_rng(1).standard_normal(7)
    z = S.euler(z0, S.schedule(9, 12.0), lambda i, z: c)
    np.testing.assert_allclose(z, z0 - c, rtol=1e-13, atol=1e-13)


def test_euler_linear_field_product_form():
    lam, z0 = 0.7, np.array([1.5, -2.0])
    sig = S.schedule(6, 3.0)
    z = S.euler(z0, sig, lambda i, z: lam * z)
    np.testing.assert_allclose(z, z0 * np.prod(1.0 + lam * np.diff(sig)), rtol=1e-13)


def test_joint_denoise_steps_each_modality_on_its_own_schedule():
    a0, v0 = np.ones(3), np.full(5, 2.0)
    sa, sv = S.schedule(5, 3.0), S.schedule(5, 12.0)
    seen = []

    def vel(i, a, v):
        seen.append(i)
        return a * 0.0 + 1.0, v * 0.0 - 2.0

    a, v = S.denoise(a0, v0, sa, sv, vel)
    assert seen == list(range(5))
    np.testing.assert_allclose(a, a0 - 1.0, rtol=1e-13)
    np.testing.assert_allclose(v, v0 + 2.0, rtol=1e-13)
    # the first pass moves audio by (sa[1]-1) and video by (sv[1]-1): different steps
    a1, v1 = S.denoise(a0, v0, sa[:2], sv[:2], lambda i, a, v: (np.ones(3), np.ones(5)))
    assert not np.isclose(a1[0] - 1.0, v1[0] - 2.0)
