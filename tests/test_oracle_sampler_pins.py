"""Pins of the sampler oracle (rectified-flow Euler with exponential sigma shift).

The pages' figure fixes the schedule: 40 passes with the video shift 12.0 and
the audio shift 3.0 evaluate 77 distinct timesteps.  The Euler update is tied
to closed forms: a constant velocity telescopes to z0 - c, and the linear field
dz/dsigma = lambda z gives the product of (1 + lambda dt) exactly.  Velocity
reuse is pinned by the pages' counts of fresh evaluations (20, 11, 8 at 20
passes for reuse 1, 2, 3), by which passes call the model, by velocity fields
linear in each modality's sigma (reproduced exactly, which a held velocity is
not), and by the known error of extrapolating a quadratic.
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


def test_fresh_evaluation_counts_of_the_pages_reuse_presets():
    g = json.load(open(GOLDEN))["velocity_reuse_20_steps"]
    for r, count in g["fresh_evaluations"].items():
        fresh = S.fresh_passes(g["steps"], int(r))
        assert int(fresh.sum()) == count
        assert fresh[0] and fresh[-1]                     # starts fresh, ends on a fresh velocity


def test_reuse_calls_the_model_only_on_fresh_passes():
    sa, sv = S.schedule(5, 3.0), S.schedule(5, 12.0)
    calls = []

    def vel(i, a, v):
        calls.append(i)
        return np.full(2, float(i + 1)), np.full(3, -float(i + 1))

    S.denoise(np.zeros(2), np.zeros(3), sa, sv, vel, reuse=2)
    assert calls == [0, 2, 4]
    calls.clear()
    S.denoise(np.zeros(2), np.zeros(3), S.schedule(20, 3.0), S.schedule(20, 12.0), vel, reuse=3)
    assert calls == [0, 3, 6, 9, 12, 15, 18, 19]


@pytest.mark.parametrize("reuse", [2, 3, 5])
def test_reuse_is_exact_on_velocities_linear_in_each_modalitys_sigma(reuse):
    """A velocity field that is a straight line in each modality's own sigma
    (and does not depend on the latents) is reproduced exactly by linear
    extrapolation once two fresh velocities exist, so the reuse loop equals the
    loop that evaluates every pass except on passes 1 .. reuse-1, which hold
    v(sigma_0): there it differs by exactly dt_i * beta * (sigma_i - sigma_0).
    A held (zero-order) velocity fails this, and so does extrapolating audio
    along the video schedule (the two schedules are not proportional)."""
    steps = 20
    sa, sv = S.schedule(steps, 3.0), S.schedule(steps, 12.0)
    r = np.random.default_rng(5)
    al_a, be_a, al_v, be_v = (r.standard_normal(n) for n in (4, 4, 6, 6))
    field = lambda i, a, v: (al_a + be_a * sa[i], al_v + be_v * sv[i])  # noqa: E731
    a0, v0 = r.standard_normal(4), r.standard_normal(6)
    fa, fv = S.denoise(a0, v0, sa, sv, field, reuse=1)
    ga, gv = S.denoise(a0, v0, sa, sv, field, reuse=reuse)
    hold = range(1, reuse)
    np.testing.assert_allclose(ga, fa - sum((sa[i + 1] - sa[i]) * be_a * (sa[i] - sa[0]) for i in hold),
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(gv, fv - sum((sv[i + 1] - sv[i]) * be_v * (sv[i] - sv[0]) for i in hold),
                               rtol=1e-12, atol=1e-12)
    # the closed form of the exact Euler sum: sum_i dt_i (alpha + beta sigma_i)
    np.testing.assert_allclose(fa, a0 + al_a * (sa[-1] - sa[0]) + be_a * np.dot(np.diff(sa), sa[:-1]),
                               rtol=1e-12, atol=1e-12)
    # a zero-order hold, written out, gives another answer on the same field
    fresh = S.fresh_passes(steps, reuse)
    held, last = a0.copy(), None
    for i in range(steps):
        if fresh[i]:
            last = al_a + be_a * sa[i]
        held = held + (sa[i + 1] - sa[i]) * last
    assert np.abs(held - ga).max() > 1e-3


def test_reuse_extrapolation_of_a_quadratic_has_the_known_error():
    """v = sigma^2 (audio) and v = -3 sigma^2 (video), reuse 3 over 7 passes:
    fresh at 0, 3 and 6; passes 1 and 2 hold v(0) (one fresh velocity so far),
    passes 4 and 5 take the straight line through passes 0 and 3, which misses
    sigma_i^2 by exactly (sigma_i - sigma_0)(sigma_i - sigma_3)."""
    steps, reuse = 7, 3
    sa, sv = S.schedule(steps, 3.0), S.schedule(steps, 12.0)
    field = lambda i, a, v: (np.array([sa[i] ** 2]), np.array([-3.0 * sv[i] ** 2]))  # noqa: E731
    fa, fv = S.denoise(np.zeros(1), np.zeros(1), sa, sv, field, reuse=1)
    ga, gv = S.denoise(np.zeros(1), np.zeros(1), sa, sv, field, reuse=reuse)
    err_a = sum((sa[i + 1] - sa[i]) * (sa[i] ** 2 - sa[0] ** 2) for i in (1, 2))
    err_a += sum((sa[i + 1] - sa[i]) * (sa[i] - sa[0]) * (sa[i] - sa[3]) for i in (4, 5))
    err_v = sum((sv[i + 1] - sv[i]) * -3.0 * (sv[i] ** 2 - sv[0] ** 2) for i in (1, 2))
    err_v += sum((sv[i + 1] - sv[i]) * -3.0 * (sv[i] - sv[0]) * (sv[i] - sv[3]) for i in (4, 5))
    np.testing.assert_allclose(fa - ga, [err_a], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(fv - gv, [err_v], rtol=1e-12, atol=1e-14)


def test_reuse_on_a_linear_field_holds_while_one_fresh_velocity_exists():
    # dz/dsigma = lam z, reuse 2 over 3 passes: fresh at 0 and 2 (the last);
    # pass 1 has a single fresh velocity to go on, so it steps along it
    lam, z0 = 0.6, 1.25
    s = S.schedule(3, 12.0)
    d = np.diff(s)
    z1 = z0 + d[0] * lam * z0
    z2 = z1 + d[1] * lam * z0
    z3 = z2 + d[2] * lam * z2
    a, v = S.denoise(np.array([z0]), np.array([z0]), s, s, lambda i, a, v: (lam * a, lam * v), reuse=2)
    np.testing.assert_allclose(a, [z3], rtol=1e-13)
    np.testing.assert_allclose(v, [z3], rtol=1e-13)


def test_reuse_one_is_plain_euler():
    sa, sv = S.schedule(6, 3.0), S.schedule(6, 12.0)
    f = lambda i, a, v: (0.3 * a - 0.1, -0.2 * v + 0.05)  # noqa: E731
    a1, v1 = S.denoise(np.ones(4), np.ones(4), sa, sv, f)
    a2, v2 = S.denoise(np.ones(4), np.ones(4), sa, sv, f, reuse=1)
    np.testing.assert_array_equal(a1, a2)
    np.testing.assert_array_equal(v1, v2)
