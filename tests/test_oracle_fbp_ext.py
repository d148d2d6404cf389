"""Pins of the oracle's FBP overrides and of its helical approximation
(oracle/fbp.py), against closed forms and invariants that do not come from
the oracle itself.

Overrides (diffct documentation, "Differentiable analytical reconstruction",
the paragraph on the complete APIs):
- a filter response of ones leaves the rows unfiltered; the response
  cos(2 pi k / P) is the two-tap average (p[u-1] + p[u+1]) / 2 with zeros past
  the row; the windowed ramp passed as a response gives the window's result;
- projection weights of ones drop the cosine weight (the result is the pinned
  ramp filter of the raw rows); per-view scalar weights scale each view;
  shared (U, V) weights equal the same weights repeated per view; the cosine
  weights passed explicitly give the default result.

Helical approximation (same page, "Helical approximation"):
- each slice's weights sum to pi (stated on the page);
- uniform sampling: the closed-form trapezoid weights when the window ends on
  a sample (1/4 of the step at each end, 1/2 inside) or half-way between two
  (1/16 and 7/16 of the step at each end);
- first moment: sum_i w_i theta_i = pi theta_c on any sampling (the hats
  reproduce linear functions), and theta_c where the source crosses the slice
  (the helix's closed form z(theta));
- incomplete windows, slices outside the source's z range and non-monotone
  samples are rejected;
- the per-slice gather reduces to the pinned weighted backprojection when the
  weights do not depend on the slice, and to it on one slice when only that
  slice has weights; its transpose passes the dot-product identity;
- a uniform ball under a helix is reconstructed near density 1, and a small
  off-centre ball lands where it is.
"""
import math

import numpy as np
import pytest

from oracle import fbp as F
from ray_driven_projector_amd import workloads as W

from test_oracle_fbp import _chords_disc, _interior


def _fan(n=60, U=48):
    fr = W.circular_fan2d(n, 60.0, 100.0)
    return W.Workload("f", W.BEAM_FAN2D, (1, 24, 24), (1, 1, 1), (U, 1), (0.8, 1), fr), W.angles(n, 2 * math.pi)


def _cone(n=40, U=24, V=12):
    fr = W.helix_cone(n, 80.0, 130.0, 0.0, 1.0)
    return W.Workload("c", W.BEAM_CONE, (6, 12, 12), (1, 1, 1), (U, V), (0.9, 0.9), fr), W.angles(n, 2 * math.pi)


# ---- filter response ----

def test_unit_response_does_not_filter():
    wl, th = _fan()
    y = np.random.default_rng(1).normal(size=wl.sino_shape)
    for pad in (1, 2, 3):
        P = pad * wl.det_shape[0]
        q = F.filter_sinogram(wl, y, th, pad_factor=pad, ang_weights=np.ones(wl.n_views),
                              projection_weights=np.ones(wl.det_shape), filter_response=np.ones(P // 2 + 1))
        assert np.allclose(q, y, rtol=0, atol=1e-12)


def test_cosine_response_is_the_two_tap_average():
    wl, th = _fan(U=37)
    y = np.random.default_rng(2).normal(size=wl.sino_shape)
    U = wl.det_shape[0]
    for pad in (2, 3):
        P = pad * U
        resp = np.cos(2 * math.pi * np.arange(P // 2 + 1) / P)
        q = F.filter_sinogram(wl, y, th, pad_factor=pad, ang_weights=np.ones(wl.n_views),
                              projection_weights=np.ones(wl.det_shape), filter_response=resp)
        z = np.pad(y, ((0, 0), (1, 1), (0, 0)))
        want = 0.5 * (z[:, :-2] + z[:, 2:])
        assert np.allclose(q, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("window", ["ram-lak", "hann"])
def test_windowed_ramp_as_response_gives_the_window(window):
    wl, th = _cone()
    y = np.random.default_rng(3).normal(size=wl.sino_shape)
    P = 2 * wl.det_shape[0]
    resp = F.ramp_multiplier(P, wl.det_spacing[0], window)
    a = F.filter_sinogram(wl, y, th, window=window)
    b = F.filter_sinogram(wl, y, th, window="shepp-logan", filter_response=resp)
    assert np.allclose(a, b, rtol=0, atol=1e-12 * np.abs(a).max())


def test_response_of_the_wrong_length_is_refused():
    wl, th = _fan()
    with pytest.raises(ValueError):
        F.filter_sinogram(wl, np.zeros(wl.sino_shape), th, filter_response=np.ones(wl.det_shape[0] + 2))


# ---- projection weights ----

def test_unit_projection_weights_drop_the_cosine_weight():
    wl, th = _cone()
    y = np.random.default_rng(4).normal(size=wl.sino_shape)
    aw = F.angular_weights(th, wl.beam)
    q = F.filter_sinogram(wl, y, th, projection_weights=np.ones(wl.det_shape))
    want = F.ramp_filter(y, wl.det_spacing[0], 2, "ram-lak", axis=1) * aw[:, None, None]
    assert np.allclose(q, want, rtol=0, atol=1e-12 * np.abs(want).max())


def test_projection_weights_scale_per_view_and_broadcast():
    wl, th = _cone()
    rng = np.random.default_rng(5)
    y = rng.normal(size=wl.sino_shape)
    c = rng.uniform(0.5, 2.0, wl.n_views)
    base = F.filter_sinogram(wl, y, th, projection_weights=np.ones(wl.det_shape))
    per_view = np.broadcast_to(c[:, None, None], wl.sino_shape)
    q = F.filter_sinogram(wl, y, th, projection_weights=per_view)
    assert np.allclose(q, c[:, None, None] * base, rtol=0, atol=1e-12 * np.abs(base).max())
    shared = rng.uniform(0.2, 1.0, wl.det_shape)
    a = F.filter_sinogram(wl, y, th, projection_weights=shared)
    b = F.filter_sinogram(wl, y, th, projection_weights=np.broadcast_to(shared, wl.sino_shape).copy())
    assert np.array_equal(a, b)
    assert not np.allclose(a, base)


def test_cosine_weights_passed_explicitly_give_the_default():
    wl, th = _fan()
    y = np.random.default_rng(6).normal(size=wl.sino_shape)
    a = F.filter_sinogram(wl, y, th)
    b = F.filter_sinogram(wl, y, th, projection_weights=F.cosine_weights(wl))
    assert np.allclose(a, b, rtol=0, atol=1e-13 * np.abs(a).max())


# ---- helical weights ----

def _helix(N=36, turns=3, per_view_z=1.0, D=9, dz=1.0, start=0.0, sid=80.0, sdd=130.0, U=40, V=24):
    """N views per turn over `turns` turns, the source rising per_view_z per view,
    angles start + k * 2 pi / N."""
    n = N * turns
    fr = W.helix_cone(n, sid, sdd, per_view_z * n, turns)
    th = start + W.angles(n, 2 * math.pi * turns)
    c, s = np.cos(th), np.sin(th)
    fr[:, 0], fr[:, 1] = sid * c, sid * s
    fr[:, 3], fr[:, 4] = -(sdd - sid) * c, -(sdd - sid) * s
    fr[:, 6], fr[:, 7] = s, -c
    wl = W.Workload("h", W.BEAM_CONE, (D, 16, 16), (dz, 1, 1), (U, V), (1.0, 1.0), fr)
    return wl, th


def test_each_slice_weights_sum_to_pi():
    wl, th = _helix()
    w = F.helical_view_weights(wl, th)
    assert w.shape == (wl.vol_shape[0], wl.n_views)
    assert np.allclose(w.sum(axis=1), math.pi, rtol=0, atol=1e-12)
    assert np.all(w >= 0)
    # jittered, descending angles with a falling source
    rng = np.random.default_rng(7)
    wl2, th2 = _helix(N=40)
    th2 = th2 + rng.uniform(-0.3, 0.3, len(th2)) * (2 * math.pi / 40)
    wl2.frames[:, 2] = -wl2.frames[:, 2]
    th2 = -th2
    w2 = F.helical_view_weights(wl2, th2)
    assert np.allclose(w2.sum(axis=1), math.pi, rtol=0, atol=1e-12)


def test_uniform_sampling_window_on_a_sample():
    # D odd, dz 1: slice centres at integers; the source rises one unit per view,
    # so theta_c falls on a sample and so do both ends of the full turn
    N = 36
    step = 2 * math.pi / N
    wl, th = _helix(N=N, D=9)
    w = F.helical_view_weights(wl, th)
    z0 = wl.frames[0, 2]
    for s, zc in enumerate(F.voxel_centres(wl)[0]):
        kc = int(round(zc - z0))                 # the centre sample
        want = np.zeros(wl.n_views)
        want[kc - N // 2 + 1:kc + N // 2] = step / 2
        want[kc - N // 2] = want[kc + N // 2] = step / 4
        assert np.allclose(w[s], want, rtol=0, atol=1e-13), s


def test_uniform_sampling_window_between_samples():
    # D even: slice centres at half-integers, theta_c half-way between samples
    N = 36
    step = 2 * math.pi / N
    wl, th = _helix(N=N, D=8)
    w = F.helical_view_weights(wl, th)
    z0 = wl.frames[0, 2]
    for s, zc in enumerate(F.voxel_centres(wl)[0]):
        k = int(math.floor(zc - z0))            # theta_c between samples k and k + 1
        lo, hi = k - N // 2, k + 1 + N // 2       # the window runs from mid(lo, lo+1) to mid(hi-1, hi)
        want = np.zeros(wl.n_views)
        want[lo + 1:hi] = step / 2
        want[lo] = want[hi] = step / 16
        want[lo + 1] = want[hi - 1] = 7 * step / 16
        assert np.allclose(w[s], want, rtol=0, atol=1e-13), s


def test_first_moment_is_pi_theta_c_at_the_crossing():
    # a helix z(theta) = z0 + h theta on jittered samples: the crossing angle of
    # slice z is (z - z0) / h, and sum_i w_i theta_i = pi theta_c
    rng = np.random.default_rng(8)
    N, turns = 50, 3
    n = N * turns
    th = np.sort(rng.uniform(0, 2 * math.pi * turns, n))
    th[0], th[-1] = 0.0, 2 * math.pi * turns
    h, z0 = 0.9, -10.0
    wl, _ = _helix(N=N, turns=turns, D=7, dz=1.3)
    wl.frames[:, 2] = z0 + h * th
    # the source z is linear in theta, so linear interpolation is exact
    w = F.helical_view_weights(wl, th)
    zc = F.voxel_centres(wl)[0]
    tc = (zc - z0) / h
    assert np.allclose(F.helical_window_centres(wl, th), tc, rtol=0, atol=1e-12)
    assert np.allclose(w @ th, math.pi * tc, rtol=1e-13, atol=1e-11)
    # no weight more than one sample beyond the window
    for s in range(len(zc)):
        far = (th < tc[s] - math.pi) | (th > tc[s] + math.pi)
        inner = np.zeros(n, bool)
        inner[1:-1] = far[:-2] & far[1:-1] & far[2:]
        assert np.all(w[s][inner] == 0)


def test_incomplete_windows_and_bad_samples_are_rejected():
    wl, th = _helix(D=9)
    # 3 turns of 36 views, source from -54 to 53: slices beyond +-35 lack a full turn
    big = W.Workload("h", W.BEAM_CONE, (80, 16, 16), (1, 1, 1), wl.det_shape, wl.det_spacing, wl.frames)
    with pytest.raises(ValueError, match="leaves the scan"):
        F.helical_view_weights(big, th)
    huge = W.Workload("h", W.BEAM_CONE, (120, 16, 16), (1, 1, 1), wl.det_shape, wl.det_spacing, wl.frames)
    with pytest.raises(ValueError, match="outside the source"):
        F.helical_view_weights(huge, th)
    flat = W.Workload("h", W.BEAM_CONE, wl.vol_shape, wl.voxel_spacing, wl.det_shape, wl.det_spacing,
                      wl.frames.copy())
    flat.frames[5, 2] = flat.frames[4, 2]
    with pytest.raises(ValueError, match="monotone"):
        F.helical_view_weights(flat, th)
    bad = th.copy()
    bad[3] = bad[2]
    with pytest.raises(ValueError, match="monotone"):
        F.helical_view_weights(wl, bad)


# ---- the per-slice gather ----

def test_slice_independent_weights_reduce_to_the_gather():
    wl, th = _helix(N=24, turns=2, D=5)
    rng = np.random.default_rng(9)
    q = rng.normal(size=wl.sino_shape)
    c = rng.uniform(0.1, 1.0, wl.n_views)
    a = F.helical_weighted_backproject(wl, q, np.tile(c, (wl.vol_shape[0], 1)), iso=(0, 0, 0))
    b = F.weighted_backproject(wl, q * c[:, None, None], iso=(0, 0, 0))
    assert np.allclose(a, b, rtol=0, atol=1e-12 * np.abs(b).max())


def test_one_weighted_slice_is_that_slice_of_the_gather():
    wl, th = _helix(N=24, turns=2, D=5)
    rng = np.random.default_rng(10)
    q = rng.normal(size=wl.sino_shape)
    c = rng.uniform(0.1, 1.0, wl.n_views)
    full = F.weighted_backproject(wl, q * c[:, None, None], iso=(0, 0, 0))
    for s in (0, 3):
        w = np.zeros((wl.vol_shape[0], wl.n_views))
        w[s] = c
        a = F.helical_weighted_backproject(wl, q, w, iso=(0, 0, 0))
        assert np.allclose(a[s], full[s], rtol=0, atol=1e-12 * np.abs(full).max())
        assert np.all(np.delete(a, s, axis=0) == 0)


def test_helical_gather_transpose_identity():
    wl, th = _helix(N=20, turns=2, D=4, U=24, V=14)
    rng = np.random.default_rng(11)
    w = rng.uniform(0, 1, (wl.vol_shape[0], wl.n_views))
    x = rng.normal(size=wl.vol_shape)
    y = rng.normal(size=wl.sino_shape)
    lhs = np.sum(F.helical_weighted_backproject(wl, y, w, iso=(0, 0, 0)) * x)
    rhs = np.sum(F.helical_weighted_backproject_T(wl, x, w, iso=(0, 0, 0)) * y)
    assert abs(lhs - rhs) <= 1e-12 * max(abs(lhs), 1.0)


# ---- reconstructions from exact line integrals ----

def _helix_scan(pitch, N=120, turns=3, D=12):
    n = N * turns
    fr = W.helix_cone(n, 100.0, 160.0, pitch * turns, turns)
    wl = W.Workload("h", W.BEAM_CONE, (D, 32, 32), (1, 1, 1), (80, 40), (0.8, 0.8), fr)
    return wl, W.angles(n, 2 * math.pi * turns)


def test_uniform_ball_under_a_helix():
    wl, th = _helix_scan(12.0)
    centre, r = (0.0, 0.0, 0.0), 10.0
    rec = F.helical_fdk(wl, _chords_disc(wl, centre, r), th, iso=(0, 0, 0))
    inside = _interior(wl, centre, r, 0.7)
    outside = ~_interior(wl, centre, r, 1.3) & _interior(wl, (0, 0, 0), 15.0, 1.0)
    assert abs(rec[inside].mean() - 1) < 0.003
    assert np.max(np.abs(rec[inside] - 1)) < 0.01
    assert np.mean(np.abs(rec[outside])) < 0.02


def test_small_ball_lands_where_it_is_under_a_low_pitch_helix():
    wl, th = _helix_scan(4.0, D=7)
    centre, r = (4.0, -2.0, 0.3), 4.0
    rec = F.helical_fdk(wl, _chords_disc(wl, centre, r), th, iso=(0, 0, 0))
    z, y, x = F.voxel_centres(wl)
    w = rec * _interior(wl, centre, r, 1.6)
    got = np.array([np.sum(w * x[None, None, :]), np.sum(w * y[None, :, None])]) / np.sum(w)
    assert np.max(np.abs(got - np.array(centre[:2]))) < 0.03, got
