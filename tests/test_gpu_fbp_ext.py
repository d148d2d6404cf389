"""GPU parity of the FBP overrides and of the helical approximation
(ct_fbp_create_ext, ct_helical_view_weights) against the float64 oracle
(oracle/fbp.py), at the 1e-5 relative L2 bar of the other FBP tests:

- a caller's filter response, on the FFT path and the direct convolution;
- a caller's projection weights, shared and per view, also with Parker's
  weights on a short fan scan;
- helical FDK over several view batches and z bands, its transpose, and a
  caller's slice weights whose zero bands must leave their slices at exactly 0.
"""
import math

import numpy as np
import pytest

import ray_driven_projector_amd as rdp
from oracle import fbp as F
from ray_driven_projector_amd import workloads as W

pytestmark = pytest.mark.gpu
TOL = 1e-5
torch = pytest.importorskip("torch")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host(t):
    return t.detach().cpu().numpy().astype(np.float64)


def rel_l2(g, o):
    g = np.asarray(g, np.float64).ravel()
    o = np.asarray(o, np.float64).ravel()
    n = np.linalg.norm(o)
    return float(np.linalg.norm(g - o) / (n if n > 0 else 1.0))


def say(*a):
    print(*a, flush=True)


def fan(n=90, U=77, span=2 * math.pi):
    fr = W.circular_fan2d(n, 60.0, 100.0, angular_range=span)
    return W.Workload("fan", W.BEAM_FAN2D, (1, 37, 41), (1, 1, 1), (U, 1), (0.8, 1), fr), W.angles(n, span)


def short_fan():
    U, n = 83, 120
    delta = math.atan(0.5 * U * 0.8 / 100.0)
    return fan(n, U, (math.pi + 2 * delta + 0.05) * n / (n - 1))


def cone(n=60, det=(53, 41)):
    fr = W.helix_cone(n, 70.0, 110.0, 0.0, 1.0)
    return W.Workload("cone", W.BEAM_CONE, (19, 27, 30), (1, 1, 1), det, (0.9, 0.8), fr), W.angles(n, 2 * math.pi)


FILTER_CASES = {"fan": lambda: fan(), "fan-pow2": lambda: fan(U=128), "cone": lambda: cone(),
                "cone-pow2": lambda: cone(det=(64, 37))}


@pytest.mark.parametrize("direct", [False, True])
@pytest.mark.parametrize("name", list(FILTER_CASES))
def test_filter_response_matches_oracle(name, direct):
    wl, th = FILTER_CASES[name]()
    U = wl.det_shape[0]
    pad = 2
    P = pad * U
    k = np.arange(P // 2 + 1)
    # a smooth positive gain times the ramp: not any of the built-in windows
    resp = F.ramp_multiplier(P, wl.det_spacing[0]) * (0.6 + 0.4 * np.cos(math.pi * k / P) ** 3)
    f = rdp.FBP.from_workload(wl, th, pad_factor=pad, filter_response=resp, direct_filter=direct)
    sino = np.random.default_rng(1).uniform(0, 1, wl.sino_shape)
    out = torch.empty(wl.sino_shape, device="cuda")
    rdp.ct_fbp_filter(f, dev(sino), out)
    ref = F.filter_sinogram(wl, sino.astype(np.float32), th, pad_factor=pad, filter_response=resp)
    e = rel_l2(host(out), ref)
    say(f"{name} direct={direct}: filter response rel_l2 {e:.2e}")
    assert e <= TOL


@pytest.mark.parametrize("per_view", [False, True])
@pytest.mark.parametrize("name", ["fan", "fan-short", "cone"])
def test_projection_weights_match_oracle(name, per_view):
    wl, th = {"fan": fan, "fan-short": short_fan, "cone": cone}[name]()
    short = name == "fan-short"
    rng = np.random.default_rng(2)
    shape = wl.sino_shape if per_view else wl.det_shape
    pw = rng.uniform(0.5, 1.5, shape)
    f = rdp.FBP.from_workload(wl, th, short_scan=short, projection_weights=pw)
    sino = rng.uniform(0, 1, wl.sino_shape)
    out = torch.empty(wl.sino_shape, device="cuda")
    rdp.ct_fbp_filter(f, dev(sino), out)
    ref = F.filter_sinogram(wl, sino.astype(np.float32), th, short_scan=short, projection_weights=pw)
    e = rel_l2(host(out), ref)
    say(f"{name} per_view={per_view}: projection weights rel_l2 {e:.2e}")
    assert e <= TOL


def helix(N=60, turns=6, pitch=16.0, D=72, hw=(20, 22), det=(48, 40)):
    """N views per turn over `turns` turns, rising `pitch` per turn; D slices of
    1 unit, so D > 64 spans two z bands of the gather."""
    n = N * turns
    fr = W.helix_cone(n, 70.0, 110.0, pitch * turns, turns)
    wl = W.Workload("helix", W.BEAM_CONE, (D, *hw), (1, 1, 1), det, (1.0, 1.0), fr)
    return wl, W.angles(n, 2 * math.pi * turns)


def test_helical_fdk_matches_oracle():
    wl, th = helix()
    sino = np.random.default_rng(3).uniform(0, 1, wl.sino_shape).astype(np.float32)
    f = rdp.FBP.helical_from_workload(wl, th, iso=(0, 0, 0))
    iso, aw = f.info()
    assert np.all(aw == 1.0)
    work = torch.empty(wl.sino_shape, device="cuda")
    vol = torch.empty(wl.vol_shape, device="cuda")
    rdp.ct_fbp_run(f, dev(sino), work, vol)
    ref = F.helical_fdk(wl, sino, th, iso=(0, 0, 0))
    e = rel_l2(host(vol), ref)
    say(f"helical FDK {wl.vol_shape}, {wl.n_views} views: rel_l2 {e:.2e}")
    assert e <= TOL
    # the filtered rows carry no angular weight
    q = F.filter_sinogram(wl, sino, th, ang_weights=np.ones(wl.n_views))
    assert rel_l2(host(work), q) <= TOL


def test_helical_fdk_of_a_ball():
    # exact line integrals of a uniform ball: the GPU result agrees with the
    # oracle and reconstructs the density
    wl, th = helix(N=90, turns=4, pitch=10.0, D=20, hw=(32, 32), det=(80, 48))
    p = F.pixel_centres(wl)
    a = wl.frames[:, None, None, 0:3]
    dvec = (p - a) / np.linalg.norm(p - a, axis=-1, keepdims=True)
    rel = -a
    t = np.sum(rel * dvec, axis=-1)
    sino = 2 * np.sqrt(np.clip(100.0 - (np.sum(rel * rel, axis=-1) - t * t), 0, None))
    f = rdp.FBP.helical_from_workload(wl, th, iso=(0, 0, 0))
    work = torch.empty(wl.sino_shape, device="cuda")
    vol = torch.empty(wl.vol_shape, device="cuda")
    rdp.ct_fbp_run(f, dev(sino), work, vol)
    ref = F.helical_fdk(wl, sino.astype(np.float32), th, iso=(0, 0, 0))
    g = host(vol)
    e = rel_l2(g, ref)
    z, y, x = F.voxel_centres(wl)
    Z, Y, X = np.meshgrid(z, y, x, indexing="ij")
    inside = X ** 2 + Y ** 2 + Z ** 2 < 49.0
    say(f"helical ball: rel_l2 {e:.2e}, interior mean {g[inside].mean():.5f}")
    assert e <= TOL
    assert abs(g[inside].mean() - 1) < 0.005


def test_helical_transpose_and_caller_weights_match_oracle():
    wl, th = helix(N=40, turns=6, D=70, hw=(13, 11), det=(40, 36))
    rng = np.random.default_rng(4)
    w = rdp.ct_helical_view_weights(wl.beam, wl.vol_shape, wl.voxel_spacing, wl.det_shape, wl.det_spacing,
                                    wl.frames, th)
    f = rdp.FBP.helical_from_workload(wl, th, iso=(0, 0, 0))
    x = rng.uniform(-1, 1, wl.vol_shape)
    out = torch.empty(wl.sino_shape, device="cuda")
    rdp.ct_fbp_backproject_transpose(f, dev(x), out)
    ref = F.helical_weighted_backproject_T(wl, x.astype(np.float32), w, iso=(0, 0, 0))
    e = rel_l2(host(out), ref)
    say(f"helical transpose: rel_l2 {e:.2e}")
    assert e <= TOL
    # the caller's own weights: random in the first band, none in the second
    # (slices 64..69), which must come out exactly 0
    cw = rng.uniform(0, 0.1, w.shape) * (rng.random(w.shape) < 0.7)
    cw[64:] = 0.0
    fc = rdp.FBP.helical_from_workload(wl, th, iso=(0, 0, 0), slice_weights=cw)
    q = rng.uniform(-1, 1, wl.sino_shape)
    vol = torch.full(wl.vol_shape, 7.0, device="cuda")
    rdp.ct_fbp_backproject(fc, dev(q), vol)
    ref = F.helical_weighted_backproject(wl, q.astype(np.float32), cw, iso=(0, 0, 0))
    g = host(vol)
    e = rel_l2(g, ref)
    say(f"caller's slice weights: rel_l2 {e:.2e}")
    assert e <= TOL
    assert np.all(g[64:] == 0.0)
