"""Range of the brick adjoint's fixed-point accumulation.

Each brick accumulates its terms in 64-bit integers whose unit is set by the
largest ray value reaching it.  Two properties are checked here:

- Dynamic range.  A ray far below the brick's largest keeps its own 24
  significant bits, so the adjoint of a sinogram is, per voxel, the sum of the
  adjoints of its parts split by magnitude, to float32-like precision:
      |g(y) - sum_c g(y_c)| <= 2^-17 sum_c g(|y_c|) + output rounding,
  whatever the parts' relative sizes (one ray a million times the rest,
  values spread over seven decades or over 2^0 .. 2^-40).  Without the range
  handling the small parts would be rounded to the large part's unit (a ray of
  1e-6 of the largest kept 3 bits).  The whole results are also checked
  against the float64 oracle (relative L2 <= 1e-5).
- No overflow.  Geometries that put many terms into each voxel (coarse voxels
  seen through a fine detector from many views) are checked against the
  oracle per voxel: |g_j - o_j| <= 1e-5 sum_i |a_ij y_i|.

The same bits come back on a second run in every case.
"""
import numpy as np
import pytest

import oracle
import ray_driven_projector_amd as rdp
from ray_driven_projector_amd import workloads as W

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
TOL = 1e-5


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host(t):
    return t.detach().cpu().numpy().astype(np.float64)


def say(*a):
    print(*a, flush=True)


def _cone():
    # a jittered cone with magnification 1.5 on a 48^3 volume (edge bricks of
    # several shapes)
    fr = W.jitter_frames(W.helix_cone(120, 150.0, 225.0, 0.0, 1.0), W.Stream(71), 0.5, 0.5)
    return W.Workload("cone 48^3", W.BEAM_CONE, (48, 48, 48), (1.0, 1.0, 1.0), (104, 80), (1.0, 1.0), fr)


def _par3d():
    fr = W.dual_axis_parallel3d(45, -70.0, 140.0 / 45)
    return W.Workload("parallel3d 40x48x44", W.BEAM_PARALLEL3D, (40, 48, 44), (1.0, 1.0, 1.0), (80, 72),
                      (1.0, 1.0), fr)


def _fan():
    return W.Workload("fan 96^2", W.BEAM_FAN2D, (1, 96, 96), (1.0, 1.0, 1.0), (160, 1), (1.0, 1.0),
                      W.circular_fan2d(180, 120.0, 200.0))


WORKLOADS = {"cone": _cone, "parallel3d": _par3d, "fan": _fan}


class Case:
    def __init__(self, wl):
        self.wl = wl
        self.og = oracle.Geometry.from_workload(wl)
        self.g = rdp.Geometry.from_workload(wl)

    def AT(self, y):
        out = torch.empty(self.g.vol_shape, device="cuda")
        rdp.ct_backproject(self.g, dev(y), out)
        return out


def _range_check(name, wl, parts, label):
    """parts: float32 sinograms of disjoint support whose sum is the input."""
    c = Case(wl)
    y = np.sum(parts, axis=0).astype(np.float32)
    gt = c.AT(y)
    g = host(gt)
    gs = [host(c.AT(p)) for p in parts]
    mag = np.sum([host(c.AT(np.abs(p))) for p in parts], axis=0)
    diff = np.abs(g - np.sum(gs, axis=0))
    bound = 2.0 ** -17 * mag + 4 * 2.0 ** -24 * (np.abs(g) + np.sum(np.abs(gs), axis=0)) + 1e-30
    worst = float(np.max(diff / bound))
    o = oracle.backproject(c.og, y.astype(np.float64))
    e = float(np.linalg.norm(g - o) / np.linalg.norm(o))
    say(f"{name} {label}: |g(y) - sum g(parts)| / bound worst {worst:.3e}; oracle relative L2 {e:.2e}")
    assert np.all(diff <= bound), (name, label, worst)
    assert e <= TOL
    assert torch.equal(gt, c.AT(y))


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_one_ray_a_million_times_larger(name):
    wl = WORKLOADS[name]()
    rng = np.random.default_rng(6)
    small = rng.uniform(0.5, 1.5, wl.sino_shape).astype(np.float32)
    big = np.zeros_like(small)
    U, V = wl.det_shape
    for k in range(0, wl.n_views, max(1, wl.n_views // 5)):
        big[k, U // 2, V // 2] = 1e6 * small[k, U // 2, V // 2]
        small[k, U // 2, V // 2] = 0.0
    _range_check(name, wl, [big, small], "one ray x 1e6")


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_log_uniform_sinogram(name):
    wl = WORKLOADS[name]()
    rng = np.random.default_rng(5)
    y = (10.0 ** rng.uniform(-7, 0, wl.sino_shape)) * np.where(rng.random(wl.sino_shape) < 0.5, -1.0, 1.0)
    y = y.astype(np.float32)
    # split by decade
    dec = np.floor(np.log10(np.abs(y.astype(np.float64)))).astype(int)
    parts = [np.where(dec == d, y, 0.0).astype(np.float32) for d in range(-7, 0)]
    _range_check(name, wl, parts, "signed 10^U[-7,0] by decade")


@pytest.mark.parametrize("name", ["cone", "parallel3d"])
def test_rays_spanning_every_exponent(name):
    """Ray i holds 2^-(i mod 41): every brick sees the whole range."""
    wl = WORKLOADS[name]()
    k = (np.arange(wl.n_rays) % 41).reshape(wl.sino_shape)
    y = np.ldexp(1.0, -k).astype(np.float32)
    parts = [np.where((k >= lo) & (k < lo + 8), y, 0.0).astype(np.float32) for lo in range(0, 41, 8)]
    _range_check(name, wl, parts, "2^-(0..40) in bands of 8 exponents")


def _overflow_check(wl, label):
    c = Case(wl)
    y = np.full(wl.sino_shape, 1.9, np.float32)
    o = oracle.backproject(c.og, y.astype(np.float64))
    bound = TOL * np.abs(o)              # y > 0: sum_i |a_ij y_i| = o_j
    gt = c.AT(y)
    g = host(gt)
    worst = float(np.max(np.abs(g - o) / np.where(bound > 0, bound, 1.0)))
    shift = rdp.ct_geom_adjoint_range(geometry=c.g)[1]
    say(f"{label}: term shift {shift}, worst per-voxel error / bound {worst:.3e}")
    assert shift > 0
    assert np.all(np.abs(g - o) <= bound + 1e-30), worst
    assert torch.equal(gt, c.AT(y))


def test_many_terms_per_voxel_2d():
    """Coarse voxels through a fine detector from many views: about 30000 x 16
    (ray, voxel) pairs per voxel, past the 64-bit range without the shift."""
    wl = W.Workload("parallel2d 16^2 of 8, 200 bins of 0.75", W.BEAM_PARALLEL2D, (1, 16, 16), (1.0, 8.0, 8.0),
                    (200, 1), (0.75, 1.0), W.circular_parallel2d(30000))
    _overflow_check(wl, "parallel2d, 30000 views")


def test_many_terms_per_voxel_3d():
    """The same in 3D: 2000 views of 6-unit voxels through a 0.4-pitch detector."""
    fr = W.dual_axis_parallel3d(1000, -80.0, 160.0 / 1000)
    wl = W.Workload("parallel3d 4x8x8 of 6, 130^2 of 0.4", W.BEAM_PARALLEL3D, (4, 8, 8), (6.0, 6.0, 6.0),
                    (130, 130), (0.4, 0.4), fr)
    _overflow_check(wl, "parallel3d, 2000 views")
