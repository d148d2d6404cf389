"""GPU parity of the line adjoint (separable tilt series) against the oracle.

Geometries whose every view has its rays in planes of one volume axis, with one
detector axis running along it at one pixel per voxel, take the line adjoint
(ct_geom_adjoint_kind reports it).  It forms chords analytically instead of
walking rays, so each of its paths is checked against the float64 oracle:
tilt series about x and y (the electron-tomography dual-axis acquisition), about
z, with mirrored pixel columns, with rays on voxel planes (half-open cells),
with anisotropic voxels, with partial bricks on every axis, over view batches
and regions, and in the SIRT and CGLS modes.  Bar: relative L2 <= 1e-5, and the
adjoint identity with the GPU forward.  (Its dynamic range and reproducibility
are checked with the brick walk's in test_gpu_fixed_point.py, whose dual-axis
workload takes the line adjoint.)
"""
import math

import numpy as np
import pytest

import oracle
import ray_driven_projector_amd as rdp
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


def tilt_about_z(n, first_deg, step_deg):
    """Parallel rays in x-y planes; e_v runs along z (one voxel plane per column)."""
    t = np.radians(first_deg + step_deg * np.arange(n))
    c, s, z = np.cos(t), np.sin(t), np.zeros(n)
    ray = np.stack([c, s, z], 1)
    eu = np.stack([-s, c, z], 1)
    ev = np.stack([z, z, np.ones(n)], 1)
    return np.concatenate([ray, np.zeros_like(ray), eu, ev], 1)


def mirrored(fr):
    """The same rays with both detector axes reversed (pixel columns run backwards)."""
    out = fr.copy()
    out[:, 6:12] *= -1.0
    return out


def shifted(fr, c):
    out = fr.copy()
    out[:, 3:6] += np.asarray(c, float)
    return out


CASES = {
    "dual_axis": dict(vol=(40, 35, 33), sp=(1.0, 1.0, 1.0), det=(50, 44), dsp=(1.0, 1.0),
                      fr=lambda: W.dual_axis_parallel3d(7, -65.0, 19.0)),
    "about_z": dict(vol=(37, 30, 28), sp=(1.0, 1.0, 1.0), det=(47, 37), dsp=(1.0, 1.0),
                    fr=lambda: tilt_about_z(9, -80.0, 20.0)),
    "mirrored": dict(vol=(33, 36, 31), sp=(1.0, 1.0, 1.0), det=(46, 40), dsp=(1.0, 1.0),
                     fr=lambda: mirrored(W.dual_axis_parallel3d(6, -50.0, 17.0))),
    # odd detectors over even volumes: pixel columns and untilted rows lie exactly
    # on voxel planes (the higher cell takes them); 45-degree rays meet cell corners
    "on_planes": dict(vol=(20, 18, 22), sp=(1.0, 1.0, 1.0), det=(31, 29), dsp=(1.0, 1.0),
                      fr=lambda: W.dual_axis_parallel3d(3, -45.0, 45.0)),
    # column planes and rows at fractional voxel positions
    "shifted": dict(vol=(34, 29, 27), sp=(1.0, 1.0, 1.0), det=(41, 38), dsp=(1.0, 1.0),
                    fr=lambda: shifted(W.dual_axis_parallel3d(5, -70.0, 33.0), (0.3, -0.2, 0.4))),
    # tilts of a few degrees, one degree apart, as in the electron-tomography
    # series: steep chord ramps (slopes up to 1 / sin 1 degree)
    "small_tilts": dict(vol=(48, 40, 44), sp=(1.0, 1.0, 1.0), det=(60, 56), dsp=(1.0, 1.0),
                        fr=lambda: W.dual_axis_parallel3d(7, -3.0, 1.0)),
    # anisotropic in-plane voxels (the pixel pitch still matches the voxels along d)
    "anisotropic": dict(vol=(26, 30, 34), sp=(1.25, 1.0, 0.8), det=(44, 40), dsp=(0.8, 1.0),
                        fr=lambda: W.dual_axis_parallel3d(3, -60.0, 40.0)),
}


def case(name):
    c = CASES[name]
    fr = c["fr"]()
    return W.Workload(name, W.BEAM_PARALLEL3D, c["vol"], c["sp"], c["det"], c["dsp"], fr)


@pytest.mark.parametrize("name", list(CASES))
def test_line_adjoint_matches_oracle(name):
    wl = case(name)
    g = rdp.Geometry.from_workload(wl)
    assert rdp.ct_geom_adjoint_kind(geometry=g) == rdp.ADJOINT_LINE
    og = oracle.Geometry.from_workload(wl)
    rng = np.random.default_rng(7)
    x = rng.uniform(0, 1, wl.vol_shape).astype(np.float32)
    y = rng.uniform(-1, 1, wl.sino_shape).astype(np.float32)
    v = torch.empty(g.vol_shape, device="cuda")
    rdp.ct_backproject(g, dev(y), v)
    e_at = rel_l2(host(v), oracle.backproject(og, y))
    s = torch.empty(g.sino_shape, device="cuda")
    rdp.ct_project(g, dev(x), s)
    lhs = float(np.dot(host(s).ravel(), y.astype(np.float64).ravel()))
    rhs = float(np.dot(x.astype(np.float64).ravel(), host(v).ravel()))
    e_id = abs(lhs - rhs) / max(abs(lhs), abs(rhs))
    say(f"{name}: A^T {e_at:.2e}, identity {e_id:.2e}")
    assert e_at <= TOL and e_id <= TOL


@pytest.mark.parametrize("name", ["dual_axis", "about_z", "small_tilts", "anisotropic"])
def test_line_sirt_weights_and_step(name):
    wl = case(name)
    g = rdp.Geometry.from_workload(wl)
    og = oracle.Geometry.from_workload(wl)
    rng = np.random.default_rng(8)
    y = oracle.project(og, rng.uniform(0, 1, wl.vol_shape))
    x0 = rng.uniform(0, 0.5, wl.vol_shape).astype(np.float32)
    R, C = oracle.sirt_weights(og)
    rt = torch.empty(g.sino_shape, device="cuda")
    ct = torch.empty(g.vol_shape, device="cuda")
    rdp.ct_sirt_weights(g, rt, ct)
    e_c = rel_l2(host(ct), C)
    xt = dev(x0)
    work = torch.empty(g.sino_shape, device="cuda")
    rdp.ct_sirt_step(g, xt, dev(y), rt, ct, 0.9, work)
    ref = oracle.sirt(og, y, x0=x0, n_iter=1, relax=0.9, weights=(R, C))
    e_x = rel_l2(host(xt), ref)
    say(f"{name}: C {e_c:.2e}, SIRT step {e_x:.2e}")
    assert e_c <= TOL and e_x <= TOL


def test_line_cgls_step():
    wl = case("dual_axis")
    g = rdp.Geometry.from_workload(wl)
    og = oracle.Geometry.from_workload(wl)
    rng = np.random.default_rng(9)
    y = oracle.project(og, rng.uniform(0, 1, wl.vol_shape)).astype(np.float32)
    vol = lambda: torch.zeros(g.vol_shape, device="cuda")
    x, s, p = vol(), vol(), vol()
    r = torch.empty(g.sino_shape, device="cuda")
    q = torch.empty(g.sino_shape, device="cuda")
    work = torch.empty(rdp.ct_cgls_workspace_size(g), dtype=torch.uint8, device="cuda")
    rdp.ct_cgls_init(g, dev(y), x, r, s, p, work)
    # one oracle step from the GPU's own start
    sc = rdp.ct_cgls_scalars(g, work)
    ref = oracle.cgls_step(og, host(x), host(r), host(s), host(p), sc["gamma"])
    rdp.ct_cgls_step(g, x, r, s, p, q, work)
    ex, es = rel_l2(host(x), ref["x"]), rel_l2(host(s), ref["s"])
    say(f"CGLS step: x {ex:.2e}, s {es:.2e}")
    assert ex <= TOL and es <= TOL


def test_line_view_batches_and_regions():
    wl = case("dual_axis")
    g = rdp.Geometry.from_workload(wl)
    og = oracle.Geometry.from_workload(wl)
    D, H, Wd = wl.vol_shape
    rng = np.random.default_rng(10)
    y = rng.uniform(0, 1, wl.sino_shape).astype(np.float32)
    vb, ve = 2, wl.n_views - 3
    r = (5, 3, 7, D - 9, H - 8, Wd - 12)
    t = torch.empty(r[3:], device="cuda")
    rdp.ct_backproject_region(g, dev(y[vb:ve]), vb, ve, r, t)
    yb = np.zeros_like(y)
    yb[vb:ve] = y[vb:ve]
    z0, y0, x0, nz, ny, nx = r
    ref = oracle.backproject(og, yb)[z0:z0 + nz, y0:y0 + ny, x0:x0 + nx]
    e = rel_l2(host(t), ref)
    say(f"region {r} views [{vb},{ve}): {e:.2e}")
    assert e <= TOL


def test_pitch_mismatch_takes_the_brick_walk():
    wl = case("dual_axis")
    wl = W.Workload("pitch", wl.beam, wl.vol_shape, wl.voxel_spacing, wl.det_shape, (0.8, 0.8), wl.frames)
    assert rdp.ct_geom_adjoint_kind(wl.beam, wl.vol_shape, wl.voxel_spacing, wl.det_shape, wl.det_spacing,
                                    wl.frames) == rdp.ADJOINT_BRICK
    g = rdp.Geometry.from_workload(wl)
    og = oracle.Geometry.from_workload(wl)
    y = np.random.default_rng(12).uniform(0, 1, wl.sino_shape).astype(np.float32)
    v = torch.empty(g.vol_shape, device="cuda")
    rdp.ct_backproject(g, dev(y), v)
    assert rel_l2(host(v), oracle.backproject(og, y)) <= TOL
