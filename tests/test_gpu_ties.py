"""Rays that lie in a lattice plane of an axis they never cross (ties).

Such a ray belongs to the cell above the plane (the half-open cells of the
reading of a ray on a cell boundary).  The frames' float64 arithmetic puts it a
few ulps to either side, and the oracle takes each ray exactly as it computes
it; so here the oracle runs on the same geometry with every ray moved 1e-7 cell
up along all three axes, which puts each tied ray into the cell above and
changes every other ray's integral by far less than the 1e-5 bar.  On dual-axis
tilt series whose pixel centres fall on lattice planes -- a detector pitch of
0.8 cell, odd detectors over even volumes at equal pitch (every pixel on a
plane), anisotropic voxels, tilts through exactly 0 (rays along z) -- the GPU's
A and A^T must match that oracle view by view, and each other through the
adjoint identity, on both adjoints (the brick walk with its ray packets, and the
line adjoint with its aligned rows).
"""
import numpy as np
import pytest

import oracle
import ray_driven_projector_amd as rdp
from ray_driven_projector_amd import workloads as W
from geom_checks import untraversed_plane_distance

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

NUDGE = 1e-7   # cells


def rel(g, o):
    g = np.asarray(g, np.float64).ravel()
    o = np.asarray(o, np.float64).ravel()
    n = np.linalg.norm(o)
    return float(np.linalg.norm(g - o) / (n if n > 0 else 1.0))


def _workload(name, voxel_spacing, det_spacing):
    fr = W.dual_axis_parallel3d(6, -60.0, 20.0)   # tilts -60 .. 40, through exactly 0
    return W.Workload(name, W.BEAM_PARALLEL3D, (20, 24, 28), voxel_spacing, (45, 37), det_spacing, fr, 0)


def _nudged(wl):
    """The same geometry with every parallel ray moved NUDGE cells up on x, y, z."""
    dz, dy, dx = wl.voxel_spacing
    fr = np.array(wl.frames, np.float64)
    fr[:, 3:6] += NUDGE * np.array([dx, dy, dz])
    return W.Workload(wl.name + " nudged", wl.beam, wl.vol_shape, wl.voxel_spacing, wl.det_shape,
                      wl.det_spacing, fr, 0)


CASES = [
    ("pitch 0.8", (1.0, 1.0, 1.0), (0.8, 0.8), rdp.ADJOINT_BRICK),
    ("odd over even", (1.0, 1.0, 1.0), (1.0, 1.0), rdp.ADJOINT_LINE),
    ("anisotropic", (1.0, 0.9, 1.1), (1.0, 1.0), rdp.ADJOINT_BRICK),
    ("anisotropic z", (1.3, 1.0, 1.0), (1.0, 1.0), rdp.ADJOINT_LINE),
]


@pytest.mark.parametrize("name,vsp,dsp,kind", CASES, ids=[c[0] for c in CASES])
def test_rays_in_lattice_planes_take_the_cell_above(name, vsp, dsp, kind):
    wl = _workload(name, vsp, dsp)
    assert untraversed_plane_distance(wl) == 0.0   # some rays lie in such planes
    g = rdp.Geometry.from_workload(wl)
    assert rdp.ct_geom_adjoint_kind(geometry=g) == kind
    og = oracle.Geometry.from_workload(_nudged(wl))
    rng = np.random.default_rng(5)
    x = rng.uniform(0, 1, wl.vol_shape).astype(np.float32)
    y = rng.uniform(0, 1, wl.sino_shape).astype(np.float32)
    sino = torch.empty(g.sino_shape, device="cuda")
    vol = torch.empty(g.vol_shape, device="cuda")
    rdp.ct_project(g, torch.from_numpy(x).cuda(), sino)
    rdp.ct_backproject(g, torch.from_numpy(y).cuda(), vol)
    torch.cuda.synchronize()
    gA, gAT = sino.cpu().numpy(), vol.cpu().numpy()
    oA = oracle.project(og, x.astype(np.float64))
    oAT = oracle.backproject(og, y.astype(np.float64))
    errs = [rel(gA[k], oA[k]) for k in range(wl.n_views)]
    print(name, "A per view", " ".join(f"{e:.1e}" for e in errs), flush=True)
    assert max(errs) <= 1e-5
    # A^T view by view (each view's rays alone), then all views
    yk = np.zeros_like(y)
    for k in range(wl.n_views):
        yk[:] = 0.0
        yk[k] = y[k]
        rdp.ct_backproject(g, torch.from_numpy(yk).cuda(), vol)
        torch.cuda.synchronize()
        e = rel(vol.cpu().numpy(), oracle.backproject(og, yk.astype(np.float64)))
        assert e <= 1e-5, (k, e)
    assert rel(gAT, oAT) <= 1e-5
    # the GPU's own pair is matched: <A x, y> = <x, A^T y>
    lhs = float(np.dot(gA.astype(np.float64).ravel(), y.astype(np.float64).ravel()))
    rhs = float(np.dot(x.astype(np.float64).ravel(), gAT.astype(np.float64).ravel()))
    assert abs(lhs - rhs) <= 1e-5 * abs(lhs)
