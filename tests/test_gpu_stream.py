"""GPU parity for the host-streaming calls (volume and sinogram in host memory).

ct_backproject_host / ct_project_host pass the data through the device in z
slabs and view batches.  Whatever the plan, the result is A^T y / A x: checked
against the float64 oracle at the 1e-5 bar, bit for bit against the device
calls where the plan reduces to them, and on a lattice of more than 2^30
voxels, which the whole-volume calls refuse.
"""
import ctypes

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


def rel_l2(g, o):
    g = np.asarray(g, np.float64).ravel()
    o = np.asarray(o, np.float64).ravel()
    n = np.linalg.norm(o)
    return float(np.linalg.norm(g - o) / (n if n > 0 else 1.0))


def say(*a):
    print(*a, flush=True)


def _tiny(beam, seed, vol, det, views, **kw):
    if beam in (W.BEAM_PARALLEL2D, W.BEAM_FAN2D):
        vol = (1, vol[1], vol[2])
        det = (det[0], 1)
    return W.tiny_workload(beam, vol, det, views, seed, **kw)


CASES = {
    "cone": dict(beam=W.BEAM_CONE, seed=51, vol=(23, 31, 27), det=(38, 29), views=11, jitter=0.5),
    "parallel3d": dict(beam=W.BEAM_PARALLEL3D, seed=52, vol=(21, 26, 33), det=(40, 28), views=12,
                       jitter=1.0),
    "fan2d": dict(beam=W.BEAM_FAN2D, seed=53, vol=(1, 41, 36), det=(77, 1), views=10),
}
# (slab, batch_views, axis): many slabs and batches, one slab, one batch,
# single planes and views, sizes past the extents (clamped), every slab axis
PLANS = [(7, 4, "z"), (1000, 3, "auto"), (5, 1000, "y"), (1, 1, "x"), (6, 5, "auto"), (4, 7, "x")]


def workload(name):
    c = dict(CASES[name])
    return _tiny(c.pop("beam"), c.pop("seed"), c.pop("vol"), c.pop("det"), c.pop("views"), **c)


def host_buf(shape, pinned):
    if pinned:
        return torch.empty(shape, dtype=torch.float32, pin_memory=True)
    return np.empty(shape, dtype=np.float32)


def as_np(t):
    return t.numpy() if isinstance(t, torch.Tensor) else t


@pytest.mark.parametrize("name", list(CASES))
def test_streamed_operators_match_oracle(name):
    wl = workload(name)
    og = oracle.Geometry.from_workload(wl)
    g = rdp.Geometry.from_workload(wl)
    x, y = W.adjoint_vectors(wl)
    ra, rb = oracle.project(og, x), oracle.backproject(og, y)
    for k, (nz, nb, ax) in enumerate(PLANS):
        pinned = k % 2 == 0
        xs = host_buf(wl.vol_shape, pinned)
        ys = host_buf(wl.sino_shape, pinned)
        as_np(xs)[...] = x
        as_np(ys)[...] = y
        sino = host_buf(wl.sino_shape, pinned)
        vol = host_buf(wl.vol_shape, pinned)
        rdp.ct_project_host(g, xs, sino, nz, nb, ax)
        rdp.ct_backproject_host(g, ys, vol, nz, nb, ax)
        ea, eb = rel_l2(as_np(sino), ra), rel_l2(as_np(vol), rb)
        say(f"{name} plan slab {nz} along {ax} batch {nb} ({'pinned' if pinned else 'pageable'}): "
            f"A {ea:.2e}, A^T {eb:.2e}")
        assert ea <= TOL and eb <= TOL


@pytest.mark.parametrize("name", ["cone", "parallel3d"])
def test_plans_that_reduce_to_device_calls_are_bitwise_equal(name):
    wl = workload(name)
    g = rdp.Geometry.from_workload(wl)
    x, y = W.adjoint_vectors(wl)
    D = wl.vol_shape[0]
    a = torch.empty(g.sino_shape, device="cuda")
    rdp.ct_project(g, dev(x), a)
    b = torch.empty(g.vol_shape, device="cuda")
    rdp.ct_backproject(g, dev(y), b)
    sino = np.empty(wl.sino_shape, np.float32)
    vol = np.empty(wl.vol_shape, np.float32)
    # one slab and one batch: the whole-volume kernels on the uploaded data
    for ax in ("z", "y", "x"):
        rdp.ct_project_host(g, x, sino, 10 ** 6, wl.n_views, ax)
        rdp.ct_backproject_host(g, y, vol, 10 ** 6, wl.n_views, ax)
        assert np.array_equal(sino, a.cpu().numpy())
        assert np.array_equal(vol, b.cpu().numpy())
    # slabs of the adjoint with one batch: each slab is its region call
    ns = 6
    _, H, Wd = wl.vol_shape
    for ax in ("z", "y", "x"):
        rdp.ct_backproject_host(g, y, vol, ns, wl.n_views, ax)
        n_ax = {"z": D, "y": H, "x": Wd}[ax]
        for a0 in range(0, n_ax, ns):
            m = min(ns, n_ax - a0)
            r = {"z": (a0, 0, 0, m, H, Wd), "y": (0, a0, 0, D, m, Wd), "x": (0, 0, a0, D, H, m)}[ax]
            t = torch.empty(r[3:], device="cuda")
            rdp.ct_backproject_region(g, dev(y), 0, wl.n_views, r, t)
            got = vol[r[0]:r[0] + r[3], r[1]:r[1] + r[4], r[2]:r[2] + r[5]]
            assert np.array_equal(got, t.cpu().numpy())
    # repeated streamed adjoint with batches: identical bits
    v2 = np.empty_like(vol)
    rdp.ct_backproject_host(g, y, vol, 5, 4)
    rdp.ct_backproject_host(g, y, v2, 5, 4)
    assert np.array_equal(vol, v2)


def test_stream_argument_errors():
    wl = workload("cone")
    g = rdp.Geometry.from_workload(wl)
    x = np.zeros(wl.vol_shape, np.float32)
    s = np.zeros(wl.sino_shape, np.float32)
    for nz, nb, ax in [(0, 1, 0), (1, 0, 0), (-3, 2, 0), (4, 4, 3), (4, 4, -2)]:
        with pytest.raises(rdp.CtError) as e:
            rdp.ct_project_host(g, x, s, nz, nb, ax)
        assert e.value.status == rdp.CT_E_ARG
        with pytest.raises(rdp.CtError) as e:
            rdp.ct_backproject_host(g, s, x, nz, nb, ax)
        assert e.value.status == rdp.CT_E_ARG
    with pytest.raises(ValueError):   # device tensors are not host buffers
        rdp.ct_project_host(g, dev(x), s, 4, 4)
    with pytest.raises(ValueError):
        rdp.ct_backproject_host(g, s, x[:-1], 4, 4)
    # overlapping host buffers
    big = np.zeros(x.size + s.size, np.float32)
    xv = big[:x.size].reshape(wl.vol_shape)
    sv = big[x.size - 8: x.size - 8 + s.size].reshape(wl.sino_shape)
    with pytest.raises(rdp.CtError) as e:
        rdp.ct_project_host(g, xv, sv, 4, 4)
    assert e.value.status == rdp.CT_E_ALIAS


def test_lattice_beyond_one_buffer():
    """A (1025, 1024, 1024) lattice (more than 2^30 voxels): the whole-volume
    calls refuse it; the streamed adjoint of a sparse sinogram matches the
    oracle's full adjoint, and the streamed forward of a sparse volume matches
    the oracle on the rays through its bright voxels."""
    shape = (1025, 1024, 1024)
    wl = W.tiny_workload(W.BEAM_CONE, shape, (160, 128), 8, 54, det_spacing=(9.0, 9.0),
                         sid=3000.0, sdd=4500.0)
    og = oracle.Geometry.from_workload(wl)
    g = rdp.Geometry.from_workload(wl)
    # whole-volume calls are refused on the host, before any launch
    st = rdp.lib().ct_project(g.handle, ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 40),
                              rdp._stream(None))
    assert st == rdp.CT_E_RANGE
    rng = np.random.default_rng(54)
    U, V = wl.det_shape
    n = wl.n_rays
    ids = np.sort(rng.choice(n, 120, replace=False))
    y = np.zeros(wl.sino_shape, np.float32)
    y.ravel()[ids] = rng.uniform(0.5, 1.5, len(ids)).astype(np.float32)
    say("lattice 1025x1024x1024: streamed adjoint")
    vol = np.empty(shape, np.float32)
    rdp.ct_backproject_host(g, y, vol, 256, 3)
    ref = oracle.backproject(og, y)
    hit = np.flatnonzero(ref.ravel())
    both = np.union1d(hit, np.flatnonzero(vol.ravel()))   # zero elsewhere on both sides
    eb = rel_l2(vol.ravel()[both], ref.ravel()[both])
    say(f"  A^T rel_l2 {eb:.2e} over {hit.size} nonzero voxels")
    assert hit.size > 10000
    del ref
    # forward of a sparse volume, checked on rays that meet its bright voxels
    xs = np.zeros(shape, np.float32)
    bright = rng.choice(hit, 40, replace=False)
    xs.ravel()[bright] = rng.uniform(1.0, 2.0, bright.size).astype(np.float32)
    say("lattice 1025x1024x1024: streamed forward")
    sino = np.empty(wl.sino_shape, np.float32)
    rdp.ct_project_host(g, xs, sino, 300, 5)
    x64 = xs.astype(np.float64)
    del xs
    rays = np.union1d(ids, np.flatnonzero(sino.ravel())[:400])
    ra = oracle.project_rays(og, x64, rays)
    ea = rel_l2(sino.ravel()[rays], ra)
    say(f"  A rel_l2 {ea:.2e} over {rays.size} rays ({int((ra != 0).sum())} nonzero)")
    assert eb <= TOL and ea <= TOL and (ra != 0).sum() > 20
