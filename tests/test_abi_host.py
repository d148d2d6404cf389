"""Host-side tests of the C ABI: exports, frame validation, view tables.

None of these launch GPU work: validation and the view table are computed on
the host before any HIP call, so they run on a CPU-only machine.
"""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import ray_driven_projector_amd as rdp
from ray_driven_projector_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _ensure_built():
    if not os.path.exists(rdp.LIB_PATH):
        from ray_driven_projector_amd import build
        build.build()


@pytest.fixture(scope="module")
def L():
    _ensure_built()
    return rdp.lib()


def test_library_exports_every_declared_symbol(L):
    with open(os.path.join(ROOT, "include", "ctproj.h")) as f:
        header = f.read()
    declared = set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(ct_\w+)\s*\(", header, re.M))
    assert declared == set(rdp.EXPORTS), declared ^ set(rdp.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name
    assert L.ct_version().startswith(b"ctproj")


def _args(wl):
    return (wl.beam, wl.vol_shape, wl.voxel_spacing, wl.det_shape, wl.det_spacing, wl.frames)


@pytest.mark.parametrize("config", [1, 2, 3, 4, 5])
def test_configs_validate(L, config):
    wl = W.make_workload(config, n_views=16)
    assert rdp.ct_geom_validate(*_args(wl)) == rdp.CT_OK, rdp.last_error()


def _variant(wl, **kw):
    a = list(_args(wl))
    names = ["beam", "vol_shape", "voxel_spacing", "det_shape", "det_spacing", "frames"]
    for k, v in kw.items():
        a[names.index(k)] = v
    return a


def test_validation_error_codes(L):
    cone = W.make_workload(3, n_views=8)
    par3 = W.make_workload(4, n_views=8)
    par2 = W.make_workload(1)
    fan = W.make_workload(2, n_views=8)
    assert L.ct_geom_validate(None) == rdp.CT_E_NULL
    # NULL frames
    d, _ = rdp.make_desc(*_args(cone))
    d.frames = ctypes.POINTER(ctypes.c_double)()
    assert L.ct_geom_validate(ctypes.byref(d)) == rdp.CT_E_NULL
    # zero views
    d, fr = rdp.make_desc(*_args(cone))
    d.n_views = 0
    assert L.ct_geom_validate(ctypes.byref(d)) == rdp.CT_E_SHAPE
    # reserved field and beam enum
    d, fr = rdp.make_desc(*_args(cone))
    d.reserved = 1
    assert L.ct_geom_validate(ctypes.byref(d)) == rdp.CT_E_ARG
    assert rdp.ct_geom_validate(*_variant(cone, beam=7)) == rdp.CT_E_ARG
    # shapes
    assert rdp.ct_geom_validate(*_variant(cone, vol_shape=(0, 8, 8))) == rdp.CT_E_SHAPE
    assert rdp.ct_geom_validate(*_variant(cone, det_shape=(8, 0))) == rdp.CT_E_SHAPE
    assert rdp.ct_geom_validate(*_variant(fan, vol_shape=(2, 512, 512))) == rdp.CT_E_SHAPE
    assert rdp.ct_geom_validate(*_variant(fan, det_shape=(736, 2))) == rdp.CT_E_SHAPE
    # lattices beyond one buffer are valid (reached by the region and streaming calls)
    assert rdp.ct_geom_validate(*_variant(cone, vol_shape=(1024, 1024, 1024))) == rdp.CT_OK
    assert rdp.ct_geom_validate(*_variant(cone, vol_shape=(1 << 20, 8, 8))) == rdp.CT_E_RANGE
    assert rdp.ct_geom_validate(*_variant(cone, det_shape=(8, 1 << 20))) == rdp.CT_E_RANGE
    # spacings
    assert rdp.ct_geom_validate(*_variant(cone, voxel_spacing=(1, -1, 1))) == rdp.CT_E_ARG
    assert rdp.ct_geom_validate(*_variant(cone, det_spacing=(0.0, 1))) == rdp.CT_E_ARG
    assert rdp.ct_geom_validate(*_variant(cone, voxel_spacing=(1, math.nan, 1))) == rdp.CT_E_NONFINITE
    # non-finite frame value
    fr = cone.frames.copy(); fr[3, 4] = math.inf
    assert rdp.ct_geom_validate(*_variant(cone, frames=fr)) == rdp.CT_E_NONFINITE
    # non-unit and non-orthogonal axes
    fr = cone.frames.copy(); fr[2, 6:9] *= 1.01
    assert rdp.ct_geom_validate(*_variant(cone, frames=fr)) == rdp.CT_E_FRAME
    fr = cone.frames.copy(); fr[2, 9:12] = fr[2, 6:9]
    assert rdp.ct_geom_validate(*_variant(cone, frames=fr)) == rdp.CT_E_FRAME
    fr = par2.frames.copy(); fr[5, 6:9] = fr[5, 0:3]
    assert rdp.ct_geom_validate(*_variant(par2, frames=fr)) == rdp.CT_E_FRAME
    # parallel3d ray tangent to the detector plane
    fr = par3.frames.copy(); fr[1, 0:3] = fr[1, 6:9]
    assert rdp.ct_geom_validate(*_variant(par3, frames=fr)) == rdp.CT_E_FRAME
    # parallel ray not unit
    fr = par3.frames.copy(); fr[1, 0:3] *= 2
    assert rdp.ct_geom_validate(*_variant(par3, frames=fr)) == rdp.CT_E_FRAME
    # cone source at the detector centre, and edge-on
    fr = cone.frames.copy(); fr[0, 0:3] = fr[0, 3:6]
    assert rdp.ct_geom_validate(*_variant(cone, frames=fr)) == rdp.CT_E_FRAME
    fr = cone.frames.copy(); fr[0, 0:3] = fr[0, 3:6] + 100 * fr[0, 6:9]
    assert rdp.ct_geom_validate(*_variant(cone, frames=fr)) == rdp.CT_E_FRAME
    # 2D frames with z components
    fr = fan.frames.copy(); fr[0, 2] = 1.0
    assert rdp.ct_geom_validate(*_variant(fan, frames=fr)) == rdp.CT_E_FRAME
    # nearer endpoint beyond 1e6 voxel spacings
    fr = cone.frames.copy(); fr[:, 0:6] *= 1e7
    assert rdp.ct_geom_validate(*_variant(cone, frames=fr)) == rdp.CT_E_RANGE
    assert "1e6" in rdp.last_error()


def test_compute_calls_reject_bad_handles_before_any_launch(L):
    nul = ctypes.c_void_p(0)
    one = ctypes.c_void_p(8)
    assert L.ct_project(None, one, one, None) == rdp.CT_E_ARG
    assert L.ct_backproject(None, one, one, None) == rdp.CT_E_ARG
    assert L.ct_backproject_atomic(None, one, one, None) == rdp.CT_E_ARG
    assert L.ct_sirt_step(None, one, one, one, one, 1.0, one, None) == rdp.CT_E_ARG
    assert L.ct_sirt_weights(None, one, one, None) == rdp.CT_E_ARG
    total = ctypes.c_uint64(0)
    assert L.ct_count_intersections(None, nul, ctypes.byref(total), None) == rdp.CT_E_ARG
    assert L.ct_geom_destroy(None) == rdp.CT_OK
    assert L.ct_geom_create(None, None) == rdp.CT_E_NULL
    r = rdp.Region(0, 0, 0, 1, 1, 1)
    assert L.ct_project_region(None, one, r, 0, 1, one, 0, None) == rdp.CT_E_ARG
    assert L.ct_backproject_region(None, one, 0, 1, r, one, 0, None) == rdp.CT_E_ARG
    plan = rdp.StreamPlan(1, 1, -1, 0)
    assert L.ct_project_host(None, one, one, plan, None) == rdp.CT_E_ARG
    assert L.ct_backproject_host(None, one, one, plan, None) == rdp.CT_E_ARG
    assert L.ct_sirt_weights_views(None, 0, 1, one, one, None) == rdp.CT_E_ARG
    assert L.ct_sirt_step_views(None, 0, 1, one, one, one, one, 1.0, 0.0, 1.0, None, one, None) == rdp.CT_E_ARG
    assert L.ct_fbp_filter(None, one, one, None) == rdp.CT_E_ARG
    assert L.ct_fbp_backproject(None, one, one, None) == rdp.CT_E_ARG
    assert L.ct_fbp_backproject_transpose(None, one, one, None) == rdp.CT_E_ARG
    assert L.ct_fbp_run(None, one, one, one, None) == rdp.CT_E_ARG
    assert L.ct_fbp_info(None, None, None) == rdp.CT_E_ARG
    assert L.ct_fbp_destroy(None) == rdp.CT_OK


def test_fbp_plan_arguments_are_checked_on_the_host(L):
    """ct_fbp_create rejects bad options before it touches the device."""
    import math
    cone = W.make_workload(3, scale=8, n_views=12)
    d, fr = rdp.make_desc(*_args(cone))
    th = np.ascontiguousarray(W.angles(12, 2 * math.pi))
    dp = ctypes.POINTER(ctypes.c_double)
    out = ctypes.c_void_p()

    def create(desc=d, angles=th, **kw):
        o = rdp.FbpOpts()
        o.window, o.pad_factor, o.short_scan, o.iso_given, o.reserved = 0, 2, 0, 0, 0
        for k, v in kw.items():
            setattr(o, k, v)
        a = angles.ctypes.data_as(dp) if angles is not None else None
        return L.ct_fbp_create(ctypes.byref(desc), a, None, ctypes.byref(o), ctypes.byref(out))

    assert create(window=5) == rdp.CT_E_ARG
    assert create(pad_factor=0) == rdp.CT_E_ARG
    assert create(pad_factor=17) == rdp.CT_E_ARG
    assert create(reserved=1) == rdp.CT_E_ARG
    assert create(angles=None) == rdp.CT_E_NULL
    bad = th.copy()
    bad[2] = math.inf
    assert create(angles=bad) == rdp.CT_E_NONFINITE
    p3 = W.make_workload(4, scale=32, n_views=4)
    d3, fr3 = rdp.make_desc(*_args(p3))
    assert create(desc=d3, angles=np.ascontiguousarray(th[:4])) == rdp.CT_E_ARG   # parallel3d
    par = W.make_workload(1, scale=2)
    dp2, fr2 = rdp.make_desc(*_args(par))
    assert create(desc=dp2, angles=np.ascontiguousarray(W.angles(90, math.pi)), short_scan=1) == rdp.CT_E_ARG
    assert L.ct_fbp_create(ctypes.byref(d), th.ctypes.data_as(dp), None, None, ctypes.byref(out)) == rdp.CT_E_NULL
    # a cone detector of 500 x (2^20 - 1): (U + 1)(V + 2) < 2^29, but the row
    # stride 8 (V + 2) passes the gather's signed 24-bit offset arithmetic
    tall = W.Workload("tall", W.BEAM_CONE, (4, 4, 4), (1.0, 1.0, 1.0), (500, (1 << 20) - 1), (1.0, 1e-5),
                      W.helix_cone(2, 100.0, 150.0, 0.0, 1.0))
    assert (500 + 1) * ((1 << 20) + 1) < 1 << 29
    dt, frt = rdp.make_desc(*_args(tall))
    assert create(desc=dt, angles=np.ascontiguousarray(W.angles(2, 2 * math.pi))) == rdp.CT_E_RANGE
    assert "2^20" in rdp.last_error()


def test_bench_refuses_several_gpus():
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def _pixel(frames, k, u, v, U, V, du, dv, is2d):
    a, c, eu, ev = frames[k, 0:3], frames[k, 3:6], frames[k, 6:9], frames[k, 9:12]
    p = c + (u - (U - 1) / 2) * du * eu
    if not is2d:
        p = p + (v - (V - 1) / 2) * dv * ev
    return a, p


@pytest.mark.parametrize("config", [1, 2, 3, 4, 5])
def test_view_table_rays_pass_through_pixels(L, config):
    wl = W.make_workload(config, n_views=12)
    T = rdp.ct_geom_view_table(*_args(wl))
    D, H, Wd = wl.vol_shape
    dz, dy, dx = wl.voxel_spacing
    s = np.array([dx, dy, dz])
    lo = -0.5 * np.array([Wd, H, D]) * s
    U, V = wl.det_shape
    du, dv = wl.det_spacing
    is2d = wl.beam in (W.BEAM_PARALLEL2D, W.BEAM_FAN2D)
    parallel = wl.beam in (W.BEAM_PARALLEL2D, W.BEAM_PARALLEL3D)
    rng = np.random.default_rng(config)
    for k in range(wl.n_views):
        t = T[k]
        for _ in range(5):
            u = int(rng.integers(0, U))
            v = 0 if is2d else int(rng.integers(0, V))
            a, p = _pixel(wl.frames, k, u, v, U, V, du, dv, is2d)
            O = t[0:3] + u * t[3:6] + v * t[6:9]
            Dv = t[9:12] + u * t[12:15] + v * t[15:18]
            to_vox = lambda q: (q - lo) / s
            if parallel:
                np.testing.assert_allclose(O, to_vox(p), atol=1e-9)
                np.testing.assert_allclose(Dv, a / s, atol=1e-12)
                ab = np.array(t[24:33]).reshape(3, 3) @ (to_vox(p) - t[0:3])
                np.testing.assert_allclose(ab[1], u, atol=1e-8)
                if not is2d:
                    np.testing.assert_allclose(ab[2], v, atol=1e-8)
            else:
                np.testing.assert_allclose(O, to_vox(a), atol=1e-9)
                np.testing.assert_allclose(O + Dv, to_vox(p), atol=1e-9)
                ab = np.array(t[24:33]).reshape(3, 3) @ (to_vox(p) - t[0:3])
                np.testing.assert_allclose(ab[0], 1.0, atol=1e-10)
                np.testing.assert_allclose(ab[1] / ab[0], u, atol=1e-8)
                if not is2d:
                    np.testing.assert_allclose(ab[2] / ab[0], v, atol=1e-8)
            # detector normal (scaled by spacing) is orthogonal to the pixel steps
            N = t[20:23]
            assert abs(np.dot(N, t[3:6] + t[12:15])) < 1e-9
            assert abs(np.dot(N, t[6:9] + t[15:18])) < 1e-9


# ---- the adjoint's fixed-point range bound ----

@pytest.mark.parametrize("beam", [W.BEAM_PARALLEL2D, W.BEAM_FAN2D, W.BEAM_CONE, W.BEAM_PARALLEL3D])
@pytest.mark.parametrize("spacing", [1.0, 3.0])
def test_adjoint_range_bound_covers_the_rays_through_each_voxel(L, beam, spacing):
    """The host bound on the (ray, voxel) pairs a voxel can collect is at least
    the true count from the oracle's brute-force matrix: per view the most
    rays crossing any one voxel, summed over the views (which bounds every
    voxel's own sum)."""
    import oracle
    vol = (5, 6, 7) if beam >= 2 else (1, 6, 7)
    det = (23, 17) if beam >= 2 else (23, 1)
    wl = W.tiny_workload(beam, vol, det, 6, 13 + beam, voxel_spacing=(spacing,) * 3,
                         det_spacing=(0.7, 0.6), sid=40.0, sdd=70.0, jitter=0.3 if beam >= 2 else 0.0)
    A = oracle.brute_matrix(oracle.Geometry.from_workload(wl))
    per_view = (A > 0).reshape(wl.n_views, -1, A.shape[1]).sum(axis=1)   # (views, voxels)
    need = per_view.max(axis=1).sum()
    bound, shift = rdp.ct_geom_adjoint_range(*_args(wl))
    assert bound >= need, (bound, need)
    assert bound <= wl.n_rays and shift == 0
    # a detector surface is bounded by its pixel count
    bs, _ = rdp.ct_geom_adjoint_range(*_args(wl), surface=True)
    assert bs == wl.n_rays


def test_adjoint_range_shift_rule(L):
    """shift = 0 below 2^16 pairs, else ceil(log2(bound)) - 16: coarse voxels
    seen by many views through a fine detector need it."""
    fr = W.circular_parallel2d(30000)
    bound, shift = rdp.ct_geom_adjoint_range(W.BEAM_PARALLEL2D, (1, 16, 16), (1.0, 8.0, 8.0), (200, 1),
                                            (0.75, 1.0), fr)
    # each voxel's image is at most 8 sqrt(2) / 0.75 pixels wide: about 16 rays a view
    assert 30000 * 8.0 / 0.75 <= bound <= 30000 * (8.0 * math.sqrt(2) / 0.75 + 1) + 1e-6
    assert shift == math.ceil(math.log2(bound)) - 16 == 3
    few = fr[:100]
    b2, s2 = rdp.ct_geom_adjoint_range(W.BEAM_PARALLEL2D, (1, 16, 16), (1.0, 8.0, 8.0), (200, 1),
                                       (0.75, 1.0), few)
    assert b2 < 2 ** 16 and s2 == 0
    # a cone source inside the volume: every ray of the view may cross one voxel
    wl = W.tiny_workload(W.BEAM_CONE, (8, 8, 8), (40, 30), 4, 3, sid=2.0, sdd=30.0)
    b3, _ = rdp.ct_geom_adjoint_range(*_args(wl))
    assert b3 == wl.n_rays
    # the five workloads need no shift; the same geometries with surfaces do
    for c in (1, 2, 3, 4, 5):
        w = W.make_workload(c)
        assert rdp.ct_geom_adjoint_range(*_args(w))[1] == 0


def test_fbp_ext_arguments_are_checked_on_the_host(L):
    """ct_fbp_create_ext rejects bad overrides before it touches the device."""
    cone = W.make_workload(3, scale=8, n_views=12)
    d, fr = rdp.make_desc(*_args(cone))
    th = np.ascontiguousarray(W.angles(12, 2 * math.pi))
    dp = ctypes.POINTER(ctypes.c_double)
    out = ctypes.c_void_p()
    D, n = cone.vol_shape[0], cone.n_views
    U, V = cone.det_shape
    sw = np.ascontiguousarray(np.full((D, n), math.pi / n))

    def create(desc=d, angles=th, aw=None, short_scan=0, **kw):
        o = rdp.FbpOpts()
        o.window, o.pad_factor, o.short_scan, o.iso_given, o.reserved = 0, 2, short_scan, 0, 0
        x = rdp.FbpExt()
        keep = []
        for k, v in kw.items():
            if isinstance(v, np.ndarray):
                v = np.ascontiguousarray(v, dtype=np.float64)
                keep.append(v)
                setattr(x, k, v.ctypes.data_as(dp))
            elif k == "reserved":
                x.reserved[0] = v
            else:
                setattr(x, k, v)
        a = angles.ctypes.data_as(dp) if angles is not None else None
        w = aw.ctypes.data_as(dp) if aw is not None else None
        return L.ct_fbp_create_ext(ctypes.byref(desc), a, w, ctypes.byref(o), ctypes.byref(x), ctypes.byref(out))

    assert create(reserved=1) == rdp.CT_E_ARG
    assert create(projection_weights_per_view=2) == rdp.CT_E_ARG
    assert create(direct_filter=3) == rdp.CT_E_ARG
    bad = np.ones(2 * U // 2 + 1)
    bad[3] = math.nan
    assert create(filter_response=bad) == rdp.CT_E_NONFINITE
    badw = np.ones((U, V))
    badw[1, 2] = math.inf
    assert create(projection_weights=badw) == rdp.CT_E_NONFINITE
    bads = sw.copy()
    bads[0, 0] = math.nan
    assert create(slice_weights=bads) == rdp.CT_E_NONFINITE
    assert create(slice_weights=sw, aw=np.ones(n)) == rdp.CT_E_ARG
    assert create(slice_weights=sw, short_scan=1) == rdp.CT_E_ARG
    fan = W.Workload("f", W.BEAM_FAN2D, (1, 16, 16), (1, 1, 1), (40, 1), (1, 1), W.circular_fan2d(12, 60.0, 100.0))
    df, frf = rdp.make_desc(*_args(fan))
    assert create(desc=df, slice_weights=np.ones((1, 12))) == rdp.CT_E_ARG
    assert "cone" in rdp.last_error()


def _helix_wl(N=36, turns=3, per_view_z=1.0, D=9, dz=1.0, start=0.0):
    n = N * turns
    fr = W.helix_cone(n, 80.0, 130.0, per_view_z * n, turns)
    th = start + W.angles(n, 2 * math.pi * turns)
    c, s = np.cos(th), np.sin(th)
    fr[:, 0], fr[:, 1] = 80.0 * c, 80.0 * s
    fr[:, 3], fr[:, 4] = -50.0 * c, -50.0 * s
    fr[:, 6], fr[:, 7] = s, -c
    return W.Workload("h", W.BEAM_CONE, (D, 16, 16), (dz, 1, 1), (40, 24), (1.0, 1.0), fr), th


def test_helical_view_weights_match_the_oracle(L):
    from oracle import fbp as F
    rng = np.random.default_rng(3)
    cases = [_helix_wl(), _helix_wl(D=8), _helix_wl(N=50, D=13, dz=0.7, start=0.3)]
    wl, th = _helix_wl(N=40, D=11)
    th = th + rng.uniform(-0.3, 0.3, len(th)) * (2 * math.pi / 40)
    wl.frames[:, 2] = -(wl.frames[:, 2] + rng.uniform(-0.2, 0.2, len(th)))
    cases.append((wl, -th))     # descending angles, falling source, jittered
    for wl, th in cases:
        got = rdp.ct_helical_view_weights(*_args(wl), th)
        want = F.helical_view_weights(wl, th)
        assert np.allclose(got, want, rtol=0, atol=1e-12), np.abs(got - want).max()
        assert np.allclose(got.sum(axis=1), math.pi, rtol=0, atol=1e-12)


def test_helical_view_weights_reject_what_the_oracle_rejects(L):
    from oracle import fbp as F
    wl, th = _helix_wl()
    cases = [(W.Workload("h", W.BEAM_CONE, (80, 16, 16), (1, 1, 1), wl.det_shape, wl.det_spacing, wl.frames), th,
              rdp.CT_E_RANGE),
             (W.Workload("h", W.BEAM_CONE, (120, 16, 16), (1, 1, 1), wl.det_shape, wl.det_spacing, wl.frames), th,
              rdp.CT_E_RANGE)]
    flat = wl.frames.copy()
    flat[5, 2] = flat[4, 2]
    cases.append((W.Workload("h", W.BEAM_CONE, wl.vol_shape, wl.voxel_spacing, wl.det_shape, wl.det_spacing, flat),
                  th, rdp.CT_E_ARG))
    bad = th.copy()
    bad[3] = bad[2]
    cases.append((wl, bad, rdp.CT_E_ARG))
    for w, t, code in cases:
        with pytest.raises(ValueError):
            F.helical_view_weights(w, t)
        with pytest.raises(rdp.CtError) as e:
            rdp.ct_helical_view_weights(*_args(w), t)
        assert e.value.status == code, (e.value, code)


def _tilt(n, first, step, axis):
    """Parallel rays tilted about one volume axis; e_v (or e_u for axis x) along it."""
    t = np.radians(first + step * np.arange(n))
    c, s, z, o = np.cos(t), np.sin(t), np.zeros(n), np.ones(n)
    if axis == "x":
        ray, eu, ev = np.stack([z, -s, c], 1), np.stack([o, z, z], 1), np.stack([z, c, s], 1)
    elif axis == "y":
        ray, eu, ev = np.stack([s, z, c], 1), np.stack([c, z, -s], 1), np.stack([z, o, z], 1)
    else:
        ray, eu, ev = np.stack([c, s, z], 1), np.stack([-s, c, z], 1), np.stack([z, z, o], 1)
    return np.concatenate([ray, np.zeros_like(ray), eu, ev], 1)


def _kind(fr, vol=(40, 36, 44), sp=(1.0, 1.0, 1.0), det=(60, 56), dsp=(1.0, 1.0), beam=W.BEAM_PARALLEL3D,
          surface=False):
    return rdp.ct_geom_adjoint_kind(beam, vol, sp, det, dsp, fr, surface=surface)


def test_line_adjoint_eligibility(L):
    """Separable tilt series take the line adjoint; anything that breaks one
    voxel plane per pixel column takes the brick walk (decided on the host)."""
    line, brick = rdp.ADJOINT_LINE, rdp.ADJOINT_BRICK
    wl4 = W.make_workload(4)
    assert rdp.ct_geom_adjoint_kind(wl4.beam, wl4.vol_shape, wl4.voxel_spacing, wl4.det_shape,
                                    wl4.det_spacing, wl4.frames) == line
    for c in (1, 2, 3, 5):
        wl = W.make_workload(c)
        assert rdp.ct_geom_adjoint_kind(wl.beam, wl.vol_shape, wl.voxel_spacing, wl.det_shape,
                                        wl.det_spacing, wl.frames) == brick, c
    for axis in "xyz":
        assert _kind(_tilt(9, -60.0, 15.0, axis)) == line, axis
    both = np.concatenate([_tilt(5, -40.0, 20.0, "x"), _tilt(5, -40.0, 20.0, "z")])
    assert _kind(both) == line                                   # two families, one geometry
    assert _kind(_tilt(9, -60.0, 15.0, "x"), surface=True) == brick
    assert _kind(_tilt(9, -60.0, 15.0, "x"), dsp=(0.8, 1.0)) == brick      # 1.25 columns per voxel plane
    assert _kind(_tilt(9, -60.0, 15.0, "x"), sp=(1.0, 1.0, 2.0)) == brick  # half a column per plane
    # pixel spacing equal to the voxel spacing along the untraversed axis is enough
    assert _kind(_tilt(9, -60.0, 15.0, "x"), sp=(1.5, 0.7, 2.0), dsp=(2.0, 1.0)) == line
    # a ray direction leaving the plane, or a row axis with a component along it
    fr = _tilt(9, -60.0, 15.0, "x")
    tilted = fr.copy()
    tilted[:, 0] = 1e-3
    tilted[:, 0:3] /= np.linalg.norm(tilted[:, 0:3], axis=1)[:, None]
    assert _kind(tilted) == brick
    # the detector axes turned by 2 degrees about the ray: neither runs along x alone
    skew = fr.copy()
    b = math.radians(2.0)
    skew[:, 6:9] = math.cos(b) * fr[:, 6:9] + math.sin(b) * fr[:, 9:12]
    skew[:, 9:12] = -math.sin(b) * fr[:, 6:9] + math.cos(b) * fr[:, 9:12]
    assert _kind(skew) == brick
    # a detector far finer than the voxels across the rays would need more staged rows
    assert _kind(_tilt(9, -60.0, 15.0, "y"), sp=(1.0, 0.25, 1.0), dsp=(1.0, 0.25)) in (line, brick)
    assert _kind(_tilt(9, -60.0, 15.0, "x"), vol=(40, 36, 44), sp=(1.0, 1.0, 1.0), det=(60, 56),
                 dsp=(1.0, 0.2)) == brick
    # 2D beams and fan/cone never do
    fan = W.make_workload(2)
    assert rdp.ct_geom_adjoint_kind(fan.beam, fan.vol_shape, fan.voxel_spacing, fan.det_shape, fan.det_spacing,
                                    fan.frames) == brick
