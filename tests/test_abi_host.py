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
