"""Python binding of libctproj, the gfx950 ray-driven projector pair.

The functions here carry the C ABI's names (include/ctproj.h) and only marshal
arguments: torch tensors are checked (device, dtype, contiguity, shape) and
their device pointers and the current HIP stream are handed to the library.
Every step of the computation runs in the library's HIP kernels.  If the
built library is missing, the first call raises; there is no fallback.

Geometry: ``Geometry`` wraps a ``ct_geom_t`` handle made from a beam type,
shapes and per-view frames (see ``workloads.py`` for the frame layout).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libctproj.so")

CT_OK, CT_E_NULL, CT_E_SHAPE, CT_E_NONFINITE, CT_E_FRAME, CT_E_RANGE, CT_E_ALIAS, \
    CT_E_NOMEM, CT_E_HIP, CT_E_ARG = range(10)
STATUS_NAMES = {0: "CT_OK", 1: "CT_E_NULL", 2: "CT_E_SHAPE", 3: "CT_E_NONFINITE",
                4: "CT_E_FRAME", 5: "CT_E_RANGE", 6: "CT_E_ALIAS", 7: "CT_E_NOMEM",
                8: "CT_E_HIP", 9: "CT_E_ARG"}
CT_PARALLEL2D, CT_FAN2D, CT_CONE, CT_PARALLEL3D = range(4)
CT_VIEW_TABLE_STRIDE = 48

# every symbol declared in include/ctproj.h
EXPORTS = ["ct_geom_validate", "ct_geom_create", "ct_geom_create_surface", "ct_geom_destroy",
           "ct_geom_view_table", "ct_geom_adjoint_range", "ct_geom_adjoint_kind",
           "ct_project", "ct_project_ws", "ct_forward_workspace_size", "ct_backproject",
           "ct_backproject_atomic", "ct_project_region",
           "ct_backproject_region", "ct_project_host", "ct_backproject_host",
           "ct_fbp_create", "ct_fbp_create_ext", "ct_helical_view_weights", "ct_fbp_destroy", "ct_fbp_info", "ct_fbp_filter", "ct_fbp_backproject",
           "ct_fbp_backproject_transpose", "ct_fbp_run", "ct_sirt_weights_views", "ct_sirt_step_views",
           "ct_sirt_weights",
           "ct_sirt_residual", "ct_sirt_update", "ct_sirt_step", "ct_sirt_update_bounded",
           "ct_sirt_step_bounded", "ct_cgls_workspace_size",
           "ct_cgls_init", "ct_cgls_step", "ct_cgls_step_noalloc", "ct_cgls_scalars", "ct_count_intersections",
           "ct_last_error", "ct_version"]


class CtError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class GeomDesc(ctypes.Structure):
    _fields_ = [("beam", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("n_views", ctypes.c_int64),
                ("vol_shape", ctypes.c_int64 * 3), ("voxel_spacing", ctypes.c_double * 3),
                ("det_shape", ctypes.c_int64 * 2), ("det_spacing", ctypes.c_double * 2),
                ("frames", ctypes.POINTER(ctypes.c_double))]


class Region(ctypes.Structure):
    _fields_ = [("z0", ctypes.c_int64), ("y0", ctypes.c_int64), ("x0", ctypes.c_int64),
                ("nz", ctypes.c_int64), ("ny", ctypes.c_int64), ("nx", ctypes.c_int64)]


class StreamPlan(ctypes.Structure):
    _fields_ = [("slab", ctypes.c_int64), ("batch_views", ctypes.c_int64),
                ("axis", ctypes.c_int32), ("reserved", ctypes.c_int32)]


AXES = {"auto": -1, "z": 0, "y": 1, "x": 2}


_lib = None


def lib():
    """Load libctproj.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run ray_driven_projector_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        P, c = ctypes.POINTER, ctypes
        vp = c.c_void_p
        st = c.c_int
        L.ct_geom_validate.argtypes = [P(GeomDesc)]
        L.ct_geom_create.argtypes = [P(GeomDesc), P(vp)]
        L.ct_geom_create_surface.argtypes = [P(GeomDesc), P(c.c_double), c.c_int, P(vp)]
        L.ct_geom_destroy.argtypes = [vp]
        L.ct_geom_view_table.argtypes = [vp, P(GeomDesc), P(c.c_double)]
        L.ct_geom_adjoint_range.argtypes = [vp, P(GeomDesc), c.c_int, P(c.c_double), P(c.c_int32)]
        L.ct_geom_adjoint_kind.argtypes = [vp, P(GeomDesc), c.c_int, P(c.c_int32)]
        L.ct_project.argtypes = [vp, vp, vp, vp]
        L.ct_project_ws.argtypes = [vp, vp, vp, vp, c.c_size_t, vp]
        L.ct_forward_workspace_size.argtypes = [vp, P(GeomDesc), P(c.c_size_t)]
        L.ct_backproject.argtypes = [vp, vp, vp, vp]
        L.ct_backproject_atomic.argtypes = [vp, vp, vp, vp]
        L.ct_project_region.argtypes = [vp, vp, Region, c.c_int64, c.c_int64, vp, c.c_int, vp]
        L.ct_backproject_region.argtypes = [vp, vp, c.c_int64, c.c_int64, Region, vp, c.c_int, vp]
        L.ct_project_host.argtypes = [vp, vp, vp, StreamPlan, vp]
        dp = P(c.c_double)
        L.ct_fbp_create.argtypes = [vp, dp, dp, vp, vp]
        L.ct_fbp_create_ext.argtypes = [vp, dp, dp, vp, vp, vp]
        L.ct_helical_view_weights.argtypes = [vp, dp, dp]
        L.ct_fbp_destroy.argtypes = [vp]
        L.ct_fbp_info.argtypes = [vp, dp, dp]
        L.ct_fbp_filter.argtypes = [vp, vp, vp, vp]
        L.ct_fbp_backproject.argtypes = [vp, vp, vp, vp]
        L.ct_fbp_backproject_transpose.argtypes = [vp, vp, vp, vp]
        L.ct_fbp_run.argtypes = [vp, vp, vp, vp, vp]
        L.ct_backproject_host.argtypes = [vp, vp, vp, StreamPlan, vp]
        L.ct_sirt_weights.argtypes = [vp, vp, vp, vp]
        L.ct_sirt_weights_views.argtypes = [vp, c.c_int64, c.c_int64, vp, vp, vp]
        L.ct_sirt_step_views.argtypes = [vp, c.c_int64, c.c_int64, vp, vp, vp, vp, c.c_float, c.c_float,
                                         c.c_float, vp, vp, vp]
        L.ct_sirt_residual.argtypes = [vp, vp, vp, vp, vp, vp]
        L.ct_sirt_update.argtypes = [vp, vp, vp, c.c_float, vp, vp]
        L.ct_sirt_step.argtypes = [vp, vp, vp, vp, vp, c.c_float, vp, vp]
        L.ct_sirt_update_bounded.argtypes = [vp, vp, vp, c.c_float, c.c_float, c.c_float, vp, vp, vp]
        L.ct_sirt_step_bounded.argtypes = [vp, vp, vp, vp, vp, c.c_float, c.c_float, c.c_float, vp,
                                           vp, vp]
        L.ct_cgls_workspace_size.argtypes = [vp, P(c.c_size_t)]
        L.ct_cgls_init.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp]
        L.ct_cgls_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp]
        L.ct_cgls_step_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp]
        L.ct_cgls_scalars.argtypes = [vp, vp, P(c.c_double), vp]
        L.ct_count_intersections.argtypes = [vp, vp, P(c.c_uint64), vp]
        for name in EXPORTS[:-2]:
            getattr(L, name).restype = st
        L.ct_last_error.restype = c.c_char_p
        L.ct_last_error.argtypes = []
        L.ct_version.restype = c.c_char_p
        L.ct_version.argtypes = []
        _lib = L
    return _lib


def _check(status: int):
    if status != CT_OK:
        raise CtError(status, lib().ct_last_error().decode())


def make_desc(beam, vol_shape, voxel_spacing, det_shape, det_spacing, frames):
    """Build a ct_geom_desc_t; returns (desc, frames_array) -- keep both alive."""
    fr = np.ascontiguousarray(frames, dtype=np.float64)
    if fr.ndim != 2 or fr.shape[1] != 12:
        raise ValueError("frames must be (n_views, 12)")
    d = GeomDesc()
    d.beam = int(beam)
    d.reserved = 0
    d.n_views = fr.shape[0]
    for k in range(3):
        d.vol_shape[k] = int(vol_shape[k])
        d.voxel_spacing[k] = float(voxel_spacing[k])
    for k in range(2):
        d.det_shape[k] = int(det_shape[k])
        d.det_spacing[k] = float(det_spacing[k])
    d.frames = fr.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    return d, fr


def ct_geom_validate(beam, vol_shape, voxel_spacing, det_shape, det_spacing, frames) -> int:
    """Host-only frame validation; returns the ct_status_t code."""
    d, fr = make_desc(beam, vol_shape, voxel_spacing, det_shape, det_spacing, frames)
    return int(lib().ct_geom_validate(ctypes.byref(d)))


def ct_geom_view_table(beam, vol_shape, voxel_spacing, det_shape, det_spacing, frames):
    """Host-computed per-view ray table (n_views x CT_VIEW_TABLE_STRIDE float64)."""
    d, fr = make_desc(beam, vol_shape, voxel_spacing, det_shape, det_spacing, frames)
    out = np.zeros((fr.shape[0], CT_VIEW_TABLE_STRIDE), dtype=np.float64)
    _check(lib().ct_geom_view_table(None, ctypes.byref(d),
                                    out.ctypes.data_as(ctypes.POINTER(ctypes.c_double))))
    return out


def ct_geom_adjoint_range(beam=None, vol_shape=None, voxel_spacing=None, det_shape=None, det_spacing=None,
                          frames=None, surface=False, geometry=None):
    """(rays_bound, shift) of the adjoint's fixed-point range: from a handle
    (geometry=) or computed on the host from the description."""
    bound = ctypes.c_double(0.0)
    shift = ctypes.c_int32(0)
    if geometry is not None:
        _check(lib().ct_geom_adjoint_range(geometry.handle, None, int(surface), ctypes.byref(bound),
                                           ctypes.byref(shift)))
    else:
        d, fr = make_desc(beam, vol_shape, voxel_spacing, det_shape, det_spacing, frames)
        _check(lib().ct_geom_adjoint_range(None, ctypes.byref(d), int(surface), ctypes.byref(bound),
                                           ctypes.byref(shift)))
    return float(bound.value), int(shift.value)


ADJOINT_BRICK, ADJOINT_LINE = 0, 1


def ct_geom_adjoint_kind(beam=None, vol_shape=None, voxel_spacing=None, det_shape=None, det_spacing=None,
                         frames=None, surface=False, geometry=None):
    """Which adjoint the geometry takes (ADJOINT_BRICK or ADJOINT_LINE): from a
    handle (geometry=) or decided on the host from the description."""
    kind = ctypes.c_int32(-1)
    if geometry is not None:
        _check(lib().ct_geom_adjoint_kind(geometry.handle, None, int(surface), ctypes.byref(kind)))
    else:
        d, fr = make_desc(beam, vol_shape, voxel_spacing, det_shape, det_spacing, frames)
        _check(lib().ct_geom_adjoint_kind(None, ctypes.byref(d), int(surface), ctypes.byref(kind)))
    return int(kind.value)


def last_error() -> str:
    return lib().ct_last_error().decode()


class Geometry:
    """A ct_geom_t handle (device tables on the current HIP device).  offsets:
    optional detector surface, float64 (U, V, 3) or (views, U, V, 3)
    (ct_geom_create_surface)."""

    def __init__(self, beam, vol_shape, voxel_spacing, det_shape, det_spacing, frames,
                 offsets=None):
        d, fr = make_desc(beam, vol_shape, voxel_spacing, det_shape, det_spacing, frames)
        h = ctypes.c_void_p()
        if offsets is None:
            _check(lib().ct_geom_create(ctypes.byref(d), ctypes.byref(h)))
        else:
            off = np.ascontiguousarray(offsets, dtype=np.float64)
            nu, nv = int(det_shape[0]), int(det_shape[1])
            if off.shape == (nu, nv, 3):
                per_view = 0
            elif off.shape == (fr.shape[0], nu, nv, 3):
                per_view = 1
            else:
                raise ValueError("offsets must be (U, V, 3) or (views, U, V, 3)")
            _check(lib().ct_geom_create_surface(ctypes.byref(d),
                                                off.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                                per_view, ctypes.byref(h)))
        self._h = h
        self.beam = int(beam)
        self.vol_shape = tuple(int(x) for x in vol_shape)
        self.sino_shape = (fr.shape[0], int(det_shape[0]), int(det_shape[1]))

    @classmethod
    def from_workload(cls, wl) -> "Geometry":
        return cls(wl.beam, wl.vol_shape, wl.voxel_spacing, wl.det_shape, wl.det_spacing, wl.frames,
                   getattr(wl, "offsets", None))

    @property
    def handle(self):
        return self._h

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().ct_geom_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):  # pragma: no cover - best effort
        try:
            self.close()
        except Exception:
            pass


WINDOWS = {"ram-lak": 0, None: 0, "shepp-logan": 1, "cosine": 2, "hamming": 3, "hann": 4, "hanning": 4}


class FbpOpts(ctypes.Structure):
    _fields_ = [("window", ctypes.c_int32), ("pad_factor", ctypes.c_int32),
                ("short_scan", ctypes.c_int32), ("iso_given", ctypes.c_int32),
                ("iso", ctypes.c_double * 3), ("reserved", ctypes.c_int64)]


class FbpExt(ctypes.Structure):
    _fields_ = [("filter_response", ctypes.POINTER(ctypes.c_double)),
                ("projection_weights", ctypes.POINTER(ctypes.c_double)),
                ("slice_weights", ctypes.POINTER(ctypes.c_double)),
                ("projection_weights_per_view", ctypes.c_int32), ("direct_filter", ctypes.c_int32),
                ("reserved", ctypes.c_int64 * 4)]


def ct_helical_view_weights(beam, vol_shape, voxel_spacing, det_shape, det_spacing, frames, angles):
    """(D, n_views) per-slice weights of the helical approximation (host, float64)."""
    d, fr = make_desc(beam, vol_shape, voxel_spacing, det_shape, det_spacing, frames)
    th = np.ascontiguousarray(angles, dtype=np.float64)
    if th.shape != (fr.shape[0],):
        raise ValueError("angles must have one value per view")
    out = np.zeros((int(vol_shape[0]), fr.shape[0]))
    dp = ctypes.POINTER(ctypes.c_double)
    _check(lib().ct_helical_view_weights(ctypes.byref(d), th.ctypes.data_as(dp), out.ctypes.data_as(dp)))
    return out


class FBP:
    """A ct_fbp_t plan: analytical FBP (parallel2d, fan2d) / FDK (cone).
    angles: n_views radians (host); angular_weights: optional override.
    filter_response (pad_factor * U // 2 + 1), projection_weights ((U, V) or
    (views, U, V)) and slice_weights ((D, views), cone) are the overrides of
    ct_fbp_create_ext; direct_filter keeps step 2 on the direct convolution."""

    def __init__(self, beam, vol_shape, voxel_spacing, det_shape, det_spacing, frames, angles=None,
                 window="ram-lak", pad_factor=2, short_scan=False, iso=None, angular_weights=None,
                 filter_response=None, projection_weights=None, slice_weights=None, direct_filter=False):
        d, fr = make_desc(beam, vol_shape, voxel_spacing, det_shape, det_spacing, frames)
        o = FbpOpts()
        o.window = WINDOWS[window]
        o.pad_factor = int(pad_factor)
        o.short_scan = int(bool(short_scan))
        o.iso_given = 0 if iso is None else 1
        if iso is not None:
            for k in range(3):
                o.iso[k] = float(iso[k])
        o.reserved = 0
        n = fr.shape[0]
        dp = ctypes.POINTER(ctypes.c_double)
        self._angles = None if angles is None else np.ascontiguousarray(angles, dtype=np.float64)
        self._aw = None if angular_weights is None else np.ascontiguousarray(angular_weights, np.float64)
        for arr, name in ((self._angles, "angles"), (self._aw, "angular_weights")):
            if arr is not None and arr.shape != (n,):
                raise ValueError(f"{name} must have one value per view")
        U, V = int(det_shape[0]), int(det_shape[1])
        x = FbpExt()
        x.direct_filter = int(bool(direct_filter))
        self._ext = []
        if filter_response is not None:
            r = np.ascontiguousarray(filter_response, dtype=np.float64)
            if r.shape != (int(pad_factor) * U // 2 + 1,):
                raise ValueError("filter_response must have pad_factor * U // 2 + 1 values")
            x.filter_response = r.ctypes.data_as(dp)
            self._ext.append(r)
        if projection_weights is not None:
            pw = np.ascontiguousarray(projection_weights, dtype=np.float64)
            if pw.shape not in ((U, V), (n, U, V)):
                raise ValueError("projection_weights must have shape (U, V) or (views, U, V)")
            x.projection_weights = pw.ctypes.data_as(dp)
            x.projection_weights_per_view = 1 if pw.ndim == 3 else 0
            self._ext.append(pw)
        if slice_weights is not None:
            sw = np.ascontiguousarray(slice_weights, dtype=np.float64)
            if sw.shape != (int(vol_shape[0]), n):
                raise ValueError("slice_weights must have shape (D, views)")
            x.slice_weights = sw.ctypes.data_as(dp)
            self._ext.append(sw)
        h = ctypes.c_void_p()
        _check(lib().ct_fbp_create_ext(ctypes.byref(d),
                                       self._angles.ctypes.data_as(dp) if self._angles is not None else None,
                                       self._aw.ctypes.data_as(dp) if self._aw is not None else None,
                                       ctypes.byref(o), ctypes.byref(x), ctypes.byref(h)))
        self._ext = None
        self._h = h
        self.vol_shape = tuple(int(x) for x in vol_shape)
        self.sino_shape = (n, int(det_shape[0]), int(det_shape[1]))

    @classmethod
    def from_workload(cls, wl, angles=None, **kw) -> "FBP":
        return cls(wl.beam, wl.vol_shape, wl.voxel_spacing, wl.det_shape, wl.det_spacing, wl.frames,
                   angles, **kw)

    @classmethod
    def helical_from_workload(cls, wl, angles, **kw) -> "FBP":
        """Helical FDK plan: the slice weights of ct_helical_view_weights for
        these unwrapped angles (or kw["slice_weights"], the caller's own)."""
        if kw.get("slice_weights") is None:
            kw["slice_weights"] = ct_helical_view_weights(wl.beam, wl.vol_shape, wl.voxel_spacing, wl.det_shape,
                                                          wl.det_spacing, wl.frames, angles)
        return cls.from_workload(wl, None, **kw)

    @property
    def handle(self):
        return self._h

    def info(self):
        """(isocentre (3,), angular weights (n_views,)) as the plan holds them."""
        iso = np.zeros(3)
        aw = np.zeros(self.sino_shape[0])
        dp = ctypes.POINTER(ctypes.c_double)
        _check(lib().ct_fbp_info(self._h, iso.ctypes.data_as(dp), aw.ctypes.data_as(dp)))
        return iso, aw

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().ct_fbp_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):  # pragma: no cover - best effort
        try:
            self.close()
        except Exception:
            pass


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(int(stream.cuda_stream))


def _ptr(t, shape, name):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (cuda) tensor")
    if t.dtype != torch.float32:
        raise ValueError(f"{name} must be float32")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


def ct_project(g: Geometry, vol, sino, stream=None):
    """sino <- A vol (overwrites every ray)."""
    _check(lib().ct_project(g.handle, _ptr(vol, g.vol_shape, "vol"),
                            _ptr(sino, g.sino_shape, "sino"), _stream(stream)))
    return sino


def ct_forward_workspace_size(g: Geometry = None, desc_args=None) -> int:
    """Bytes of ct_project_ws workspace, from a handle or (desc_args: beam,
    vol_shape, voxel_spacing, det_shape, det_spacing, frames) on the host."""
    n = ctypes.c_size_t(0)
    if g is not None:
        _check(lib().ct_forward_workspace_size(g.handle, None, ctypes.byref(n)))
    else:
        d, fr = make_desc(*desc_args)
        _check(lib().ct_forward_workspace_size(None, ctypes.byref(d), ctypes.byref(n)))
    return int(n.value)


def ct_project_ws(g: Geometry, vol, sino, work, stream=None):
    """Forward projection with the volume copies in `work` (a device tensor of
    at least ct_forward_workspace_size(g) bytes, 256-byte aligned, or None when
    that size is 0); the handle is only read."""
    if work is None:
        ptr, nb = None, 0
    else:
        import torch
        if not isinstance(work, torch.Tensor) or not work.is_cuda or not work.is_contiguous():
            raise ValueError("work must be a contiguous device tensor")
        ptr, nb = ctypes.c_void_p(work.data_ptr()), work.numel() * work.element_size()
    _check(lib().ct_project_ws(g.handle, _ptr(vol, g.vol_shape, "vol"), _ptr(sino, g.sino_shape, "sino"), ptr,
                               nb, _stream(stream)))


def ct_backproject(g: Geometry, sino, vol, stream=None):
    """vol <- A^T sino (brick-binned, overwrites every voxel)."""
    _check(lib().ct_backproject(g.handle, _ptr(sino, g.sino_shape, "sino"),
                                _ptr(vol, g.vol_shape, "vol"), _stream(stream)))
    return vol


def ct_project_region(g: Geometry, vol_region, region, view_begin, view_end, sino_batch,
                      accumulate=False, stream=None):
    """sino_batch (+)= A of the region's voxels for views [view_begin, view_end).
    region = (z0, y0, x0, nz, ny, nx)."""
    z0, y0, x0, nz, ny, nx = (int(v) for v in region)
    r = Region(z0, y0, x0, nz, ny, nx)
    _check(lib().ct_project_region(g.handle, _ptr(vol_region, (nz, ny, nx), "vol_region"), r,
                                   int(view_begin), int(view_end),
                                   _ptr(sino_batch, (int(view_end) - int(view_begin),) + g.sino_shape[1:],
                                        "sino_batch"), int(bool(accumulate)), _stream(stream)))
    return sino_batch


def ct_backproject_region(g: Geometry, sino_batch, view_begin, view_end, region, vol_region,
                          accumulate=False, stream=None):
    """vol_region (+)= A^T of the batch's rays restricted to the region."""
    z0, y0, x0, nz, ny, nx = (int(v) for v in region)
    r = Region(z0, y0, x0, nz, ny, nx)
    _check(lib().ct_backproject_region(g.handle,
                                       _ptr(sino_batch, (int(view_end) - int(view_begin),) + g.sino_shape[1:],
                                            "sino_batch"), int(view_begin), int(view_end), r,
                                       _ptr(vol_region, (nz, ny, nx), "vol_region"),
                                       int(bool(accumulate)), _stream(stream)))
    return vol_region


def _host_ptr(t, shape, name, writable):
    """Host buffer (a CPU torch tensor, pinned or not, or a numpy array)."""
    import torch
    if isinstance(t, np.ndarray):
        if t.dtype != np.float32 or not t.flags.c_contiguous or (writable and not t.flags.writeable):
            raise ValueError(f"{name} must be a writable C-contiguous float32 array" if writable
                             else f"{name} must be a C-contiguous float32 array")
        p = t.ctypes.data
    elif isinstance(t, torch.Tensor):
        if t.is_cuda:
            raise ValueError(f"{name} must be a host (cpu) tensor")
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 tensor")
        p = t.data_ptr()
    else:
        raise TypeError(f"{name} must be a torch tensor or a numpy array")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(p)


def ct_backproject_host(g: Geometry, sino, vol, slab, batch_views, axis="auto", stream=None):
    """vol = A^T sino with both in host memory, streamed through the device in
    slabs of `slab` planes along `axis` ("z", "y", "x" or "auto") and batches
    of batch_views views."""
    plan = StreamPlan(int(slab), int(batch_views), AXES[axis] if isinstance(axis, str) else int(axis), 0)
    _check(lib().ct_backproject_host(g.handle, _host_ptr(sino, g.sino_shape, "sino", False),
                                     _host_ptr(vol, g.vol_shape, "vol", True), plan, _stream(stream)))
    return vol


def ct_project_host(g: Geometry, vol, sino, slab, batch_views, axis="auto", stream=None):
    """sino = A vol with both in host memory (slabs and view batches)."""
    plan = StreamPlan(int(slab), int(batch_views), AXES[axis] if isinstance(axis, str) else int(axis), 0)
    _check(lib().ct_project_host(g.handle, _host_ptr(vol, g.vol_shape, "vol", False),
                                 _host_ptr(sino, g.sino_shape, "sino", True), plan, _stream(stream)))
    return sino


def ct_fbp_filter(f: FBP, sino, filtered, stream=None):
    """filtered = angular weight x ramp filter of the pre-weighted sinogram."""
    _check(lib().ct_fbp_filter(f.handle, _ptr(sino, f.sino_shape, "sino"),
                               _ptr(filtered, f.sino_shape, "filtered"), _stream(stream)))
    return filtered


def ct_fbp_backproject(f: FBP, filtered, vol, stream=None):
    """vol = voxel-driven interpolating weighted backprojection of filtered."""
    _check(lib().ct_fbp_backproject(f.handle, _ptr(filtered, f.sino_shape, "filtered"),
                                    _ptr(vol, f.vol_shape, "vol"), _stream(stream)))
    return vol


def ct_fbp_backproject_transpose(f: FBP, vol, sino, stream=None):
    """sino = transpose of the weighted backprojection applied to vol."""
    _check(lib().ct_fbp_backproject_transpose(f.handle, _ptr(vol, f.vol_shape, "vol"),
                                              _ptr(sino, f.sino_shape, "sino"), _stream(stream)))
    return sino


def ct_fbp_run(f: FBP, sino, work, vol, stream=None):
    """vol = FBP / FDK of sino (work holds the filtered sinogram)."""
    _check(lib().ct_fbp_run(f.handle, _ptr(sino, f.sino_shape, "sino"), _ptr(work, f.sino_shape, "work"),
                            _ptr(vol, f.vol_shape, "vol"), _stream(stream)))
    return vol


def ct_backproject_atomic(g: Geometry, sino, vol, stream=None):
    """vol <- A^T sino (one lane per ray, global float atomics)."""
    _check(lib().ct_backproject_atomic(g.handle, _ptr(sino, g.sino_shape, "sino"),
                                       _ptr(vol, g.vol_shape, "vol"), _stream(stream)))
    return vol


def ct_sirt_weights(g: Geometry, row_inv, col_inv, stream=None):
    _check(lib().ct_sirt_weights(g.handle, _ptr(row_inv, g.sino_shape, "row_inv"),
                                 _ptr(col_inv, g.vol_shape, "col_inv"), _stream(stream)))
    return row_inv, col_inv


def ct_sirt_residual(g: Geometry, x, y, row_inv, work_sino, stream=None):
    _check(lib().ct_sirt_residual(g.handle, _ptr(x, g.vol_shape, "x"), _ptr(y, g.sino_shape, "y"),
                                  _ptr(row_inv, g.sino_shape, "row_inv"),
                                  _ptr(work_sino, g.sino_shape, "work_sino"), _stream(stream)))
    return work_sino


def ct_sirt_update(g: Geometry, work_sino, col_inv, relax, x, stream=None):
    _check(lib().ct_sirt_update(g.handle, _ptr(work_sino, g.sino_shape, "work_sino"),
                                _ptr(col_inv, g.vol_shape, "col_inv"), float(relax),
                                _ptr(x, g.vol_shape, "x"), _stream(stream)))
    return x


def ct_sirt_step(g: Geometry, x, y, row_inv, col_inv, relax, work_sino, stream=None):
    _check(lib().ct_sirt_step(g.handle, _ptr(x, g.vol_shape, "x"), _ptr(y, g.sino_shape, "y"),
                              _ptr(row_inv, g.sino_shape, "row_inv"),
                              _ptr(col_inv, g.vol_shape, "col_inv"), float(relax),
                              _ptr(work_sino, g.sino_shape, "work_sino"), _stream(stream)))
    return x


def _mask_ptr(g: Geometry, mask):
    import torch
    if mask is None:
        return ctypes.c_void_p(0)
    if not isinstance(mask, torch.Tensor) or not mask.is_cuda or mask.dtype != torch.uint8 \
            or not mask.is_contiguous() or tuple(mask.shape) != tuple(g.vol_shape):
        raise ValueError("mask must be a contiguous uint8 device tensor of volume shape")
    return ctypes.c_void_p(mask.data_ptr())


def ct_sirt_update_bounded(g: Geometry, work_sino, col_inv, relax, lo, hi, mask, x, stream=None):
    """x <- clamp(x + relax * col_inv * A^T work_sino, lo, hi) where mask != 0."""
    _check(lib().ct_sirt_update_bounded(g.handle, _ptr(work_sino, g.sino_shape, "work_sino"),
                                        _ptr(col_inv, g.vol_shape, "col_inv"), float(relax),
                                        float(lo), float(hi), _mask_ptr(g, mask),
                                        _ptr(x, g.vol_shape, "x"), _stream(stream)))
    return x


def ct_sirt_step_bounded(g: Geometry, x, y, row_inv, col_inv, relax, lo, hi, mask, work_sino,
                         stream=None):
    _check(lib().ct_sirt_step_bounded(g.handle, _ptr(x, g.vol_shape, "x"), _ptr(y, g.sino_shape, "y"),
                                      _ptr(row_inv, g.sino_shape, "row_inv"),
                                      _ptr(col_inv, g.vol_shape, "col_inv"), float(relax), float(lo),
                                      float(hi), _mask_ptr(g, mask),
                                      _ptr(work_sino, g.sino_shape, "work_sino"), _stream(stream)))
    return x


def ct_sirt_weights_views(g: Geometry, view_begin, view_end, row_inv_batch, col_inv, stream=None):
    """R and C of the views [view_begin, view_end) (one ordered subset)."""
    vb, ve = int(view_begin), int(view_end)
    bshape = (ve - vb,) + g.sino_shape[1:]
    _check(lib().ct_sirt_weights_views(g.handle, vb, ve, _ptr(row_inv_batch, bshape, "row_inv_batch"),
                                       _ptr(col_inv, g.vol_shape, "col_inv"), _stream(stream)))
    return row_inv_batch, col_inv


def ct_sirt_step_views(g: Geometry, view_begin, view_end, x, y_batch, row_inv_batch, col_inv, relax=1.0,
                       lo=-float("inf"), hi=float("inf"), mask=None, work_batch=None, stream=None):
    """One ordered-subset (SART) step on the views [view_begin, view_end)."""
    vb, ve = int(view_begin), int(view_end)
    bshape = (ve - vb,) + g.sino_shape[1:]
    _check(lib().ct_sirt_step_views(g.handle, vb, ve, _ptr(x, g.vol_shape, "x"),
                                    _ptr(y_batch, bshape, "y_batch"),
                                    _ptr(row_inv_batch, bshape, "row_inv_batch"),
                                    _ptr(col_inv, g.vol_shape, "col_inv"), float(relax), float(lo),
                                    float(hi), _mask_ptr(g, mask), _ptr(work_batch, bshape, "work_batch"),
                                    _stream(stream)))
    return x


def ct_cgls_workspace_size(g: Geometry) -> int:
    """Bytes of device workspace the CGLS calls need for this geometry."""
    n = ctypes.c_size_t(0)
    _check(lib().ct_cgls_workspace_size(g.handle, ctypes.byref(n)))
    return int(n.value)


def _work_ptr(g: Geometry, work):
    import torch
    if not isinstance(work, torch.Tensor) or not work.is_cuda or not work.is_contiguous():
        raise ValueError("work must be a contiguous device tensor")
    if work.numel() * work.element_size() < ct_cgls_workspace_size(g):
        raise ValueError("work is smaller than ct_cgls_workspace_size(g)")
    return ctypes.c_void_p(work.data_ptr())


def ct_cgls_init(g: Geometry, y, x, r, s, p, work, stream=None):
    """CGLS start: r = y - A x, s = A^T r, p = s, scalars into work."""
    _check(lib().ct_cgls_init(g.handle, _ptr(y, g.sino_shape, "y"), _ptr(x, g.vol_shape, "x"),
                              _ptr(r, g.sino_shape, "r"), _ptr(s, g.vol_shape, "s"),
                              _ptr(p, g.vol_shape, "p"), _work_ptr(g, work), _stream(stream)))


def ct_cgls_step(g: Geometry, x, r, s, p, q, work, stream=None):
    """One CGLS iteration on (x, r, s, p, q, work), in place."""
    _check(lib().ct_cgls_step(g.handle, _ptr(x, g.vol_shape, "x"), _ptr(r, g.sino_shape, "r"),
                              _ptr(s, g.vol_shape, "s"), _ptr(p, g.vol_shape, "p"),
                              _ptr(q, g.sino_shape, "q"), _work_ptr(g, work), _stream(stream)))


def ct_cgls_step_noalloc(g: Geometry, x, r, s, p, q, state, stream=None):
    """One CGLS iteration with the partial sums in the library's static device
    scratch; state: a device tensor whose first 256 bytes hold the scalars
    (e.g. the workspace ct_cgls_init filled)."""
    import torch
    if not isinstance(state, torch.Tensor) or not state.is_cuda or not state.is_contiguous():
        raise ValueError("state must be a contiguous device tensor")
    if state.numel() * state.element_size() < 256:
        raise ValueError("state must hold at least 256 bytes")
    _check(lib().ct_cgls_step_noalloc(g.handle, _ptr(x, g.vol_shape, "x"), _ptr(r, g.sino_shape, "r"),
                                      _ptr(s, g.vol_shape, "s"), _ptr(p, g.vol_shape, "p"),
                                      _ptr(q, g.sino_shape, "q"), ctypes.c_void_p(state.data_ptr()),
                                      _stream(stream)))


def ct_cgls_scalars(g: Geometry, work, stream=None) -> dict:
    """gamma = ||A^T r||^2, alpha, beta, qq = ||q||^2 and rr = ||r||^2 (syncs the stream)."""
    out = (ctypes.c_double * 5)()
    _check(lib().ct_cgls_scalars(g.handle, _work_ptr(g, work), out, _stream(stream)))
    return dict(zip(("gamma", "alpha", "beta", "qq", "rr"), list(out)))


def ct_count_intersections(g: Geometry, per_ray=None, stream=None) -> int:
    """Number of (ray, voxel) pairs the traversal visits: per ray the lattice-plane
    crossings inside the volume plus one, from float64 entry and exit cells
    (equal to the pairs of positive length except where a ray crosses two planes
    at exactly the same point).  Syncs the stream."""
    import torch
    total = ctypes.c_uint64(0)
    p = ctypes.c_void_p(0)
    if per_ray is not None:
        if per_ray.dtype not in (torch.int32, torch.uint32) or not per_ray.is_cuda \
                or not per_ray.is_contiguous() or tuple(per_ray.shape) != tuple(g.sino_shape):
            raise ValueError("per_ray must be a contiguous int32 device tensor of sinogram shape")
        p = ctypes.c_void_p(per_ray.data_ptr())
    _check(lib().ct_count_intersections(g.handle, p, ctypes.byref(total), _stream(stream)))
    return int(total.value)


def version() -> str:
    return lib().ct_version().decode()
