"""Float64 CPU oracle of the ray-driven projector pair (test infrastructure).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark may use this package; the product path never does.  It shares
no code with the HIP library.  The arithmetic lives in ``ct_oracle.c`` (plain
C, float64); this module only marshals numpy arrays and composes the SIRT
iteration from the oracle's A and A^T.

Sources (diffct documentation):
  - "Trajectories and Geometry" > "Trajectory format": frames, axes, pixel
    centres, volume and sinogram layouts.
  - "Differentiable analytical reconstruction": cell-constant Siddon forward
    operator with the matched adjoint.
  - "API Reference" > "Numerical Solvers": a SIRT solver built on A and A^T
    (no formula on the page; the standard SIRT update is used, see ``sirt``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ct_oracle.c")
_LIB = os.path.join(_HERE, "libctoracle.so")


# plain gcc, IEEE float64: no contraction into fused multiply-adds, no fast math
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread"]


def compile_library(src: str, out: str, extra=()) -> str:
    """Compile one oracle C source into a shared library at `out`."""
    cmd = ["gcc", *CFLAGS, *extra, "-I", _HERE, "-o", out + ".tmp", src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build(force: bool = True) -> str:
    """Compile ct_oracle.c into libctoracle.so."""
    if force or not os.path.exists(_LIB):
        compile_library(_SRC, _LIB)
    return _LIB


class _Geom(ctypes.Structure):
    _fields_ = [("beam", ctypes.c_int), ("n_views", ctypes.c_int64),
                ("nz", ctypes.c_int64), ("ny", ctypes.c_int64), ("nx", ctypes.c_int64),
                ("sz", ctypes.c_double), ("sy", ctypes.c_double), ("sx", ctypes.c_double),
                ("nu", ctypes.c_int64), ("nv", ctypes.c_int64),
                ("su", ctypes.c_double), ("sv", ctypes.c_double),
                ("frames", ctypes.POINTER(ctypes.c_double)),
                ("offsets", ctypes.POINTER(ctypes.c_double)), ("offsets_per_view", ctypes.c_int)]


class _Ray(ctypes.Structure):
    _fields_ = [("o", ctypes.c_double * 3), ("d", ctypes.c_double * 3),
                ("tmin", ctypes.c_double), ("tmax", ctypes.c_double)]


_lib = None


def bind(L):
    """Declare the C signatures on a loaded copy of the oracle library."""
    P = ctypes.POINTER
    dp = P(ctypes.c_double)
    ip = P(ctypes.c_int64)
    L.ora_ray_of.argtypes = [P(_Geom), ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, P(_Ray)]
    L.ora_box_chord.argtypes = [P(_Ray), dp, dp]
    L.ora_box_chord.restype = ctypes.c_double
    L.ora_trace.argtypes = [P(_Geom), P(_Ray), dp, ip, ip]
    L.ora_trace.restype = ctypes.c_double
    L.ora_project.argtypes = [P(_Geom), dp, dp, ctypes.c_int, ip, ip]
    L.ora_project_rays.argtypes = [P(_Geom), dp, ip, ctypes.c_int64, dp, ip, ctypes.c_int]
    L.ora_backproject.argtypes = [P(_Geom), dp, dp, ctypes.c_int]
    L.ora_brute_matrix.argtypes = [P(_Geom), dp]
    L.ora_column_dot.argtypes = [P(_Geom), ctypes.c_int64, dp, ctypes.c_int]
    L.ora_column_dot.restype = ctypes.c_double
    L.ora_row_chords.argtypes = [P(_Geom), dp, ctypes.c_int]
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = bind(ctypes.CDLL(_LIB))
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _dptr(a: np.ndarray):
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _iptr(a: np.ndarray):
    assert a.dtype == np.int64 and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


class Geometry:
    """Oracle geometry: shapes + frames (n_views x 12 float64), and optionally a
    detector surface: per-pixel offsets (o_u, o_v, o_n) of shape (U, V, 3), or
    (views, U, V, 3) per view (2D: V = 1)."""

    def __init__(self, beam, vol_shape, voxel_spacing, det_shape, det_spacing, frames,
                 offsets=None):
        self.frames = np.ascontiguousarray(frames, dtype=np.float64)
        d, h, w = (int(x) for x in vol_shape)
        dz, dy, dx = (float(x) for x in voxel_spacing)
        nu, nv = (int(x) for x in det_shape)
        du, dv = (float(x) for x in det_spacing)
        self.vol_shape = (d, h, w)
        self.sino_shape = (self.frames.shape[0], nu, nv)
        per_view = 0
        self.offsets = None
        optr = ctypes.POINTER(ctypes.c_double)()
        if offsets is not None:
            self.offsets = np.ascontiguousarray(offsets, dtype=np.float64)
            if self.offsets.shape == (nu, nv, 3):
                per_view = 0
            elif self.offsets.shape == (self.frames.shape[0], nu, nv, 3):
                per_view = 1
            else:
                raise ValueError("offsets must be (U, V, 3) or (views, U, V, 3)")
            optr = _dptr(self.offsets)
        self._g = _Geom(int(beam), self.frames.shape[0], d, h, w, dz, dy, dx, nu, nv, du, dv,
                        _dptr(self.frames), optr, per_view)

    @classmethod
    def from_workload(cls, wl) -> "Geometry":
        return cls(wl.beam, wl.vol_shape, wl.voxel_spacing, wl.det_shape, wl.det_spacing, wl.frames,
                   getattr(wl, "offsets", None))

    @property
    def n_rays(self) -> int:
        return int(np.prod(self.sino_shape))

    @property
    def n_voxels(self) -> int:
        return int(np.prod(self.vol_shape))

    def ray(self, view: int, u: int, v: int):
        r = _Ray()
        lib().ora_ray_of(ctypes.byref(self._g), view, u, v, ctypes.byref(r))
        return np.array(r.o[:]), np.array(r.d[:]), r.tmin, r.tmax


def _as64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def project(g: Geometry, vol, nthreads: int | None = None, with_counts: bool = False):
    """Forward projection A x (float64); optionally returns (sino, nnz, ties)."""
    x = _as64(vol).reshape(g.vol_shape)
    out = np.zeros(g.sino_shape, dtype=np.float64)
    nnz = ctypes.c_int64(0)
    ties = ctypes.c_int64(0)
    lib().ora_project(ctypes.byref(g._g), _dptr(x), _dptr(out), nthreads or default_threads(),
                      ctypes.byref(nnz), ctypes.byref(ties))
    if with_counts:
        return out, int(nnz.value), int(ties.value)
    return out


def project_rays(g: Geometry, vol, ray_ids, nthreads: int | None = None, with_counts=False):
    """Forward values of selected rays (flat ids into the sinogram)."""
    x = _as64(vol).reshape(g.vol_shape)
    ids = np.ascontiguousarray(ray_ids, dtype=np.int64)
    out = np.zeros(ids.shape[0], dtype=np.float64)
    cnt = np.zeros(ids.shape[0], dtype=np.int64)
    lib().ora_project_rays(ctypes.byref(g._g), _dptr(x), _iptr(ids), ids.shape[0], _dptr(out),
                           _iptr(cnt), nthreads or default_threads())
    return (out, cnt) if with_counts else out


def backproject(g: Geometry, sino, nthreads: int | None = None) -> np.ndarray:
    """Adjoint A^T y (float64), by the separately coded merged-list method."""
    y = _as64(sino).reshape(g.sino_shape)
    out = np.zeros(g.vol_shape, dtype=np.float64)
    lib().ora_backproject(ctypes.byref(g._g), _dptr(y), _dptr(out), nthreads or default_threads())
    return out


def row_chords(g: Geometry, nthreads: int | None = None) -> np.ndarray:
    """Per ray, the chord of the whole volume box: the row sums A 1 in closed form."""
    out = np.zeros(g.sino_shape, dtype=np.float64)
    lib().ora_row_chords(ctypes.byref(g._g), _dptr(out), nthreads or default_threads())
    return out


def brute_matrix(g: Geometry) -> np.ndarray:
    """Dense A (n_rays x n_voxels) from per-cell chords (tiny grids only)."""
    if g.n_rays * g.n_voxels > 5e7:
        raise ValueError("brute-force matrix too large")
    A = np.zeros((g.n_rays, g.n_voxels), dtype=np.float64)
    lib().ora_brute_matrix(ctypes.byref(g._g), _dptr(A))
    return A


def column_dot(g: Geometry, j: int, sino, nthreads: int | None = None) -> float:
    """(A^T y)_j by per-cell chords of voxel j over every ray."""
    y = _as64(sino).reshape(g.sino_shape)
    return float(lib().ora_column_dot(ctypes.byref(g._g), int(j), _dptr(y),
                                      nthreads or default_threads()))


def box_chord(o, d, tmin, tmax, lo, hi) -> float:
    r = _Ray((ctypes.c_double * 3)(*o), (ctypes.c_double * 3)(*d), tmin, tmax)
    lo = np.ascontiguousarray(lo, dtype=np.float64)
    hi = np.ascontiguousarray(hi, dtype=np.float64)
    return float(lib().ora_box_chord(ctypes.byref(r), _dptr(lo), _dptr(hi)))


# ----------------------------------------------------------------------------
# SIRT.  The pages name a SIRT solver built on A and A^T but print no formula;
# this is the standard simultaneous iterative reconstruction update
#     x <- x + relax * C A^T R (y - A x),
# R = 1 / (A 1) per ray, C = 1 / (A^T 1) per voxel, each 0 where the sum is 0.
# ----------------------------------------------------------------------------

def sirt_weights(g: Geometry, nthreads: int | None = None):
    rs = project(g, np.ones(g.vol_shape), nthreads)
    cs = backproject(g, np.ones(g.sino_shape), nthreads)
    R = np.zeros_like(rs)
    C = np.zeros_like(cs)
    R[rs > 0] = 1.0 / rs[rs > 0]
    C[cs > 0] = 1.0 / cs[cs > 0]
    return R, C


def sirt(g: Geometry, y, x0=None, n_iter: int = 1, relax: float = 1.0,
         weights=None, nthreads: int | None = None, lo: float = -np.inf, hi: float = np.inf,
         mask=None) -> np.ndarray:
    """SIRT; with lo/hi/mask the bounded, masked variant of the ASTRA options
    printed in the ASTRA guide (MinConstraint, MaxConstraint, ReconstructionMask):
    after each update x is clipped to [lo, hi], and voxels where mask == 0 keep
    their previous value."""
    y = _as64(y).reshape(g.sino_shape)
    x = np.zeros(g.vol_shape) if x0 is None else _as64(x0).reshape(g.vol_shape).copy()
    R, C = weights if weights is not None else sirt_weights(g, nthreads)
    for _ in range(n_iter):
        e = R * (y - project(g, x, nthreads))
        xn = x + relax * C * backproject(g, e, nthreads)
        xn = np.clip(xn, lo, hi)
        if mask is not None:
            xn = np.where(np.asarray(mask).reshape(g.vol_shape) != 0, xn, x)
        x = xn
    return x


# ----------------------------------------------------------------------------
# CGLS.  The pages ship a CGLS solver and time it per iteration ("Performance";
# "API Reference" > "Numerical Solvers"), keeping x, s, p and r, q with float64
# norms ("Large Volumes and Chunked Execution" > "Runnable iterative
# reconstruction"), but print no formula.  This is the standard conjugate
# gradient method on the normal equations A^T A x = A^T y in its least-squares
# form (Hestenes-Stiefel / Bjorck):
#     r = y - A x,  s = A^T r,  p = s,  gamma = ||s||^2
#     repeat:  q = A p;  alpha = gamma / ||q||^2;  x += alpha p;  r -= alpha q;
#              s = A^T r;  gamma' = ||s||^2;  beta = gamma' / gamma;
#              p = s + beta p;  gamma = gamma'
# with alpha = 0 when q = 0 and beta = 0 when gamma = 0.
# ----------------------------------------------------------------------------

def cgls_step(g: Geometry, x, r, s, p, gamma: float, nthreads: int | None = None) -> dict:
    """One CGLS iteration from the state (x, r, s, p, gamma): returns the new
    x, r, s, p, the q = A p it used, and alpha, beta, gamma, qq = ||q||^2,
    rr = ||r||^2 (after the step)."""
    x = _as64(x).reshape(g.vol_shape)
    r = _as64(r).reshape(g.sino_shape)
    p = _as64(p).reshape(g.vol_shape)
    q = project(g, p, nthreads)
    qq = float(np.sum(q * q))
    alpha = gamma / qq if qq > 0 else 0.0
    x = x + alpha * p
    r = r - alpha * q
    s = backproject(g, r, nthreads)
    gnew = float(np.sum(s * s))
    beta = gnew / gamma if gamma > 0 else 0.0
    p = s + beta * p
    return {"x": x, "r": r, "s": s, "p": p, "q": q, "alpha": alpha, "beta": beta, "gamma": gnew,
            "qq": qq, "rr": float(np.sum(r * r))}


def cgls(g: Geometry, y, x0=None, n_iter: int = 1, nthreads: int | None = None):
    """Returns (x, hist): hist holds per iteration alpha, beta, gamma (after the
    step), qq = ||q||^2 and rr = ||r||^2 (after the step), plus the start's
    gamma0 and rr0."""
    y = _as64(y).reshape(g.sino_shape)
    x = np.zeros(g.vol_shape) if x0 is None else _as64(x0).reshape(g.vol_shape).copy()
    r = y - project(g, x, nthreads)
    s = backproject(g, r, nthreads)
    p = s.copy()
    gamma = float(np.sum(s * s))
    hist = {"gamma0": gamma, "rr0": float(np.sum(r * r)),
            "alpha": [], "beta": [], "gamma": [], "qq": [], "rr": []}
    for _ in range(n_iter):
        st = cgls_step(g, x, r, s, p, gamma, nthreads)
        x, r, s, p, gamma = st["x"], st["r"], st["s"], st["p"], st["gamma"]
        for k in ("alpha", "beta", "gamma", "qq", "rr"):
            hist[k].append(st[k])
    return x, hist
