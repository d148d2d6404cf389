"""Seeded synthetic inputs: acquisition frames and voxel phantoms.

This module is the only code that both the CPU oracle side and the HIP side
consume.  It holds no projection arithmetic: it draws random numbers, builds
per-view frames (source or ray direction, detector centre, detector axes) and
rasterises ellipse/ellipsoid phantoms.  Every array it returns is plain numpy.

Frame convention (diffct documentation, "Trajectories and Geometry" >
"Trajectory format"): Cartesian (x, y, z) coordinates with the origin at the
volume centre; one row per view.  The rows handed to the library are
``n_views x 12`` float64: ``[a(3), c(3), e_u(3), e_v(3)]`` where ``a`` is the
source position (fan, cone) or the unit ray direction (parallel, parallel3d),
``c`` the detector centre, ``e_u``/``e_v`` unit detector axes.  2D beams keep
all z components at 0 and ``e_v`` = 0.

Random numbers: a counter-based splitmix64 stream (Steele, Lea and Flood,
"Fast splittable pseudorandom number generators", OOPSLA 2014): the k-th draw
of stream ``s`` is ``mix(seed_s + (k + 1) * 0x9E3779B97F4A7C15)``, turned into a
double in [0, 1) from its top 53 bits.  Seeds are ``1000 * config + stream``
with stream 1 = phantom shapes, 2 = per-view jitter, 3 and 4 = adjoint-test
vectors, 5 = phantom background noise.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BEAM_PARALLEL2D = 0
BEAM_FAN2D = 1
BEAM_CONE = 2
BEAM_PARALLEL3D = 3
BEAM_NAMES = {BEAM_PARALLEL2D: "parallel2d", BEAM_FAN2D: "fan2d",
              BEAM_CONE: "cone", BEAM_PARALLEL3D: "parallel3d"}

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def _mix64(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


class Stream:
    """Counter-based splitmix64 stream of doubles in [0, 1)."""

    def __init__(self, seed: int):
        self.seed = np.uint64(seed & 0xFFFFFFFFFFFFFFFF)
        self.pos = 0

    def raw(self, n: int) -> np.ndarray:
        k = np.arange(self.pos + 1, self.pos + 1 + n, dtype=np.uint64)
        self.pos += n
        with np.errstate(over="ignore"):
            return _mix64(self.seed + k * _GOLDEN)

    def uniform(self, n: int, lo: float = 0.0, hi: float = 1.0) -> np.ndarray:
        u = (self.raw(n) >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)
        return lo + (hi - lo) * u


def seed_of(config: int, stream: int) -> int:
    return 1000 * config + stream


# --------------------------------------------------------------------------
# Geometry description shared by both sides (shapes + frames only)
# --------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    beam: int
    vol_shape: tuple            # (D, H, W); 2D: D = 1
    voxel_spacing: tuple        # (dz, dy, dx); 2D: dz = 1
    det_shape: tuple            # (U, V); 2D: V = 1
    det_spacing: tuple          # (du, dv)
    frames: np.ndarray          # (n_views, 12) float64
    config: int = 0
    meta: dict = field(default_factory=dict)
    offsets: np.ndarray | None = None   # detector surface: (U, V, 3) or (views, U, V, 3)

    @property
    def n_views(self) -> int:
        return int(self.frames.shape[0])

    @property
    def sino_shape(self) -> tuple:
        return (self.n_views, int(self.det_shape[0]), int(self.det_shape[1]))

    @property
    def n_rays(self) -> int:
        return self.n_views * int(self.det_shape[0]) * int(self.det_shape[1])

    @property
    def n_voxels(self) -> int:
        d, h, w = self.vol_shape
        return int(d) * int(h) * int(w)

    def subset_views(self, views) -> "Workload":
        views = np.asarray(views, dtype=np.int64)
        off = self.offsets
        if off is not None and off.ndim == 4:
            off = np.ascontiguousarray(off[views])
        return Workload(self.name + f"[{len(views)} views]", self.beam, self.vol_shape,
                        self.voxel_spacing, self.det_shape, self.det_spacing,
                        np.ascontiguousarray(self.frames[views]), self.config, dict(self.meta), off)


def cylinder_offsets(det_shape, det_spacing, radius: float, two_d: bool = False) -> np.ndarray:
    """Per-pixel local offsets (o_u, o_v, o_n) of a cylindrical detector: the
    pixel at physical detector coordinates (u, v) sits at angle u / radius on a
    cylinder of that radius whose axis is e_v, bending towards the source
    (negative normal offsets), after the diffct documentation's example
    ("Trajectories and Geometry" > "Parameterized detector surfaces").  A radius
    equal to the source-detector distance centres the cylinder on the source.
    Shape (U, V, 3); 2D: V = 1 and o_v = 0."""
    nu, nv = int(det_shape[0]), int(det_shape[1])
    du, dv = float(det_spacing[0]), float(det_spacing[1])
    u = (np.arange(nu) - 0.5 * (nu - 1)) * du
    v = np.zeros(1) if two_d else (np.arange(nv) - 0.5 * (nv - 1)) * dv
    uu, vv = np.meshgrid(u, v, indexing="ij")
    ang = uu / radius
    return np.ascontiguousarray(np.stack((radius * np.sin(ang), vv, radius * (np.cos(ang) - 1.0)),
                                         axis=-1), dtype=np.float64)


def with_surface(wl: "Workload", offsets: np.ndarray, label: str) -> "Workload":
    """The same acquisition with a parameterized detector surface."""
    return Workload(wl.name + f", {label} detector", wl.beam, wl.vol_shape, wl.voxel_spacing,
                    wl.det_shape, wl.det_spacing, wl.frames, wl.config, dict(wl.meta),
                    np.ascontiguousarray(offsets, dtype=np.float64))


def _frames(a, c, eu, ev) -> np.ndarray:
    n = a.shape[0]
    f = np.zeros((n, 12), dtype=np.float64)
    f[:, 0:3] = a
    f[:, 3:6] = c
    f[:, 6:9] = eu
    f[:, 9:12] = ev
    return f


def _pad3(v2: np.ndarray) -> np.ndarray:
    out = np.zeros((v2.shape[0], 3))
    out[:, :2] = v2
    return out


# Angles: theta_k = theta0 + k * range / n (endpoint excluded), radians.
def angles(n_views: int, angular_range: float, start: float = 0.0) -> np.ndarray:
    return start + angular_range * np.arange(n_views, dtype=np.float64) / n_views


def circular_parallel2d(n_views: int, angular_range: float = math.pi) -> np.ndarray:
    th = angles(n_views, angular_range)
    ray = _pad3(np.stack([np.cos(th), np.sin(th)], 1))
    eu = _pad3(np.stack([np.sin(th), -np.cos(th)], 1))
    return _frames(ray, np.zeros_like(ray), eu, np.zeros_like(ray))


def circular_fan2d(n_views: int, sid: float, sdd: float,
                   angular_range: float = 2 * math.pi) -> np.ndarray:
    th = angles(n_views, angular_range)
    r = np.stack([np.cos(th), np.sin(th)], 1)
    src = _pad3(sid * r)
    det = _pad3(-(sdd - sid) * r)
    eu = _pad3(np.stack([np.sin(th), -np.cos(th)], 1))
    return _frames(src, det, eu, np.zeros_like(src))


def helix_cone(n_views: int, sid: float, sdd: float, z_range: float = 0.0,
               n_turns: float = 1.0) -> np.ndarray:
    th = angles(n_views, 2 * math.pi * n_turns)
    z = -z_range / 2 + z_range * np.arange(n_views, dtype=np.float64) / n_views
    c, s = np.cos(th), np.sin(th)
    src = np.stack([sid * c, sid * s, z], 1)
    det = np.stack([-(sdd - sid) * c, -(sdd - sid) * s, z], 1)
    eu = np.stack([s, -c, np.zeros_like(c)], 1)
    ev = np.tile(np.array([0.0, 0.0, 1.0]), (n_views, 1))
    return _frames(src, det, eu, ev)


def dual_axis_parallel3d(n_per_series: int = 140, first_deg: float = -70.0,
                         step_deg: float = 1.0) -> np.ndarray:
    """Two tilt series of parallel rays around the z (beam) axis.

    Series X tilts the ray about the x axis, series Y about the y axis; at zero
    tilt both look straight along z.  Tilts are first_deg + k * step_deg.
    """
    tau = np.radians(first_deg + step_deg * np.arange(n_per_series, dtype=np.float64))
    s, c = np.sin(tau), np.cos(tau)
    z0 = np.zeros_like(s)
    o = np.ones_like(s)
    ray_x = np.stack([z0, -s, c], 1)
    eu_x = np.stack([o, z0, z0], 1)
    ev_x = np.stack([z0, c, s], 1)
    ray_y = np.stack([s, z0, c], 1)
    eu_y = np.stack([c, z0, -s], 1)
    ev_y = np.stack([z0, o, z0], 1)
    ray = np.concatenate([ray_x, ray_y])
    return _frames(ray, np.zeros_like(ray), np.concatenate([eu_x, eu_y]),
                   np.concatenate([ev_x, ev_y]))


def _rodrigues(axis: np.ndarray, ang: np.ndarray) -> np.ndarray:
    """Rotation matrices (n, 3, 3) about unit axes by angles (radians)."""
    k = axis
    kx, ky, kz = k[:, 0], k[:, 1], k[:, 2]
    K = np.zeros((k.shape[0], 3, 3))
    K[:, 0, 1], K[:, 0, 2] = -kz, ky
    K[:, 1, 0], K[:, 1, 2] = kz, -kx
    K[:, 2, 0], K[:, 2, 1] = -ky, kx
    s = np.sin(ang)[:, None, None]
    c = np.cos(ang)[:, None, None]
    eye = np.eye(3)[None]
    return eye + s * K + (1 - c) * (K @ K)


def jitter_frames(frames: np.ndarray, stream: Stream, shift: float,
                  angle_deg: float) -> np.ndarray:
    """Per-view jitter: source and detector centre move by U[-shift, shift]^3;
    (e_u, e_v) turn together about a uniform random unit axis by an angle in
    U[-angle_deg, angle_deg] degrees, so they stay orthonormal."""
    n = frames.shape[0]
    out = frames.copy()
    d_src = stream.uniform(3 * n, -shift, shift).reshape(n, 3)
    d_det = stream.uniform(3 * n, -shift, shift).reshape(n, 3)
    zz = stream.uniform(n, -1.0, 1.0)
    ph = stream.uniform(n, 0.0, 2 * math.pi)
    rr = np.sqrt(np.maximum(0.0, 1 - zz * zz))
    axis = np.stack([rr * np.cos(ph), rr * np.sin(ph), zz], 1)
    ang = np.radians(stream.uniform(n, -angle_deg, angle_deg))
    R = _rodrigues(axis, ang)
    out[:, 0:3] += d_src
    out[:, 3:6] += d_det
    out[:, 6:9] = np.einsum("nij,nj->ni", R, frames[:, 6:9])
    out[:, 9:12] = np.einsum("nij,nj->ni", R, frames[:, 9:12])
    return out


# --------------------------------------------------------------------------
# Phantoms: voxel value = sum of intensity * [voxel centre inside the shape]
# --------------------------------------------------------------------------

def _axis_centres(n: int, s: float) -> np.ndarray:
    return (np.arange(n, dtype=np.float64) + 0.5 - n / 2.0) * s


def _rot_from_uniforms(u1: float, u2: float, u3: float) -> np.ndarray:
    """Uniform random rotation from three uniforms (Shoemake's unit quaternion)."""
    a, b = math.sqrt(1 - u1), math.sqrt(u1)
    w, x, y, z = (a * math.sin(2 * math.pi * u2), a * math.cos(2 * math.pi * u2),
                  b * math.sin(2 * math.pi * u3), b * math.cos(2 * math.pi * u3))
    return np.array([
        [1 - 2 * (y * y + z * z), 2 * (x * y - z * w), 2 * (x * z + y * w)],
        [2 * (x * y + z * w), 1 - 2 * (x * x + z * z), 2 * (y * z - x * w)],
        [2 * (x * z - y * w), 2 * (y * z + x * w), 1 - 2 * (x * x + y * y)],
    ])


def ellipse_phantom(shape_hw, spacing_yx, n_ellipses: int, stream: Stream,
                    centre_frac=0.6, axes_frac=(0.05, 0.5)) -> np.ndarray:
    """2D phantom (1, H, W) float32 of random ellipses."""
    h, w = shape_hw
    sy, sx = spacing_yx
    half = 0.5 * min(h * sy, w * sx)
    ys, xs = _axis_centres(h, sy), _axis_centres(w, sx)
    img = np.zeros((h, w), dtype=np.float64)
    p = stream.uniform(6 * n_ellipses).reshape(n_ellipses, 6)
    for cx, cy, ax, ay, th, inten in p:
        cx = (2 * cx - 1) * centre_frac * half
        cy = (2 * cy - 1) * centre_frac * half
        ax = (axes_frac[0] + (axes_frac[1] - axes_frac[0]) * ax) * half
        ay = (axes_frac[0] + (axes_frac[1] - axes_frac[0]) * ay) * half
        th = th * math.pi
        r = max(ax, ay)
        iy = np.nonzero(np.abs(ys - cy) <= r)[0]
        ix = np.nonzero(np.abs(xs - cx) <= r)[0]
        if iy.size == 0 or ix.size == 0:
            continue
        Y, X = np.meshgrid(ys[iy] - cy, xs[ix] - cx, indexing="ij")
        c, s = math.cos(th), math.sin(th)
        qx = c * X + s * Y
        qy = -s * X + c * Y
        inside = (qx / ax) ** 2 + (qy / ay) ** 2 <= 1.0
        img[iy[0]:iy[-1] + 1, ix[0]:ix[-1] + 1] += inten * inside
    return img.astype(np.float32)[None]


def ellipsoid_phantom(shape_dhw, spacing_zyx, n_ellipsoids: int, stream: Stream,
                      centre_frac=0.6, axes_frac=(0.05, 0.5),
                      background: np.ndarray | None = None) -> np.ndarray:
    """3D phantom (D, H, W) float32 of randomly rotated ellipsoids."""
    d, h, w = shape_dhw
    sz, sy, sx = spacing_zyx
    half = 0.5 * min(d * sz, h * sy, w * sx)
    zs, ys, xs = _axis_centres(d, sz), _axis_centres(h, sy), _axis_centres(w, sx)
    vol = np.zeros((d, h, w), dtype=np.float32)
    if background is not None:
        vol += background.astype(np.float32)
    p = stream.uniform(10 * n_ellipsoids).reshape(n_ellipsoids, 10)
    for row in p:
        c = (2 * row[0:3] - 1) * centre_frac * half                  # (x, y, z)
        ax = (axes_frac[0] + (axes_frac[1] - axes_frac[0]) * row[3:6]) * half
        R = _rot_from_uniforms(*row[6:9])
        inten = np.float32(row[9])
        r = float(ax.max())
        iz = np.nonzero(np.abs(zs - c[2]) <= r)[0]
        iy = np.nonzero(np.abs(ys - c[1]) <= r)[0]
        ix = np.nonzero(np.abs(xs - c[0]) <= r)[0]
        if iz.size == 0 or iy.size == 0 or ix.size == 0:
            continue
        X = (xs[ix] - c[0])[None, None, :]
        Y = (ys[iy] - c[1])[None, :, None]
        Z = (zs[iz] - c[2])[:, None, None]
        # body coordinates q = R^T (p - c); inside if sum (q_i / a_i)^2 <= 1
        acc = np.zeros((iz.size, iy.size, ix.size))
        for i in range(3):
            q = R[0, i] * X + R[1, i] * Y + R[2, i] * Z
            acc += (q / ax[i]) ** 2
        sl = (slice(iz[0], iz[-1] + 1), slice(iy[0], iy[-1] + 1), slice(ix[0], ix[-1] + 1))
        vol[sl] += inten * (acc <= 1.0).astype(np.float32)
    return vol


# --------------------------------------------------------------------------
# The five synthetic workloads (and reduced variants for CPU-sized checks)
# --------------------------------------------------------------------------

def make_workload(config: int, scale: int = 1, n_views: int | None = None) -> Workload:
    """Workload C<config> (1..5).  ``scale`` divides the volume and detector
    extents per axis (detector spacing and voxel spacing are multiplied by it
    so the physical acquisition stays the same); ``n_views`` optionally keeps
    only the first views (C4: the first views of each series)."""
    if config == 1:
        nv = 90
        fr = circular_parallel2d(nv, math.pi)
        wl = Workload("C1 parallel2d 64^2, 90 views, 96 bins", BEAM_PARALLEL2D,
                      (1, 64 // scale, 64 // scale), (1.0, 1.0 * scale, 1.0 * scale),
                      (96 // scale, 1), (1.0 * scale, 1.0), fr, 1)
    elif config == 2:
        fr = circular_fan2d(360, 500.0, 1000.0)
        wl = Workload("C2 fan2d 512^2, 360 views, 736 bins", BEAM_FAN2D,
                      (1, 512 // scale, 512 // scale), (1.0, 1.0 * scale, 1.0 * scale),
                      (736 // scale, 1), (1.0 * scale, 1.0), fr, 2)
    elif config == 3:
        fr = helix_cone(360, 320.0, 512.0, 40.0, 1.0)
        wl = Workload("C3 cone helix 128^3, 360 views, 384x256", BEAM_CONE,
                      (128 // scale,) * 3, (1.0 * scale,) * 3,
                      (384 // scale, 256 // scale), (0.8 * scale, 0.8 * scale), fr, 3)
    elif config == 4:
        fr = dual_axis_parallel3d(140, -70.0, 1.0)
        wl = Workload("C4 parallel3d dual-axis 512^3, 280 views, 512x512", BEAM_PARALLEL3D,
                      (512 // scale,) * 3, (1.0 * scale,) * 3,
                      (512 // scale, 512 // scale), (1.0 * scale, 1.0 * scale), fr, 4)
    elif config == 5:
        base = helix_cone(720, 1000.0, 1500.0, 0.0, 1.0)
        fr = jitter_frames(base, Stream(seed_of(5, 2)), 0.5, 0.5)
        wl = Workload("C5 cone circular jittered 512^3, 720 views, 1024x768", BEAM_CONE,
                      (512 // scale,) * 3, (1.0 * scale,) * 3,
                      (1024 // scale, 768 // scale), (1.0 * scale, 1.0 * scale), fr, 5)
    else:
        raise ValueError(f"unknown config {config}")
    if scale != 1:
        wl.name += f" (reduced {scale}x per axis)"
    if n_views is not None and n_views < wl.n_views:
        if config == 4:
            h = wl.n_views // 2
            k = max(1, n_views // 2)
            idx = np.concatenate([np.arange(k), h + np.arange(k)])
        else:
            idx = np.arange(n_views)
        wl = wl.subset_views(idx)
    return wl


def make_phantom(wl: Workload) -> np.ndarray:
    """Float32 phantom of the workload's volume shape (config recipe)."""
    cfg = wl.config
    st = Stream(seed_of(cfg, 1))
    d, h, w = wl.vol_shape
    if cfg in (1, 2) or d == 1:
        return ellipse_phantom((h, w), wl.voxel_spacing[1:], 10, st)
    if cfg == 3:
        bg = Stream(seed_of(cfg, 5)).uniform(d * h * w).reshape(d, h, w)
        return ellipsoid_phantom((d, h, w), wl.voxel_spacing, 20, st, background=bg)
    return ellipsoid_phantom((d, h, w), wl.voxel_spacing, 200, st, axes_frac=(0.03, 0.3))


def adjoint_vectors(wl: Workload):
    """x ~ U[0,1] volume-shaped and y ~ U[0,1] sinogram-shaped, float32."""
    x = Stream(seed_of(wl.config, 3)).uniform(wl.n_voxels).astype(np.float32).reshape(wl.vol_shape)
    y = Stream(seed_of(wl.config, 4)).uniform(wl.n_rays).astype(np.float32).reshape(wl.sino_shape)
    return x, y


def tiny_workload(beam: int, vol_shape, det_shape, n_views: int, seed: int,
                  voxel_spacing=(1.0, 1.0, 1.0), det_spacing=(1.0, 1.0),
                  sid: float = 30.0, sdd: float = 50.0, jitter: float = 0.0) -> Workload:
    """Small random-angle workloads for brute-force checks."""
    st = Stream(seed)
    th0 = st.uniform(1, 0.0, 2 * math.pi)[0]
    if beam == BEAM_PARALLEL2D:
        fr = circular_parallel2d(n_views, math.pi)
    elif beam == BEAM_FAN2D:
        fr = circular_fan2d(n_views, sid, sdd)
    elif beam == BEAM_CONE:
        fr = helix_cone(n_views, sid, sdd, z_range=2.0, n_turns=1.0)
    else:
        fr = dual_axis_parallel3d(max(1, n_views // 2), -65.0, 130.0 / max(1, n_views // 2))
    if beam in (BEAM_PARALLEL2D, BEAM_FAN2D):
        # rotate the whole orbit by a random start angle
        c, s = math.cos(th0), math.sin(th0)
        R = np.array([[c, -s, 0], [s, c, 0], [0, 0, 1.0]])
        for k in (0, 3, 6):
            fr[:, k:k + 3] = fr[:, k:k + 3] @ R.T
    if jitter > 0 and beam in (BEAM_CONE, BEAM_PARALLEL3D):
        fr = jitter_frames(fr, st, jitter if beam == BEAM_CONE else 0.0, 3.0)
        if beam == BEAM_PARALLEL3D:
            # keep rays orthogonal to nothing in particular: tilt the rays too
            fr[:, 0:3] = np.einsum("nij,nj->ni", _rodrigues(
                np.tile([[0.0, 0.0, 1.0]], (fr.shape[0], 1)),
                st.uniform(fr.shape[0], -0.3, 0.3)), fr[:, 0:3])
    return Workload(f"tiny {BEAM_NAMES[beam]}", beam, tuple(vol_shape), tuple(voxel_spacing),
                    tuple(det_shape), tuple(det_spacing), fr, 0)
