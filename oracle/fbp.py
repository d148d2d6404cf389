"""Float64 oracle of analytical FBP / FDK (test infrastructure).

TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the benchmark's
CPU-baseline leg; the product path never imports it.  Plain numpy, float64,
written to read like the definitions; it shares no code with the HIP library.

What is computed (diffct documentation, "Differentiable analytical
reconstruction", the "Analytical Reconstruction Helpers" and "Ramp Filter
Options" sections of the API reference, and the FBP/FDK example pages):

  1. pre-weights on the sinogram: the fan/cone cosine weight of each pixel and,
     for short scans, Parker's weights;
  2. a ramp filter along the detector u axis, zero-padded to pad_factor * U
     samples and applied as a real-FFT multiplier, optionally windowed;
  3. angular quadrature weights per view (a full fan/cone turn carries the 1/2
     redundancy factor);
  4. a voxel-driven, interpolating weighted backprojection (not the Siddon
     adjoint): each voxel gathers, per view, the bilinearly interpolated
     filtered value where its centre projects on the detector, times the
     FDK distance weight R D / U(x)^2 (fan/cone) or 1 (parallel).
  The transpose of step 4 scatters the same interpolation coefficients.

Readings where the pages give no formula (each listed in the design notes):
  - Ram-Lak: the band-limited ramp of Ramachandran and Lakshminarayanan sampled
    in space (Kak and Slaney, "Principles of Computerized Tomographic Imaging",
    ch. 3): h[0] = 1/(4 d^2), h[n] = -1/(pi n d)^2 for odd n, 0 for even n != 0,
    taken P-periodic (n in [-P/2, P/2)); the multiplier is d * DFT_P(h).
    Windows of the normalised frequency f = k / P in [0, 1/2]: Shepp-Logan
    sin(pi f)/(pi f), cosine cos(pi f), Hamming 0.54 + 0.46 cos(2 pi f), Hann
    0.5 + 0.5 cos(2 pi f).
  - Cosine weight |(p - a).n| / |p - a| for pixel centre p, source a and unit
    detector normal n.
  - Angular weights: half the angular gap to the two neighbouring views,
    periodic over the scan's period (2 pi for full fan/cone turns and for
    redundant parallel turns, pi for parallel half turns), non-periodic
    (one-sided at the ends) for short scans; times 1/2 for redundant full turns.
  - FDK weight R D / U(x)^2 with U(x) = (x - a).n, D = (c - a).n and
    R = (iso - a).n; the isocentre, when not given, is the point nearest (least
    squares) to the lines through each source along its detector normal.
  - Parker weights (Parker 1982) with beta the scan angle from the first view
    and gamma the in-plane fan angle of the column, signed in the sense of
    rotation; delta is the largest |gamma|.
  - Interpolation treats detector samples outside [0, U-1] x [0, V-1] as 0.
  - Fan/cone: a point at or behind the source (U(x) <= 0) lies on no ray of
    that view (the rays run from the source towards the detector) and gathers
    nothing from it.
  - Overrides (same page, the paragraph on the complete APIs): a caller's
    projection weights take the place of the cosine weight of step 1 (Parker's
    weights, when asked for, still multiply); a caller's filter response, of
    length pad_factor * U // 2 + 1 in physical units, takes the place of the
    windowed multiplier of step 2.

Helical approximation (same page, "Helical approximation"): the rows are
filtered once (steps 1-2, no angular weight), and each axial slice s is then
gathered as in step 4 with its own per-view weights w[s, i].  Reading of the
window: the source crosses the slice centre z_s at the angle theta_c(s), found
by linear interpolation of the (source z, unwrapped angle) samples; the slice
integrates over the full turn [theta_c - pi, theta_c + pi] with the 1/2
redundancy factor, by the trapezoidal rule on the sampled angles, i.e.
w[s, i] = 1/2 * integral over the window of the hat function of sample i (the
piecewise-linear interpolation basis on the angles).  The hats sum to 1 on the
scanned range, so each slice's weights sum to pi.  A slice whose centre lies
outside the source's z range, or whose window leaves the scanned angles, is
rejected.
"""
from __future__ import annotations

import math

import numpy as np

PARALLEL2D, FAN2D, CONE, PARALLEL3D = 0, 1, 2, 3
WINDOWS = ("ram-lak", "shepp-logan", "cosine", "hamming", "hann")


# ---------------------------------------------------------------------------
# ramp filter
# ---------------------------------------------------------------------------

def ramlak_kernel(P: int, spacing: float) -> np.ndarray:
    """The P-periodic band-limited ramp h[n], n = 0..P-1 (n >= P/2 stands for n - P)."""
    n = np.arange(P)
    n = np.where(n >= P // 2 + (P % 2), n - P, n)   # signed index in [-P/2, P/2)
    h = np.zeros(P)
    h[n == 0] = 1.0 / (4.0 * spacing * spacing)
    odd = (n % 2) != 0
    h[odd] = -1.0 / (math.pi * n[odd] * spacing) ** 2
    return h


def window_values(P: int, window: str) -> np.ndarray:
    """Window at the rFFT frequencies k / P, k = 0..P//2."""
    f = np.arange(P // 2 + 1) / P
    if window in (None, "ram-lak"):
        return np.ones_like(f)
    if window == "shepp-logan":
        return np.sinc(f)          # numpy's sinc is sin(pi f) / (pi f)
    if window == "cosine":
        return np.cos(math.pi * f)
    if window == "hamming":
        return 0.54 + 0.46 * np.cos(2 * math.pi * f)
    if window in ("hann", "hanning"):
        return 0.5 + 0.5 * np.cos(2 * math.pi * f)
    raise ValueError(f"unknown window {window!r}")


def ramp_multiplier(P: int, spacing: float, window: str = "ram-lak") -> np.ndarray:
    """Real rFFT multiplier (length P//2 + 1) in physical units (1 / length)."""
    h = ramlak_kernel(P, spacing)
    M = spacing * np.fft.rfft(h).real
    return M * window_values(P, window)


def ramp_filter(p: np.ndarray, spacing: float, pad_factor: int = 2, window: str = "ram-lak",
                axis: int = 1, response=None) -> np.ndarray:
    """Filter along `axis` (zero-padded to pad_factor * N, rFFT multiplier, cropped).
    response: the caller's multiplier (length pad_factor * N // 2 + 1), in place
    of the windowed ramp."""
    p = np.moveaxis(np.asarray(p, dtype=np.float64), axis, -1)
    N = p.shape[-1]
    P = pad_factor * N
    if response is None:
        M = ramp_multiplier(P, spacing, window)
    else:
        M = np.asarray(response, dtype=np.float64)
        if M.shape != (P // 2 + 1,):
            raise ValueError(f"filter response must have pad_factor * U // 2 + 1 = {P // 2 + 1} values")
    q = np.fft.irfft(np.fft.rfft(p, n=P, axis=-1) * M, n=P, axis=-1)[..., :N]
    return np.moveaxis(q, -1, axis)


# ---------------------------------------------------------------------------
# geometry helpers
# ---------------------------------------------------------------------------

def _three_d(beam: int) -> bool:
    return beam in (CONE, PARALLEL3D)


def detector_normals(frames: np.ndarray, beam: int) -> np.ndarray:
    """Unit detector normal per view, oriented from the source side to the detector."""
    a, c, eu, ev = frames[:, 0:3], frames[:, 3:6], frames[:, 6:9], frames[:, 9:12]
    if _three_d(beam):
        n = np.cross(eu, ev)
    else:
        n = np.stack([eu[:, 1], -eu[:, 0], np.zeros(len(eu))], 1)
    n = n / np.linalg.norm(n, axis=1, keepdims=True)
    if beam in (FAN2D, CONE):
        toward = np.einsum("ij,ij->i", c - a, n)
    else:
        toward = np.einsum("ij,ij->i", a, n)     # parallel: along the ray direction
    return n * np.where(toward < 0, -1.0, 1.0)[:, None]


def pixel_centres(wl) -> np.ndarray:
    """(views, U, V, 3) world positions of the flat detector's pixel centres."""
    fr = wl.frames
    U, V = wl.det_shape
    du, dv = wl.det_spacing
    ou = (np.arange(U) - 0.5 * (U - 1)) * du
    ov = (np.arange(V) - 0.5 * (V - 1)) * dv if _three_d(wl.beam) else np.zeros(V)
    c, eu, ev = fr[:, 3:6], fr[:, 6:9], fr[:, 9:12]
    return (c[:, None, None, :] + ou[None, :, None, None] * eu[:, None, None, :]
            + ov[None, None, :, None] * ev[:, None, None, :])


def cosine_weights(wl) -> np.ndarray:
    """|(p - a).n| / |p - a| per pixel for fan/cone; ones for parallel beams."""
    if wl.beam not in (FAN2D, CONE):
        return np.ones(wl.sino_shape)
    p = pixel_centres(wl)
    a = wl.frames[:, None, None, 0:3]
    n = detector_normals(wl.frames, wl.beam)[:, None, None, :]
    d = p - a
    return np.abs(np.sum(d * n, axis=-1)) / np.linalg.norm(d, axis=-1)


def isocentre(wl) -> np.ndarray:
    """Least-squares point nearest to the lines a_i + t n_i (fan/cone; origin for
    parallel beams).  2D: in the z = 0 plane."""
    if wl.beam not in (FAN2D, CONE):
        return np.zeros(3)
    a = wl.frames[:, 0:3]
    n = detector_normals(wl.frames, wl.beam)
    dim = 3 if wl.beam == CONE else 2
    Asum = np.zeros((dim, dim))
    bsum = np.zeros(dim)
    for ai, ni in zip(a[:, :dim], n[:, :dim]):
        Pm = np.eye(dim) - np.outer(ni, ni) / np.dot(ni, ni)
        Asum += Pm
        bsum += Pm @ ai
    x = np.linalg.lstsq(Asum, bsum, rcond=None)[0]
    out = np.zeros(3)
    out[:dim] = x
    return out


def angular_weights(angles, beam: int, short_scan: bool = False, redundant=None) -> np.ndarray:
    """Quadrature weight per view (see the module notes)."""
    th = np.asarray(angles, dtype=np.float64)
    n = len(th)
    if redundant is None:
        redundant = beam in (FAN2D, CONE) and not short_scan
    if n == 1:
        return np.array([math.pi if not redundant else math.pi])
    if short_scan:
        w = np.empty(n)
        w[1:-1] = 0.5 * (th[2:] - th[:-2])
        w[0] = 0.5 * (th[1] - th[0])
        w[-1] = 0.5 * (th[-1] - th[-2])
        w = np.abs(w)
    else:
        period = 2 * math.pi if (beam in (FAN2D, CONE) or redundant) else math.pi
        sgn = 1.0 if th[-1] >= th[0] else -1.0
        nxt = np.concatenate([th[1:], [th[0] + sgn * period]])
        prv = np.concatenate([[th[-1] - sgn * period], th[:-1]])
        w = np.abs(0.5 * (nxt - prv))
    return w * (0.5 if redundant else 1.0)


def rotation_sense(wl) -> float:
    """+1 if the source moves counter-clockwise about z (seen from +z), else -1."""
    a = wl.frames[:, 0:2]
    cr = a[:-1, 0] * a[1:, 1] - a[:-1, 1] * a[1:, 0]
    return 1.0 if cr.sum() >= 0 else -1.0


def fan_angles(wl) -> np.ndarray:
    """(views, U) in-plane angle between the central ray and the ray through the
    centre of column u, positive in the sense of rotation."""
    p = pixel_centres(wl)[:, :, 0, :]             # v at the first row: only x, y matter
    a = wl.frames[:, None, 0:3]
    n = detector_normals(wl.frames, wl.beam)[:, None, :]
    d = (p - a)[..., :2]
    d0 = np.broadcast_to(n[..., :2], d.shape)
    cross = d0[..., 0] * d[..., 1] - d0[..., 1] * d[..., 0]
    dot = np.sum(d0 * d, axis=-1)
    return rotation_sense(wl) * np.arctan2(cross, dot)


def parker(beta: np.ndarray, gamma: np.ndarray, delta: float) -> np.ndarray:
    """Parker's short-scan weight w(beta, gamma) for a half fan angle delta."""
    beta = np.asarray(beta, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    w = np.zeros(np.broadcast(beta, gamma).shape)
    b = np.broadcast_to(beta, w.shape)
    g = np.broadcast_to(gamma, w.shape)
    r1 = (b >= 0) & (b < 2 * (delta - g))
    r2 = (b >= 2 * (delta - g)) & (b <= math.pi - 2 * g)
    r3 = (b > math.pi - 2 * g) & (b <= math.pi + 2 * delta)
    with np.errstate(divide="ignore", invalid="ignore"):
        w = np.where(r1, np.sin(math.pi / 4 * b / (delta - g)) ** 2, w)
        w = np.where(r2, 1.0, w)
        w = np.where(r3, np.sin(math.pi / 4 * (math.pi + 2 * delta - b) / (delta + g)) ** 2, w)
    return w


def parker_weights(wl, angles) -> np.ndarray:
    """(views, U) Parker weights of a fan/cone short scan."""
    th = np.asarray(angles, dtype=np.float64)
    beta = np.abs(th - th[0])
    gam = fan_angles(wl)
    delta = float(np.max(np.abs(gam)))
    return parker(beta[:, None], gam, delta)


# ---------------------------------------------------------------------------
# filtering and the weighted backprojection
# ---------------------------------------------------------------------------

def filter_sinogram(wl, sino, angles, window="ram-lak", pad_factor=2, short_scan=False,
                    ang_weights=None, projection_weights=None, filter_response=None) -> np.ndarray:
    """Steps 1-3: pre-weights, ramp filter along u, angular weights.
    projection_weights ((U, V) or (views, U, V)) replace the cosine weight;
    filter_response replaces the windowed multiplier."""
    if projection_weights is None:
        pre = cosine_weights(wl)
    else:
        pw = np.asarray(projection_weights, dtype=np.float64)
        if pw.shape not in (tuple(wl.det_shape), tuple(wl.sino_shape)):
            raise ValueError("projection weights must have shape (U, V) or (views, U, V)")
        pre = np.broadcast_to(pw, wl.sino_shape)
    p = np.asarray(sino, dtype=np.float64) * pre
    if short_scan:
        p = p * parker_weights(wl, angles)[:, :, None]
    q = ramp_filter(p, wl.det_spacing[0], pad_factor, window, axis=1, response=filter_response)
    w = angular_weights(angles, wl.beam, short_scan) if ang_weights is None else \
        np.asarray(ang_weights, dtype=np.float64)
    return q * w[:, None, None]


def voxel_centres(wl):
    D, H, Wd = wl.vol_shape
    dz, dy, dx = wl.voxel_spacing
    x = -0.5 * Wd * dx + (np.arange(Wd) + 0.5) * dx
    y = -0.5 * H * dy + (np.arange(H) + 0.5) * dy
    z = -0.5 * D * dz + (np.arange(D) + 0.5) * dz if _three_d(wl.beam) else np.zeros(1)
    return z, y, x


def _projection(wl, view, X, iso):
    """Detector coordinates (u, v in pixel units) and weight of the world points X (..., 3)."""
    fr = wl.frames[view]
    a, c, eu, ev = fr[0:3], fr[3:6], fr[6:9], fr[9:12]
    n = detector_normals(wl.frames[view:view + 1], wl.beam)[0]
    U, V = wl.det_shape
    du, dv = wl.det_spacing
    if wl.beam in (FAN2D, CONE):
        Ux = (X - a) @ n
        D = np.dot(c - a, n)
        R = np.dot(iso - a, n)
        front = Ux > 0
        Us = np.where(front, Ux, 1.0)            # points on no ray: any finite stand-in
        P = a + (X - a) * (D / Us)[..., None]
        wgt = np.where(front, R * D / Us ** 2, 0.0)
    else:
        # parallel: slide X along the ray direction onto the detector plane
        t = ((c - X) @ n) / np.dot(a, n)
        P = X + t[..., None] * a
        wgt = np.ones(X.shape[:-1])
    u = (P - c) @ eu / du + 0.5 * (U - 1)
    v = (P - c) @ ev / dv + 0.5 * (V - 1) if _three_d(wl.beam) else np.zeros(X.shape[:-1])
    return u, v, wgt


def _bilinear_taps(u, v, U, V):
    """Four (index_u, index_v, coefficient) taps; samples outside the detector are 0."""
    iu = np.floor(u).astype(np.int64)
    iv = np.floor(v).astype(np.int64)
    au = u - iu
    av = v - iv
    taps = []
    for su, cu in ((0, 1 - au), (1, au)):
        for sv, cv in ((0, 1 - av), (1, av)):
            ju, jv = iu + su, iv + sv
            ok = (ju >= 0) & (ju < U) & (jv >= 0) & (jv < V)
            taps.append((np.where(ok, ju, 0), np.where(ok, jv, 0), np.where(ok, cu * cv, 0.0)))
    return taps


def weighted_backproject(wl, q, iso=None) -> np.ndarray:
    """Step 4: f(x) = sum_i weight_i(x) * interp(q_i, u_i(x), v_i(x))."""
    q = np.asarray(q, dtype=np.float64)
    iso = isocentre(wl) if iso is None else np.asarray(iso, dtype=np.float64)
    z, y, x = voxel_centres(wl)
    Z, Y, Xg = np.meshgrid(z, y, x, indexing="ij")
    X = np.stack([Xg, Y, Z], axis=-1)
    U, V = wl.det_shape
    out = np.zeros(X.shape[:-1])
    for i in range(wl.n_views):
        u, v, wgt = _projection(wl, i, X, iso)
        val = np.zeros_like(out)
        for ju, jv, cf in _bilinear_taps(u, v, U, V):
            val += cf * q[i, ju, jv]
        out += wgt * val
    return out.reshape(wl.vol_shape)


def weighted_backproject_voxels(wl, q, voxel_ids, iso=None) -> np.ndarray:
    """weighted_backproject evaluated at the given flat voxel indices only."""
    q = np.asarray(q, dtype=np.float64)
    iso = isocentre(wl) if iso is None else np.asarray(iso, dtype=np.float64)
    z, y, x = voxel_centres(wl)
    D, H, Wd = wl.vol_shape
    ids = np.asarray(voxel_ids, dtype=np.int64)
    X = np.stack([x[ids % Wd], y[(ids // Wd) % H], z[ids // (Wd * H)]], axis=-1)
    U, V = wl.det_shape
    out = np.zeros(len(ids))
    for i in range(wl.n_views):
        u, v, wgt = _projection(wl, i, X, iso)
        val = np.zeros_like(out)
        for ju, jv, cf in _bilinear_taps(u, v, U, V):
            val += cf * q[i, ju, jv]
        out += wgt * val
    return out


def weighted_backproject_T(wl, vol, iso=None) -> np.ndarray:
    """Transpose of weighted_backproject: scatter of the same coefficients."""
    vol = np.asarray(vol, dtype=np.float64).reshape(wl.vol_shape)
    iso = isocentre(wl) if iso is None else np.asarray(iso, dtype=np.float64)
    z, y, x = voxel_centres(wl)
    Z, Y, Xg = np.meshgrid(z, y, x, indexing="ij")
    X = np.stack([Xg, Y, Z], axis=-1)
    U, V = wl.det_shape
    out = np.zeros(wl.sino_shape)
    for i in range(wl.n_views):
        u, v, wgt = _projection(wl, i, X, iso)
        for ju, jv, cf in _bilinear_taps(u, v, U, V):
            np.add.at(out[i], (ju.ravel(), jv.ravel()), (wgt * cf * vol).ravel())
    return out


def fbp(wl, sino, angles, window="ram-lak", pad_factor=2, short_scan=False, iso=None,
        ang_weights=None, projection_weights=None, filter_response=None) -> np.ndarray:
    """FBP (parallel2d, fan2d) or FDK (cone): filter, then the weighted backprojection."""
    q = filter_sinogram(wl, sino, angles, window, pad_factor, short_scan, ang_weights,
                        projection_weights, filter_response)
    return weighted_backproject(wl, q, iso)


# ---------------------------------------------------------------------------
# helical approximation
# ---------------------------------------------------------------------------

def _hat_integral(t, i, lo, hi) -> float:
    """Integral over [lo, hi] of the hat function of node i on the increasing nodes t."""
    total = 0.0
    if i > 0:                                   # rising side, 0 at t[i-1] to 1 at t[i]
        a, b = max(lo, t[i - 1]), min(hi, t[i])
        if b > a:
            L = t[i] - t[i - 1]
            total += ((b - t[i - 1]) ** 2 - (a - t[i - 1]) ** 2) / (2 * L)
    if i < len(t) - 1:                          # falling side, 1 at t[i] to 0 at t[i+1]
        a, b = max(lo, t[i]), min(hi, t[i + 1])
        if b > a:
            L = t[i + 1] - t[i]
            total += ((t[i + 1] - a) ** 2 - (t[i + 1] - b) ** 2) / (2 * L)
    return total


def helical_window_centres(wl, angles) -> np.ndarray:
    """theta_c per slice: the unwrapped angle at which the source crosses the
    slice centre, by linear interpolation of the (source z, angle) samples."""
    th = np.asarray(angles, dtype=np.float64)
    zs = wl.frames[:, 2]
    if wl.beam != CONE:
        raise ValueError("the helical approximation is a cone-beam method")
    if len(th) != wl.n_views or len(th) < 2:
        raise ValueError("one unwrapped angle per view, at least two views")
    dth, dz = np.diff(th), np.diff(zs)
    if not (np.all(dth > 0) or np.all(dth < 0)):
        raise ValueError("the unwrapped angles must be strictly monotone")
    if not (np.all(dz > 0) or np.all(dz < 0)):
        raise ValueError("the source z must be strictly monotone")
    sz = 1.0 if dz[0] > 0 else -1.0
    z_c = voxel_centres(wl)[0]
    out = np.empty(len(z_c))
    for s, zc in enumerate(z_c):
        key = sz * zs
        if not (key[0] <= sz * zc <= key[-1]):
            raise ValueError(f"slice {s} (z = {zc}) lies outside the source's z range")
        k = min(int(np.searchsorted(key, sz * zc, side="right")) - 1, len(th) - 2)
        f = (zc - zs[k]) / (zs[k + 1] - zs[k])
        out[s] = th[k] + f * (th[k + 1] - th[k])
    return out


def helical_view_weights(wl, angles) -> np.ndarray:
    """(D, views) per-slice weights: half the integral of each sample's hat
    function over the full turn centred at the slice's theta_c."""
    th = np.asarray(angles, dtype=np.float64)
    centres = helical_window_centres(wl, angles)
    sa = 1.0 if th[-1] > th[0] else -1.0
    t = sa * th                                # increasing
    tol = 1e-9 * (1.0 + np.max(np.abs(t)))
    w = np.zeros((len(centres), len(th)))
    for s, tc in enumerate(sa * centres):
        lo, hi = tc - math.pi, tc + math.pi
        if lo < t[0] - tol or hi > t[-1] + tol:
            raise ValueError(f"slice {s}: the full turn about its crossing angle leaves the scan")
        lo, hi = max(lo, t[0]), min(hi, t[-1])
        for i in range(len(t)):
            w[s, i] = 0.5 * _hat_integral(t, i, lo, hi)
    return w


def helical_weighted_backproject(wl, q, weights, iso=None) -> np.ndarray:
    """Step 4 with per-slice view weights: f_s(x) = sum_i w[s, i] * weight_i(x) *
    interp(q_i, u_i(x), v_i(x)) for the voxels x of slice s."""
    q = np.asarray(q, dtype=np.float64)
    wts = np.asarray(weights, dtype=np.float64)
    if wts.shape != (wl.vol_shape[0], wl.n_views):
        raise ValueError("weights must have shape (D, views)")
    iso = isocentre(wl) if iso is None else np.asarray(iso, dtype=np.float64)
    z, y, x = voxel_centres(wl)
    Z, Y, Xg = np.meshgrid(z, y, x, indexing="ij")
    X = np.stack([Xg, Y, Z], axis=-1)
    U, V = wl.det_shape
    out = np.zeros(X.shape[:-1])
    for i in range(wl.n_views):
        u, v, wgt = _projection(wl, i, X, iso)
        val = np.zeros_like(out)
        for ju, jv, cf in _bilinear_taps(u, v, U, V):
            val += cf * q[i, ju, jv]
        out += wts[:, i][:, None, None] * wgt * val
    return out


def helical_weighted_backproject_T(wl, vol, weights, iso=None) -> np.ndarray:
    """Transpose of helical_weighted_backproject."""
    vol = np.asarray(vol, dtype=np.float64).reshape(wl.vol_shape)
    wts = np.asarray(weights, dtype=np.float64)
    if wts.shape != (wl.vol_shape[0], wl.n_views):
        raise ValueError("weights must have shape (D, views)")
    iso = isocentre(wl) if iso is None else np.asarray(iso, dtype=np.float64)
    z, y, x = voxel_centres(wl)
    Z, Y, Xg = np.meshgrid(z, y, x, indexing="ij")
    X = np.stack([Xg, Y, Z], axis=-1)
    U, V = wl.det_shape
    out = np.zeros(wl.sino_shape)
    for i in range(wl.n_views):
        u, v, wgt = _projection(wl, i, X, iso)
        g = wts[:, i][:, None, None] * wgt * vol
        for ju, jv, cf in _bilinear_taps(u, v, U, V):
            np.add.at(out[i], (ju.ravel(), jv.ravel()), (cf * g).ravel())
    return out


def helical_fdk(wl, sino, angles, window="ram-lak", pad_factor=2, iso=None, projection_weights=None,
                filter_response=None) -> np.ndarray:
    """Filter the rows once (no angular weight), then gather each slice with its
    helical view weights."""
    q = filter_sinogram(wl, sino, angles, window, pad_factor, False, np.ones(wl.n_views),
                        projection_weights, filter_response)
    return helical_weighted_backproject(wl, q, helical_view_weights(wl, angles), iso)
