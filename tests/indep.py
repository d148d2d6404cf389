"""Independent geometric helpers used to pin the oracle.

These are deliberately written with different algorithms from the oracle:
chords come from intersecting the line with the six face rectangles of a box
(not the slab method), and line integrals come from dense midpoint sampling
of points along the ray, each mapped to its cell by the lattice definition.
"""
from __future__ import annotations

import itertools
import math

import numpy as np


def face_chord(o, d, tmin, tmax, lo, hi) -> float:
    """Length of {o + t d : tmin <= t <= tmax} inside the closed box [lo, hi],
    from the line's hits on the box's face rectangles."""
    o = np.asarray(o, float)
    d = np.asarray(d, float)
    ts = []
    for ax in range(3):
        if d[ax] == 0.0:
            continue
        for plane in (lo[ax], hi[ax]):
            t = (plane - o[ax]) / d[ax]
            p = o + t * d
            ok = True
            for b in range(3):
                if b == ax:
                    continue
                eps = 1e-12 * max(1.0, abs(hi[b] - lo[b]))
                if p[b] < lo[b] - eps or p[b] > hi[b] + eps:
                    ok = False
            if ok:
                ts.append(t)
    # lines parallel to a face pair must lie between its planes
    for ax in range(3):
        if d[ax] == 0.0 and not (lo[ax] <= o[ax] < hi[ax]):
            return 0.0
    if len(ts) < 2:
        # the line may start/end inside (segments): include interior end points
        pass
    inside = lambda t: all(lo[b] - 1e-12 <= o[b] + t * d[b] <= hi[b] + 1e-12 for b in range(3))
    cand = list(ts)
    for t in (tmin, tmax):
        if math.isfinite(t) and inside(t):
            cand.append(t)
    cand = [t for t in cand if tmin - 1e-15 <= t <= tmax + 1e-15]
    if len(cand) < 2:
        return 0.0
    return (max(cand) - min(cand)) * float(np.linalg.norm(d))


def lattice(vol_shape, spacing):
    """(n, s, lo) per axis in x, y, z order from (D,H,W) and (dz,dy,dx)."""
    d, h, w = vol_shape
    sz, sy, sx = spacing
    n = np.array([w, h, d], dtype=np.int64)
    s = np.array([sx, sy, sz], dtype=float)
    lo = -0.5 * n * s
    return n, s, lo


def sampled_line_integral(o, d, tmin, tmax, vol, spacing, n_samples=400_000):
    """Midpoint-rule line integral of the cell-constant volume along the ray.

    The ray is first limited to the volume's bounding box with face_chord's
    hit points; points are then mapped to cells by floor((p - lo) / s)."""
    vol = np.asarray(vol, float)
    n, s, lo = lattice(vol.shape, spacing)
    hi = lo + n * s
    o = np.asarray(o, float)
    d = np.asarray(d, float)
    # bounding interval via a generous scan of face hits
    ts = []
    for ax in range(3):
        if d[ax] != 0.0:
            ts += [(lo[ax] - o[ax]) / d[ax], (hi[ax] - o[ax]) / d[ax]]
    if not ts:
        return 0.0, 0.0
    a = max(min(ts), tmin)
    b = min(max(ts), tmax)
    if not b > a:
        return 0.0, 0.0
    dt = (b - a) / n_samples
    t = a + (np.arange(n_samples) + 0.5) * dt
    p = o[None, :] + t[:, None] * d[None, :]
    idx = np.floor((p - lo[None, :]) / s[None, :]).astype(np.int64)
    ok = np.all((idx >= 0) & (idx < n[None, :]), axis=1)
    vals = np.zeros(n_samples)
    ii = idx[ok]
    vals[ok] = vol[ii[:, 2], ii[:, 1], ii[:, 0]]
    L = float(np.linalg.norm(d))
    integral = vals.sum() * dt * L
    # error bound: each cell boundary crossed can misattribute at most one
    # sample interval's worth of length times the jump in value
    n_bound = int(np.count_nonzero(np.any(idx[1:] != idx[:-1], axis=1)))
    bound = (n_bound + 2) * dt * L * (np.abs(vol).max() if vol.size else 0.0)
    return integral, bound


def cell_boxes(vol_shape, spacing):
    n, s, lo = lattice(vol_shape, spacing)
    for iz, iy, ix in itertools.product(range(n[2]), range(n[1]), range(n[0])):
        blo = lo + np.array([ix, iy, iz]) * s
        yield (iz, iy, ix), blo, blo + s
