"""Host-side checks of test geometries (no oracle, no device)."""
import numpy as np


def untraversed_plane_distance(wl):
    """Smallest distance (in cells) from a ray to a lattice plane of an axis the
    ray never crosses (direction component exactly 0), over every such ray of a
    flat-detector parallel geometry; 0 when some ray lies in such a plane (a tie,
    where a ray belongs to the cell above the plane)."""
    D, H, Wd = wl.vol_shape
    dz, dy, dx = wl.voxel_spacing
    n, sp = np.array([Wd, H, D], float), np.array([dx, dy, dz])
    lo = -0.5 * n * sp
    U, V = wl.det_shape
    su, sv = wl.det_spacing
    fr = np.asarray(wl.frames, np.float64)
    ou = (np.arange(U) - 0.5 * (U - 1)) * su
    ov = (np.arange(V) - 0.5 * (V - 1)) * sv
    best = np.inf
    for ray, c, eu, ev in zip(fr[:, 0:3], fr[:, 3:6], fr[:, 6:9], fr[:, 9:12]):
        for k in np.nonzero(ray == 0.0)[0]:
            p = c[k] + ou[:, None] * eu[k] + ov[None, :] * ev[k]
            q = (p - lo[k]) / sp[k]
            best = min(best, float(np.abs(q - np.rint(q)).min()))
    return best
