"""GPU parity of ordered-subset SIRT / SART (ct_sirt_weights_views,
ct_sirt_step_views) against the oracle's SIRT step applied subset by subset
(each subset with its own row and column weights), with and without bounds
and a mask; the whole view range reproduces the bounded SIRT step bit for bit.
"""
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


def host(t):
    return t.detach().cpu().numpy().astype(np.float64)


def rel_l2(g, o):
    g = np.asarray(g, np.float64).ravel()
    o = np.asarray(o, np.float64).ravel()
    return float(np.linalg.norm(g - o) / np.linalg.norm(o))


def say(*a):
    print(*a, flush=True)


def gpu_os(wl, y, subsets, epochs, lo=-np.inf, hi=np.inf, mask=None, relax=1.0):
    g = rdp.Geometry.from_workload(wl)
    x = torch.zeros(wl.vol_shape, device="cuda")
    U, V = wl.det_shape
    w = {}
    for vb, ve in subsets:
        r = torch.empty((ve - vb, U, V), device="cuda")
        c = torch.empty(wl.vol_shape, device="cuda")
        rdp.ct_sirt_weights_views(g, vb, ve, r, c)
        w[(vb, ve)] = (r, c)
    m = None if mask is None else torch.from_numpy(mask.astype(np.uint8)).cuda()
    for _ in range(epochs):
        for vb, ve in subsets:
            r, c = w[(vb, ve)]
            work = torch.empty((ve - vb, U, V), device="cuda")
            rdp.ct_sirt_step_views(g, vb, ve, x, dev(y[vb:ve]), r, c, relax, lo, hi, m, work)
    return host(x)


def oracle_os(wl, y, subsets, epochs, lo=-np.inf, hi=np.inf, mask=None, relax=1.0):
    x = np.zeros(wl.vol_shape)
    geo = {s: oracle.Geometry.from_workload(wl.subset_views(np.arange(*s))) for s in subsets}
    wts = {s: oracle.sirt_weights(geo[s]) for s in subsets}
    for _ in range(epochs):
        for s in subsets:
            x = oracle.sirt(geo[s], y[s[0]:s[1]], x0=x, n_iter=1, relax=relax, weights=wts[s], lo=lo,
                            hi=hi, mask=mask)
    return x


def test_ordered_subsets_on_reduced_c2_bounded_masked():
    wl = W.make_workload(2, scale=4)          # 128^2 fan beam, 360 views, 184 bins
    og = oracle.Geometry.from_workload(wl)
    y = oracle.project(og, W.make_phantom(wl)).astype(np.float32)
    subsets = [(k, min(k + 45, wl.n_views)) for k in range(0, wl.n_views, 45)]
    D, H, Wd = wl.vol_shape
    yy, xx = np.mgrid[0:H, 0:Wd]
    mask = ((xx - Wd / 2 + 0.5) ** 2 + (yy - H / 2 + 0.5) ** 2 < (0.45 * Wd) ** 2)[None]
    g = gpu_os(wl, y, subsets, 2, lo=0.0, hi=0.8, mask=mask, relax=0.9)
    o = oracle_os(wl, y, subsets, 2, lo=0.0, hi=0.8, mask=mask, relax=0.9)
    e = rel_l2(g, o)
    say(f"C2/4 OS-SIRT, 8 subsets x 2 epochs, bounded + masked: rel_l2 {e:.2e}")
    assert e <= TOL
    assert np.all(g[~np.broadcast_to(mask, g.shape)] == 0.0)   # masked-out voxels keep x0 = 0


def test_single_view_subsets_are_sart():
    wl = W.tiny_workload(W.BEAM_CONE, (14, 17, 19), (26, 21), 12, 61, jitter=0.5)
    og = oracle.Geometry.from_workload(wl)
    x_true = np.random.default_rng(2).uniform(0, 1, wl.vol_shape)
    y = oracle.project(og, x_true).astype(np.float32)
    subsets = [(k, k + 1) for k in range(wl.n_views)]
    g = gpu_os(wl, y, subsets, 1, relax=0.5)
    o = oracle_os(wl, y, subsets, 1, relax=0.5)
    e = rel_l2(g, o)
    say(f"single-view SART, 12 views: rel_l2 {e:.2e}")
    assert e <= TOL


def test_whole_range_is_the_bounded_sirt_step():
    wl = W.tiny_workload(W.BEAM_PARALLEL3D, (15, 18, 20), (24, 22), 10, 62, jitter=1.0)
    g = rdp.Geometry.from_workload(wl)
    og = oracle.Geometry.from_workload(wl)
    y = dev(oracle.project(og, np.random.default_rng(3).uniform(0, 1, wl.vol_shape)))
    r1, c1 = torch.empty(g.sino_shape, device="cuda"), torch.empty(g.vol_shape, device="cuda")
    r2, c2 = torch.empty(g.sino_shape, device="cuda"), torch.empty(g.vol_shape, device="cuda")
    rdp.ct_sirt_weights(g, r1, c1)
    rdp.ct_sirt_weights_views(g, 0, wl.n_views, r2, c2)
    assert torch.equal(r1, r2) and torch.equal(c1, c2)
    x1 = torch.full(g.vol_shape, 0.1, device="cuda")
    x2 = x1.clone()
    w1, w2 = torch.empty(g.sino_shape, device="cuda"), torch.empty(g.sino_shape, device="cuda")
    rdp.ct_sirt_step_bounded(g, x1, y, r1, c1, 1.0, 0.0, 0.5, None, w1)
    rdp.ct_sirt_step_views(g, 0, wl.n_views, x2, y, r2, c2, 1.0, 0.0, 0.5, None, w2)
    assert torch.equal(x1, x2)


def test_subset_argument_errors():
    wl = W.tiny_workload(W.BEAM_FAN2D, (1, 12, 12), (20, 1), 8, 63)
    g = rdp.Geometry.from_workload(wl)
    U, V = wl.det_shape
    c = torch.empty(wl.vol_shape, device="cuda")
    for vb, ve in [(3, 3), (-1, 2), (6, 9)]:
        r = torch.empty((max(ve - vb, 1), U, V), device="cuda")
        with pytest.raises((rdp.CtError, ValueError)):
            rdp.ct_sirt_weights_views(g, vb, ve, r, c)
    r = torch.empty((2, U, V), device="cuda")
    x = torch.zeros(wl.vol_shape, device="cuda")
    with pytest.raises(rdp.CtError) as e:
        rdp.ct_sirt_step_views(g, 0, 2, x, r, r.clone(), c, 1.0, 1.0, 0.0, None, r.clone())
    assert e.value.status == rdp.CT_E_ARG   # lo > hi
    with pytest.raises(rdp.CtError) as e:
        rdp.ct_sirt_step_views(g, 0, 2, x, r, r.clone(), c, 1.0, -np.inf, np.inf, None, r)
    assert e.value.status == rdp.CT_E_ALIAS  # work aliases y
