"""The allocation-free CGLS step (ct_cgls_step_noalloc) against ct_cgls_step.

Both run the same kernels; the only difference is where the per-block partial
sums live (the library's static device scratch instead of the caller's
workspace), so from the same state they must give the same bits.  Two calls
in a row on different geometries, the second with fewer blocks than the
first, show that the shared scratch carries nothing over between calls.
"""
import ctypes

import numpy as np
import pytest

import ray_driven_projector_amd as rdp
from ray_driven_projector_amd import workloads as W

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _state(g, y):
    """A started CGLS state: (x, r, s, p, q, workspace) after ct_cgls_init."""
    x = torch.zeros(g.vol_shape, device="cuda")
    r = torch.empty(g.sino_shape, device="cuda")
    s = torch.empty(g.vol_shape, device="cuda")
    p = torch.empty(g.vol_shape, device="cuda")
    q = torch.empty(g.sino_shape, device="cuda")
    wk = torch.empty(rdp.ct_cgls_workspace_size(g), dtype=torch.uint8, device="cuda")
    rdp.ct_cgls_init(g, dev(y), x, r, s, p, wk)
    return x, r, s, p, q, wk


def _compare(wl, steps):
    g = rdp.Geometry.from_workload(wl)
    y = W.Stream(99).uniform(wl.n_rays, 0.0, 1.0).reshape(wl.sino_shape).astype(np.float32)
    a = _state(g, y)
    b = _state(g, y)
    for _ in range(steps):
        rdp.ct_cgls_step(g, *a)
        rdp.ct_cgls_step_noalloc(g, *b[:5], b[5])
        torch.cuda.synchronize()
        for name, ta, tb in zip("xrspq", a[:5], b[:5]):
            assert torch.equal(ta, tb), name
        sa, sb = rdp.ct_cgls_scalars(g, a[5]), rdp.ct_cgls_scalars(g, b[5])
        assert sa == sb, (sa, sb)
    return g


def test_noalloc_step_matches_the_workspace_step_on_two_geometries():
    # first the larger geometry (more forward blocks), then a smaller one
    big = W.tiny_workload(W.BEAM_CONE, (40, 44, 48), (256, 192), 120, 5, sid=150.0, sdd=240.0, jitter=0.3)
    small = W.tiny_workload(W.BEAM_PARALLEL3D, (9, 12, 10), (14, 11), 8, 6)
    gb = _compare(big, 2)
    gs = _compare(small, 2)
    assert rdp.ct_cgls_workspace_size(gs) < rdp.ct_cgls_workspace_size(gb)


def test_noalloc_step_rejects_geometries_beyond_the_scratch():
    # cone views (one ray per lane, no packets) on a 2048 x 2048 detector with 257
    # views: 128 x 128 x 257 > 2^22 forward blocks
    fr = W.helix_cone(257, 40.0, 80.0)
    g = rdp.Geometry(W.BEAM_CONE, (8, 8, 8), (1.0, 1.0, 1.0), (2048, 2048), (0.01, 0.01), fr)
    assert rdp.ct_cgls_workspace_size(g) // 8 - 32 > 2 ** 22
    # the check comes before any launch: far-apart stand-in addresses never read
    base = 1 << 46
    ptrs = [ctypes.c_void_p(base + k * (1 << 34)) for k in range(6)]
    st = rdp.lib().ct_cgls_step_noalloc(g.handle, *ptrs, None)
    assert st == rdp.CT_E_RANGE
    assert "static scratch" in rdp.last_error()
