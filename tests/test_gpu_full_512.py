"""Whole-output parity at 512^3: every ray of the sinogram and every voxel of
the volume against the float64 oracle, in the launch shapes the benchmark
times.

- Dual-axis parallel3d (512^3, 280 views of 512 x 512): A of the phantom,
  the row and column weights, A^T of a dense sinogram (both adjoints), and one
  whole SIRT iteration from a nonzero start, x0 = phantom / 2, so the fused
  residual gathers a full volume.  The oracle's A x0 is exactly half its A of
  the phantom (a power-of-two scale commutes with every float64 rounding).
- Jittered circular cone at one GPU's share of the views (the first 90 of
  720, full 512^3 volume and 1024 x 768 detector): A of the phantom and A^T of
  that sinogram.

Bar: relative L2 <= 1e-5 per sinogram / volume, as everywhere.  The oracle
results are computed once per module (minutes of host time on a many-core
box); each test computes only what it needs first, so progress shows test by
test.
"""
import json
import os

import numpy as np
import pytest

import oracle
import ray_driven_projector_amd as rdp
from ray_driven_projector_amd import workloads as W

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]
TOL = 1e-5
torch = pytest.importorskip("torch")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nnz_configs.json")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host(t):
    return t.detach().cpu().numpy().astype(np.float64)


def rel_l2(g, o):
    g = np.asarray(g, np.float64).ravel()
    o = np.asarray(o, np.float64).ravel()
    n = np.linalg.norm(o)
    return float(np.linalg.norm(g - o) / (n if n > 0 else 1.0))


def say(*a):
    print(*a, flush=True)


class Case:
    """One workload on both sides, with the oracle's results cached on demand."""

    def __init__(self, wl):
        self.wl = wl
        self.og = oracle.Geometry.from_workload(wl)
        self.g = rdp.Geometry.from_workload(wl)
        self.phantom = W.make_phantom(wl)
        self._memo = {}

    def memo(self, key, fn):
        if key not in self._memo:
            self._memo[key] = fn()
        return self._memo[key]

    def y64(self):
        """Oracle A of the phantom, with its intersection count."""
        return self.memo("y64", lambda: oracle.project(self.og, self.phantom, with_counts=True))

    def empty_sino(self):
        return torch.empty(self.g.sino_shape, device="cuda", dtype=torch.float32)

    def empty_vol(self):
        return torch.empty(self.g.vol_shape, device="cuda", dtype=torch.float32)


@pytest.fixture(scope="module")
def c4():
    return Case(W.make_workload(4))


@pytest.fixture(scope="module")
def c5share():
    return Case(W.make_workload(5).subset_views(np.arange(90)))


# ---------------------------------------------------------------------------
# dual-axis parallel3d
# ---------------------------------------------------------------------------

def test_c4_forward_whole_sinogram(c4):
    y64, nnz, ties = c4.y64()
    out = c4.empty_sino()
    rdp.ct_project(c4.g, dev(c4.phantom), out)
    e = rel_l2(host(out), y64)
    say(f"C4 A whole sinogram rel_l2 = {e:.3e} ({y64.size} rays)")
    assert e <= TOL
    # the GPU's count against the oracle's (no exact ties on this workload)
    assert ties == 0
    assert rdp.ct_count_intersections(c4.g) == nnz
    with open(GOLDEN) as f:
        assert json.load(f)["c4"]["nnz"] == nnz


def _c4_weights(c4):
    def make():
        rs = oracle.row_chords(c4.og)
        cs = oracle.backproject(c4.og, np.ones(c4.wl.sino_shape))
        R = np.where(rs > 0, 1.0 / np.where(rs > 0, rs, 1.0), 0.0)
        C = np.where(cs > 0, 1.0 / np.where(cs > 0, cs, 1.0), 0.0)
        return R, C
    return c4.memo("weights", make)


def test_c4_sirt_weights_whole(c4):
    R, C = _c4_weights(c4)
    rinv, cinv = c4.empty_sino(), c4.empty_vol()
    rdp.ct_sirt_weights(c4.g, rinv, cinv)
    er, ec = rel_l2(host(rinv), R), rel_l2(host(cinv), C)
    say(f"C4 row weights rel_l2 = {er:.3e}, column weights rel_l2 = {ec:.3e}")
    assert er <= TOL and ec <= TOL


def _c4_residual(c4):
    """x0 = phantom / 2 (exact in float32), e = R (y - A x0) with y the oracle's
    A of the phantom rounded to float32; the oracle's A x0 = y64 / 2 exactly."""
    def make():
        y64, _, _ = c4.y64()
        R, _ = _c4_weights(c4)
        y32 = y64.astype(np.float32)
        e64 = R * (y32.astype(np.float64) - 0.5 * y64)
        return y32, e64
    return c4.memo("residual", make)


def _c4_adjoint_of_residual(c4):
    def make():
        _, e64 = _c4_residual(c4)
        e32 = e64.astype(np.float32)
        return e32, oracle.backproject(c4.og, e32)
    return c4.memo("bt", make)


def test_c4_adjoint_whole_volume(c4):
    e32, bt = _c4_adjoint_of_residual(c4)
    out = c4.empty_vol()
    for atomic in (False, True):
        (rdp.ct_backproject_atomic if atomic else rdp.ct_backproject)(c4.g, dev(e32), out)
        e = rel_l2(host(out), bt)
        say(f"C4 A^T ({'atomic' if atomic else 'brick'}) whole volume rel_l2 = {e:.3e}")
        assert e <= TOL


def test_c4_sirt_iteration_whole_volume(c4):
    y32, e64 = _c4_residual(c4)
    _, bt = _c4_adjoint_of_residual(c4)
    _, C = _c4_weights(c4)
    x0 = (0.5 * c4.phantom).astype(np.float32)
    x1 = x0.astype(np.float64) + C * bt
    rinv, cinv = c4.empty_sino(), c4.empty_vol()
    rdp.ct_sirt_weights(c4.g, rinv, cinv)
    yd, work = dev(y32), c4.empty_sino()
    # the fused residual alone: the forward gather of a nonzero volume
    rdp.ct_sirt_residual(c4.g, dev(x0), yd, rinv, work)
    er = rel_l2(host(work), e64)
    # the whole iteration
    x = dev(x0)
    rdp.ct_sirt_step(c4.g, x, yd, rinv, cinv, 1.0, work)
    ex = rel_l2(host(x), x1)
    # the update alone on the oracle's residual
    xu = dev(x0)
    rdp.ct_sirt_update(c4.g, dev(e64), cinv, 1.0, xu)
    eu = rel_l2(host(xu), x1)
    say(f"C4 SIRT from x0 = phantom/2: residual rel_l2 = {er:.3e}, iterate {ex:.3e}, update {eu:.3e}")
    assert er <= TOL and ex <= TOL and eu <= TOL
    # bounded and masked, against the same composition clipped and masked
    lo, hi = 0.05, 0.35
    rng = np.random.default_rng(12)
    mask = (rng.random(c4.wl.vol_shape) < 0.7).astype(np.uint8)
    xb = dev(x0)
    rdp.ct_sirt_step_bounded(c4.g, xb, yd, rinv, cinv, 1.0, lo, hi, torch.from_numpy(mask).cuda(), work)
    ref = np.where(mask != 0, np.clip(x1, lo, hi), x0.astype(np.float64))
    xbg = host(xb)
    eb = rel_l2(xbg, ref)
    say(f"C4 bounded masked SIRT iterate rel_l2 = {eb:.3e}")
    assert eb <= TOL
    assert np.array_equal(xbg[mask == 0], x0[mask == 0].astype(np.float64))


def test_c4_adjoint_identity_whole(c4):
    x, y = W.adjoint_vectors(c4.wl)
    ax, aty = c4.empty_sino(), c4.empty_vol()
    rdp.ct_project(c4.g, dev(x), ax)
    rdp.ct_backproject(c4.g, dev(y), aty)
    lhs = float(torch.sum(ax.double() * dev(y).double()))
    rhs = float(torch.sum(dev(x).double() * aty.double()))
    e = abs(lhs - rhs) / abs(lhs)
    say(f"C4 adjoint identity {e:.3e}")
    assert e <= TOL


# ---------------------------------------------------------------------------
# jittered cone, one GPU's share of the views
# ---------------------------------------------------------------------------

def test_c5_share_forward_whole_sinogram(c5share):
    y64, nnz, _ = c5share.y64()
    out = c5share.empty_sino()
    rdp.ct_project(c5share.g, dev(c5share.phantom), out)
    g = host(out)
    e = rel_l2(g, y64)
    say(f"C5 (views 0..89) A whole sinogram rel_l2 = {e:.3e} ({y64.size} rays, nnz {nnz})")
    assert e <= TOL
    total = rdp.ct_count_intersections(c5share.g)
    say(f"C5 share intersections: gpu {total}, oracle {nnz}")
    assert abs(total - nnz) <= 1e-6 * nnz        # exact ties aside


def test_c5_share_adjoint_whole_volume(c5share):
    y64, _, _ = c5share.y64()
    y32 = y64.astype(np.float32)
    ref = c5share.memo("bt", lambda: oracle.backproject(c5share.og, y32))
    out = c5share.empty_vol()
    for atomic in (False, True):
        (rdp.ct_backproject_atomic if atomic else rdp.ct_backproject)(c5share.g, dev(y32), out)
        e = rel_l2(host(out), ref)
        say(f"C5 (views 0..89) A^T ({'atomic' if atomic else 'brick'}) whole volume rel_l2 = {e:.3e}")
        assert e <= TOL
