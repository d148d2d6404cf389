"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Bar (float32 arithmetic): relative L2 error ||g - o|| / ||o|| <= 1e-5 per
sinogram / volume / SIRT iterate, and the adjoint identity
|<Ax, y> - <x, A^T y>| / |<Ax, y>| <= 1e-5 on the GPU.  Full-size 512^3 cases
compare sampled rays (computed one by one by the oracle), the adjoint of
sparse sinograms (whose exact result the oracle computes in full), per-voxel
column sums and the adjoint identity.
"""
import math

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
    n = np.linalg.norm(o)
    return float(np.linalg.norm(g - o) / (n if n > 0 else 1.0))


def say(*a):
    print(*a, flush=True)


class Pair:
    """The same workload on both sides."""

    def __init__(self, wl):
        self.wl = wl
        self.og = oracle.Geometry.from_workload(wl)
        self.g = rdp.Geometry.from_workload(wl)

    def A_dev(self, x):
        out = torch.empty(self.g.sino_shape, device="cuda", dtype=torch.float32)
        rdp.ct_project(self.g, dev(x), out)
        return out

    def A(self, x):
        return host(self.A_dev(x))

    def AT(self, y, atomic=False):
        out = torch.empty(self.g.vol_shape, device="cuda", dtype=torch.float32)
        (rdp.ct_backproject_atomic if atomic else rdp.ct_backproject)(self.g, dev(y), out)
        return host(out)


def _tiny(beam, seed, vol, det, views, **kw):
    if beam in (W.BEAM_PARALLEL2D, W.BEAM_FAN2D):
        vol = (1, vol[1], vol[2])
        det = (det[0], 1)
    return W.tiny_workload(beam, vol, det, views, seed, **kw)


ALL_BEAMS = [W.BEAM_PARALLEL2D, W.BEAM_FAN2D, W.BEAM_CONE, W.BEAM_PARALLEL3D]


@pytest.mark.parametrize("beam", ALL_BEAMS)
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_tiny_grids_match_brute_force(beam, seed):
    wl = _tiny(beam, 40 + 7 * seed + beam, vol=(7, 9, 11), det=(13, 7), views=6,
               voxel_spacing=(1.1, 0.9, 1.0), det_spacing=(1.05, 0.95),
               jitter=0.3 if beam >= 2 else 0.0)
    say("tiny", W.BEAM_NAMES[beam], seed)
    p = Pair(wl)
    Am = oracle.brute_matrix(p.og)
    rng = np.random.default_rng(seed)
    x = rng.uniform(0, 1, wl.vol_shape).astype(np.float32)
    y = rng.uniform(0, 1, wl.sino_shape).astype(np.float32)
    ref_f = Am @ x.astype(np.float64).ravel()
    ref_b = Am.T @ y.astype(np.float64).ravel()
    gf = p.A(x)
    assert rel_l2(gf, ref_f) <= TOL
    assert np.max(np.abs(gf.ravel() - ref_f)) <= 1e-5 * max(1.0, np.abs(ref_f).max())
    for atomic in (False, True):
        gb = p.AT(y, atomic)
        assert rel_l2(gb, ref_b) <= TOL, atomic
        assert np.max(np.abs(gb.ravel() - ref_b)) <= 1e-5 * max(1.0, np.abs(ref_b).max())


@pytest.mark.parametrize("beam", [W.BEAM_CONE, W.BEAM_PARALLEL3D])
def test_adjoint_beyond_the_footprint_cache(beam):
    # 1100 views: more than the brick kernel keeps footprints for (1024), so
    # pass 2 recomputes them; the adjoint and the SIRT update still match
    wl = _tiny(beam, 77 + beam, vol=(9, 10, 11), det=(12, 9), views=1100,
               jitter=0.3 if beam == W.BEAM_CONE else 0.0)
    p = Pair(wl)
    rng = np.random.default_rng(8)
    y = rng.uniform(0, 1, wl.sino_shape).astype(np.float32)
    e = rel_l2(p.AT(y), oracle.backproject(p.og, y))
    say(f"{W.BEAM_NAMES[beam]} with 1100 views: A^T rel_l2 {e:.2e}")
    assert e <= TOL


@pytest.mark.parametrize("beam", [W.BEAM_CONE, W.BEAM_PARALLEL3D, W.BEAM_FAN2D])
def test_several_tiles_with_ragged_tails(beam):
    # volume not a multiple of the 16^3 (2D: 64^2) bricks, detector not a
    # multiple of the 16 x 16 (2D: 256) ray tiles
    vol = (37, 45, 41) if beam >= 2 else (1, 150, 133)
    det = (53, 35) if beam >= 2 else (301, 1)
    wl = W.tiny_workload(beam, vol, det, 17, 900 + beam, sid=80.0, sdd=140.0, jitter=0.2,
                         det_spacing=(1.1, 1.2))
    say("ragged", W.BEAM_NAMES[beam])
    p = Pair(wl)
    rng = np.random.default_rng(5)
    x = rng.uniform(0, 1, wl.vol_shape).astype(np.float32)
    y = rng.uniform(0, 1, wl.sino_shape).astype(np.float32)
    assert rel_l2(p.A(x), oracle.project(p.og, x)) <= TOL
    ob = oracle.backproject(p.og, y)
    assert rel_l2(p.AT(y), ob) <= TOL
    assert rel_l2(p.AT(y, atomic=True), ob) <= TOL


_FULL = {}


def full_pair(config):
    if config not in _FULL:
        wl = W.make_workload(config)
        _FULL[config] = (Pair(wl), W.make_phantom(wl))
    return _FULL[config]


@pytest.mark.parametrize("config", [1, 2, 3])
def test_small_configs_full_parity(config):
    say("config", config)
    p, phantom = full_pair(config)
    ref, nnz, ties = oracle.project(p.og, phantom, with_counts=True)
    g = p.A(phantom)
    e = rel_l2(g, ref)
    say(f"C{config} A rel_l2 = {e:.3e}")
    assert e <= TOL
    ob = oracle.backproject(p.og, ref.astype(np.float32))
    for atomic in (False, True):
        gb = p.AT(ref.astype(np.float32), atomic)
        eb = rel_l2(gb, ob)
        say(f"C{config} AT({'atomic' if atomic else 'brick'}) rel_l2 = {eb:.3e}")
        assert eb <= TOL
    cnt = rdp.ct_count_intersections(p.g)
    say(f"C{config} nnz oracle {nnz} gpu {cnt} ties {ties}")
    # equal up to cells of zero length at exact plane-crossing ties
    assert nnz <= cnt <= nnz + 2 * ties


@pytest.mark.parametrize("config", [1, 2, 3, 4, 5])
def test_gpu_adjoint_identity(config):
    say("adjoint identity", config)
    p, _ = full_pair(config) if config <= 3 else (Pair(W.make_workload(config)), None)
    x, y = W.adjoint_vectors(p.wl)
    ax = p.A(x)
    aty = p.AT(y)
    lhs = float(np.dot(ax.ravel(), y.astype(np.float64).ravel()))
    rhs = float(np.dot(x.astype(np.float64).ravel(), aty.ravel()))
    say(f"C{config} <Ax,y>={lhs:.10e} <x,ATy>={rhs:.10e} rel={abs(lhs - rhs) / abs(lhs):.2e}")
    assert abs(lhs - rhs) <= TOL * abs(lhs)


def test_sirt_c2_ten_iterations():
    p, phantom = full_pair(2)
    y = oracle.project(p.og, phantom).astype(np.float32)
    R, C = oracle.sirt_weights(p.og)
    xo = oracle.sirt(p.og, y, n_iter=10, relax=1.0, weights=(R, C))
    g = p.g
    rinv = torch.empty(g.sino_shape, device="cuda")
    cinv = torch.empty(g.vol_shape, device="cuda")
    rdp.ct_sirt_weights(g, rinv, cinv)
    assert rel_l2(host(rinv), R) <= TOL
    assert rel_l2(host(cinv), C) <= TOL
    x = torch.zeros(g.vol_shape, device="cuda")
    yd = dev(y)
    work = torch.empty(g.sino_shape, device="cuda")
    for _ in range(10):
        rdp.ct_sirt_step(g, x, yd, rinv, cinv, 1.0, work)
    e = rel_l2(host(x), xo)
    say(f"C2 SIRT x10 rel_l2 = {e:.3e}")
    assert e <= TOL


def test_bounded_masked_sirt_c2_ten_iterations():
    """Box constraints and a reconstruction mask (a disc, so whole corner bricks
    are skipped), with bounds that are active on both sides."""
    p, phantom = full_pair(2)
    y = oracle.project(p.og, phantom).astype(np.float32)
    R, C = oracle.sirt_weights(p.og)
    _, H, Wd = p.wl.vol_shape
    yy, xx = np.mgrid[0:H, 0:Wd]
    mask = (((yy + 0.5 - H / 2) ** 2 + (xx + 0.5 - Wd / 2) ** 2) < 200.0 ** 2).astype(np.uint8)
    mask = mask.reshape(p.wl.vol_shape)
    x0 = np.full(p.wl.vol_shape, 0.05, np.float32)
    lo, hi = 0.02, 0.6
    xo = oracle.sirt(p.og, y, x0=x0, n_iter=10, relax=1.0, weights=(R, C), lo=lo, hi=hi, mask=mask)
    assert np.any(xo[mask != 0] == lo) and np.any(xo[mask != 0] == hi)
    g = p.g
    rinv = torch.empty(g.sino_shape, device="cuda")
    cinv = torch.empty(g.vol_shape, device="cuda")
    rdp.ct_sirt_weights(g, rinv, cinv)
    x = dev(x0)
    yd, md = dev(y), torch.from_numpy(mask).cuda()
    work = torch.empty(g.sino_shape, device="cuda")
    for _ in range(10):
        rdp.ct_sirt_step_bounded(g, x, yd, rinv, cinv, 1.0, lo, hi, md, work)
    xg = host(x)
    assert np.array_equal(xg[mask == 0], x0[mask == 0].astype(np.float64))
    e = rel_l2(xg, xo)
    say(f"C2 bounded masked SIRT x10 rel_l2 = {e:.3e}")
    assert e <= TOL
    # no bounds, no mask: the same bits as the plain step
    xa, xb = dev(x0), dev(x0)
    rdp.ct_sirt_step(g, xa, yd, rinv, cinv, 1.0, work)
    rdp.ct_sirt_step_bounded(g, xb, yd, rinv, cinv, 1.0, -math.inf, math.inf, None, work)
    assert torch.equal(xa, xb)
    with pytest.raises(rdp.CtError) as ei:
        rdp.ct_sirt_step_bounded(g, x, yd, rinv, cinv, 1.0, 1.0, 0.0, md, work)
    assert ei.value.status == rdp.CT_E_ARG


def _sample_rays(wl, n, seed):
    rng = np.random.default_rng(seed)
    return np.unique(rng.integers(0, wl.n_rays, n)).astype(np.int64)


@pytest.mark.parametrize("config", [4, 5])
def test_full_size_forward_sampled_rays(config):
    say("full-size forward", config)
    wl = W.make_workload(config)
    p = Pair(wl)
    phantom = W.make_phantom(wl)
    ids = _sample_rays(wl, 4000, config)
    g = host(p.A_dev(phantom).view(-1)[torch.from_numpy(ids).cuda()])
    ref, cnt = oracle.project_rays(p.og, phantom, ids, with_counts=True)
    e = rel_l2(g, ref)
    say(f"C{config} A sampled rel_l2 = {e:.3e} over {len(ids)} rays")
    assert e <= TOL
    per = torch.zeros(wl.sino_shape, device="cuda", dtype=torch.int32)
    total = rdp.ct_count_intersections(p.g, per)
    pc = per.view(-1)[torch.from_numpy(ids).cuda()].cpu().numpy()
    assert np.array_equal(pc.astype(np.int64), cnt)
    say(f"C{config} nnz (gpu count) = {total}")


def _rays_through_points(wl, pts, views):
    """Flat ids of the 3x3 pixels around where the ray through each point lands,
    from the frames by the pixel-centre formula (independent of both sides)."""
    U, V = wl.det_shape
    du, dv = wl.det_spacing
    ids = []
    for k in views:
        a, c, eu, ev = (wl.frames[k, i:i + 3] for i in (0, 3, 6, 9))
        n = np.cross(eu, ev)
        for p in pts:
            if wl.beam == W.BEAM_CONE:
                t = np.dot(c - a, n) / np.dot(p - a, n)
                hitp = a + t * (p - a)
            else:
                hitp = p - np.dot(p - c, n) / np.dot(a, n) * a
            u = np.dot(hitp - c, eu) / du + (U - 1) / 2
            v = np.dot(hitp - c, ev) / dv + (V - 1) / 2
            for uu in range(int(round(u)) - 1, int(round(u)) + 2):
                for vv in range(int(round(v)) - 1, int(round(v)) + 2):
                    if 0 <= uu < U and 0 <= vv < V:
                        ids.append((k * U + uu) * V + vv)
    return np.unique(np.array(ids, dtype=np.int64))


@pytest.mark.parametrize("config", [4, 5])
def test_full_size_forward_sparse_volume(config):
    """A few isolated bright voxels: each ray value is then one or two single
    chord lengths, so every piece length is checked, not an average."""
    say("full-size forward sparse volume", config)
    wl = W.make_workload(config)
    p = Pair(wl)
    rng = np.random.default_rng(50 + config)
    D, H, Wd = wl.vol_shape
    vol = np.zeros(wl.vol_shape, np.float32)
    cells = [(int(rng.integers(40, D - 40)), int(rng.integers(40, H - 40)), int(rng.integers(40, Wd - 40)))
             for _ in range(12)]
    pts = []
    for z, y, x in cells:
        vol[z, y, x] = 1.0
        pts.append(np.array([x + 0.5 - Wd / 2, y + 0.5 - H / 2, z + 0.5 - D / 2]))
    views = rng.choice(wl.n_views, 24, replace=False)
    ids = _rays_through_points(wl, pts, views)
    g = host(p.A_dev(vol).view(-1)[torch.from_numpy(ids).cuda()])
    ref = oracle.project_rays(p.og, vol, ids)
    assert np.count_nonzero(ref) > 100
    e = rel_l2(g, ref)
    say(f"C{config} A sparse-volume rel_l2 = {e:.3e} over {len(ids)} rays "
        f"(max abs err {np.abs(g - ref).max():.2e})")
    assert e <= TOL


@pytest.mark.parametrize("config", [4, 5])
def test_full_size_adjoint_sparse_sinogram(config):
    say("full-size adjoint sparse", config)
    wl = W.make_workload(config)
    p = Pair(wl)
    ids = _sample_rays(wl, 3000, 100 + config)
    y = np.zeros(wl.n_rays, dtype=np.float32)
    y[ids] = np.random.default_rng(config).uniform(0.5, 1.5, len(ids)).astype(np.float32)
    y = y.reshape(wl.sino_shape)
    ob = oracle.backproject(p.og, y)
    for atomic in (False, True):
        gb = p.AT(y, atomic)
        e = rel_l2(gb, ob)
        say(f"C{config} AT sparse ({'atomic' if atomic else 'brick'}) rel_l2 = {e:.3e}")
        assert e <= TOL


@pytest.mark.parametrize("config", [4, 5])
def test_full_size_adjoint_sampled_columns(config):
    say("full-size adjoint columns", config)
    wl = W.make_workload(config)
    p = Pair(wl)
    _, y = W.adjoint_vectors(wl)
    gb = p.AT(y).ravel()
    rng = np.random.default_rng(7 + config)
    D, H, Wd = wl.vol_shape
    js = []
    for _ in range(3):
        z, yy, x = (int(rng.integers(D // 4, 3 * D // 4)), int(rng.integers(H // 4, 3 * H // 4)),
                    int(rng.integers(Wd // 4, 3 * Wd // 4)))
        js.append((z * H + yy) * Wd + x)
    ref = np.array([oracle.column_dot(p.og, j, y) for j in js])
    got = gb[js]
    say(f"C{config} columns gpu {got} oracle {ref}")
    assert rel_l2(got, ref) <= TOL


def test_sirt_step_c4_matches_composition():
    """One SIRT iteration at 512^3 from x0 = 0 with a sparse measurement: the
    exact iterate is C * A^T (R * y).  R on the sampled rays and C on sampled
    voxels come from the oracle's chords and column sums; A^T of the sparse
    weighted residual from the oracle in full.  The plain step and the bounded,
    masked step are both checked."""
    wl = W.make_workload(4)
    p = Pair(wl)
    g = p.g
    rinv = torch.empty(g.sino_shape, device="cuda")
    cinv = torch.empty(g.vol_shape, device="cuda")
    rdp.ct_sirt_weights(g, rinv, cinv)
    ids = _sample_rays(wl, 2000, 44)
    ones = np.ones(wl.vol_shape)
    rs = oracle.project_rays(p.og, ones, ids)
    R_s = np.where(rs > 0, 1 / np.where(rs > 0, rs, 1), 0)
    assert rel_l2(host(rinv).ravel()[ids], R_s) <= TOL
    y = np.zeros(wl.n_rays, dtype=np.float32)
    y[ids] = 1.0 + (np.arange(len(ids)) % 7).astype(np.float32)
    y = y.reshape(wl.sino_shape)
    e_ref = np.zeros(wl.n_rays)
    e_ref[ids] = R_s * y.ravel()[ids]
    bt = oracle.backproject(p.og, e_ref.reshape(wl.sino_shape)).ravel()
    support = np.flatnonzero(bt > 0)
    rng = np.random.default_rng(3)
    js = [int(j) for j in rng.choice(support, 4, replace=False)]
    cs = np.array([oracle.column_dot(p.og, j, np.ones(wl.sino_shape)) for j in js])
    x_ref = bt[js] / cs
    assert rel_l2(host(cinv).ravel()[js], 1 / cs) <= TOL
    work = torch.empty(g.sino_shape, device="cuda")
    x = torch.zeros(g.vol_shape, device="cuda")
    rdp.ct_sirt_step(g, x, dev(y), rinv, cinv, 1.0, work)
    xg = host(x).ravel()
    say(f"C4 SIRT step sampled voxels gpu {xg[js]} oracle {x_ref}")
    assert rel_l2(xg[js], x_ref) <= TOL
    # voxels that no measured ray crosses with positive length stay (nearly) 0:
    # a ray grazing a voxel edge may leave a piece of rounding length there
    assert np.abs(xg[bt == 0]).max() <= 1e-5 * np.abs(xg).max()
    # bounded and masked: the mask keeps two of the four sampled voxels, the
    # upper bound cuts the larger of them
    mask = np.zeros(wl.n_voxels, np.uint8)
    keep = sorted(js, key=lambda j: x_ref[js.index(j)])[2:]
    mask[keep] = 1
    mask[support[: len(support) // 2]] = 1
    hi = float(np.mean([x_ref[js.index(j)] for j in keep]))
    xb = torch.zeros(g.vol_shape, device="cuda")
    rdp.ct_sirt_step_bounded(g, xb, dev(y), rinv, cinv, 1.0, 0.0, hi,
                             torch.from_numpy(mask.reshape(wl.vol_shape)).cuda(), work)
    xbg = host(xb).ravel()
    exp = np.array([min(x_ref[k], hi) if mask[j] else 0.0 for k, j in enumerate(js)])
    say(f"C4 bounded masked step gpu {xbg[js]} expected {exp}")
    assert rel_l2(xbg[js], exp) <= TOL
    assert not np.any(xbg[mask == 0])

# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("beam", [W.BEAM_CONE, W.BEAM_PARALLEL3D, W.BEAM_FAN2D])
def test_zero_gradient_at_the_calibrated_point(beam):
    # The gradient of 1/2 ||A x - y||^2 is A^T (A x - y) (diffct docs,
    # "Differentiable analytical reconstruction"); at y = A x it vanishes.  The
    # forward is deterministic, so on the GPU the residual is exactly zero, and
    # a SIRT step (and CGLS's r = y - A x) leave the calibrated x unchanged.
    wl = _tiny(beam, 91 + beam, vol=(12, 13, 14), det=(17, 15), views=24,
               jitter=0.3 if beam >= 2 else 0.0)
    p = Pair(wl)
    x = dev(np.random.default_rng(12).uniform(0, 1, wl.vol_shape))
    y = torch.empty(p.g.sino_shape, device="cuda")
    rdp.ct_project(p.g, x, y)
    work = torch.empty(p.g.sino_shape, device="cuda")
    ones = torch.ones(p.g.sino_shape, device="cuda")
    rdp.ct_sirt_residual(p.g, x, y, ones, work)
    assert torch.count_nonzero(work).item() == 0
    r, c = torch.empty(p.g.sino_shape, device="cuda"), torch.empty(p.g.vol_shape, device="cuda")
    rdp.ct_sirt_weights(p.g, r, c)
    x2 = x.clone()
    rdp.ct_sirt_step(p.g, x2, y, r, c, 1.0, work)
    assert torch.equal(x2, x)
    g = torch.empty(p.g.vol_shape, device="cuda")
    rdp.ct_backproject(p.g, work, g)
    assert torch.count_nonzero(g).item() == 0


def test_all_rays_miss():
    wl = W.tiny_workload(W.BEAM_PARALLEL3D, (8, 8, 8), (6, 5), 4, 3)
    wl.frames[:, 3:6] += np.array([500.0, 0, 0])  # detector far to the side, rays along ~z
    p = Pair(wl)
    x = np.ones(wl.vol_shape, np.float32)
    s = torch.full(p.g.sino_shape, 7.0, device="cuda")
    rdp.ct_project(p.g, dev(x), s)
    assert float(s.abs().max()) == 0.0
    v = torch.full(p.g.vol_shape, 7.0, device="cuda")
    rdp.ct_backproject(p.g, dev(np.ones(wl.sino_shape)), v)
    assert float(v.abs().max()) == 0.0
    assert rdp.ct_count_intersections(p.g) == 0


def test_rays_on_lattice_planes_follow_half_open_cells():
    # odd detector of unit pitch: untilted parallel3d rays lie exactly on planes
    fr = W.dual_axis_parallel3d(3, -10.0, 10.0)
    wl = W.Workload("planes", W.BEAM_PARALLEL3D, (6, 7, 8), (1, 1, 1), (9, 9), (1.0, 1.0), fr)
    p = Pair(wl)
    rng = np.random.default_rng(2)
    x = rng.uniform(0, 1, wl.vol_shape).astype(np.float32)
    y = rng.uniform(0, 1, wl.sino_shape).astype(np.float32)
    assert rel_l2(p.A(x), oracle.project(p.og, x)) <= TOL
    ob = oracle.backproject(p.og, y)
    assert rel_l2(p.AT(y), ob) <= TOL
    assert rel_l2(p.AT(y, atomic=True), ob) <= TOL


@pytest.mark.parametrize("beam", [W.BEAM_FAN2D, W.BEAM_CONE])
@pytest.mark.parametrize("n", [23, 24])
def test_fan_cone_rays_with_zero_direction_components(beam, n):
    # four views exactly along the axes (frames rounded, so cos and sin are 0 or
    # +-1) and an odd, centred detector: the central rays have direction
    # components that are exactly zero.  Footprints that straddle an axis plane
    # take the per-ray sign handling and the near-zero clip, the others the
    # footprint-wide mirroring; an even volume puts the central rays on lattice
    # planes (half-open cells).
    if beam == W.BEAM_CONE:
        fr = np.round(W.helix_cone(4, 40.0, 70.0, 0.0), 12)
        vol, det = (n, n, n), (31, 29)
    else:
        fr = np.round(W.circular_fan2d(4, 40.0, 70.0), 12)
        vol, det = (1, n, n), (31, 1)
    assert np.all((fr == 0.0) | (np.abs(fr) >= 1.0))
    wl = W.Workload(f"axis views {n}", beam, vol, (1.0, 1.0, 1.0), det, (1.0, 1.0), fr)
    say("axis views", W.BEAM_NAMES[beam], n)
    p = Pair(wl)
    rng = np.random.default_rng(11 + n)
    x = rng.uniform(0, 1, wl.vol_shape).astype(np.float32)
    y = rng.uniform(0, 1, wl.sino_shape).astype(np.float32)
    assert rel_l2(p.A(x), oracle.project(p.og, x)) <= TOL
    ob = oracle.backproject(p.og, y)
    assert rel_l2(p.AT(y), ob) <= TOL
    assert rel_l2(p.AT(y, atomic=True), ob) <= TOL


@pytest.mark.parametrize("where", ["source_inside", "detector_inside"])
def test_cone_segment_ends_inside_volume(where):
    fr = W.helix_cone(9, 30.0, 50.0, 0.0)
    if where == "source_inside":
        fr[:, 0:3] *= 0.1     # sources inside the 24^3 box
    else:
        fr[:, 3:6] *= 0.2     # detector centres inside the box
    wl = W.Workload(where, W.BEAM_CONE, (24, 24, 24), (1, 1, 1), (20, 18), (1.3, 1.3), fr)
    p = Pair(wl)
    rng = np.random.default_rng(9)
    x = rng.uniform(0, 1, wl.vol_shape).astype(np.float32)
    y = rng.uniform(0, 1, wl.sino_shape).astype(np.float32)
    assert rel_l2(p.A(x), oracle.project(p.og, x)) <= TOL
    ob = oracle.backproject(p.og, y)
    assert rel_l2(p.AT(y), ob) <= TOL
    assert rel_l2(p.AT(y, atomic=True), ob) <= TOL


def test_alias_and_shape_errors_are_reported():
    wl = W.make_workload(1)
    g = rdp.Geometry.from_workload(wl)
    buf = torch.zeros(max(wl.n_rays, wl.n_voxels) + 8, device="cuda")
    vol = buf[: wl.n_voxels].view(wl.vol_shape)
    sino = buf[8: 8 + wl.n_rays].view(wl.sino_shape)
    with pytest.raises(rdp.CtError) as ei:
        rdp.ct_project(g, vol, sino)
    assert ei.value.status == rdp.CT_E_ALIAS
    with pytest.raises(rdp.CtError) as ei:
        rdp.ct_backproject(g, sino, vol)
    assert ei.value.status == rdp.CT_E_ALIAS
    with pytest.raises(ValueError):
        rdp.ct_project(g, torch.zeros(3, device="cuda"), torch.zeros(wl.sino_shape, device="cuda"))


def test_outputs_are_overwritten_not_accumulated():
    p, phantom = full_pair(3)
    y = oracle.project(p.og, phantom).astype(np.float32)
    yd = dev(y)
    for fn in (rdp.ct_backproject, rdp.ct_backproject_atomic):
        a = torch.full(p.g.vol_shape, 123.0, device="cuda")
        b = torch.full(p.g.vol_shape, -5.0, device="cuda")
        fn(p.g, yd, a)
        fn(p.g, yd, b)
        if fn is rdp.ct_backproject:
            # integer on-chip sums: the same bits whatever the order of the adds
            assert torch.equal(a, b)
        else:
            # equal up to the float32 order of the atomic adds
            assert rel_l2(host(a), host(b)) <= 1e-6
    s1 = torch.full(p.g.sino_shape, 9.0, device="cuda")
    s2 = torch.full(p.g.sino_shape, -9.0, device="cuda")
    rdp.ct_project(p.g, dev(phantom), s1)
    rdp.ct_project(p.g, dev(phantom), s2)
    assert torch.equal(s1, s2)
