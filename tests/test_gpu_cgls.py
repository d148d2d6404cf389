"""GPU CGLS through the C ABI against the float64 oracle CGLS.

The iterate after k steps and the step scalars are compared with the oracle
started from the same data.  Tolerance, derived from the arithmetic: CGLS
feeds each step's rounding into the next search direction, with an
amplification that depends on the problem's conditioning.  So the bar is the
oracle's own spread when every A and A^T application is perturbed within the
per-application parity bar (relative 1e-5: element-wise noise, or a scale
error per application): the largest deviation of the iterate (and of each
scalar) over the perturbed float64 runs, times 2, and never below 1e-5.  The GPU's own A and A^T stay well inside 1e-5, so a
correct GPU CGLS lands inside that spread.  At 512^3 one step is checked piece
by piece on sampled rays and voxels against the oracle and through identities
of the recurrence.
"""
import numpy as np
import pytest

import oracle
import ray_driven_projector_amd as rdp
from geom_checks import untraversed_plane_distance
from ray_driven_projector_amd import workloads as W

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host(t):
    return t.detach().cpu().numpy().astype(np.float64)


def rel(g, o):
    g = np.asarray(g, np.float64).ravel()
    o = np.asarray(o, np.float64).ravel()
    n = np.linalg.norm(o)
    return float(np.linalg.norm(g - o) / (n if n > 0 else 1.0))


def say(*a):
    print(*a, flush=True)


class GpuCgls:
    def __init__(self, wl, y, x0=None):
        self.g = g = rdp.Geometry.from_workload(wl)
        self.x = torch.zeros(g.vol_shape, device="cuda") if x0 is None else dev(x0)
        self.y = dev(y)
        self.r = torch.empty(g.sino_shape, device="cuda")
        self.q = torch.empty(g.sino_shape, device="cuda")
        self.s = torch.empty(g.vol_shape, device="cuda")
        self.p = torch.empty(g.vol_shape, device="cuda")
        self.work = torch.empty(rdp.ct_cgls_workspace_size(g), dtype=torch.uint8, device="cuda")
        rdp.ct_cgls_init(g, self.y, self.x, self.r, self.s, self.p, self.work)

    def step(self):
        rdp.ct_cgls_step(self.g, self.x, self.r, self.s, self.p, self.q, self.work)

    def scalars(self):
        return rdp.ct_cgls_scalars(self.g, self.work)


def _tiny(beam, seed):
    vol, det = (9, 11, 13), (15, 9)
    if beam in (W.BEAM_PARALLEL2D, W.BEAM_FAN2D):
        vol, det = (1, 23, 19), (31, 1)
    return W.tiny_workload(beam, vol, det, 8, seed, voxel_spacing=(1.1, 0.9, 1.0),
                           jitter=0.3 if beam >= 2 else 0.0)


SCALARS = ("alpha", "beta", "gamma", "qq", "rr")


def _perturbed_spread(og, y, x0, n_iter, ref_x, hist, seeds=(1, 2, 3), delta=1e-5):
    """Largest relative deviation of the float64 oracle CGLS (iterate, and each
    scalar per step) when every A / A^T output o is perturbed within the
    per-application bar: o * (1 + delta*N(0,1)) element by element (noise), or
    o * (1 + delta*N(0,1)) with one draw per application (a scale error, the
    kind that does not average out of the norms)."""
    P, B = oracle.project, oracle.backproject
    dx = 0.0
    ds = {k: np.zeros(n_iter) for k in SCALARS}
    for kind in ("noise", "scale"):
        for sd in seeds:
            rng = np.random.default_rng(sd)

            def pert(o):
                f = rng.standard_normal(o.shape) if kind == "noise" else rng.standard_normal()
                return o * (1 + delta * f)

            oracle.project = lambda g, v, nt=None, **kw: pert(P(g, v, nt, **kw))
            oracle.backproject = lambda g, v, nt=None: pert(B(g, v, nt))
            try:
                xp, hp = oracle.cgls(og, y, x0=x0, n_iter=n_iter)
            finally:
                oracle.project, oracle.backproject = P, B
            dx = max(dx, rel(xp, ref_x))
            for k in SCALARS:
                ds[k] = np.maximum(ds[k], np.abs(np.array(hp[k]) - np.array(hist[k])) /
                                   np.maximum(np.abs(np.array(hist[k])), 1e-300))
    return dx, ds


def _compare(wl, y, n_iter, x0=None, label="", seeds=(1, 2, 3)):
    og = oracle.Geometry.from_workload(wl)
    run = GpuCgls(wl, y, x0)
    sc0 = run.scalars()
    ref_x, hist = oracle.cgls(og, y, x0=x0, n_iter=n_iter)
    assert abs(sc0["gamma"] - hist["gamma0"]) <= 1e-5 * hist["gamma0"]
    assert abs(sc0["rr"] - hist["rr0"]) <= 1e-5 * hist["rr0"]
    dx, ds = _perturbed_spread(og, y, x0, n_iter, ref_x, hist, seeds)
    for k in range(1, n_iter + 1):
        run.step()
        sc = run.scalars()
        for name in SCALARS:
            o = hist[name][k - 1]
            tol = max(1e-5, 2 * ds[name][k - 1])
            assert abs(sc[name] - o) <= tol * abs(o) + 1e-30, (label, k, name, sc[name], o, tol)
    e = rel(host(run.x), ref_x)
    tol = max(1e-5, 2 * dx)
    say(f"{label} CGLS x_{n_iter} rel_l2 = {e:.3e} (bar {tol:.3e}: oracle spread {dx:.3e} "
        f"under 1e-5 operator noise)")
    assert e <= tol
    return run


@pytest.mark.parametrize("beam", [W.BEAM_PARALLEL2D, W.BEAM_FAN2D, W.BEAM_CONE, W.BEAM_PARALLEL3D])
def test_cgls_tiny_matches_oracle(beam):
    wl = _tiny(beam, 70 + beam)
    rng = np.random.default_rng(beam)
    y = rng.uniform(0, 1, wl.sino_shape).astype(np.float32)
    x0 = rng.uniform(0, 1, wl.vol_shape).astype(np.float32) if beam % 2 else None
    _compare(wl, y, 5, x0=x0, label=f"tiny {W.BEAM_NAMES[beam]}")


def test_cgls_c2_five_iterations():
    wl = W.make_workload(2)
    og = oracle.Geometry.from_workload(wl)
    y = oracle.project(og, W.make_phantom(wl)).astype(np.float32)
    _compare(wl, y, 5, label="C2")


def test_cgls_c2_ten_iterations_residual():
    """Beyond a handful of steps CGLS on this consistent 512^2 problem amplifies
    any rounding by about 100x per step (the float64 oracle perturbed by 1e-9
    moves x_10 by 6e-5), so no float32 run can track the float64 iterate there.
    What must hold: the residual norm decreases at every step, the recurrence
    residual stays the true residual, and the final residual is as small as
    the oracle's (within its own spread under float32-level perturbations)."""
    wl = W.make_workload(2)
    og = oracle.Geometry.from_workload(wl)
    y = oracle.project(og, W.make_phantom(wl)).astype(np.float32)
    _, hist = oracle.cgls(og, y, n_iter=10)
    run = GpuCgls(wl, y)
    rr = [run.scalars()["rr"]]
    for _ in range(10):
        run.step()
        rr.append(run.scalars()["rr"])
    say("C2 CGLS rr gpu", ["%.4e" % v for v in rr], "oracle rr_10 %.4e" % hist["rr"][-1])
    assert all(b <= a * (1 + 1e-6) for a, b in zip(rr, rr[1:]))
    ax = torch.empty(run.g.sino_shape, device="cuda")
    rdp.ct_project(run.g, run.x, ax)
    true_rr = float(((run.y.double() - ax.double()) ** 2).sum())
    assert abs(true_rr - rr[-1]) <= 1e-3 * rr[-1]
    assert 0.5 <= rr[-1] / hist["rr"][-1] <= 2.0


def test_cgls_c3_two_iterations():
    wl = W.make_workload(3)
    og = oracle.Geometry.from_workload(wl)
    y = oracle.project(og, W.make_phantom(wl)).astype(np.float32)
    _compare(wl, y, 2, label="C3", seeds=(1,))


def test_cgls_is_reproducible_and_zero_data_is_stationary():
    wl = _tiny(W.BEAM_CONE, 5)
    y = np.random.default_rng(1).uniform(0, 1, wl.sino_shape).astype(np.float32)
    a, b = GpuCgls(wl, y), GpuCgls(wl, y)
    for _ in range(3):
        a.step()
        b.step()
    assert torch.equal(a.x, b.x) and torch.equal(a.p, b.p) and torch.equal(a.r, b.r)
    # y = 0 from x = 0: every vector and scalar is 0 and stays 0 (alpha = beta = 0)
    z = GpuCgls(wl, np.zeros(wl.sino_shape, np.float32))
    z.step()
    sc = z.scalars()
    assert sc["gamma"] == 0 and sc["alpha"] == 0 and sc["beta"] == 0
    assert float(z.x.abs().max()) == 0.0


def test_cgls_argument_errors():
    wl = _tiny(W.BEAM_FAN2D, 3)
    y = np.ones(wl.sino_shape, np.float32)
    run = GpuCgls(wl, y)
    g = run.g
    with pytest.raises(rdp.CtError) as ei:
        rdp.ct_cgls_step(g, run.x, run.r, run.x, run.p, run.q, run.work)   # s aliases x
    assert ei.value.status == rdp.CT_E_ALIAS
    small = torch.empty(8, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        rdp.ct_cgls_step(g, run.x, run.r, run.s, run.p, run.q, small)


def _sample_rays(wl, n, seed):
    return np.sort(np.random.default_rng(seed).choice(wl.n_rays, n, replace=False))


@pytest.mark.parametrize("config", [4, 5])
def test_cgls_full_size_first_step(config):
    """One CGLS step at 512^3 in the launch shapes the benchmark uses, from
    x0 = 0 with a sparse seeded measurement (2000 rays), so that the oracle
    computes s0 = A^T y in full.  Checked: s0 against the oracle, q = A s0 on
    the measured rays and on random rays against the oracle applied to its own
    s0, and the recurrence from the GPU vectors in float64: alpha =
    gamma/||q||^2, x1 = alpha s0, r1 = y - alpha q, ||r1||^2 = ||r0||^2 - alpha gamma."""
    say("CGLS full size", config)
    wl = W.make_workload(config)
    og = oracle.Geometry.from_workload(wl)
    ids_y = _sample_rays(wl, 2000, 60 + config)
    y = np.zeros(wl.n_rays, np.float32)
    y[ids_y] = 1.0 + (np.arange(len(ids_y)) % 7).astype(np.float32)
    y = y.reshape(wl.sino_shape)
    s0_ref = oracle.backproject(og, y)
    run = GpuCgls(wl, y)
    sc0 = run.scalars()
    s0h = host(run.s)
    es = rel(s0h, s0_ref)
    say(f"C{config} CGLS s0 rel_l2 = {es:.3e}")
    assert es <= 1e-5
    g_ref = float(np.sum(s0_ref * s0_ref))
    assert abs(sc0["gamma"] - g_ref) <= 1e-5 * g_ref
    rr0 = float(np.sum(y.astype(np.float64) ** 2))
    assert abs(sc0["rr"] - rr0) <= 1e-12 * rr0
    run.step()
    sc = run.scalars()
    ids = np.unique(np.concatenate([ids_y, _sample_rays(wl, 2000, 31 + config)]))
    qh = host(run.q).ravel()
    ref_q = oracle.project_rays(og, s0_ref, ids)
    eq = rel(qh[ids], ref_q)
    say(f"C{config} CGLS q sampled rel_l2 = {eq:.3e}")
    assert eq <= 1e-5
    qd = run.q.double()
    qq = float((qd * qd).sum())
    assert abs(sc["qq"] - qq) <= 1e-9 * qq
    alpha = sc0["gamma"] / qq
    assert abs(sc["alpha"] - alpha) <= 1e-12 * alpha
    # x1 = alpha s0 (one float32 rounding), r1 = y - alpha q (float32 fma)
    assert rel(host(run.x), np.float32(alpha) * s0h.astype(np.float32)) <= 1e-6
    r1 = dev(y).double() - float(np.float32(alpha)) * qd
    assert float((run.r.double() - r1).norm() / r1.norm()) <= 1e-6
    rr1 = sc0["rr"] - alpha * sc0["gamma"]
    say(f"C{config} CGLS ||r1||^2 {sc['rr']:.6e} recurrence {rr1:.6e}")
    assert abs(sc["rr"] - rr1) <= 1e-4 * sc0["rr"]


def _step_local(wl, y, steps, x0=None):
    """Each GPU step against one oracle step from the GPU's own state: the
    oracle reads the GPU's (x, r, s, p, gamma) after step k and takes step k+1;
    the GPU's state after step k+1 must match it to 1e-5.  No amplification
    across steps enters this bar, only the rounding of one step."""
    gc = GpuCgls(wl, y, x0)
    og = oracle.Geometry.from_workload(wl)
    worst = 0.0
    for k in range(steps):
        x, r, s, p = host(gc.x), host(gc.r), host(gc.s), host(gc.p)
        gamma = gc.scalars()["gamma"]
        ref = oracle.cgls_step(og, x, r, s, p, gamma)
        gc.step()
        sc = gc.scalars()
        errs = {n: rel(host(getattr(gc, n)), ref[n]) for n in ("x", "r", "s", "p", "q")}
        errs.update({n: abs(sc[n] - ref[n]) / max(abs(ref[n]), 1e-300) for n in SCALARS})
        say(f"{wl.name} step {k + 1}: " + ", ".join(f"{n} {v:.1e}" for n, v in errs.items()))
        for n, v in errs.items():
            assert v <= 1e-5, (k + 1, n, v)
        worst = max(worst, max(errs.values()))
    return worst


@pytest.mark.parametrize("beam", [W.BEAM_PARALLEL2D, W.BEAM_FAN2D, W.BEAM_CONE, W.BEAM_PARALLEL3D])
def test_step_local_parity_tiny(beam):
    wl = _tiny(beam, 60 + beam)
    rng = np.random.default_rng(beam)
    y = rng.uniform(0, 1, wl.sino_shape).astype(np.float32)
    _step_local(wl, y, 6)
    x0 = rng.uniform(0, 1, wl.vol_shape).astype(np.float32)
    _step_local(wl, y, 3, x0=x0)


def test_step_local_parity_packets():
    # Dual-axis parallel views: every ray lies in planes of x or y and a detector
    # axis runs along that axis alone, so the CGLS forward (A p with ||q||^2, and
    # the start r = y - A x) runs in packets of rays that share their walk, and so
    # does the brick adjoint (anisotropic voxels keep it off the line adjoint).  A
    # 46 x 38 detector leaves ragged packet tiles; the tilts avoid 0 and the
    # spacings keep every ray clear of the planes it runs along.
    fr = W.dual_axis_parallel3d(6, -61.0, 130.0 / 6)
    wl = W.Workload("packets parallel3d", W.BEAM_PARALLEL3D, (20, 24, 28), (1.0, 0.93, 1.07), (46, 38),
                    (1.0, 1.0), fr, 0)
    for ray, eu, ev in zip(fr[:, 0:3], fr[:, 6:9], fr[:, 9:12]):
        d = int(np.argmin(np.abs(ray)))
        assert ray[d] == 0.0
        assert any(np.count_nonzero(e) == 1 and e[d] != 0.0 for e in (eu, ev))
    assert untraversed_plane_distance(wl) > 1e-3
    assert rdp.ct_geom_adjoint_kind(wl.beam, wl.vol_shape, wl.voxel_spacing, wl.det_shape, wl.det_spacing,
                                    wl.frames) == rdp.ADJOINT_BRICK
    rng = np.random.default_rng(71)
    y = rng.uniform(0, 1, wl.sino_shape).astype(np.float32)
    _step_local(wl, y, 4)
    x0 = rng.uniform(0, 1, wl.vol_shape).astype(np.float32)
    _step_local(wl, y, 2, x0=x0)


@pytest.mark.parametrize("config", [2, 3])
def test_step_local_parity_c2_c3(config):
    wl = W.make_workload(config)
    og = oracle.Geometry.from_workload(wl)
    y = oracle.project(og, W.make_phantom(wl)).astype(np.float32)
    _step_local(wl, y, 6 if config == 2 else 3)
