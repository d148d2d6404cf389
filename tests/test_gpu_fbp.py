"""GPU parity of analytical FBP / FDK (ct_fbp_*) against the float64 oracle
(oracle/fbp.py): the filtered sinogram, the interpolating weighted
backprojection, its transpose and the whole pipeline, at the 1e-5 relative L2
bar; full-size FDK of the 512^3 cone acquisition on sampled rows and voxels;
and the argument errors.
"""
import math

import numpy as np
import pytest

import ray_driven_projector_amd as rdp
from oracle import fbp as F
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


def fan_wl(n=90, U=77, vol=(1, 37, 41), sid=60.0, sdd=100.0, du=0.8, span=2 * math.pi):
    fr = W.circular_fan2d(n, sid, sdd, angular_range=span)
    return W.Workload("fan", W.BEAM_FAN2D, vol, (1, 1, 1), (U, 1), (du, 1), fr), W.angles(n, span)


def par_wl(n=75, U=61, vol=(1, 29, 33)):
    fr = W.circular_parallel2d(n, math.pi)
    return W.Workload("par", W.BEAM_PARALLEL2D, vol, (1, 1, 1), (U, 1), (0.7, 1), fr), W.angles(n, math.pi)


def cone_wl(n=60, det=(53, 41), vol=(19, 27, 30), sid=70.0, sdd=110.0, jitter=0.0, spacing=(1, 1, 1)):
    fr = W.helix_cone(n, sid, sdd, 0.0, 1.0)
    if jitter:
        fr = W.jitter_frames(fr, W.Stream(77), jitter, jitter)
    return W.Workload("cone", W.BEAM_CONE, vol, spacing, det, (0.9, 0.8), fr), W.angles(n, 2 * math.pi)


def short_fan():
    sid, sdd, U, du, n = 60.0, 100.0, 83, 0.8, 120
    delta = math.atan(0.5 * U * du / sdd)
    span = (math.pi + 2 * delta + 0.05) * n / (n - 1)
    return fan_wl(n, U, (1, 31, 35), sid, sdd, du, span)


CASES = {
    "parallel": par_wl,
    "fan": fan_wl,
    "fan-short": short_fan,
    "cone": cone_wl,
    "cone-jittered-aniso": lambda: cone_wl(jitter=0.4, spacing=(1.2, 0.9, 1.0)),
    # more views than one backprojection batch holds: batches of 86, 86, 85
    "cone-257-views": lambda: cone_wl(n=257, det=(31, 23), vol=(12, 17, 19)),
    # power-of-two padded rows take the FFT filter
    "parallel-pow2": lambda: par_wl(U=64),
    "fan-pow2": lambda: fan_wl(U=128),
    "cone-pow2": lambda: cone_wl(det=(64, 37)),
}


def plan(wl, th, **kw):
    return rdp.FBP.from_workload(wl, th, **kw)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("window,pad", [("ram-lak", 2), ("shepp-logan", 1), ("hann", 4),
                                        ("cosine", 2), ("hamming", 3)])
def test_filter_matches_oracle(name, window, pad):
    wl, th = CASES[name]()
    short = name == "fan-short"
    if "pow2" in name and pad == 3:
        pad = 2
    f = plan(wl, th, window=window, pad_factor=pad, short_scan=short)
    iso, aw = f.info()
    assert np.allclose(iso, F.isocentre(wl), atol=1e-9)
    assert np.allclose(aw, F.angular_weights(th, wl.beam, short), rtol=1e-12, atol=0)
    rng = np.random.default_rng(3)
    sino = rng.uniform(0, 2, wl.sino_shape).astype(np.float32)
    out = torch.empty(wl.sino_shape, device="cuda")
    rdp.ct_fbp_filter(f, dev(sino), out)
    ref = F.filter_sinogram(wl, sino, th, window, pad, short)
    e = rel_l2(host(out), ref)
    say(f"{name} {window} pad {pad}: filter rel_l2 {e:.2e}")
    assert e <= TOL


@pytest.mark.parametrize("name", list(CASES))
def test_backprojection_and_transpose_match_oracle(name):
    wl, th = CASES[name]()
    f = plan(wl, th, short_scan=name == "fan-short")
    rng = np.random.default_rng(4)
    q = rng.standard_normal(wl.sino_shape).astype(np.float32)
    vol = torch.empty(wl.vol_shape, device="cuda")
    rdp.ct_fbp_backproject(f, dev(q), vol)
    eb = rel_l2(host(vol), F.weighted_backproject(wl, q))
    x = rng.uniform(0, 1, wl.vol_shape).astype(np.float32)
    s = torch.empty(wl.sino_shape, device="cuda")
    rdp.ct_fbp_backproject_transpose(f, dev(x), s)
    et = rel_l2(host(s), F.weighted_backproject_T(wl, x))
    # the GPU pair is itself transposed
    lhs = float(np.dot(host(vol).ravel(), x.astype(np.float64).ravel()))
    rhs = float(np.dot(q.astype(np.float64).ravel(), host(s).ravel()))
    ei = abs(lhs - rhs) / max(abs(lhs), abs(rhs))
    say(f"{name}: B {eb:.2e}, B^T {et:.2e}, identity {ei:.2e}")
    assert eb <= TOL and et <= TOL and ei <= TOL


def _disc_chords(wl, centre, radius):
    p = F.pixel_centres(wl)
    a = wl.frames[:, None, None, 0:3]
    if wl.beam in (F.FAN2D, F.CONE):
        o, d = np.broadcast_to(a, p.shape), p - a
    else:
        o, d = p, np.broadcast_to(a, p.shape)
    d = d / np.linalg.norm(d, axis=-1, keepdims=True)
    rel = np.asarray(centre, float) - o
    t = np.sum(rel * d, axis=-1)
    return 2 * np.sqrt(np.clip(radius ** 2 - (np.sum(rel * rel, axis=-1) - t * t), 0, None))


@pytest.mark.parametrize("name", list(CASES))
def test_pipeline_matches_oracle(name):
    wl, th = CASES[name]()
    short = name == "fan-short"
    sino = _disc_chords(wl, (2.0, -1.5, 0.5 if wl.beam == W.BEAM_CONE else 0.0), 9.0).astype(np.float32)
    f = plan(wl, th, window="shepp-logan", short_scan=short)
    work = torch.empty(wl.sino_shape, device="cuda")
    vol = torch.empty(wl.vol_shape, device="cuda")
    rdp.ct_fbp_run(f, dev(sino), work, vol)
    ref = F.fbp(wl, sino, th, window="shepp-logan", short_scan=short)
    e = rel_l2(host(vol), ref)
    say(f"{name}: FBP/FDK rel_l2 {e:.2e}")
    assert e <= TOL


@pytest.mark.parametrize("name", ["cone-pow2", "fan-pow2"])
def test_fft_and_direct_filters_agree(name):
    wl, th = CASES[name]()
    f = plan(wl, th, window="shepp-logan", pad_factor=2)
    fd = plan(wl, th, window="shepp-logan", pad_factor=2, direct_filter=True)
    sino = dev(np.random.default_rng(6).uniform(0, 1, wl.sino_shape))
    a = torch.empty(wl.sino_shape, device="cuda")
    b = torch.empty(wl.sino_shape, device="cuda")
    rdp.ct_fbp_filter(f, sino, a)
    rdp.ct_fbp_filter(fd, sino, b)
    e = rel_l2(host(a), host(b))
    say(f"{name}: FFT vs direct filter {e:.2e}")
    assert e <= 2e-6


@pytest.mark.parametrize("beam", ["fan", "cone"])
def test_voxels_behind_the_source_gather_nothing(beam):
    # The orbit (radius 12) runs inside the volume, so in every view some
    # voxels lie behind the source.  One view at a time (the other views' data
    # zero): voxels behind that view's source get exactly 0; in front, away
    # from the source plane, the result matches the oracle.  Near that plane
    # the magnification D / U and the weight R D / U^2 grow without bound, and
    # the float32 gather parts from the float64 oracle by more than the bar
    # (1.3e-5 over U >= 3 and 1.2e-5 over U >= 6 in one fan view, with a
    # random filtered sinogram), so the comparison takes U >= 10
    # (magnification <= 6).
    if beam == "fan":
        wl, th = fan_wl(n=72, U=77, vol=(1, 29, 33), sid=12.0, sdd=60.0)
    else:
        wl, th = cone_wl(n=60, det=(53, 41), vol=(19, 27, 30), sid=12.0, sdd=60.0)
    f = plan(wl, th)
    q = np.random.default_rng(9).standard_normal(wl.sino_shape).astype(np.float32)
    z, y, x = F.voxel_centres(wl)
    Z, Y, X = np.meshgrid(z, y, x, indexing="ij")
    P = np.stack([X, Y, Z], -1)
    n = F.detector_normals(wl.frames, wl.beam)
    vol = torch.empty(wl.vol_shape, device="cuda")
    for i in (0, wl.n_views // 3, (2 * wl.n_views) // 3 + 1):
        qi = np.zeros_like(q)
        qi[i] = q[i]
        rdp.ct_fbp_backproject(f, dev(qi), vol)
        g = host(vol)
        ref = F.weighted_backproject(wl, qi)
        Ux = (P - wl.frames[i, 0:3]) @ n[i]
        behind, front = Ux <= -0.5, Ux >= 10.0
        assert behind.sum() >= 20 and front.sum() >= 100
        assert np.all(g[behind] == 0.0) and np.all(ref[behind] == 0.0)
        e = rel_l2(g[front], ref[front])
        say(f"{beam} view {i}: {behind.sum()} voxels behind the source get 0; in front rel_l2 {e:.2e}")
        assert e <= TOL


def test_given_isocentre_and_angular_weights():
    wl, th = cone_wl(jitter=0.3)
    iso = np.array([0.7, -0.4, 0.2])
    aw = np.random.default_rng(9).uniform(0.05, 0.15, wl.n_views)
    f = plan(wl, None, iso=iso, angular_weights=aw)
    got_iso, got_aw = f.info()
    assert np.array_equal(got_iso, iso) and np.array_equal(got_aw, aw)
    sino = np.random.default_rng(8).uniform(0, 1, wl.sino_shape).astype(np.float32)
    work = torch.empty(wl.sino_shape, device="cuda")
    vol = torch.empty(wl.vol_shape, device="cuda")
    rdp.ct_fbp_run(f, dev(sino), work, vol)
    ref = F.fbp(wl, sino, th, iso=iso, ang_weights=aw)
    assert rel_l2(host(vol), ref) <= TOL


def test_full_size_fdk_of_the_512_cone_acquisition():
    """C5's acquisition (512^3, 720 jittered views, 1024 x 768) in the launch
    shapes the benchmark uses: the filter on 6 views' rows against the oracle
    (angular weights of the full scan), and the backprojection of a seeded
    sinogram on 400 sampled voxels."""
    wl = W.make_workload(5)
    th = W.angles(wl.n_views, 2 * math.pi)
    f = plan(wl, th, window="ram-lak", pad_factor=2)
    rng = np.random.default_rng(11)
    sino = rng.uniform(0, 1, wl.sino_shape).astype(np.float32)
    out = torch.empty(wl.sino_shape, device="cuda")
    rdp.ct_fbp_filter(f, dev(sino), out)
    views = np.array([0, 1, 137, 360, 611, 719])
    sub = wl.subset_views(views)
    aw = F.angular_weights(th, wl.beam)[views]
    ref = F.filter_sinogram(sub, sino[views], th[views], "ram-lak", 2, ang_weights=aw)
    ef = rel_l2(host(out[torch.from_numpy(views).cuda()]), ref)
    del out
    q = rng.standard_normal(wl.sino_shape).astype(np.float32)
    vol = torch.empty(wl.vol_shape, device="cuda")
    rdp.ct_fbp_backproject(f, dev(q), vol)
    ids = rng.choice(wl.n_voxels, 400, replace=False)
    eb = rel_l2(host(vol).ravel()[ids], F.weighted_backproject_voxels(wl, q, ids))
    say(f"C5 FDK: filter rel_l2 {ef:.2e} (6 views), B rel_l2 {eb:.2e} (400 voxels)")
    assert ef <= TOL and eb <= TOL


def test_fbp_argument_errors():
    wl, th = cone_wl()
    desc_args = (wl.beam, wl.vol_shape, wl.voxel_spacing, wl.det_shape, wl.det_spacing, wl.frames)
    with pytest.raises(rdp.CtError) as e:   # parallel3d has no FBP here
        rdp.FBP(W.BEAM_PARALLEL3D, wl.vol_shape, wl.voxel_spacing, wl.det_shape, wl.det_spacing,
                W.dual_axis_parallel3d(5, -60, 20), np.zeros(10))
    assert e.value.status == rdp.CT_E_ARG
    pw, pth = par_wl()
    with pytest.raises(rdp.CtError) as e:   # Parker weights need a fan or cone
        rdp.FBP.from_workload(pw, pth, short_scan=True)
    assert e.value.status == rdp.CT_E_ARG
    fw, fth = fan_wl(n=60, span=math.pi)   # half a turn is too short for a short scan
    with pytest.raises(rdp.CtError) as e:
        rdp.FBP.from_workload(fw, fth, short_scan=True)
    assert e.value.status == rdp.CT_E_ARG
    for kw in ({"pad_factor": 0}, {"pad_factor": 17}):
        with pytest.raises(rdp.CtError) as e:
            rdp.FBP(*desc_args, th, **kw)
        assert e.value.status == rdp.CT_E_ARG
    bad = np.array(th)
    bad[3] = np.nan
    with pytest.raises(rdp.CtError) as e:
        rdp.FBP(*desc_args, bad)
    assert e.value.status == rdp.CT_E_NONFINITE
    f = rdp.FBP(*desc_args, th)
    s = torch.zeros(wl.sino_shape, device="cuda")
    with pytest.raises(rdp.CtError) as e:
        rdp.ct_fbp_filter(f, s, s)
    assert e.value.status == rdp.CT_E_ALIAS
    with pytest.raises(ValueError):
        rdp.ct_fbp_backproject(f, s, torch.zeros((3, 3, 3), device="cuda"))
