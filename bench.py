#!/usr/bin/env python3
"""Benchmark of the ray-driven projector pair on one MI355X.

A step is one SIRT iteration on the 512^3 parallel3d dual-axis workload (C4:
280 views, 512 x 512 detector): the forward projection with the residual
epilogue (ct_sirt_residual) and the brick-binned adjoint with the update
epilogue (ct_sirt_update), i.e. every hot-path kernel of the iteration.  The
SIRT weights are computed once before timing.  Inputs live in HBM before the
timed region starts.

Printed value: ray-voxel intersections per second over the step (each
intersection is visited once by A and once by A^T, so 2 * nnz per step),
in G/s; ms_per_step is the time of one SIRT iteration.  --workload c5 instead
times A + A^T (ct_project + ct_backproject) on the 512^3 jittered circular
cone (720 views, 1024 x 768); its A^T input is a dense seeded sinogram (every
ray nonzero), since rays whose value is 0 add nothing and are skipped by the
adjoint, which would make a sparse sinogram look faster.  --workload c4cgls /
c5cgls time CGLS iterations (ct_cgls_step: A p with ||q||^2, r -= alpha q,
A^T r with ||s||^2 and x += alpha p, p = s + beta p) on the same workloads
from y = A phantom, after ct_cgls_init.  --workload c5cyl times A + A^T on C5's
acquisition with a cylindrical detector centred on the source (radius 1500,
the parameterized-surface path).  --workload c5fdk times FDK on C5's
acquisition (ct_fbp_filter: cosine weights, Ram-Lak ramp filter padded to 2U,
angular weights; ct_fbp_backproject: the interpolating weighted
backprojection, six launches of 120 views, each after a pair-interleaving
copy of its views) of y = A phantom; its value is voxel-view updates per second
(512^3 voxels x 720 views per step), and the backprojection is bound by
instruction issue, so its roofline is against the fp32 vector peak, per launch.  --workload c1 / c2 / c3 time A + A^T
(dense seeded A^T input) on the small configurations (2D parallel 64^2, 2D fan
512^2, helical cone 128^3), whose throughput is reported for completeness.

Roofline: algorithmic HBM bytes of the dominant kernel per launch divided by
its average duration (HIP events on the launch stream), against 8 TB/s;
"traffic" is the HBM bytes per launch from committed rocprofv3 counter runs
(profiles/traffic_*.json) when they were taken on the current kernel code.
CPU baseline: the float64 oracle on a bounded sample of views, same unit.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12
# fp32 vector peak without packed-math: 256 CUs x 4 SIMDs x 16 lanes x 2 flops (FMA) x 2.4 GHz
ALU_PEAK = 256 * 4 * 16 * 2 * 2.4e9
# FDK backprojection flops per voxel-view: three affine forms (9 FMA = 18), a
# reciprocal (1), u and v (2), the weight K / w^2 (2), two fractional parts (2),
# the bilinear interpolation (3 lerps of sub + FMA = 9) and the accumulation (2)
FDK_FLOPS_PER_UPDATE = 36


KERNEL_SOURCES = ("ct_kernels.hip", "ct_abi.hip", "ct_geometry.cpp", "ct_fbp.hip", "ct_launch.h", "ct_internal.h")


def _kernel_source_hash() -> str:
    """Hash of the library's code with comments and blank space removed, so
    that counter summaries stay valid across edits that change no code."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "ray_driven_projector_amd", "csrc", f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def _traffic(kernel: str, workload: str, per_launch_bytes_unused=None):
    """HBM bytes per launch measured by rocprofv3 counters, if a summary taken on
    the current kernel sources is committed under profiles/; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            d = json.load(f)
        if d.get("source_hash") != _kernel_source_hash():
            return None
        return float(d["hbm_bytes_per_launch"])
    except Exception:
        return None


def cpu_baseline(wl, n_views_sample: int):
    """Float64 oracle on evenly spaced views of the workload (A then A^T)."""
    import numpy as np

    import oracle
    from ray_driven_projector_amd import workloads as W

    views = sorted(set(int(round(v)) for v in np.linspace(0, wl.n_views - 1, n_views_sample)))
    sub = wl.subset_views(views)
    og = oracle.Geometry.from_workload(sub)
    x = W.make_phantom(wl)
    nt = oracle.default_threads()
    t0 = time.perf_counter()
    sino, nnz, _ = oracle.project(og, x, nthreads=nt, with_counts=True)
    t1 = time.perf_counter()
    # A^T of a dense sinogram (no ray is zero, so none is skipped)
    dense = sino + 1.0
    t2 = time.perf_counter()
    oracle.backproject(og, dense, nthreads=nt)
    t3 = time.perf_counter()
    ta, tat = t1 - t0, t3 - t2
    rate = 2 * nnz / (ta + tat) / 1e9
    return {"value": rate, "unit": "G ray-voxel intersections/s", "cores": nt, "kind": "oracle",
            "sample": f"{len(views)} of {wl.n_views} views of the same workload: A, then A^T of a "
                      f"dense sinogram, {nnz} intersections each; A {ta:.2f} s, A^T {tat:.2f} s"}


def cpu_baseline_fdk(wl, angles, n_vox: int):
    """Float64 oracle of the FDK backprojection on a bounded sample of voxels
    (all views), in voxel-view updates per second."""
    import numpy as np

    from oracle import fbp as F

    rng = np.random.default_rng(7)
    ids = rng.choice(wl.n_voxels, n_vox, replace=False)
    q = rng.standard_normal(wl.sino_shape).astype(np.float32)
    t0 = time.perf_counter()
    F.weighted_backproject_voxels(wl, q, ids)
    dt = time.perf_counter() - t0
    return {"value": n_vox * wl.n_views / dt / 1e9, "unit": "G voxel-view updates/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{n_vox} random voxels of the 512^3 volume, all {wl.n_views} views (numpy, "
                      f"one thread): {dt:.2f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", choices=["c1", "c2", "c3", "c4", "c5", "c4cgls", "c5cgls", "c5cyl", "c5fdk"],
                    default="c4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-views", type=int, default=16)
    ap.add_argument("--extra", action="store_true", help="also time A, A^T and atomic A^T alone")
    ap.add_argument("--host-stream", type=int, nargs=2, metavar=("SLAB", "BATCH_VIEWS"),
                    help="also time A and A^T with volume and sinogram in pinned host memory "
                         "(PCIe-inclusive; reported apart from value)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a 1 GiB device copy first (reference kernel for HBM counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print("bench.py: runs on one GPU; several GPUs (views or space sharding) are not "
              "implemented. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import ray_driven_projector_amd as rdp
    from ray_driven_projector_amd import workloads as W

    if not os.path.exists(rdp.LIB_PATH):
        from ray_driven_projector_amd import build as b
        b.build()
    torch.cuda.set_device(0)
    # the box's device-copy bandwidth (1 GiB read + 1 GiB written), the second
    # yardstick for the roofline fraction; with --copy-calibration it is also
    # the reference kernel for the HBM counters
    src = torch.ones(1 << 28, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    copy_ms = []
    for _ in range(1 if args.copy_calibration else 5):
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        dst.copy_(src)
        c1.record()
        torch.cuda.synchronize()
        copy_ms.append(c0.elapsed_time(c1))
    copy_bw = 2 * (1 << 30) / (float(np.median(copy_ms)) * 1e-3)
    del src, dst
    cfg = int(args.workload[1])
    cgls = args.workload.endswith("cgls")
    wl = W.make_workload(cfg)
    if args.workload == "c5cyl":
        wl = W.with_surface(wl, W.cylinder_offsets(wl.det_shape, wl.det_spacing, 1500.0), "cylindrical")
    print(f"# workload: {wl.name}", file=sys.stderr, flush=True)
    phantom = W.make_phantom(wl)
    g = rdp.Geometry.from_workload(wl)
    stream = torch.cuda.current_stream()
    x_true = torch.from_numpy(phantom).cuda()
    y = torch.empty(g.sino_shape, device="cuda")
    rdp.ct_project(g, x_true, y)                     # synthetic measurement
    nnz = rdp.ct_count_intersections(g)
    M, N = wl.n_rays, wl.n_voxels
    print(f"# nnz={nnz} rays={M} voxels={N}", file=sys.stderr, flush=True)

    ev = lambda: torch.cuda.Event(enable_timing=True)
    fdk = args.workload == "c5fdk"
    if fdk:
        fdk_angles = W.angles(wl.n_views, 2 * np.pi)
        fplan = rdp.FBP.from_workload(wl, fdk_angles, window="ram-lak", pad_factor=2)
        work = torch.empty(g.sino_shape, device="cuda")
        vol = torch.empty(g.vol_shape, device="cuda")
        names = ("fbp_filter", "fbp_backproject")
        U = wl.det_shape[0]
        flops_per = {"fbp_filter": 2 * U * M, "fbp_backproject": FDK_FLOPS_PER_UPDATE * N * wl.n_views}
        # ct_fbp_backproject gathers in equal batches of at most 128 views, one
        # launch each (after a pair-interleaving copy of the batch)
        n_batch = -(-wl.n_views // 128)
        kern_names = {"fbp_filter": "fbp_fft_filter_kernel",
                      "fbp_backproject": f"fbp_bp_kernel<false, false, 4> ({n_batch} launches per call)"}

        def step(evs):
            evs[0].record(stream)
            rdp.ct_fbp_filter(fplan, y, work, stream)
            evs[1].record(stream)
            rdp.ct_fbp_backproject(fplan, work, vol, stream)
            evs[2].record(stream)
    elif cgls:
        x = torch.zeros(g.vol_shape, device="cuda")
        r = torch.empty(g.sino_shape, device="cuda")
        q = torch.empty(g.sino_shape, device="cuda")
        s_ = torch.empty(g.vol_shape, device="cuda")
        p_ = torch.empty(g.vol_shape, device="cuda")
        work = torch.empty(rdp.ct_cgls_workspace_size(g), dtype=torch.uint8, device="cuda")
        rdp.ct_cgls_init(g, y, x, r, s_, p_, work, stream)
        names = ("cgls_step", "none")
        # forward (A p, ||q||^2) + r update + adjoint (A^T r, ||s||^2, x update) + p update
        bytes_per = {"cgls_step": (4 * nnz + 4 * M) + 12 * M + (4 * nnz + 4 * M + 16 * N) + 12 * N,
                     "none": 0}
        kern_names = {"cgls_step": "one CGLS iteration (all kernels)", "none": ""}

        def step(evs):
            evs[0].record(stream)
            rdp.ct_cgls_step(g, x, r, s_, p_, q, work, stream)
            evs[1].record(stream)
            evs[2].record(stream)
    elif cfg == 4:
        rinv = torch.empty(g.sino_shape, device="cuda")
        cinv = torch.empty(g.vol_shape, device="cuda")
        rdp.ct_sirt_weights(g, rinv, cinv)
        x = torch.zeros(g.vol_shape, device="cuda")
        work = torch.empty(g.sino_shape, device="cuda")
        names = ("sirt_residual", "sirt_update")
        bytes_per = {"sirt_residual": 4 * nnz + 12 * M, "sirt_update": 4 * nnz + 4 * M + 12 * N}
        kern_names = {"sirt_residual": "ray_kernel<1, false, false>",
                      "sirt_update": "brick_kernel<16, 16, 32, 512, 1, false>"}

        def step(evs):
            evs[0].record(stream)
            rdp.ct_sirt_residual(g, x, y, rinv, work, stream)
            evs[1].record(stream)
            rdp.ct_sirt_update(g, work, cinv, 1.0, x, stream)
            evs[2].record(stream)
    else:
        xs = x_true
        gen = torch.Generator(device="cuda")
        gen.manual_seed(5005)
        y = 0.5 + torch.rand(g.sino_shape, device="cuda", generator=gen)   # dense A^T input
        sino = torch.empty(g.sino_shape, device="cuda")
        vol = torch.empty(g.vol_shape, device="cuda")
        names = ("project", "backproject")
        bytes_per = {"project": 4 * nnz + 4 * M, "backproject": 4 * nnz + 4 * M + 4 * N}
        sf = "true" if wl.offsets is not None else "false"
        two_d = wl.beam in (W.BEAM_PARALLEL2D, W.BEAM_FAN2D)
        kern_names = {"project": f"ray_kernel<0, {'true' if two_d else 'false'}, {sf}>",
                      "backproject": (f"brick_kernel<64, 64, 1, 256, 0, {sf}>" if two_d else
                                      f"brick_kernel<16, 16, 32, 512, 0, {sf}>")}

        def step(evs):
            evs[0].record(stream)
            rdp.ct_project(g, xs, sino, stream)
            evs[1].record(stream)
            rdp.ct_backproject(g, y, vol, stream)
            evs[2].record(stream)

    for _ in range(args.warmup):
        step([ev(), ev(), ev()])
    torch.cuda.synchronize()
    all_evs = [[ev(), ev(), ev()] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(all_evs[k])
        print(f"# step {k} enqueued", file=sys.stderr, flush=True) if k == 0 else None
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    k_ms = {names[0]: [], names[1]: []}
    for e in all_evs:
        k_ms[names[0]].append(e[0].elapsed_time(e[1]))
        k_ms[names[1]].append(e[1].elapsed_time(e[2]))
    ms_step = (t1 - t0) * 1e3 / args.steps
    avg = {k: float(np.mean(v)) for k, v in k_ms.items()}
    if cgls:
        avg.pop("none")
    dom = max(avg, key=avg.get)
    if fdk:
        achieved = flops_per[dom] / (avg[dom] * 1e-3)
        value = N * wl.n_views / (ms_step * 1e-3) / 1e9
    else:
        achieved = bytes_per[dom] / (avg[dom] * 1e-3)
        value = 2 * nnz / (ms_step * 1e-3) / 1e9

    extra = {}
    if args.extra:
        out_s = torch.empty(g.sino_shape, device="cuda")
        out_v = torch.empty(g.vol_shape, device="cuda")
        for name, fn, a, b in (("A", rdp.ct_project, x_true, out_s), ("AT", rdp.ct_backproject, y, out_v),
                               ("AT_atomic", rdp.ct_backproject_atomic, y, out_v)):
            fn(g, a, b, stream)
            ts = []
            for _ in range(3 if name != "AT_atomic" else 1):
                e0, e1 = ev(), ev()
                e0.record(stream)
                fn(g, a, b, stream)
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            extra[f"{name}_ms"] = float(np.median(ts))
            extra[f"{name}_G_intersections_per_s"] = nnz / (np.median(ts) * 1e-3) / 1e9

    res = {
        "metric": ("G voxel-view updates/s of FDK at 512^3" if fdk else
                   "G ray-voxel intersections/s for A and A^T; ms per SIRT iteration at 512^3"),
        "value": round(value, 3),
        "unit": "G voxel-view updates/s" if fdk else "G ray-voxel intersections/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": (wl.name + (", FDK (Ram-Lak, pad 2) of y = A phantom" if fdk else
                                    ", one CGLS iteration (from y = A phantom)" if cgls else
                                    ", one SIRT iteration (A with residual + A^T with update)"
                                    if cfg == 4 else ", A + A^T")),
            "volume": list(wl.vol_shape), "views": wl.n_views, "detector": list(wl.det_shape),
            "intersections_per_pass": nnz, "rays": M, "voxels": N,
        },
        "ms_per_sirt_iteration": round(ms_step, 3) if (cfg == 4 and not cgls) else None,
        "ms_per_cgls_iteration": round(ms_step, 3) if cgls else None,
        "kernel_ms": {k: round(v, 3) for k, v in avg.items()},
        "roofline": ({
            "bound": "alu", "kernel": kern_names[dom], "achieved": round(achieved / 1e12, 2),
            "peak": round(ALU_PEAK / 1e12, 1), "unit": "TFLOP/s", "frac": round(achieved / ALU_PEAK, 4),
            "traffic": _traffic(dom, args.workload),
            "algorithmic_flops_per_launch": flops_per[dom] // (n_batch if dom == "fbp_backproject" else 1),
            "launches_per_call": n_batch if dom == "fbp_backproject" else 1,
        } if fdk else {
            "bound": "hbm", "kernel": kern_names[dom], "achieved": round(achieved / 1e9, 1),
            "peak": HBM_PEAK / 1e9, "unit": "GB/s", "frac": round(achieved / HBM_PEAK, 4),
            "traffic": _traffic(dom, args.workload),
            "algorithmic_bytes_per_launch": bytes_per[dom],
            "copy_bw": round(copy_bw / 1e9, 1), "frac_vs_copy": round(achieved / copy_bw, 4),
        }),
    }
    res.update(extra)
    if args.host_stream:
        nz, nb = args.host_stream
        hx = torch.from_numpy(phantom).pin_memory()
        hy = y.cpu().pin_memory()
        hs = torch.empty(g.sino_shape, pin_memory=True)
        hv = torch.empty(g.vol_shape, pin_memory=True)
        hres = {"plan": {"slab": nz, "batch_views": nb, "axis": "auto"}, "host_memory": "pinned"}
        for name, fn, a, b in (("A", rdp.ct_project_host, hx, hs), ("AT", rdp.ct_backproject_host, hy, hv)):
            fn(g, a, b, nz, nb, stream=stream)
            ts = []
            for _ in range(3):
                t = time.perf_counter()
                fn(g, a, b, nz, nb, stream=stream)
                ts.append((time.perf_counter() - t) * 1e3)
            hres[f"{name}_ms"] = round(float(np.median(ts)), 2)
        n_bt = -(-wl.n_views // nb)
        vb, sb = 4 * N, 4 * M
        n_sl_a = -(-wl.vol_shape[0] // nz)   # the adjoint slabs along z; the forward's
        hres["pcie_bytes"] = {"A": vb * n_bt + sb,   # axis is the library's choice
                              "AT": sb * (n_sl_a if n_bt > 1 else 1) + vb}
        res["host_stream"] = hres
    if fdk:
        res["kernel_ms_note"] = "fbp_filter: pre-weights + ramp + angular weights; fbp_backproject: gather"
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        res["cpu_baseline"] = (cpu_baseline_fdk(wl, fdk_angles, 100000) if fdk else
                               cpu_baseline(wl, args.cpu_views))
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
