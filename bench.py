#!/usr/bin/env python3
"""Benchmark of the ray-driven projector pair on one MI355X.

Default run (one JSON line):

- The timed step is one SIRT iteration on the 512^3 parallel3d dual-axis
  workload (280 views, 512 x 512 detector): the forward projection with the
  residual epilogue (ct_sirt_residual) and the brick-binned adjoint with the
  update epilogue (ct_sirt_update; the line adjoint on this tilt series),
  every hot-path kernel of the iteration.
  The SIRT weights are computed once before timing; inputs live in HBM before
  the timed region starts.  value = ray-voxel intersections per second over
  the step (each intersection is visited once by A and once by A^T: 2 nnz per
  step), in G/s; ms_per_step is the time of one SIRT iteration.
- "configs": all five synthetic workloads (2D parallel 64^2, 2D fan 512^2,
  helical cone 128^3, the 512^3 dual-axis parallel3d, the 512^3 jittered
  cone): A of the phantom and A^T of a dense seeded sinogram (every ray
  nonzero, since the adjoint skips rays whose value is 0), each the median of
  7 launches after 3 warm-ups (the diffct documentation's protocol,
  "Performance"), in ms and G intersections/s, with each kernel's ALU
  roofline fraction.  nnz is the oracle's exact count
  (tests/golden/nnz_configs.json, checked against the frames and the GPU's
  own count).
- "roofline": the dominant kernel of the step.  The projector kernels are
  bound by instruction issue and latency, not by HBM (the rocprofv3 counters
  put the VALU busy at 0.6-1.0 while they fetch 1-2.5 TB/s from HBM), so the
  roofline is the ALU one: algorithmic lane operations per launch over the launch's duration
  against 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 39.3 T lane-ops/s (one
  wave64 VALU instruction per SIMD every 4 cycles; packed math does not apply
  to this integer and compare work).  The algorithmic work per intersection
  is that of the walk that runs: a Siddon step is 10 lane operations of
  bookkeeping and length (minimum of the next crossings, the compares, the
  index and position updates, the loop test, the length) plus 2 for the
  multiply-add, 12 in all (10 to 14 by the model the bound was derived
  from); where four rays share one walk (parallel views with an untraversed
  axis whose pixel step runs along it, as on the dual-axis workload) the 10
  are shared, 10 / 4 + 2 = 4.5.  Where the adjoint runs as the line kernel
  (every view's rays lie in planes of one volume axis, as on the dual-axis
  workload) no ray is walked: a ray's chord through an in-plane cell is formed
  once (6 lane operations: offset, distance to the window edge, slope, the two
  clamps, the step to the next row) and shared by the 32 voxels of the thread's
  line through that cell, so 6 / 32 + 2.  The kernels spend more (the measured
  figure, from committed counters, is given beside it).  The effective-HBM view (4
  bytes per intersection against 8 TB/s, most of them served by the caches)
  is kept as "effective_hbm_frac".
- "traffic" and the measured VALU instructions come from rocprofv3 counter
  runs committed in profiles/counters.json; they are reported only while the
  library's device code object is the one they were taken on (its SHA-256).
- "solvers": one CGLS iteration on C4 and on C5 (from y = A phantom) and the
  FDK (Ram-Lak, pad 2) of C5's acquisition, in ms, timed the same way.
- "cpu_baseline": the float64 oracle on a bounded sample of views of the same
  workload (A, then A^T of a dense sinogram), same unit.

--workload c1|c2|c3|c4|c5 times A + A^T of one workload (c4: the SIRT step);
c4cgls / c5cgls time CGLS iterations, c5cyl A + A^T with a cylindrical
detector, c5fdk the FDK (filter + interpolating backprojection).

--ingest-counters WL=DIR ... (no GPU) reads rocprofv3 --pmc CSV output (one
directory per workload, holding the passes' *_counter_collection.csv files),
takes each hot kernel's last dispatch (the timed step), scales FETCH_SIZE and
WRITE_SIZE by what they read for the --copy-calibration copy, and writes
profiles/counters.json (keyed to the current device code) and a Markdown
table beside it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import struct
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12
# VALU issue: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz lane operations per second
VALU_PEAK = 256 * 4 * 16 * 2.4e9
# algorithmic lane operations per ray-voxel intersection (see the module notes):
# walk bookkeeping and length, shared by the rays of a packet, plus the
# multiply-add of each ray
WALK_OPS, RAY_OPS, PACKET = 10, 2, 4
OPS_PER_INTERSECTION = WALK_OPS + RAY_OPS
OPS_PACKET = WALK_OPS / PACKET + RAY_OPS
# line adjoint: one chord per (ray, in-plane cell), shared along a 32-voxel line
CHORD_OPS, LINE_SEG = 6, 32
OPS_LINE = CHORD_OPS / LINE_SEG + RAY_OPS
# fp32 vector peak without packed math, for the FDK gather: VALU_PEAK x 2 (FMA)
ALU_PEAK = 2 * VALU_PEAK
# FDK backprojection flops per voxel-view: three affine forms (9 FMA = 18), a
# reciprocal (1), u and v (2), the weight K / w^2 (2), two fractional parts (2),
# the bilinear interpolation (3 lerps of sub + FMA = 9) and the accumulation (2)
FDK_FLOPS_PER_UPDATE = 36
GOLDEN_NNZ = os.path.join(ROOT, "tests", "golden", "nnz_configs.json")
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")


def code_object_hash() -> str:
    """SHA-256 (16 hex digits) of the device code in libctproj.so: the bytes of
    its .hip_fatbin section (the offload bundle of the gfx950 code object)."""
    path = os.path.join(ROOT, "ray_driven_projector_amd", "libctproj.so")
    with open(path, "rb") as f:
        data = f.read()
    shoff, = struct.unpack_from("<Q", data, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", data, 0x3A)
    hdrs = [struct.unpack_from("<IIQQQQIIQQ", data, shoff + i * shentsize) for i in range(shnum)]
    names = hdrs[shstrndx][4]
    for h in hdrs:
        name = data[names + h[0]: data.index(b"\0", names + h[0])]
        if name == b".hip_fatbin":
            return hashlib.sha256(data[h[4]: h[4] + h[5]]).hexdigest()[:16]
    raise RuntimeError("libctproj.so has no .hip_fatbin section")


def counters(key: str):
    """Counter figures for `key` ("<workload>/<kernel role>") from
    profiles/counters.json, if they were taken on the current device code."""
    try:
        with open(COUNTERS) as f:
            d = json.load(f)
        if d.get("code_object") != code_object_hash():
            return None
        return d["entries"].get(key)
    except (OSError, ValueError, KeyError):
        return None


# kernel-name patterns of the hot kernels and the role each plays
ROLES = (("ray_kernel<0,", "project"), ("ray_kernel<1,", "sirt_residual"), ("ray_kernel<4,", "backproject_atomic"),
         ("ray_packet_kernel<0>", "project"), ("ray_packet_kernel<1>", "sirt_residual"),
         ("ray_kernel<5,", "cgls_project"), ("brick_kernel<", "backproject"), ("line_kernel<", "backproject"),
         ("fbp_bp_kernel<", "fbp_backproject"),
         ("fbp_fft_filter_kernel", "fbp_filter"), ("fbp_filter_kernel", "fbp_filter"))
BRICK_MODES = {"0": "backproject", "1": "sirt_update", "2": "colinv", "3": "cgls_adjoint"}
COPY_BYTES = 1 << 30   # the --copy-calibration copy reads and writes 1 GiB
# the rocprofv3 --pmc passes the counters come from: (output name, counters, extra bench flag)
PMC_PASSES = (("sq", "SQ_INSTS_VALU SQ_INSTS_LDS SQ_INSTS_SALU SQ_WAVES SQ_INSTS_VMEM_RD SQ_LDS_BANK_CONFLICT "
               "GRBM_GUI_ACTIVE", ""),
              ("tcc", "TCC_HIT_sum TCC_MISS_sum", ""),
              ("fetch", "FETCH_SIZE", " --copy-calibration"),
              ("write", "WRITE_SIZE", " --copy-calibration"))


def kernel_role(name: str):
    for pat, role in ROLES:
        if pat in name:
            if role == "backproject" and pat == "brick_kernel<":   # <BX, BY, BZ, NT, MODE, SURF, PERSP, REC>
                args = name.split("brick_kernel<", 1)[1].split(">", 1)[0].split(",")
                return BRICK_MODES.get(args[4].strip())
            if role == "backproject":   # line_kernel<MODE, SHAPE>
                args = name.split("line_kernel<", 1)[1].split(">", 1)[0].split(",")
                return BRICK_MODES.get(args[0].strip())
            return role
    return None


def ingest_counters(specs, out_path=COUNTERS):
    """Write profiles/counters.json (and counters.md) from rocprofv3 --pmc runs."""
    import csv
    import glob
    entries, notes = {}, []
    for spec in specs:
        wl, d = spec.split("=", 1)
        disp = {}
        for path in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            run = os.path.basename(path)
            with open(path) as f:
                for r in csv.DictReader(f):
                    k = (run, int(r["Dispatch_Id"]))
                    e = disp.setdefault(k, {"name": r["Kernel_Name"], "c": {},
                                            "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
                    e["c"][r["Counter_Name"]] = e["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        # the calibration copy: the largest FETCH_SIZE / WRITE_SIZE among the copy kernels
        fscale = wscale = None
        for (run, _), e in disp.items():
            if "copy" not in e["name"].lower():
                continue
            if "FETCH_SIZE" in e["c"] and e["c"]["FETCH_SIZE"] * 1024 > COPY_BYTES / 2:
                fscale = COPY_BYTES / (e["c"]["FETCH_SIZE"] * 1024)
            if "WRITE_SIZE" in e["c"] and e["c"]["WRITE_SIZE"] * 1024 > COPY_BYTES / 2:
                wscale = COPY_BYTES / (e["c"]["WRITE_SIZE"] * 1024)
        notes.append(f"{wl}: FETCH_SIZE x{fscale if fscale is None else round(fscale, 3)}, "
                     f"WRITE_SIZE x{wscale if wscale is None else round(wscale, 3)}")
        last = {}
        for (run, did), e in sorted(disp.items()):
            role = kernel_role(e["name"])
            if role:
                last.setdefault(role, {})
                last[role][run] = e          # the last dispatch of each run
        for role, runs in last.items():
            c, names = {}, set()
            for e in runs.values():
                c.update(e["c"])
                names.add(e["name"])
            ent = {"kernel": sorted(names)[0]}
            if "SQ_INSTS_VALU" in c:
                ent["valu_insts"] = c["SQ_INSTS_VALU"]
            for k, v in (("SQ_INSTS_LDS", "lds_insts"), ("SQ_INSTS_SALU", "salu_insts"), ("SQ_WAVES", "waves"),
                         ("SQ_INSTS_VMEM_RD", "vmem_rd_insts"), ("SQ_LDS_BANK_CONFLICT", "lds_bank_conflict")):
                if k in c:
                    ent[v] = c[k]
            if "GRBM_GUI_ACTIVE" in c:
                cyc = c["GRBM_GUI_ACTIVE"] / 8          # the counter sums the 8 XCDs
                ent["cycles"] = cyc
                if "SQ_INSTS_VALU" in c:
                    ent["valu_busy"] = round(c["SQ_INSTS_VALU"] * 4 / (1024 * cyc), 3)
            if "TCC_HIT_sum" in c and "TCC_MISS_sum" in c:
                ent["l2_hit"] = round(c["TCC_HIT_sum"] / max(1.0, c["TCC_HIT_sum"] + c["TCC_MISS_sum"]), 3)
            if "FETCH_SIZE" in c and fscale:
                ent["fetch_bytes"] = int(c["FETCH_SIZE"] * 1024 * fscale)
            if "WRITE_SIZE" in c and wscale:
                ent["write_bytes"] = int(c["WRITE_SIZE"] * 1024 * wscale)
            if "fetch_bytes" in ent and "write_bytes" in ent:
                ent["hbm_bytes"] = ent["fetch_bytes"] + ent["write_bytes"]
            entries[f"{wl}/{role}"] = ent
    doc = {"code_object": code_object_hash(), "scales": notes, "entries": entries}
    with open(out_path, "w") as f:
        json.dump(doc, f, indent=1, sort_keys=True)
    md = os.path.splitext(out_path)[0] + ".md"
    with open(md, "w") as f:
        f.write("# rocprofv3 counters of the hot kernels (generated by bench.py --ingest-counters)\n\n")
        f.write(f"Device code object: {doc['code_object']} (SHA-256 of libctproj.so's .hip_fatbin, first 16 hex).\n")
        f.write("Calibration (1 GiB device copy): " + "; ".join(notes) + ".\n\n")
        f.write("| key | kernel | VALU instr (wave) | VALU busy | LDS instr | cycles (M) | L2 hit | HBM fetch GB | "
                "HBM write GB |\n|---|---|---|---|---|---|---|---|---|\n")
        for k in sorted(entries):
            e = entries[k]
            g = lambda x, fmt: (fmt.format(e[x]) if x in e else "")
            name = e["kernel"].replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]
            f.write(f"| {k} | `{name}` | {g('valu_insts', '{:.3e}')} | "
                    f"{g('valu_busy', '{}')} | {g('lds_insts', '{:.3e}')} | "
                    f"{(format(e['cycles'] / 1e6, '.1f') if 'cycles' in e else '')} | {g('l2_hit', '{}')} | "
                    f"{(format(e['fetch_bytes'] / 1e9, '.2f') if 'fetch_bytes' in e else '')} | "
                    f"{(format(e['write_bytes'] / 1e9, '.2f') if 'write_bytes' in e else '')} |\n")
        f.write("\nEach workload `<wl>` takes four passes of one step each (`--extra` on the parallel workload adds "
                "the SIRT, weight and atomic-adjoint kernels), from /tmp, `<repo>` the repository root, `<out>` any output folder:\n\n")
        for out, pmc, cal in PMC_PASSES:
            f.write(f"    rocprofv3 --pmc {pmc} --output-format csv -d <out>/<wl> -o {out} -- "
                    f"python3 <repo>/bench.py --workload <wl> --steps 1 --warmup 0 --no-cpu-baseline [--extra]{cal}\n")
        f.write("\nthen `python3 bench.py --ingest-counters " +
                " ".join(f"{s.split('=', 1)[0]}=<out>/{s.split('=', 1)[0]}" for s in specs) + "`.\n"
                "VALU busy = SQ_INSTS_VALU x 4 cycles / (1024 SIMDs x GRBM_GUI_ACTIVE / 8 XCDs); "
                "HBM bytes = FETCH_SIZE / WRITE_SIZE in KiB x the calibration factor, which makes the counter read "
                "1 GiB for a 1 GiB device-to-device copy in the same run.\n")
    print(f"wrote {out_path} and {md}: {len(entries)} entries", flush=True)


def golden_nnz(wl, config: int):
    """The oracle's exact intersection count of the workload, if the stored
    one was made for these frames."""
    try:
        with open(GOLDEN_NNZ) as f:
            e = json.load(f)[f"c{config}"]
    except (OSError, ValueError, KeyError):
        return None
    import numpy as np
    sha = hashlib.sha256(np.ascontiguousarray(wl.frames, dtype=np.float64).tobytes()).hexdigest()
    return int(e["nnz"]) if e.get("frames_sha256") == sha else None


def packet_views(wl) -> bool:
    """Every view of the workload runs in packets (parallel, flat, a detector
    axis along an untraversed volume axis: the view table's packet slot)."""
    import ray_driven_projector_amd as rdp
    t = rdp.ct_geom_view_table(wl.beam, wl.vol_shape, wl.voxel_spacing, wl.det_shape, wl.det_spacing,
                               wl.frames)
    return bool((t[:, 47] >= 0).all()) and getattr(wl, "offsets", None) is None


def line_adjoint(wl) -> bool:
    """The workload's adjoint runs as the line kernel (decided by the library
    from the geometry description)."""
    import ray_driven_projector_amd as rdp
    return rdp.ct_geom_adjoint_kind(wl.beam, wl.vol_shape, wl.voxel_spacing, wl.det_shape, wl.det_spacing,
                                    wl.frames, surface=getattr(wl, "offsets", None) is not None) \
        == rdp.ADJOINT_LINE


def alu_roofline(kernel: str, nnz: int, ms: float, key: str, packets: bool = False, line: bool = False):
    per = OPS_LINE if line else (OPS_PACKET if packets else OPS_PER_INTERSECTION)
    ops = int(per * nnz)
    achieved = ops / (ms * 1e-3)
    c = counters(key)
    out = {"bound": "alu", "kernel": kernel, "achieved": round(achieved / 1e12, 2),
           "peak": round(VALU_PEAK / 1e12, 2), "unit": "T lane-ops/s", "frac": round(achieved / VALU_PEAK, 4),
           "traffic": None, "algorithmic_ops_per_launch": ops,
           "ops_per_intersection": per,
           "effective_hbm_frac": round(4 * nnz / (ms * 1e-3) / HBM_PEAK, 4)}
    if c:
        out["traffic"] = c.get("hbm_bytes")
        if c.get("valu_insts"):
            lanes = 64 * c["valu_insts"]
            out["measured_lane_ops_per_intersection"] = round(lanes / nnz, 2)
            out["measured_valu_frac"] = round(lanes / (ms * 1e-3) / VALU_PEAK, 4)
    return out


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


def cpu_baseline_fdk(wl, n_vox: int):
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


def say(msg: str):
    print(f"# {msg}", file=sys.stderr, flush=True)


class Timer:
    """HIP events on the launch stream around each launch."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def median_ms(self, fn, warmup=3, reps=7):
        torch = self.torch
        for _ in range(warmup):
            fn()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(self.stream)
            fn()
            e1.record(self.stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ts.sort()
        return ts[len(ts) // 2]


def kernel_names(wl, W, mode=0):
    """(forward, adjoint) kernel names; mode 0: A and A^T, 1: the SIRT pair."""
    two_d = wl.beam in (W.BEAM_PARALLEL2D, W.BEAM_FAN2D)
    persp = wl.beam in (W.BEAM_FAN2D, W.BEAM_CONE)
    sf = "true" if getattr(wl, "offsets", None) is not None else "false"
    shape = "16, 16, 1, 256" if two_d else "16, 16, 32, 512"
    fwd = (f"ray_packet_kernel<{mode}>" if packet_views(wl) else
           f"ray_kernel<{mode}, {'true' if two_d else 'false'}, {sf}>")
    if line_adjoint(wl):
        return fwd, f"line_kernel<{mode}, shape> (line adjoint)"
    return fwd, f"brick_kernel<{shape}, {mode}, {sf}, {'true' if persp else 'false'}> (packets of {PACKET})" \
        if packet_views(wl) else f"brick_kernel<{shape}, {mode}, {sf}, {'true' if persp else 'false'}>"


def config_pair(cfg, rdp, W, torch, stream, timer):
    """A of the phantom and A^T of a dense seeded sinogram on workload C<cfg>."""
    wl = W.make_workload(cfg)
    g = rdp.Geometry.from_workload(wl)
    x = torch.from_numpy(W.make_phantom(wl)).cuda()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5000 + cfg)
    y = 0.5 + torch.rand(g.sino_shape, device="cuda", generator=gen)
    sino = torch.empty(g.sino_shape, device="cuda")
    vol = torch.empty(g.vol_shape, device="cuda")
    gpu_nnz = rdp.ct_count_intersections(g)
    nnz = golden_nnz(wl, cfg)
    ms_a = timer.median_ms(lambda: rdp.ct_project(g, x, sino, stream))
    ms_at = timer.median_ms(lambda: rdp.ct_backproject(g, y, vol, stream))
    n = nnz if nnz is not None else gpu_nnz
    ka, kat = kernel_names(wl, W)
    pk = packet_views(wl)
    out = {"workload": wl.name, "nnz": n, "nnz_source": "oracle" if nnz is not None else "gpu count",
           "gpu_count_matches": gpu_nnz == n,
           "A_ms": round(ms_a, 4), "AT_ms": round(ms_at, 4),
           "A_G_intersections_per_s": round(n / (ms_a * 1e-3) / 1e9, 1),
           "AT_G_intersections_per_s": round(n / (ms_at * 1e-3) / 1e9, 1),
           "A_roofline": alu_roofline(ka, n, ms_a, f"c{cfg}/project", pk),
           "AT_roofline": alu_roofline(kat, n, ms_at, f"c{cfg}/backproject", pk, line_adjoint(wl))}
    del g, x, y, sino, vol
    torch.cuda.empty_cache()
    return out


def solver_lines(rdp, W, torch, np, stream, timer):
    """The solvers around the projector pair, timed beside the SIRT step: one
    CGLS iteration on C4 and on C5 (from y = A phantom, median of the timed
    steps after two warm-up steps), and the FDK (Ram-Lak, pad 2) of C5's
    acquisition (filter + backprojection)."""
    out = {}
    for cfg, reps in ((4, 7), (5, 3)):
        wl = W.make_workload(cfg)
        g = rdp.Geometry.from_workload(wl)
        y = torch.empty(g.sino_shape, device="cuda")
        rdp.ct_project(g, torch.from_numpy(W.make_phantom(wl)).cuda(), y, stream)
        x = torch.zeros(g.vol_shape, device="cuda")
        r = torch.empty(g.sino_shape, device="cuda")
        q = torch.empty(g.sino_shape, device="cuda")
        s_ = torch.empty(g.vol_shape, device="cuda")
        p_ = torch.empty(g.vol_shape, device="cuda")
        work = torch.empty(rdp.ct_cgls_workspace_size(g), dtype=torch.uint8, device="cuda")
        rdp.ct_cgls_init(g, y, x, r, s_, p_, work, stream)
        ms = timer.median_ms(lambda: rdp.ct_cgls_step(g, x, r, s_, p_, q, work, stream), warmup=2, reps=reps)
        out[f"c{cfg}_cgls_ms_per_iteration"] = round(ms, 3)
        del x, r, q, s_, p_, work
        if cfg == 5:
            angles = W.angles(wl.n_views, 2 * np.pi)
            fplan = rdp.FBP.from_workload(wl, angles, window="ram-lak", pad_factor=2)
            filt = torch.empty(g.sino_shape, device="cuda")
            vol = torch.empty(g.vol_shape, device="cuda")

            def fdk():
                rdp.ct_fbp_filter(fplan, y, filt, stream)
                rdp.ct_fbp_backproject(fplan, filt, vol, stream)
            ms = timer.median_ms(fdk, warmup=1, reps=3)
            out["c5_fdk_ms"] = round(ms, 3)
            out["c5_fdk_G_voxel_view_updates_per_s"] = round(wl.n_voxels * wl.n_views / (ms * 1e-3) / 1e9, 1)
            del fplan, filt, vol
        del g, y
        torch.cuda.empty_cache()
    return out


def default_run(args, rdp, W, torch, np):
    stream = torch.cuda.current_stream()
    timer = Timer(torch, stream)
    wl = W.make_workload(4)
    say(f"workload: {wl.name}")
    g = rdp.Geometry.from_workload(wl)
    x_true = torch.from_numpy(W.make_phantom(wl)).cuda()
    y = torch.empty(g.sino_shape, device="cuda")
    rdp.ct_project(g, x_true, y)                     # synthetic measurement
    gpu_nnz = rdp.ct_count_intersections(g)
    nnz = golden_nnz(wl, 4)
    if nnz is None:
        nnz = gpu_nnz
    M, N = wl.n_rays, wl.n_voxels
    say(f"nnz={nnz} (gpu count {gpu_nnz}) rays={M} voxels={N}")
    rinv = torch.empty(g.sino_shape, device="cuda")
    cinv = torch.empty(g.vol_shape, device="cuda")
    rdp.ct_sirt_weights(g, rinv, cinv)
    x = torch.zeros(g.vol_shape, device="cuda")
    work = torch.empty(g.sino_shape, device="cuda")
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def step(evs):
        evs[0].record(stream)
        rdp.ct_sirt_residual(g, x, y, rinv, work, stream)
        evs[1].record(stream)
        rdp.ct_sirt_update(g, work, cinv, 1.0, x, stream)
        evs[2].record(stream)

    for _ in range(args.warmup):
        step([ev(), ev(), ev()])
    torch.cuda.synchronize()
    all_evs = [[ev(), ev(), ev()] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(all_evs[k])
        if k == 0:
            say("step 0 enqueued")
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_res = float(np.mean([e[0].elapsed_time(e[1]) for e in all_evs]))
    ms_upd = float(np.mean([e[1].elapsed_time(e[2]) for e in all_evs]))
    ms_step = (t1 - t0) * 1e3 / args.steps
    value = 2 * nnz / (ms_step * 1e-3) / 1e9
    pk = packet_views(wl)
    kres, kupd = kernel_names(wl, W, 1)
    kernels = {"sirt_residual": (kres, ms_res), "sirt_update": (kupd, ms_upd)}
    dom = max(kernels, key=lambda k: kernels[k][1])
    res = {
        "metric": "G ray-voxel intersections/s for A and A^T; ms per SIRT iteration at 512^3",
        "value": round(value, 3),
        "unit": "G ray-voxel intersections/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name + ", one SIRT iteration (A with residual + A^T with update)",
                   "volume": list(wl.vol_shape), "views": wl.n_views, "detector": list(wl.det_shape),
                   "intersections_per_pass": nnz, "rays": M, "voxels": N},
        "ms_per_sirt_iteration": round(ms_step, 3),
        "kernel_ms": {k: round(v[1], 3) for k, v in kernels.items()},
        "roofline": alu_roofline(kernels[dom][0], nnz, kernels[dom][1], f"c4/{dom}", pk,
                                 line_adjoint(wl) and dom == "sirt_update"),
        "roofline_other": {k: alu_roofline(v[0], nnz, v[1], f"c4/{k}", pk, line_adjoint(wl) and k == "sirt_update")
                           for k, v in kernels.items() if k != dom},
    }
    del g, x_true, y, rinv, cinv, x, work
    torch.cuda.empty_cache()
    configs = {}
    for cfg in (1, 2, 3, 4, 5):
        say(f"config C{cfg}: A and A^T")
        configs[f"c{cfg}"] = config_pair(cfg, rdp, W, torch, stream, timer)
    res["configs"] = configs
    say("solvers: CGLS on C4 and C5, FDK on C5")
    res["solvers"] = solver_lines(rdp, W, torch, np, stream, timer)
    res["device_code"] = code_object_hash()
    if not args.no_cpu_baseline:
        say("cpu baseline (oracle) ...")
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_views)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


def single_run(args, rdp, W, torch, np):
    """One workload's line: --workload c1..c5 (A + A^T; c4: the SIRT step),
    c4cgls / c5cgls (CGLS iterations), c5cyl (cylindrical detector), c5fdk."""
    stream = torch.cuda.current_stream()
    cfg = int(args.workload[1])
    cgls = args.workload.endswith("cgls")
    fdk = args.workload == "c5fdk"
    wl = W.make_workload(cfg)
    if args.workload == "c5cyl":
        wl = W.with_surface(wl, W.cylinder_offsets(wl.det_shape, wl.det_spacing, 1500.0), "cylindrical")
    say(f"workload: {wl.name}")
    phantom = W.make_phantom(wl)
    g = rdp.Geometry.from_workload(wl)
    x_true = torch.from_numpy(phantom).cuda()
    y = torch.empty(g.sino_shape, device="cuda")
    rdp.ct_project(g, x_true, y)
    gpu_nnz = rdp.ct_count_intersections(g)
    nnz = golden_nnz(wl, cfg) if args.workload != "c5cyl" else None
    nnz = gpu_nnz if nnz is None else nnz
    M, N = wl.n_rays, wl.n_voxels
    say(f"nnz={nnz} (gpu count {gpu_nnz}) rays={M} voxels={N}")
    ev = lambda: torch.cuda.Event(enable_timing=True)
    ka, kat = kernel_names(wl, W)
    if fdk:
        angles = W.angles(wl.n_views, 2 * np.pi)
        fplan = rdp.FBP.from_workload(wl, angles, window="ram-lak", pad_factor=2)
        work = torch.empty(g.sino_shape, device="cuda")
        vol = torch.empty(g.vol_shape, device="cuda")
        names = ("fbp_filter", "fbp_backproject")
        n_batch = -(-wl.n_views // 128)   # gather launches of at most 128 views each

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
        ka, kat = kernel_names(wl, W, 1)

        def step(evs):
            evs[0].record(stream)
            rdp.ct_sirt_residual(g, x, y, rinv, work, stream)
            evs[1].record(stream)
            rdp.ct_sirt_update(g, work, cinv, 1.0, x, stream)
            evs[2].record(stream)
    else:
        gen = torch.Generator(device="cuda")
        gen.manual_seed(5005)
        yd = 0.5 + torch.rand(g.sino_shape, device="cuda", generator=gen)   # dense A^T input
        sino = torch.empty(g.sino_shape, device="cuda")
        vol = torch.empty(g.vol_shape, device="cuda")
        names = ("project", "backproject")

        def step(evs):
            evs[0].record(stream)
            rdp.ct_project(g, x_true, sino, stream)
            evs[1].record(stream)
            rdp.ct_backproject(g, yd, vol, stream)
            evs[2].record(stream)

    for _ in range(args.warmup):
        step([ev(), ev(), ev()])
    torch.cuda.synchronize()
    all_evs = [[ev(), ev(), ev()] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(all_evs[k])
        if k == 0:
            say("step 0 enqueued")
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = [float(np.mean([e[0].elapsed_time(e[1]) for e in all_evs])),
          float(np.mean([e[1].elapsed_time(e[2]) for e in all_evs]))]
    ms_step = (t1 - t0) * 1e3 / args.steps
    kernel_ms = {names[0]: round(ms[0], 3)}
    if not cgls:
        kernel_ms[names[1]] = round(ms[1], 3)
    res = {
        "metric": ("G voxel-view updates/s of FDK at 512^3" if fdk else
                   "G ray-voxel intersections/s for A and A^T; ms per SIRT iteration at 512^3"),
        "value": round((N * wl.n_views if fdk else 2 * nnz) / (ms_step * 1e-3) / 1e9, 3),
        "unit": "G voxel-view updates/s" if fdk else "G ray-voxel intersections/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name + (", FDK (Ram-Lak, pad 2) of y = A phantom" if fdk else
                                          ", one CGLS iteration (from y = A phantom)" if cgls else
                                          ", one SIRT iteration" if cfg == 4 else ", A + A^T"),
                   "volume": list(wl.vol_shape), "views": wl.n_views, "detector": list(wl.det_shape),
                   "intersections_per_pass": nnz, "rays": M, "voxels": N},
        "kernel_ms": kernel_ms,
        "device_code": code_object_hash(),
    }
    if fdk:
        flops = FDK_FLOPS_PER_UPDATE * N * wl.n_views // n_batch
        achieved = flops / (ms[1] / n_batch * 1e-3)
        c = counters("c5fdk/fbp_backproject")
        res["roofline"] = {"bound": "alu", "kernel": f"fbp_bp_kernel<false, false, 4, false> ({n_batch} launches per call)",
                           "achieved": round(achieved / 1e12, 2), "peak": round(ALU_PEAK / 1e12, 1),
                           "unit": "TFLOP/s", "frac": round(achieved / ALU_PEAK, 4),
                           "traffic": c.get("hbm_bytes") if c else None,
                           "algorithmic_flops_per_launch": flops,
                           "peak_note": "fp32 FMA rate without packed math (packed FP32 is not used)"}
    elif cgls:
        res["ms_per_cgls_iteration"] = round(ms_step, 3)
    else:
        dom = 0 if ms[0] >= ms[1] else 1
        kern = (ka, kat)[dom]
        res["roofline"] = alu_roofline(kern, nnz, ms[dom], f"c{cfg}/{names[dom]}",
                                       packet_views(wl) and args.workload != "c5cyl",
                                       dom == 1 and line_adjoint(wl))
        if cfg == 4:
            res["ms_per_sirt_iteration"] = round(ms_step, 3)
    if args.extra:
        out_s = torch.empty(g.sino_shape, device="cuda")
        out_v = torch.empty(g.vol_shape, device="cuda")
        timer = Timer(torch, stream)
        for name, fn, a_, b_ in (("A", rdp.ct_project, x_true, out_s), ("AT", rdp.ct_backproject, y, out_v),
                                 ("AT_atomic", rdp.ct_backproject_atomic, y, out_v)):
            t = timer.median_ms(lambda: fn(g, a_, b_, stream), warmup=1, reps=3 if name != "AT_atomic" else 1)
            res[f"{name}_ms"] = round(t, 3)
    if args.host_stream:
        nz, nb = args.host_stream
        hx = torch.from_numpy(phantom).pin_memory()
        hy = y.cpu().pin_memory()
        hs = torch.empty(g.sino_shape, pin_memory=True)
        hv = torch.empty(g.vol_shape, pin_memory=True)
        hres = {"plan": {"slab": nz, "batch_views": nb, "axis": "auto"}, "host_memory": "pinned"}
        for name, fn, a_, b_ in (("A", rdp.ct_project_host, hx, hs), ("AT", rdp.ct_backproject_host, hy, hv)):
            fn(g, a_, b_, nz, nb, stream=stream)
            ts = []
            for _ in range(3):
                t = time.perf_counter()
                fn(g, a_, b_, nz, nb, stream=stream)
                ts.append((time.perf_counter() - t) * 1e3)
            hres[f"{name}_ms"] = round(float(np.median(ts)), 2)
        n_bt = -(-wl.n_views // nb)
        vb, sb = 4 * N, 4 * M
        n_sl_a = -(-wl.vol_shape[0] // nz)
        hres["pcie_bytes"] = {"A": vb * n_bt + sb, "AT": sb * (n_sl_a if n_bt > 1 else 1) + vb}
        res["host_stream"] = hres
    if not args.no_cpu_baseline:
        say("cpu baseline (oracle) ...")
        res["cpu_baseline"] = cpu_baseline_fdk(wl, 100000) if fdk else cpu_baseline(wl, args.cpu_views)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=["c1", "c2", "c3", "c4", "c5", "c4cgls", "c5cgls", "c5cyl", "c5fdk"],
                    default=None, help="time one workload alone (default: the SIRT step plus all five configs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-views", type=int, default=16)
    ap.add_argument("--extra", action="store_true", help="also time A, A^T and atomic A^T alone")
    ap.add_argument("--host-stream", type=int, nargs=2, metavar=("SLAB", "BATCH_VIEWS"),
                    help="also time A and A^T with volume and sinogram in pinned host memory "
                         "(PCIe-inclusive; reported apart from value)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a 1 GiB device copy first (the reference kernel for HBM counters)")
    ap.add_argument("--ingest-counters", nargs="+", metavar="WL=DIR",
                    help="write profiles/counters.json from rocprofv3 --pmc output directories (no GPU)")
    args = ap.parse_args()
    if args.ingest_counters:
        ingest_counters(args.ingest_counters)
        return

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
    if args.copy_calibration:
        # a plain 1 GiB device copy (1 GiB read + 1 GiB written): the reference
        # kernel that scales the FETCH_SIZE / WRITE_SIZE counters
        src = torch.ones(1 << 28, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.workload is None:
        default_run(args, rdp, W, torch, np)
    else:
        single_run(args, rdp, W, torch, np)


if __name__ == "__main__":
    main()
