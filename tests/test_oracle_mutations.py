"""Mutation check of the oracle pins.

Each entry plants one plausible slip in a copy of the oracle (on the CPU: a
mutated copy of oracle/ct_oracle.c compiled into its own library, or a mutated
copy of an oracle Python module executed in that module's namespace) and runs
the pin tests against it in a child pytest process.  Every mutant must make
at least one pin fail; a mutant that survives would mean a slip of that kind
in the oracle could go unnoticed.

The slips: pixel-centre offsets, the sign of a detector axis, transposed
volume indices, a dropped length factor, wrong start cells and crossing
parameters, the half-open cell rule, the lattice origin, the adjoint's piece
midpoint and its last piece, ray-id decoding of the sampled-ray forward, the
surface normal, the row-chord layout, the brute-force cell boxes, SIRT and
CGLS recurrences, the ramp filter's taps and windows, the FDK weights,
interpolation and sampled-voxel decoding; the filter-response and
projection-weight overrides; the helical window's width, redundancy half,
quadrature, crossing angle and per-slice indexing.

Equivalent mutations (changes that cannot alter any result) are not listed:
for instance the start-cell rule of an axis at its entry face, where the
traversal's first crossing is the entry itself and the clamp puts the cell
back, or the sign of a parallel ray's direction (the rays are infinite lines).
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
C_SRC = os.path.join(ROOT, "oracle", "ct_oracle.c")
PY_SRC = {"oracle": os.path.join(ROOT, "oracle", "__init__.py"),
          "oracle.fbp": os.path.join(ROOT, "oracle", "fbp.py")}

PINS = os.path.join("tests", "test_oracle_pins.py")
FBP_PINS = os.path.join("tests", "test_oracle_fbp.py")
EXT_PINS = os.path.join("tests", "test_oracle_fbp_ext.py")
# the two sampled-line-integral pins take most of the pin file's time; every
# mutant below is caught without them
FAST = "not sampled_line_integral"

# (name, target, old, new, pin file): target "c" = ct_oracle.c, else a module
MUTANTS = [
    ("pixel offset U", "c", "0.5 * (double)(g->nu - 1)) * g->su", "0.5 * (double)(g->nu)) * g->su", PINS),
    ("pixel offset V", "c", "0.5 * (double)(g->nv - 1)) * g->sv", "0.5 * (double)(g->nv - 2)) * g->sv",
     PINS),
    ("sign of e_v", "c", "p[k] = c[k] + ou * eu[k] + (three_d ? ov * ev[k] : 0.0);",
     "p[k] = c[k] + ou * eu[k] - (three_d ? ov * ev[k] : 0.0);", PINS),
    ("forward index z/y transposed", "c", "sum += len * vol[(i[2] * n[1] + i[1]) * n[0] + i[0]];",
     "sum += len * vol[(i[1] * n[2] + i[2]) * n[0] + i[0]];", PINS),
    ("forward drops |d|", "c", "double len = (tn - t) * L;", "double len = (tn - t);", PINS),
    ("forward start cell, rising axis", "c", "c = (int64_t)floor(q); step[k] = 1;",
     "c = (int64_t)ceil(q); step[k] = 1;", PINS),
    ("forward first crossing", "c",
     "if (r->d[k] > 0)      next[k] = (lo[k] + (double)(c + 1) * s[k] - r->o[k]) / r->d[k];",
     "if (r->d[k] > 0)      next[k] = (lo[k] + (double)(c + 2) * s[k] - r->o[k]) / r->d[k];", PINS),
    ("closed cells in the clip", "c", "if (!(r->o[k] >= lo[k] && r->o[k] < hi[k])) return 0;",
     "if (!(r->o[k] >= lo[k] && r->o[k] <= hi[k])) return 0;", PINS),
    ("lattice origin off by half a cell", "c", "lo[a] = -0.5 * (double)n[a] * s[a];",
     "lo[a] = -0.5 * (double)(n[a] - 1) * s[a];", PINS),
    ("adjoint drops |d|", "c", "+= gap * L * y;", "+= gap * y;", PINS),
    ("adjoint cell from the piece start", "c", "double tm = 0.5 * (merged[q] + merged[q + 1]);",
     "double tm = merged[q];", PINS),
    ("adjoint index z/y transposed", "c", "c->vol[(cell[2] * n[1] + cell[1]) * n[0] + cell[0]]",
     "c->vol[(cell[1] * n[2] + cell[2]) * n[0] + cell[0]]", PINS),
    ("adjoint drops the last piece", "c", "merged[nm++] = tb;", "(void)tb;", PINS),
    ("sampled rays: u and v decoded swapped", "c",
     "int64_t v = id % g->nv;\n        int64_t u = (id / g->nv) % g->nu;",
     "int64_t u = id % g->nu;\n        int64_t v = (id / g->nu) % g->nv;", PINS),
    ("sampled rays: counts not kept", "c", "if (c->nnz_per) c->nnz_per[k] = nnz;",
     "if (c->nnz_per) c->nnz_per[k] = nnz + (k == 0);", PINS),
    ("2D surface normal flipped", "c", "n[0] = eu[1];\n            n[1] = -eu[0];",
     "n[0] = -eu[1];\n            n[1] = eu[0];", PINS),
    ("3D surface normal, x component", "c", "n[0] = eu[1] * ev[2] - eu[2] * ev[1];",
     "n[0] = eu[2] * ev[1] - eu[1] * ev[2];", PINS),
    ("row chords in (view, V, U) order", "c",
     "c->out[(view * g->nu + u) * g->nv + v] = ora_box_chord(&r, lo, hi);",
     "c->out[(view * g->nv + v) * g->nu + u] = ora_box_chord(&r, lo, hi);", PINS),
    ("brute-force cell decode", "c",
     "int64_t ix = j % n[0], iy = (j / n[0]) % n[1], iz = j / (n[0] * n[1]);",
     "int64_t ix = j % n[0], iy = (j / n[0]) % n[2], iz = j / (n[0] * n[2]);", PINS),
    ("box chord drops |d|", "c", "return (b - a) * norm3(r->d);", "return (b - a);", PINS),
    ("SIRT without row weights", "oracle", "e = R * (y - project(g, x, nthreads))",
     "e = (y - project(g, x, nthreads))", PINS),
    ("SIRT row weights not inverted", "oracle", "R[rs > 0] = 1.0 / rs[rs > 0]", "R[rs > 0] = rs[rs > 0]",
     PINS),
    ("SIRT mask inverted", "oracle", "np.asarray(mask).reshape(g.vol_shape) != 0, xn, x)",
     "np.asarray(mask).reshape(g.vol_shape) == 0, xn, x)", PINS),
    ("CGLS ||p||^2 for ||q||^2", "oracle", "qq = float(np.sum(q * q))", "qq = float(np.sum(p * p))", PINS),
    ("CGLS beta inverted", "oracle", "beta = gnew / gamma if gamma > 0 else 0.0",
     "beta = gamma / gnew if gnew > 0 else 0.0", PINS),
    ("CGLS sign of the r update", "oracle", "r = r - alpha * q", "r = r + alpha * q", PINS),
    ("CGLS p = s + beta s", "oracle", "p = s + beta * p", "p = s + beta * s", PINS),
    ("CGLS x += alpha s", "oracle", "x = x + alpha * p", "x = x + alpha * s", PINS),
    ("Ram-Lak centre tap", "oracle.fbp", "h[n == 0] = 1.0 / (4.0 * spacing * spacing)",
     "h[n == 0] = 1.0 / (2.0 * spacing * spacing)", FBP_PINS),
    ("Ram-Lak odd taps", "oracle.fbp", "h[odd] = -1.0 / (math.pi * n[odd] * spacing) ** 2",
     "h[odd] = -2.0 / (math.pi * n[odd] * spacing) ** 2", FBP_PINS),
    ("cosine window at twice the frequency", "oracle.fbp", "return np.cos(math.pi * f)",
     "return np.cos(2 * math.pi * f)", FBP_PINS),
    ("Shepp-Logan window at twice the frequency", "oracle.fbp", "return np.sinc(f)", "return np.sinc(2 * f)",
     FBP_PINS),
    ("Hamming coefficients", "oracle.fbp", "return 0.54 + 0.46 * np.cos(2 * math.pi * f)",
     "return 0.46 + 0.54 * np.cos(2 * math.pi * f)", FBP_PINS),
    ("Hann as cosine", "oracle.fbp", "return 0.5 + 0.5 * np.cos(2 * math.pi * f)",
     "return np.cos(math.pi * f)", FBP_PINS),
    ("no cosine pre-weight", "oracle.fbp", "pre = cosine_weights(wl)", "pre = np.ones(wl.sino_shape)", FBP_PINS),
    ("Parker fan angle sign", "oracle.fbp", "return rotation_sense(wl) * np.arctan2(cross, dot)",
     "return -rotation_sense(wl) * np.arctan2(cross, dot)", FBP_PINS),
    ("angular weights without the redundancy half", "oracle.fbp",
     "return w * (0.5 if redundant else 1.0)", "return w", FBP_PINS),
    ("half a bin in u", "oracle.fbp", "u = (P - c) @ eu / du + 0.5 * (U - 1)", "u = (P - c) @ eu / du + 0.5 * U",
     FBP_PINS),
    ("half a bin in v", "oracle.fbp", "v = (P - c) @ ev / dv + 0.5 * (V - 1)", "v = (P - c) @ ev / dv + 0.5 * V",
     FBP_PINS),
    ("FDK weight (R/U)^2", "oracle.fbp", "wgt = np.where(front, R * D / Us ** 2, 0.0)",
     "wgt = np.where(front, (R / Us) ** 2, 0.0)", FBP_PINS),
    ("points behind the source gather", "oracle.fbp", "front = Ux > 0", "front = Ux > -1e300", FBP_PINS),
    ("bilinear coefficients swapped", "oracle.fbp", "for su, cu in ((0, 1 - au), (1, au)):",
     "for su, cu in ((0, au), (1, 1 - au)):", FBP_PINS),
    ("sampled voxels: x and y decoded swapped", "oracle.fbp",
     "X = np.stack([x[ids % Wd], y[(ids // Wd) % H], z[ids // (Wd * H)]], axis=-1)",
     "X = np.stack([x[(ids // H) % Wd], y[ids % H], z[ids // (Wd * H)]], axis=-1)", FBP_PINS),
    ("scatter index u/v swapped", "oracle.fbp", "np.add.at(out[i], (ju.ravel(), jv.ravel()), (wgt * cf * vol)",
     "np.add.at(out[i], (jv.ravel() % U, ju.ravel() % V), (wgt * cf * vol)", FBP_PINS),
    ("filter response ignored", "oracle.fbp", "M = np.asarray(response, dtype=np.float64)",
     "M = ramp_multiplier(P, spacing, window)", EXT_PINS),
    ("projection weights ignored", "oracle.fbp", "pre = np.broadcast_to(pw, wl.sino_shape)",
     "pre = cosine_weights(wl)", EXT_PINS),
    ("helical window of half a turn", "oracle.fbp", "lo, hi = tc - math.pi, tc + math.pi",
     "lo, hi = tc - math.pi / 2, tc + math.pi / 2", EXT_PINS),
    ("helical weights without the redundancy half", "oracle.fbp",
     "w[s, i] = 0.5 * _hat_integral(t, i, lo, hi)", "w[s, i] = _hat_integral(t, i, lo, hi)", EXT_PINS),
    ("hat integral, rising side over L", "oracle.fbp",
     "total += ((b - t[i - 1]) ** 2 - (a - t[i - 1]) ** 2) / (2 * L)",
     "total += ((b - t[i - 1]) ** 2 - (a - t[i - 1]) ** 2) / L", EXT_PINS),
    ("crossing angle of the sample below", "oracle.fbp", "out[s] = th[k] + f * (th[k + 1] - th[k])",
     "out[s] = th[k]", EXT_PINS),
    ("crossing fraction from the upper sample", "oracle.fbp", "f = (zc - zs[k]) / (zs[k + 1] - zs[k])",
     "f = (zs[k + 1] - zc) / (zs[k + 1] - zs[k])", EXT_PINS),
    ("slice weights of the mirrored slice", "oracle.fbp", "out += wts[:, i][:, None, None] * wgt * val",
     "out += wts[::-1, i][:, None, None] * wgt * val", EXT_PINS),
    ("helical scatter drops the slice weights", "oracle.fbp", "g = wts[:, i][:, None, None] * wgt * vol",
     "g = wgt * vol", EXT_PINS),
    ("helical FDK keeps the angular weights", "oracle.fbp",
     "q = filter_sinogram(wl, sino, angles, window, pad_factor, False, np.ones(wl.n_views),",
     "q = filter_sinogram(wl, sino, angles, window, pad_factor, False, None,", EXT_PINS),
]


def _source(target):
    return C_SRC if target == "c" else PY_SRC[target]


@pytest.mark.parametrize("name,target,old,new,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutation_applies_once(name, target, old, new, pins):
    with open(_source(target)) as f:
        assert f.read().count(old) == 1, f"{name}: the text to mutate must occur exactly once"


def _run_mutant(tmp, idx, name, target, old, new, pins):
    with open(_source(target)) as f:
        src = f.read()
    mutated = src.replace(old, new)
    env = dict(os.environ)
    env.pop("ORACLE_MUTANT_LIB", None)
    env.pop("ORACLE_MUTANT_PY", None)
    if target == "c":
        path = os.path.join(tmp, f"m{idx}.c")
        with open(path, "w") as f:
            f.write(mutated)
        lib = oracle.compile_library(path, os.path.join(tmp, f"libm{idx}.so"))
        env["ORACLE_MUTANT_LIB"] = lib
    else:
        path = os.path.join(tmp, f"m{idx}.py")
        with open(path, "w") as f:
            f.write(mutated)
        env["ORACLE_MUTANT_PY"] = f"{target}={path}"
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "tests.mutant_plugin", "-m", "not gpu",
           "-k", FAST, pins]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    failed = [ln for ln in r.stdout.splitlines() if ln.startswith("FAILED")]
    return name, r.returncode, failed, r.stdout[-2000:]


def test_every_mutant_fails_a_pin(tmp_path):
    # the unmutated oracle passes the same selection (a control run)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "tests.mutant_plugin", "-m", "not gpu",
                        "-k", FAST, PINS, FBP_PINS, EXT_PINS], cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]
    with ThreadPoolExecutor(max_workers=min(8, oracle.default_threads())) as ex:
        results = list(ex.map(lambda a: _run_mutant(str(tmp_path), *a),
                              [(i, *m) for i, m in enumerate(MUTANTS)]))
    survivors = []
    for name, rc, failed, tail in results:
        print(f"{name:45s} rc={rc} caught by {failed[0] if failed else '-'}")
        # rc 1: tests failed; a negative rc would be a crash of the mutated oracle
        if rc != 1 or not failed:
            survivors.append((name, rc, tail))
    assert not survivors, survivors
