"""Write tests/golden/nnz_configs.json: the exact intersection counts of the
five synthetic workloads, from the float64 oracle's forward traversal.

An intersection is a (ray, voxel) pair whose float64 piece length is positive
(the oracle's count; the lengths do not depend on the voxel values, so the
traversal runs on a volume of ones).  The oracle also reports its tie events
(a ray lying in a lattice plane, or crossing two planes at one point).  Each
entry carries a SHA-256 of the workload's frames so a reader can tell that it
was made for the same geometry.

Calls only the oracle and the seeded input generators.  Run from the
repository root:

    python tests/golden/make_nnz.py            # all five workloads
    python tests/golden/make_nnz.py 1 2 3      # a subset (merged into the file)

The 512^3 workloads take minutes on a many-core host (about 3e11 walk steps
for the jittered cone).
"""
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from ray_driven_projector_amd import workloads as W  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "nnz_configs.json")


def frames_sha(wl) -> str:
    return hashlib.sha256(np.ascontiguousarray(wl.frames, dtype=np.float64).tobytes()).hexdigest()


def count(config: int) -> dict:
    wl = W.make_workload(config)
    g = oracle.Geometry.from_workload(wl)
    t0 = time.time()
    _, nnz, ties = oracle.project(g, np.ones(wl.vol_shape), with_counts=True)
    return {"workload": wl.name, "nnz": int(nnz), "ties": int(ties), "rays": int(wl.n_rays),
            "voxels": int(wl.n_voxels), "frames_sha256": frames_sha(wl),
            "oracle_seconds": round(time.time() - t0, 1), "threads": oracle.default_threads()}


def main(argv):
    configs = [int(a) for a in argv] or [1, 2, 3, 4, 5]
    data = {}
    if os.path.exists(OUT):
        with open(OUT) as f:
            data = json.load(f)
    for c in configs:
        data[f"c{c}"] = count(c)
        print(f"c{c}: {data[f'c{c}']}", flush=True)
        with open(OUT, "w") as f:
            json.dump(data, f, indent=1, sort_keys=True)
            f.write("\n")


if __name__ == "__main__":
    main(sys.argv[1:])
