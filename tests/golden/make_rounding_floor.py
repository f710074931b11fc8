"""Write rounding_floor.json: the bf16 rounding-placement model's error vs the
fp64 oracle on each named workload (sampled slices for stacks).

Calls only oracle/ (ns_oracle and the rounding model) and the seeded input
recipes.  Run from the repository root:

    python tests/golden/make_rounding_floor.py [NAME ...]

With names, only those workloads are recomputed and merged into the existing
file.
"""

import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from ns_inputs import WORKLOADS, make_workload  # noqa: E402
from oracle import newton_schulz  # noqa: E402
from oracle.rounding_model import ns_bf16_model  # noqa: E402

SAMPLES = {"experts16_1536x2048": [0, 7, 15], "experts128_1536x2048": [0, 63, 127],
           "experts32_7168x2048": [0, 31], "experts128_2048x768": [0, 64, 127]}
NAMES = ["iid_256x512", "lowrank64_4096x4096", "mlp_4096x14336", "experts16_1536x2048", "experts128_1536x2048",
         "experts32_7168x2048", "square_8192x8192", "experts128_2048x768"]


def rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def main(names):
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "rounding_floor.json")
    out = {"what": "relative Frobenius error vs the fp64 oracle of the CPU bf16 rounding model "
                   "(oracle/rounding_model.py). 'shipped': the diagonal split with the normalisation "
                   "folded into the first step (X0 never rounded), the placement the HIP kernels use; "
                   "'literal': bf16 A, B and X with a stored bf16 X0, the plain reading",
           "workloads": {}}
    if names:
        with open(path) as f:
            out["workloads"] = json.load(f)["workloads"]
    for name in names or NAMES:
        t0 = time.time()
        w = WORKLOADS[name]
        x = make_workload(name)
        xs = x.reshape(-1, w.rows, w.cols)
        rec = {}
        for i in SAMPLES.get(name, [0]):
            xi = xs[i]
            ref = newton_schulz(xi.double().numpy())          # oracle reads the given tensor
            xb = xi.to(torch.bfloat16).double().numpy()         # the bf16 path's input
            rec[str(i)] = {"shipped": rel(ns_bf16_model(xb), ref),
                           "literal": rel(ns_bf16_model(xb, placement="literal", fold_norm=False), ref)}
        out["workloads"][name] = rec
        print(name, rec, f"{time.time() - t0:.0f}s", flush=True)
    # the transposed MLP weight has the same floor (NS(Xᵀ) = NS(X)ᵀ)
    out["workloads"]["mlp_14336x4096"] = out["workloads"]["mlp_4096x14336"]
    with open(path, "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main(sys.argv[1:])
