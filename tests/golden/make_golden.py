"""Write tests/golden/tiny_f32.json from the oracle alone.

    python tests/golden/make_golden.py

The tiny fp32 workload (one 8x8 latent frame, C=16, one layer d=64, two
heads, Jacobi block 16, tau 1e-3, seed 0): the oracle's forward of x ~ N(0,1)
(seed 2) and its block-Jacobi inverse of z ~ N(0,1) (seed 1).  The pages print
no worked numbers for this path, so this fixture pins the oracle against
itself over time: a change to its arithmetic shows here and must name the
passage that justifies it.
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

from autoregressive_normalizing_flow_amd import synth  # noqa: E402
from oracle import af_oracle as O  # noqa: E402


def main():
    w = synth.WORKLOADS["tiny_f32"]
    p = O.to64(synth.make_params(w.block, 0)[0])
    x = synth.normal((1, 64, 16), 2)
    z = synth.normal((1, 64, 16), 1)
    zf, ld = O.forward_block(p, x, 2)
    xj, it = O.inverse_jacobi_block(p, z, 2, 16, 1e-3)
    xs = O.inverse_sequential_block(p, z, 2)
    out = {
        "workload": "tiny_f32", "seed_params": 0, "seed_z": 1, "seed_x": 2,
        "forward_logdet": float(ld[0]),
        "forward_z_first_token": zf[0, 0].tolist(),
        "forward_z_last_token": zf[0, -1].tolist(),
        "forward_z_sum": float(zf.sum()), "forward_z_sumsq": float((zf ** 2).sum()),
        "jacobi_iters": it.tolist(),
        "jacobi_x_last_token": xj[0, -1].tolist(),
        "jacobi_x_sumsq": float((xj ** 2).sum()),
        "sequential_x_last_token": xs[0, -1].tolist(),
    }
    with open(os.path.join(HERE, "tiny_f32.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
