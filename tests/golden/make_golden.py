"""Writes tests/golden/*.json from the fp64 oracle only.

The pages print no worked example, so the stored values are oracle output on
seeded inputs, kept to catch any later change of the oracle's arithmetic:
  c1_step.json     one Muon step on the single fp32 256x512 workload
  small_cases.json tiny matrices (ragged, tall, square, T = 0..6) with their full NS output
Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import muon_oracle as O  # noqa: E402
import workloads as WL  # noqa: E402


def c1_step():
    wl = WL.workload(1)
    W = WL.draw(wl, 0, 0, WL.KIND_W).value
    g = WL.draw(wl, 0, 0, WL.KIND_G).value
    h = wl.hyper
    r = O.muon_step_ref(W, g, np.zeros_like(W), lr=h.lr, beta=h.beta, wd=h.wd,
                        ns_steps=h.ns_steps, coeffs=h.coeffs, eps=h.eps, param_dtype="f32")
    U = r["U"]
    return {
        "workload": wl.name, "shape": list(W.shape),
        "nu": r["nu"],
        "U_fro": float(np.linalg.norm(U)),
        "U_sum": float(U.sum()),
        "U_corner": U[:4, :4].tolist(),
        "U_last_row_head": U[-1, :8].tolist(),
        "X_rms": float(np.sqrt(np.mean(r["X"] ** 2))),
        "W_new_stored_sum": float(r["W_new_stored"].sum()),
    }


def small_cases():
    out = []
    for k, (shape, T) in enumerate([((3, 5), 5), ((5, 3), 5), ((4, 4), 2), ((2, 7), 0),
                                    ((6, 2), 6), ((1, 4), 5)]):
        M = WL.draw_custom([7, k], shape, WL.F32).value
        X0, _ = O.frobenius_normalize(M)
        out.append({"seed": [7, k], "shape": list(shape), "T": T,
                    "X": O.ns_direct(X0, T).tolist()})
    return out


if __name__ == "__main__":
    with open(os.path.join(HERE, "c1_step.json"), "w") as f:
        json.dump(c1_step(), f, indent=1)
    with open(os.path.join(HERE, "small_cases.json"), "w") as f:
        json.dump(small_cases(), f, indent=1)
    print("wrote golden fixtures")
