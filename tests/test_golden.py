"""The stored oracle fixtures (tests/golden, written by make_golden.py from the
oracle alone) still match the oracle, and the small cases also match the SVD
closed form of the NS polynomial."""
import json
import os

import numpy as np

from oracle import muon_oracle as O
import workloads as WL

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_c1_step_fixture():
    want = json.load(open(os.path.join(GOLD, "c1_step.json")))
    wl = WL.workload(1)
    W = WL.draw(wl, 0, 0, WL.KIND_W).value
    g = WL.draw(wl, 0, 0, WL.KIND_G).value
    h = wl.hyper
    r = O.muon_step_ref(W, g, np.zeros_like(W), lr=h.lr, beta=h.beta, wd=h.wd,
                        ns_steps=h.ns_steps, coeffs=h.coeffs, eps=h.eps)
    assert abs(r["nu"] - want["nu"]) <= 1e-12 * want["nu"]
    assert abs(np.linalg.norm(r["U"]) - want["U_fro"]) <= 1e-12 * want["U_fro"]
    assert np.allclose(r["U"][:4, :4], np.array(want["U_corner"]), rtol=1e-11, atol=1e-16)
    assert np.allclose(r["U"][-1, :8], np.array(want["U_last_row_head"]), rtol=1e-11, atol=1e-16)


def test_small_case_fixtures_and_svd():
    for case in json.load(open(os.path.join(GOLD, "small_cases.json"))):
        M = WL.draw_custom(case["seed"], tuple(case["shape"]), WL.F32).value
        X0, _ = O.frobenius_normalize(M)
        got = O.ns_direct(X0, case["T"])
        assert np.allclose(got, np.array(case["X"]), rtol=1e-12, atol=1e-15)
        U, S, Vt = np.linalg.svd(X0, full_matrices=False)
        s = S.copy()
        for _ in range(case["T"]):
            s = 3.4445 * s - 4.7750 * s ** 3 + 2.0315 * s ** 5
        assert np.allclose(got, (U * s) @ Vt, rtol=1e-11, atol=1e-13)


def test_workload_generator_is_deterministic_and_stored_exactly():
    wl = WL.workload(2)
    a = WL.draw(wl, 3, 1, WL.KIND_G, shape=(8, 16))
    b = WL.draw(wl, 3, 1, WL.KIND_G, shape=(8, 16))
    assert np.array_equal(a.raw, b.raw)
    assert a.raw.dtype == np.uint16
    # stored value is exactly the bf16 pattern
    back = (a.raw.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(back, a.value)
    c = WL.draw(wl, 3, 2, WL.KIND_G, shape=(8, 16))
    assert not np.array_equal(a.raw, c.raw)
