"""The per-row / per-column bound of the full-size parity tests catches what
the relative Frobenius bound alone lets through.

A defect is planted, on the CPU, into a copy of an oracle update: evenly
spread noise at 1.0e-2 relative Frobenius error (about what bf16 rounding
gives) plus one zeroed column of a 1024 x 4096 update.  The zeroed column
adds ~1.6e-2 in quadrature, so the Frobenius error stays under 2e-2, while
that column's line error is 1 and fails the 2.5 x 2e-2 line bound."""
import numpy as np
import pytest

import workloads as WL
from oracle import muon_oracle as O


def _oracle_update(shape):
    W = WL.draw_custom([5, 0], shape, WL.BF16, "normal", 0.02)
    G = WL.draw_custom([5, 1], shape, WL.BF16, "normal", 0.02)
    return O.muon_step_ref(W.value, G.value, np.zeros(shape), param_dtype="bf16")["U"]


@pytest.fixture(scope="module")
def U_ref():
    return _oracle_update((1024, 4096))


def _noisy(U, rel, seed):
    rng = np.random.default_rng(seed)
    n = rng.standard_normal(U.shape)
    return U + n * (rel * np.linalg.norm(U) / np.linalg.norm(n))


def test_even_noise_passes_both_bounds(U_ref):
    from gpu_util import check_lines, rel, REL_TOL
    U = _noisy(U_ref, 1.0e-2, 1)
    assert rel(U, U_ref) <= REL_TOL[WL.BF16]
    row, col = check_lines(U, U_ref, REL_TOL[WL.BF16], "noise only")
    assert row < 0.02 and col < 0.02


@pytest.mark.parametrize("axis", [0, 1])
def test_zeroed_line_passes_frobenius_but_fails_line_bound(U_ref, axis):
    from gpu_util import check_lines, rel, REL_TOL
    U = _noisy(U_ref, 1.0e-2, 2)
    if axis == 0:
        U[:, 1234] = 0.0          # one column of 1024 elements
    else:
        # a 2 x 512 strip: as many elements as one column, an eighth of two rows
        U[100:102, 2048:2560] = 0.0
    e = rel(U, U_ref)
    assert e <= REL_TOL[WL.BF16], e
    with pytest.raises(AssertionError, match="worst"):
        check_lines(U, U_ref, REL_TOL[WL.BF16], "planted defect")
