"""The per-row / per-column bound of the full-size parity tests catches what
the relative Frobenius bound alone lets through, and is wide enough for what
bf16 rounding itself does to single lines.

A defect is planted, on the CPU, into a copy of an oracle update: evenly
spread noise at 1.0e-2 relative Frobenius error (about what bf16 rounding
gives) plus one zeroed column of a 1024 x 4096 update.  The zeroed column
adds ~1.6e-2 in quadrature, so the Frobenius error stays under 2e-2, while
that column's line error is 1 and fails the 5 x 2e-2 line bound.

The bound's width: a numpy model of the bf16 path's operand rounding (every
NS operand and product output rounded to bf16 where the kernels store bf16,
fp64 accumulation; a model for sizing the bound, not the oracle) on the
heavy-tailed workload's 512 x 512 matrix 137 gives a worst row near 0.05,
five times the 1e-2 Frobenius error, while Gaussian inputs stay within 2x."""
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


def _bf16_model(W, g, T=5, a=3.4445, b=-4.7750, c=2.0315, lr=0.02, wd=0.01, beta=0.95):
    """Nesterov direction from zero momentum, rounded to fp32 then bf16; per NS
    step A, B (with a I folded in) and X' rounded to bf16, the last X' kept."""
    def bf(x):
        return O.round_to_bf16(np.asarray(x, np.float64))
    rows, cols = W.shape
    d = (g + beta * g).astype(np.float32).astype(np.float64)
    r = 1.0 / (np.sqrt(np.sum(d * d)) + 1e-7)
    X = bf(d.T if rows > cols else d)
    for k in range(T):
        A = bf((r * r if k == 0 else 1.0) * (X @ X.T))
        B = bf(c * (A @ A) + b * A + a * np.eye(A.shape[0]))
        Xn = (r if k == 0 else 1.0) * (B @ X)
        X = Xn if k == T - 1 else bf(Xn)
    X = X.T if rows > cols else X
    return -lr * (wd * W + 0.2 * np.sqrt(max(rows, cols)) * X)


@pytest.mark.parametrize("cfg,idx,lo,hi", [(3, 137, 4.0, 5.5), (5, 0, 1.0, 2.0)])
def test_bf16_rounding_worst_line_sizes_the_bound(cfg, idx, lo, hi):
    from gpu_util import line_errors, LINE_FACTOR, REL_TOL
    wl = WL.workload(cfg)
    W, G = WL.draw(wl, idx, 0, WL.KIND_W), WL.draw(wl, idx, 0, WL.KIND_G)
    ref = O.muon_step_ref(W.value, G.value, np.zeros(W.value.shape), param_dtype="bf16")["U"]
    U = _bf16_model(W.value, G.value)
    e = np.linalg.norm(U - ref) / np.linalg.norm(ref)
    worst = max(line_errors(U - ref, ref))
    assert 5e-3 < e < REL_TOL[WL.BF16]
    assert lo * e < worst < hi * e, (worst, e)
    assert worst <= LINE_FACTOR * REL_TOL[WL.BF16]
