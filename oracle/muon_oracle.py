"""fp64 CPU oracle for the Muon per-owner update step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers or constants); both sides receive the
same seeded inputs from ``workloads``.

Every quantity is fp64.  Inputs are read exactly from their stored fp32 /
bf16 values.  The functions follow the method as the pages describe it:

* "DeepSpeed now supports Muon" (setupai.cc, section "technical deep dive"):
  Muon orthogonalizes the momentum-based update with Newton-Schulz
  iterations, is applied to 2-D weight matrices (conv filters flattened),
  needs decoupled weight decay and a per-parameter update scale, and that
  scale is chosen by RMS matching so AdamW's lr and wd carry over.
* DMuon announcement (wjxwpt.net), improvement 2 "shape-adaptive execution
  stack", item 1: the NS iteration can be moved from the m x n matrix space
  into the m x m Gram space.  The page is cut off mid-sentence there; the
  recursion in ``ns_gram`` is the plainest reading (every iterate is a
  polynomial in G = X0 X0^T, so it is exact in exact arithmetic).
* DMuon announcement, "three improvements" preamble: DMuon does not change
  the parameter update rule, so every execution form must give this result.

Where the pages are silent the readings are:
  momentum   SGD-Nesterov: buf <- beta*buf + g, d <- g + beta*buf (with
             nesterov=False the plain buffer: d <- buf, the library's option).
  normalize  X0 = d / (||d||_F + eps), eps = 1e-7.
  polynomial odd quintic X <- a X + b (X X^T) X + c (X X^T)^2 X, the same
             (a, b, c) each step unless a per-step schedule is given.
  orientation work on the smaller side (transpose when rows > cols).
  scale      s = 0.2 * sqrt(max(rows, cols)).
  apply      U = -lr * (wd * W + s * X_T);  W_new = W + U  (old W in both).

Pins (tests/test_oracle_pins.py) tie every function here to something other
than itself: the SVD closed form of the matrix polynomial, convergence of the
cubic iteration to scipy's polar factor, Gram == direct, orientation and
orthogonal equivariance, the momentum closed forms (Nesterov and plain), the
whole step on shared singular vectors (both momentum forms), RMS = 0.2 for an exact
polar factor, and the zero-gradient / lr = 0 / ns_steps = 0 special cases.
No function here is parity-unpinned.
"""
from __future__ import annotations

from typing import Iterable, Sequence

import numpy as np

QUINTIC = (3.4445, -4.7750, 2.0315)
CUBIC = (1.5, -0.5, 0.0)


def coeff_schedule(coeffs, ns_steps: int) -> np.ndarray:
    """(a, b, c) per step as a (T, 3) fp64 array.

    A single triple is used for every step; a (T, 3) array is a per-step schedule."""
    c = np.asarray(coeffs, dtype=np.float64)
    if c.ndim == 1:
        if c.shape[0] != 3:
            raise ValueError("coeffs must be (a, b, c) or a (T, 3) schedule")
        return np.tile(c, (ns_steps, 1))
    if c.shape != (ns_steps, 3):
        raise ValueError(f"schedule shape {c.shape} != ({ns_steps}, 3)")
    return c


def nesterov_momentum(buf: np.ndarray, g: np.ndarray, beta: float):
    """One Nesterov momentum step (the 'momentum-based update' Muon orthogonalizes).

    buf_new = beta*buf + g;  d = g + beta*buf_new.  Returns (buf_new, d)."""
    buf = np.asarray(buf, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    buf_new = beta * buf + g
    d = g + beta * buf_new
    return buf_new, d


def plain_momentum(buf: np.ndarray, g: np.ndarray, beta: float):
    """Plain (heavy-ball) momentum, the library's option with Nesterov off:
    buf_new = beta*buf + g;  d = buf_new.  Returns (buf_new, d)."""
    buf = np.asarray(buf, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    buf_new = beta * buf + g
    return buf_new, buf_new.copy()


def frobenius_normalize(d: np.ndarray, eps: float = 1e-7):
    """X0 = d / (||d||_F + eps): puts every singular value of X0 in [0, 1]."""
    d = np.asarray(d, dtype=np.float64)
    nu = float(np.sqrt(np.sum(d * d)))
    return d / (nu + eps), nu


def ns_direct(X0: np.ndarray, ns_steps: int, coeffs=QUINTIC) -> np.ndarray:
    """Newton-Schulz in matrix space: per step A = X X^T, B = b A + c A^2, X <- a X + B X.

    Runs on the smaller side (a tall matrix is transposed, iterated, transposed back)."""
    X = np.asarray(X0, dtype=np.float64)
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T
    sched = coeff_schedule(coeffs, ns_steps)
    for a, b, c in sched:
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X.T.copy() if tall else X


def ns_gram(X0: np.ndarray, ns_steps: int, coeffs=QUINTIC) -> np.ndarray:
    """Newton-Schulz carried out in the m x m Gram space (m = smaller side).

    With G = X0 X0^T every iterate is X_k = Q_k X0, Q_k a polynomial in G, so
    A_k = X_k X_k^T = Q_k G Q_k.  One step is H = a I + b A + c A^2,
    Q <- H Q, A <- H A H; the result is X_T = Q_T X0."""
    X = np.asarray(X0, dtype=np.float64)
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T
    m = X.shape[0]
    sched = coeff_schedule(coeffs, ns_steps)
    I = np.eye(m)
    G = X @ X.T
    A = G
    Q = I
    for k, (a, b, c) in enumerate(sched):
        H = a * I + b * A + c * (A @ A)
        Q = H @ Q
        if k + 1 < len(sched):
            A = H @ A @ H
    out = Q @ X
    return out.T.copy() if tall else out


def orthogonalize_ref(M, ns_steps: int = 5, coeffs=QUINTIC, eps: float = 1e-7,
                      form: str = "direct") -> np.ndarray:
    """The orthogonalization Muon applies to its update, on its own: M scaled to
    unit Frobenius norm (plus eps), then ns_steps Newton-Schulz steps.
    "DeepSpeed now supports Muon" (setupai.cc), technical deep dive."""
    X0, _ = frobenius_normalize(M, eps)
    if form == "direct":
        return ns_direct(X0, ns_steps, coeffs)
    if form == "gram":
        return ns_gram(X0, ns_steps, coeffs)
    raise ValueError(form)


def rms_scale(rows: int, cols: int, base: float = 0.2) -> float:
    """Update scale chosen by RMS matching: an exact polar factor of a full-rank
    rows x cols matrix has RMS 1/sqrt(max(rows, cols)), so s*X has RMS `base`."""
    return base * float(np.sqrt(max(rows, cols)))


def apply_update(W: np.ndarray, X: np.ndarray, lr: float, wd: float, s: float):
    """Decoupled weight decay plus the scaled orthogonal step, both on the old W.

    Returns (U, W_new) with U = -lr*(wd*W + s*X) and W_new = W + U."""
    W = np.asarray(W, dtype=np.float64)
    U = -lr * (wd * W + s * np.asarray(X, dtype=np.float64))
    return U, W + U


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 -> nearest bf16 (ties to even), returned as fp64 values.

    Direct rounding on the fp64 bit pattern (no fp32 intermediate); valid for
    finite values inside bf16's normal range."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    u = x.view(np.uint64)
    drop = np.uint64(45)                 # 52 fp64 mantissa bits -> 7 bf16 bits
    lsb = (u >> drop) & np.uint64(1)
    half = np.uint64((1 << 44) - 1)
    r = ((u + half + lsb) >> drop) << drop
    return r.view(np.float64)


def round_to_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def muon_step_ref(W, g, buf, *, lr: float = 0.02, beta: float = 0.95, wd: float = 0.01,
                  ns_steps: int = 5, coeffs=QUINTIC, eps: float = 1e-7,
                  rms_base: float = 0.2, form: str = "direct", param_dtype: str = "f32",
                  nesterov: bool = True):
    """One Muon update of one matrix, every step in fp64.

    nesterov=False orthogonalizes the plain momentum buffer instead of the
    Nesterov direction (the library's option of the same name).

    Returns a dict: U (the update), buf_new, W_new (fp64), W_new_stored (rounded to
    the parameter dtype), X (the NS output), nu (the Frobenius norm of d)."""
    W = np.asarray(W, dtype=np.float64)
    rows, cols = W.shape
    buf_new, d = (nesterov_momentum if nesterov else plain_momentum)(buf, g, beta)
    X0, nu = frobenius_normalize(d, eps)
    if form == "direct":
        X = ns_direct(X0, ns_steps, coeffs)
    elif form == "gram":
        X = ns_gram(X0, ns_steps, coeffs)
    else:
        raise ValueError(form)
    s = rms_scale(rows, cols, rms_base)
    U, W_new = apply_update(W, X, lr, wd, s)
    stored = round_to_bf16(W_new) if param_dtype == "bf16" else round_to_f32(W_new)
    return {"U": U, "buf_new": buf_new, "W_new": W_new, "W_new_stored": stored,
            "X": X, "nu": nu}


def muon_steps_ref(Ws: Sequence[np.ndarray], grads: Iterable[Sequence[np.ndarray]],
                   bufs: Sequence[np.ndarray], **kw):
    """Several consecutive steps over a list of matrices (fresh grads per step,
    momenta carried over, weights carried over in their stored dtype).

    ``grads`` yields one list of per-matrix gradients per step.  Returns the last
    step's per-matrix result dicts and the carried state."""
    Ws = [np.asarray(w, dtype=np.float64) for w in Ws]
    bufs = [np.asarray(b, dtype=np.float64) for b in bufs]
    last = None
    for step_grads in grads:
        last = []
        for i, g in enumerate(step_grads):
            r = muon_step_ref(Ws[i], g, bufs[i], **kw)
            Ws[i] = r["W_new_stored"]
            bufs[i] = round_to_f32(r["buf_new"])
            last.append(r)
    return last, Ws, bufs

