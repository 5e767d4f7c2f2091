"""Helpers of the GPU parity tests: seeded inputs to device tensors, results back
to exact fp64, and the oracle driven on the same stored values."""
import numpy as np
import torch

import workloads as WL
from oracle import muon_oracle as O

REL_TOL = {WL.F32: 1e-4, WL.BF16: 2e-2}
# A row or column of U may carry at most this multiple of the Frobenius
# tolerance, measured as the norm of the line's error over max(the line's own
# norm, the RMS norm of all lines).  With Gaussian inputs bf16 rounding gives
# worst lines within about 2x the Frobenius error; heavy-tailed (Student-t)
# gradients concentrate it on the lines that carry the outliers, up to about
# 5x (0.05 on a 512 x 512 matrix, which a numpy model of the bf16 operand
# rounding reproduces: tests/test_line_check_cpu.py).  A wrong row, column or
# strip has a line error near 1, ten times the bound.
LINE_FACTOR = 5.0
LINE_MIN_LEN = 256


def line_errors(d, ref):
    """(largest row error, largest column error) of d = U - U_ref against ref,
    each line's error norm over max(its own norm, the RMS norm of the lines)."""
    out = []
    for ax in (1, 0):
        err = np.sqrt(np.sum(d * d, axis=ax))
        nrm = np.sqrt(np.sum(ref * ref, axis=ax))
        rms = np.sqrt(np.mean(nrm * nrm))
        out.append(float(np.max(err / np.maximum(nrm, rms))) if rms > 0 else float(np.max(err)))
    return out


def check_lines(U, ref, tol, what):
    """Asserts the per-row and per-column bound on lines of >= LINE_MIN_LEN
    elements (rows when there are that many columns, and vice versa)."""
    row, col = line_errors(U - ref, ref)
    rows, cols = ref.shape
    if cols >= LINE_MIN_LEN:
        assert row <= LINE_FACTOR * tol, f"{what}: worst row error {row:.3e} > {LINE_FACTOR * tol:.1e}"
    if rows >= LINE_MIN_LEN:
        assert col <= LINE_FACTOR * tol, f"{what}: worst column error {col:.3e} > {LINE_FACTOR * tol:.1e}"
    return row, col


def to_device(stored):
    if stored.dtype == WL.F32:
        return torch.from_numpy(np.ascontiguousarray(stored.raw)).cuda()
    bits = np.ascontiguousarray(stored.raw).view(np.int16)
    return torch.from_numpy(bits).view(torch.bfloat16).cuda()


def to_f64(t):
    t = t.detach()
    if t.dtype == torch.bfloat16:
        bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return WL.bf16_bits_to_f64(bits)
    return t.float().cpu().numpy().astype(np.float64)


def rel(a, b):
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a - b))


def make_state(shapes, dtype, seed, grad_law="normal", grad_scale=0.02, w_scale=0.02,
               buf_scale=0.0):
    """Seeded params / grads / momenta for arbitrary shapes (edge and ragged cases)."""
    Ws, Gs, Bs = [], [], []
    for i, shp in enumerate(shapes):
        Ws.append(WL.draw_custom([seed, i, 0], shp, dtype, "normal", w_scale))
        Gs.append(WL.draw_custom([seed, i, 1], shp, dtype, grad_law, grad_scale))
        if buf_scale:
            Bs.append(WL.draw_custom([seed, i, 2], shp, WL.F32, "normal", buf_scale))
        else:
            Bs.append(WL.Stored(np.zeros(shp), np.zeros(shp, np.float32), WL.F32))
    return Ws, Gs, Bs


def device_state(Ws, Gs, Bs):
    return [to_device(w) for w in Ws], [to_device(g) for g in Gs], [to_device(b) for b in Bs]


def run_and_compare(plan, Ws, Gs, Bs, dtype, *, lr=0.02, beta=0.95, wd=0.01, ns_steps=5,
                    coeffs=None, check=None, tol=None, nesterov=True):
    """One GPU step through the C ABI vs the oracle on the same stored inputs.

    check: indices of matrices to compare (default all).  Returns per-matrix errors."""
    P, G, M = device_state(Ws, Gs, Bs)
    idx = range(len(Ws)) if check is None else check
    cap = [None] * len(Ws)
    for i in idx:
        cap[i] = torch.empty(Ws[i].value.shape, dtype=torch.float32, device="cuda")
    plan.set_update_capture(cap)
    plan.step(P, G, M, lr=lr, beta=beta, wd=wd, ns_steps=ns_steps, coeffs=coeffs)
    torch.cuda.synchronize()
    plan.set_update_capture(None)
    co = O.QUINTIC if coeffs is None else coeffs
    tol = REL_TOL[dtype] if tol is None else tol
    errs = []
    for i in idx:
        ref = O.muon_step_ref(Ws[i].value, Gs[i].value, Bs[i].value, lr=lr, beta=beta, wd=wd,
                              ns_steps=ns_steps, coeffs=co, param_dtype=dtype, nesterov=nesterov)
        U = cap[i].cpu().numpy().astype(np.float64)
        e_u = rel(U, ref["U"])
        e_buf = rel(to_f64(M[i]), ref["buf_new"])
        Wn = to_f64(P[i])
        e_dw = rel(Wn - Ws[i].value, ref["U"])
        errs.append({"i": i, "err_U": e_u, "err_buf": e_buf, "err_dW": e_dw})
        assert np.all(np.isfinite(U)), f"matrix {i}: non-finite update"
        assert e_u <= tol, f"matrix {i} {Ws[i].value.shape}: rel err of U {e_u:.3e} > {tol}"
        check_lines(U, ref["U"], tol, f"matrix {i} {Ws[i].value.shape}")
        assert e_buf <= 1e-6, f"matrix {i}: momentum rel err {e_buf:.3e}"
        # the stored weights are W + U rounded to the parameter dtype: allow the error of U
        # plus twice the rounding floor that the oracle's own rounding of W + U shows
        floor = rel(ref["W_new_stored"] - ref["W_new"], np.zeros_like(ref["U"])) / max(
            np.linalg.norm(ref["U"]), 1e-300)
        assert e_dw <= tol + 2.5 * floor + 1e-7, \
            f"matrix {i}: weight delta rel err {e_dw:.3e} (rounding floor {floor:.3e})"
    return errs
