"""muon_step_noalloc (no device allocation) against the plan-based muon_step.

The entry point runs one matrix with the workspace in the library's static
per-device scratch array.  Its configuration equals a plan forced to the
direct form, tile plan 5 and one lane, so on the bf16 path the weights and
momenta it writes are bitwise those of that plan's step; on the fp32 path
(128 x 128 tiles, while a plan may pick 64 x 64) they are compared within the
fp32 tolerance.  Both are also graded against the fp64 oracle.  Two calls in
a row, the second on a smaller matrix (the array keeps the first call's
contents), then a larger-than-the-array matrix is refused with nothing
enqueued, and no call changes the device's free memory."""
import numpy as np
import pytest

import workloads as WL

pytestmark = pytest.mark.gpu


def _state(shape, dtype, seed):
    from gpu_util import to_device
    W = WL.draw_custom([seed, 0], shape, dtype)
    G = WL.draw_custom([seed, 1], shape, dtype)
    B = WL.draw_custom([seed, 2], shape, WL.F32, "normal", 0.01)
    return W, G, B, to_device(W), to_device(G), to_device(B)


def _plan_step(M, shape, dtype, W, G, B, **kw):
    from gpu_util import to_device
    plan = M.MuonPlan([shape], dtype, tune="off", form="direct", lanes=1,
                      tile=5 if dtype == WL.BF16 else None)
    P, Gd, Bd = to_device(W), to_device(G), to_device(B)
    plan.step([P], [Gd], [Bd], **kw)
    import torch
    torch.cuda.synchronize()
    plan.close()
    return P, Bd


@pytest.mark.parametrize("dtype,shapes", [
    (WL.BF16, [(1024, 4096), (300, 700)]),
    (WL.BF16, [(4096, 1024), (129, 2000)]),
    (WL.F32, [(256, 512), (100, 333)]),
    (WL.F32, [(1024, 512), (77, 64)]),
])
def test_noalloc_equals_plan_step_two_calls(dtype, shapes):
    import torch
    import matrix_orthogonalizing_optimizer_muon_amd as M
    from gpu_util import to_f64, rel, REL_TOL, check_lines
    from oracle import muon_oracle as O

    tol = REL_TOL[dtype]
    for c, shape in enumerate(shapes):
        W, G, B, P, Gd, Bd = _state(shape, dtype, 300 + c)
        free0 = torch.cuda.mem_get_info()[0]
        M.step_noalloc(P, Gd, Bd, lr=0.02, beta=0.95, wd=0.01, ns_steps=5)
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] == free0 or c == 0   # the first call may load the module
        Pp, Bp = _plan_step(M, shape, dtype, W, G, B)
        assert torch.equal(Bd, Bp), "momentum"
        if dtype == WL.BF16:
            assert torch.equal(P.view(torch.int16), Pp.view(torch.int16)), f"weights {shape}"
        else:
            e = rel(to_f64(P) - W.value, to_f64(Pp) - W.value)
            assert e <= tol, f"weight delta vs plan {shape}: {e:.3e}"
        ref = O.muon_step_ref(W.value, G.value, B.value, param_dtype=dtype)
        e_dw = rel(to_f64(P) - W.value, ref["U"])
        e_b = rel(to_f64(Bd), ref["buf_new"])
        print(f"noalloc {dtype} {shape}: weight delta vs oracle {e_dw:.3e}, momentum {e_b:.1e}", flush=True)
        floor = np.linalg.norm(ref["W_new_stored"] - ref["W_new"]) / np.linalg.norm(ref["U"])
        assert e_dw <= tol + 2.5 * floor + 1e-7
        assert e_b <= 1e-6


def test_noalloc_ns_steps_zero_plain_momentum_and_coeffs():
    import torch
    import matrix_orthogonalizing_optimizer_muon_amd as M
    for dtype in (WL.BF16, WL.F32):
        shape = (200, 520)
        for kw in ({"ns_steps": 0}, {"nesterov": False}, {"coeffs": (1.5, -0.5, 0.0), "ns_steps": 7}):
            W, G, B, P, Gd, Bd = _state(shape, dtype, 400)
            M.step_noalloc(P, Gd, Bd, **kw)
            torch.cuda.synchronize()
            plan_kw = {k: v for k, v in kw.items() if k != "nesterov"}
            plan = M.MuonPlan([shape], dtype, tune="off", form="direct", lanes=1,
                              nesterov=kw.get("nesterov", True), tile=5 if dtype == WL.BF16 else None)
            from gpu_util import to_device, to_f64, rel
            Pp, Gp, Bp = to_device(W), to_device(G), to_device(B)
            plan.step([Pp], [Gp], [Bp], **plan_kw)
            torch.cuda.synchronize()
            plan.close()
            assert torch.equal(Bd, Bp), (dtype, kw)
            if dtype == WL.BF16:
                assert torch.equal(P.view(torch.int16), Pp.view(torch.int16)), (dtype, kw)
            else:
                assert rel(to_f64(P) - W.value, to_f64(Pp) - W.value) <= 1e-4, (dtype, kw)


def test_noalloc_refuses_oversize_and_bad_arguments():
    import torch
    import matrix_orthogonalizing_optimizer_muon_amd as M
    big = (4096, 4096)   # bf16 workspace 4 (m n + m m) = 128 MiB > 64 MiB
    P = torch.zeros(big, dtype=torch.bfloat16, device="cuda")
    G = torch.zeros_like(P)
    B = torch.zeros(big, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    with pytest.raises(M.MuonError, match="MUON_ENOMEM"):
        M.step_noalloc(P, G, B)
    with pytest.raises(M.MuonError, match="MUON_EINVAL"):
        M.step_noalloc(P[:10, :10].contiguous(), G[:10, :10].contiguous(), B[:10, :10].contiguous(),
                       ns_steps=-1)
    torch.cuda.synchronize()
    assert torch.count_nonzero(P).item() == 0 and torch.count_nonzero(B).item() == 0
