"""Parity of muon_orthogonalize (NS alone, through the C ABI) with the fp64 oracle.

Tolerance (relative Frobenius error of the fp32 output): 2e-2 on the bf16-MFMA
path, 1e-4 on the fp32 path, as for the update of muon_step."""
import numpy as np
import pytest

import workloads as WL

pytestmark = pytest.mark.gpu

TOL = {WL.BF16: 2e-2, WL.F32: 1e-4}


@pytest.fixture(scope="module")
def M():
    import matrix_orthogonalizing_optimizer_muon_amd as mod
    return mod


def _run(M, shapes, dtype, ns_steps=5, coeffs=None, seed=0, **plan_kw):
    import torch
    from gpu_util import to_device, rel
    from oracle import muon_oracle as O
    plan_kw.setdefault("tune", "off")
    plan = M.MuonPlan(shapes, dtype, **plan_kw)
    ins = [WL.draw_custom([seed, i, 5], s, dtype, "normal", 0.02) for i, s in enumerate(shapes)]
    X = [to_device(st) for st in ins]
    outs = [torch.full(s, float("nan"), dtype=torch.float32, device="cuda") for s in shapes]
    plan.orthogonalize(X, outs, ns_steps=ns_steps, coeffs=coeffs)
    torch.cuda.synchronize()
    assert plan.flags() == 0
    sched = O.QUINTIC if coeffs is None else coeffs
    errs = []
    for i, st in enumerate(ins):
        want = O.orthogonalize_ref(st.value, ns_steps, sched)
        got = outs[i].cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(got)), i
        errs.append(rel(got, want))
    plan.close()
    return errs


@pytest.mark.parametrize("dtype", [WL.BF16, WL.F32])
def test_orthogonalize_ragged_tall_and_wide(M, dtype):
    shapes = [(300, 700), (700, 300), (129, 1000), (520, 520), (64, 2048), (33, 65)]
    errs = _run(M, shapes, dtype, seed=1)
    print(dtype, ["%.2e" % e for e in errs])
    assert max(errs) <= TOL[dtype]


@pytest.mark.parametrize("T", [0, 1, 2])
def test_orthogonalize_few_steps(M, T):
    errs = _run(M, [(256, 512), (512, 256), (100, 300)], WL.BF16, ns_steps=T, seed=2 + T)
    assert max(errs) <= TOL[WL.BF16]


def test_orthogonalize_schedule_gram_and_lanes(M):
    sched = [(3.4445, -4.7750, 2.0315), (1.5, -0.5, 0.0), (2.0, -1.5, 0.5), (3.4445, -4.7750, 2.0315)]
    shapes = [(200, 1500), (1500, 200), (256, 1024), (384, 640), (640, 384)]
    errs = _run(M, shapes, WL.BF16, ns_steps=4, coeffs=sched, seed=9, form="gram")
    assert max(errs) <= TOL[WL.BF16]
    errs = _run(M, shapes, WL.BF16, ns_steps=4, coeffs=sched, seed=9, lanes=3, tile=2)
    assert max(errs) <= TOL[WL.BF16]


def test_orthogonalize_then_step_on_the_same_plan(M):
    """The step after an orthogonalization (different pointers, same workspace)
    still matches the oracle: the per-chunk pointer upload is refreshed."""
    import torch
    from gpu_util import make_state, run_and_compare
    shapes = [(256, 768), (768, 256)]
    plan = M.MuonPlan(shapes, "bf16", tune="off")
    X = [torch.randn(s, device="cuda").to(torch.bfloat16) for s in shapes]
    outs = [torch.empty(s, dtype=torch.float32, device="cuda") for s in shapes]
    plan.orthogonalize(X, outs)
    torch.cuda.synchronize()
    Ws, Gs, Bs = make_state(shapes, WL.BF16, seed=44, buf_scale=0.01)
    run_and_compare(plan, Ws, Gs, Bs, WL.BF16)


def test_orthogonalize_argument_errors(M):
    import torch
    plan = M.MuonPlan([(64, 128)], "bf16", tune="off")
    x = [torch.zeros(64, 128, dtype=torch.bfloat16, device="cuda")]
    o = [torch.zeros(64, 128, dtype=torch.float32, device="cuda")]
    with pytest.raises(ValueError):
        plan.orthogonalize(x, [torch.zeros(64, 128, dtype=torch.bfloat16, device="cuda")])
    with pytest.raises(M.MuonError):
        plan.orthogonalize(x, o, ns_steps=65)
    with pytest.raises(M.MuonError):
        plan.orthogonalize(x, o, ns_steps=1, coeffs=[(float("nan"), 0.0, 0.0)])
    # a zero input gives a zero output (no NaN: the norm gets eps)
    plan.orthogonalize(x, o)
    torch.cuda.synchronize()
    assert torch.count_nonzero(o[0]).item() == 0 and plan.flags() == 0
