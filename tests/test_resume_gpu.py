"""Checkpoint / resume: the only state carried between steps is the caller's
momenta (and the weights), and a plan is re-derived byte-identically from the
same shapes and tune cache.  So a run interrupted after step k (weights and
momenta saved to the host, the plan destroyed) and resumed with a new plan and
new device buffers gives, at step k+1, bitwise the tensors of the
uninterrupted run."""
import numpy as np
import pytest

import workloads as WL

pytestmark = pytest.mark.gpu


def _grads(shapes, dtype, step):
    from gpu_util import to_device
    return [to_device(WL.draw_custom([77, i, step], s, dtype)) for i, s in enumerate(shapes)]


@pytest.mark.parametrize("dtype,shapes", [
    (WL.BF16, [(1024, 4096), (4096, 1024), (512, 512), (300, 700), (700, 300), (129, 2000)]),
    (WL.F32, [(256, 512), (512, 256), (100, 333)]),
])
def test_resume_after_step_k_is_bitwise_equal(dtype, shapes, tmp_path):
    import torch
    import matrix_orthogonalizing_optimizer_muon_amd as M
    from gpu_util import to_device

    cache = str(tmp_path / "tune.txt")
    K = 3
    W0 = [to_device(WL.draw_custom([76, i], s, dtype)) for i, s in enumerate(shapes)]

    def fresh_state():
        return [w.clone() for w in W0], [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]

    # uninterrupted: K + 1 steps on one plan
    plan = M.MuonPlan(shapes, dtype, tune="once", cache_path=cache)
    ref_plan_bytes = plan.serialize()
    P, B = fresh_state()
    for k in range(K + 1):
        plan.step(P, _grads(shapes, dtype, k), B)
    torch.cuda.synchronize()
    want_P = [p.cpu() for p in P]
    want_B = [b.cpu() for b in B]
    plan.close()

    # interrupted after step K: save, destroy the plan, resume on new buffers
    plan = M.MuonPlan(shapes, dtype, tune="once", cache_path=cache)
    P, B = fresh_state()
    for k in range(K):
        plan.step(P, _grads(shapes, dtype, k), B)
    torch.cuda.synchronize()
    saved_P = [p.cpu().clone() for p in P]
    saved_B = [b.cpu().clone() for b in B]
    plan.close()
    del P, B
    torch.cuda.empty_cache()

    plan2 = M.MuonPlan(shapes, dtype, tune="once", cache_path=cache)
    assert plan2.serialize() == ref_plan_bytes     # cache hit: the same plan
    # new allocations (a padding tensor first, so the pointers differ)
    pad = torch.empty(12345, device="cuda")
    P2 = [p.to("cuda") for p in saved_P]
    B2 = [b.to("cuda") for b in saved_B]
    plan2.step(P2, _grads(shapes, dtype, K), B2)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        assert torch.equal(P2[i].cpu().view(torch.int16) if dtype == WL.BF16 else P2[i].cpu(),
                           want_P[i].view(torch.int16) if dtype == WL.BF16 else want_P[i]), i
        assert torch.equal(B2[i].cpu(), want_B[i]), i
    del pad
    plan2.close()
