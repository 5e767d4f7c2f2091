"""Parity at the full workload sizes, in the launch configuration bench.py times.

Each test builds the plan over every matrix of a workload the way bench.py does
(form and tile plan timed once per shape, cached in a fresh file), steps all of
them at once, and compares the fp32 update of a sample of matrices - drawn from
the seeded host generator - with the fp64 oracle one by one.  The other
matrices get device-generated values of the same laws (their values do not
change which kernels run).  Tolerance: 2e-2 relative Frobenius error of U."""
import time

import numpy as np
import pytest

import workloads as WL

pytestmark = pytest.mark.gpu


def _step_and_check(wl, sample, tmp_path):
    import torch
    import matrix_orthogonalizing_optimizer_muon_amd as M
    from gpu_util import to_device, to_f64, rel
    from oracle import muon_oracle as O

    t0 = time.time()
    plan = M.MuonPlan(wl.shapes, wl.dtype, tune="once", cache_path=str(tmp_path / "tune.txt"))
    print(f"{wl.name}: plan {time.time() - t0:.1f}s, choices "
          f"{sorted({(min(s), max(s), plan.matrix_choice(i)['form'], plan.matrix_choice(i)['tile']) for i, s in enumerate(wl.shapes)})}",
          flush=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4321 + wl.cfg)
    P, G, B = [], [], []
    host = {}
    for i, (r, c) in enumerate(wl.shapes):
        if i in sample:
            Wst, Gst = WL.draw(wl, i, 0, WL.KIND_W), WL.draw(wl, i, 0, WL.KIND_G)
            host[i] = (Wst, Gst)
            P.append(to_device(Wst))
            G.append(to_device(Gst))
        else:
            P.append((torch.randn(r, c, device="cuda", generator=gen) * wl.w_scale).to(torch.bfloat16))
            G.append((torch.randn(r, c, device="cuda", generator=gen) * wl.grad_scale).to(torch.bfloat16))
        B.append(torch.zeros(r, c, device="cuda", dtype=torch.float32))
    cap = [torch.empty(s, dtype=torch.float32, device="cuda") if i in sample else None
           for i, s in enumerate(wl.shapes)]
    plan.set_update_capture(cap)
    plan.step(P, G, B)
    torch.cuda.synchronize()
    plan.set_update_capture(None)
    assert plan.flags() == 0
    print(f"{wl.name}: step done {time.time() - t0:.1f}s", flush=True)
    worst = 0.0
    for i in sample:
        Wst, Gst = host[i]
        ref = O.muon_step_ref(Wst.value, Gst.value, np.zeros(Wst.value.shape), param_dtype="bf16")
        e = rel(cap[i].cpu().numpy().astype(np.float64), ref["U"])
        eb = rel(to_f64(B[i]), ref["buf_new"])
        print(f"  matrix {i} {wl.shapes[i]}: rel err U {e:.3e}, momentum {eb:.1e}", flush=True)
        worst = max(worst, e)
        assert e <= 2e-2, f"matrix {i} {wl.shapes[i]}: {e:.3e}"
        assert eb <= 1e-6
    plan.close()
    return worst


def test_vla_mixed_shapes_full_size(tmp_path):
    wl = WL.workload(3)
    # backbone layer 0 (QKV, O, up, down) and action-expert layer 0
    sample = [0, 1, 2, 3, 96, 97, 98, 99]
    _step_and_check(wl, sample, tmp_path)


def test_llama7b_matrix_set_full_size(tmp_path):
    wl = WL.workload(4)
    # layer 0 O projection (4096 x 4096) and gate (11008 x 4096, iterated transposed)
    sample = [1, 2]
    _step_and_check(wl, sample, tmp_path)


def test_moe_stack_full_size(tmp_path):
    wl = WL.workload(5)
    # two experts' gate/up/down and the first 512 x 16384 matrix
    sample = [0, 1, 2, 1535, 1536]
    _step_and_check(wl, sample, tmp_path)
