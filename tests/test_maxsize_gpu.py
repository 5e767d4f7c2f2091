"""The largest matrices the planner accepts (m_pad * n_pad = 2^30 bf16
elements: 16384 x 65536 and its transpose), checked where the oracle cannot
run whole.  The gradient is zero except one seeded 64 x 256 block, so d, X0
and every NS iterate are zero outside that block: the normalization sees only
the block's entries, and zero rows and columns stay zero through X X^T,
a I + b A + c A A and B X.  Inside the block the update must match the fp64
oracle's step on the block with the full matrix's RMS scale (bf16 bar);
everywhere else it is -lr wd W in fp32 and the new weight is W + U rounded to
bf16, within fp32 rounding; the momentum is exactly g (zero start)."""
import numpy as np
import pytest

import workloads as WL
from oracle import muon_oracle as O

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,cols,r0,c0,bh,bw", [
    (16384, 65536, 8000, 40000, 64, 256),   # wide: canonical = stored
    (65536, 16384, 40000, 8000, 256, 64),   # tall: iterated as its transpose
])
def test_max_size_matrix_with_one_nonzero_block(rows, cols, r0, c0, bh, bw):
    import torch
    import matrix_orthogonalizing_optimizer_muon_amd as M
    from gpu_util import rel, to_device, to_f64
    print(f"max-size case {rows}x{cols}", flush=True)
    lr, beta, wd = 0.02, 0.95, 0.01
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2024)
    W = (torch.randn(rows, cols, device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
    W_old = W.clone()
    Gb = WL.draw_custom([130, rows, 1], (bh, bw), WL.BF16)
    G = torch.zeros(rows, cols, dtype=torch.bfloat16, device="cuda")
    G[r0:r0 + bh, c0:c0 + bw] = to_device(Gb)
    B = torch.zeros(rows, cols, dtype=torch.float32, device="cuda")
    U = torch.empty(rows, cols, dtype=torch.float32, device="cuda")
    plan = M.MuonPlan([(rows, cols)], "bf16", tune="off")
    plan.set_update_capture([U])
    plan.step([W], [G], [B], lr=lr, beta=beta, wd=wd)
    torch.cuda.synchronize()
    assert not plan.flags()
    assert torch.equal(B, G.float())
    # inside the block: the oracle's step on the block, full-matrix RMS scale
    W_blk = to_f64(W_old[r0:r0 + bh, c0:c0 + bw])
    _, d = O.nesterov_momentum(np.zeros((bh, bw)), Gb.value, beta)
    X0, _ = O.frobenius_normalize(d)
    X = O.ns_direct(X0, 5)
    U_ref, _ = O.apply_update(W_blk, X, lr, wd, O.rms_scale(rows, cols))
    err = rel(U[r0:r0 + bh, c0:c0 + bw].double().cpu().numpy(), U_ref)
    print(f"block update rel err {err:.3e}", flush=True)
    assert err <= 2e-2
    # everywhere else: x = 0, so U = -lr (wd W) and W_new = bf16(W + U)
    want = (W_old.float() * wd) * (-lr)
    U[r0:r0 + bh, c0:c0 + bw] = 0
    want[r0:r0 + bh, c0:c0 + bw] = 0
    tol = 2 * torch.finfo(torch.float32).eps * float(want.abs().max())
    assert float((U - want).abs().max()) <= tol
    W_want = (W_old.float() + want).to(torch.bfloat16)
    W[r0:r0 + bh, c0:c0 + bw] = 0
    W_want[r0:r0 + bh, c0:c0 + bw] = 0
    diff = (W.float() - W_want.float()).abs()
    ulp = W_want.float().abs() * 2.0 ** -7
    assert bool((diff <= ulp).all())
    assert float((diff == 0).float().mean()) >= 0.999
    plan.close()
    del W, W_old, G, B, U, want, W_want, diff, ulp
    torch.cuda.empty_cache()
