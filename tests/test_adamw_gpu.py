"""Parity of the fused multi-tensor AdamW kernel (through the C ABI) with the
fp64 oracle, over three consecutive steps.

Bars: moments (fp32) within 4 fp32 ulp of the magnitudes of the two terms they
sum (beta m and (1 - beta) g, or g^2), per element; fp32 parameters: the
step p_new - p_old within 1e-5 relative Frobenius error; bf16 parameters:
every element within one bf16 ulp of the oracle's rounded value and at least
99% equal to it (the kernel rounds an fp32 result, the oracle an fp64 one)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import matrix_orthogonalizing_optimizer_muon_amd as mod
    return mod


def _bf16_round(x):
    import torch
    return torch.from_numpy(np.asarray(x, np.float64)).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()


def _ulp_bf16(x):
    e = np.floor(np.log2(np.maximum(np.abs(x), 1e-38)))
    return 2.0 ** (e - 7)


@pytest.mark.parametrize("hp", [dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01),
                                dict(lr=0.02, beta1=0.9, beta2=0.95, eps=1e-6, wd=0.1)])
def test_adamw_matches_oracle(M, hp):
    import torch
    from oracle import adamw_oracle as A
    sizes = [1, 7, 2048, 2049, 100003, 32768 + 3, 4096]
    dtypes = ["bf16", "f32", "bf16", "f32", "bf16", "bf16", "f32"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(77)
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}
    # the last tensor sits at an odd element offset: no 16-byte alignment
    back = torch.zeros(4097, device="cuda", dtype=torch.float32)
    P = [(torch.randn(n, device="cuda", generator=gen) * 0.02).to(tdt[d]) for n, d in zip(sizes[:-1], dtypes[:-1])]
    P.append(back[1:])
    P[-1].copy_(torch.randn(4096, device="cuda", generator=gen) * 0.02)
    Mo = [torch.zeros(n, device="cuda") for n in sizes]
    Vo = [torch.zeros(n, device="cuda") for n in sizes]
    plan = M.AdamWPlan(sizes, dtypes)
    for t in (1, 2, 3):
        G = [(torch.randn(n, device="cuda", generator=gen) * 10 ** (-t)).to(tdt[d]) for n, d in zip(sizes, dtypes)]
        before = [(p.double().cpu().numpy(), m.double().cpu().numpy(), v.double().cpu().numpy())
                  for p, m, v in zip(P, Mo, Vo)]
        plan.step(P, G, Mo, Vo, step=t, **hp)
        torch.cuda.synchronize()
        for i, (d, (p0, m0, v0)) in enumerate(zip(dtypes, before)):
            g = G[i].double().cpu().numpy()
            pr, mr, vr = A.adamw_step_ref(p0, g, m0, v0, step=t, **hp)
            # fp32 sums of two terms: a few ulp of the terms' magnitudes (the sum
            # itself may cancel, so a bound relative to it would not hold)
            b1, b2 = hp["beta1"], hp["beta2"]
            mb = 4 * 2.0 ** -24 * (b1 * np.abs(m0) + (1 - b1) * np.abs(g)) + 1e-30
            vb = 4 * 2.0 ** -24 * (b2 * v0 + (1 - b2) * g * g) + 1e-30
            assert np.all(np.abs(Mo[i].double().cpu().numpy() - mr) <= mb), f"tensor {i} exp_avg, step {t}"
            assert np.all(np.abs(Vo[i].double().cpu().numpy() - vr) <= vb), f"tensor {i} exp_avg_sq, step {t}"
            pg = P[i].double().cpu().numpy()
            if d == "f32":
                err = np.linalg.norm((pg - p0) - (pr - p0)) / np.linalg.norm(pr - p0)
                assert err <= 1e-5, (i, t, err)
            else:
                want = _bf16_round(pr)
                assert np.all(np.abs(pg - want) <= _ulp_bf16(want) * 1.0001), (i, t)
                assert np.mean(pg == want) >= 0.99, (i, t, np.mean(pg == want))
    plan.close()


def test_adamw_errors(M):
    import torch
    with pytest.raises(M.MuonError):
        M.AdamWPlan([0], ["f32"])
    plan = M.AdamWPlan([16], ["f32"])
    p = [torch.zeros(16, device="cuda")]
    with pytest.raises(M.MuonError):
        plan.step(p, [torch.zeros(16, device="cuda")], [torch.zeros(16, device="cuda")],
                  [torch.zeros(16, device="cuda")], lr=1e-3, step=0)
    with pytest.raises(M.MuonError):
        plan.step(p, [torch.zeros(16, device="cuda")], [torch.zeros(16, device="cuda")],
                  [torch.zeros(16, device="cuda")], lr=1e-3, beta1=1.0)
    with pytest.raises(ValueError):
        plan.step(p, [torch.zeros(15, device="cuda")], [torch.zeros(16, device="cuda")],
                  [torch.zeros(16, device="cuda")], lr=1e-3)
