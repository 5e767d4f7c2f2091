"""Pins for the AdamW oracle: torch's own AdamW (fp64, CPU) as a library
routine, and closed forms a slip in any term would break."""
import numpy as np
import pytest

from oracle import adamw_oracle as A


def _rng(seed):
    return np.random.default_rng(seed)


@pytest.mark.parametrize("hp", [dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01),
                                dict(lr=0.02, beta1=0.8, beta2=0.95, eps=1e-6, wd=0.1),
                                dict(lr=0.5, beta1=0.0, beta2=0.5, eps=1e-3, wd=0.0)])
def test_matches_torch_adamw_fp64_over_steps(hp):
    import torch
    r = _rng(3)
    p0 = r.standard_normal(257)
    grads = [r.standard_normal(257) * 10 ** r.uniform(-3, 1) for _ in range(6)]
    tp = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([tp], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["wd"])
    p, m, v = p0.copy(), np.zeros(257), np.zeros(257)
    for t, g in enumerate(grads, start=1):
        tp.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        p, m, v = A.adamw_step_ref(p, g, m, v, step=t, **hp)
        np.testing.assert_allclose(p, tp.detach().numpy(), rtol=1e-13, atol=1e-15)
        st = opt.state[tp]
        np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-13, atol=1e-300)
        np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-13, atol=1e-300)


def test_first_step_from_zero_moments():
    r = _rng(5)
    p, g = r.standard_normal(100), r.standard_normal(100)
    lr, wd, eps = 0.01, 0.1, 1e-8
    pn, m, v = A.adamw_step_ref(p, g, np.zeros(100), np.zeros(100), lr=lr, wd=wd, eps=eps,
                                beta1=0.9, beta2=0.999, step=1)
    # m_hat = g, v_hat = g^2: the step is lr * g / (|g| + eps)
    np.testing.assert_allclose(pn, p - lr * wd * p - lr * g / (np.abs(g) + eps), rtol=1e-14)
    np.testing.assert_allclose(m, 0.1 * g, rtol=1e-15)
    np.testing.assert_allclose(v, 0.001 * g * g, rtol=1e-14)


def test_constant_gradient_keeps_bias_corrected_moments():
    g = np.array([0.5, -2.0, 3e-3, 0.0])
    p, m, v = np.ones(4), np.zeros(4), np.zeros(4)
    lr, eps = 0.1, 1e-8
    for t in range(1, 8):
        prev = p
        p, m, v = A.adamw_step_ref(p, g, m, v, lr=lr, wd=0.0, eps=eps, beta1=0.9, beta2=0.99, step=t)
        np.testing.assert_allclose(prev - p, lr * g / (np.abs(g) + eps), rtol=1e-12, atol=1e-18)


def test_zero_betas_and_zero_gradient():
    g = np.array([1.0, -4.0])
    p, m, v = A.adamw_step_ref(np.zeros(2), g, np.full(2, 7.0), np.full(2, 9.0), lr=1.0, wd=0.0,
                               eps=0.0, beta1=0.0, beta2=0.0, step=3)
    np.testing.assert_allclose(p, -np.sign(g))
    np.testing.assert_allclose(m, g)
    np.testing.assert_allclose(v, g * g)
    # zero gradient and zero moments: decoupled decay only
    p, m, v = A.adamw_step_ref(np.full(3, 2.0), np.zeros(3), np.zeros(3), np.zeros(3), lr=0.1, wd=0.5,
                               step=1)
    np.testing.assert_allclose(p, 2.0 * (1 - 0.05))
