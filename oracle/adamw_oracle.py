"""fp64 CPU oracle for the fused AdamW step (the non-matrix half of the hybrid).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests (and bench's CPU leg, if any) use it.  It
shares no code with the library.

"DeepSpeed now supports Muon" (setupai.cc), technical deep dive: Muon is
usually run together with AdamW, Muon on the weight matrices and AdamW on the
other parameters (embeddings, biases, the final classifier).  The pages do not
write AdamW out, so this is AdamW as published (Loshchilov and Hutter,
"Decoupled Weight Decay Regularization"), with the weight decay applied to the
old parameter and scaled by the learning rate:

    m_t = beta1 m_{t-1} + (1 - beta1) g_t
    v_t = beta2 v_{t-1} + (1 - beta2) g_t^2
    m_hat = m_t / (1 - beta1^t),   v_hat = v_t / (1 - beta2^t)
    p_t = p_{t-1} - lr wd p_{t-1} - lr m_hat / (sqrt(v_hat) + eps)

Pins (tests/test_adamw_oracle.py): torch.optim.AdamW on fp64 CPU tensors over
several steps (a library routine), the first step from zero moments
(m_hat = g, v_hat = g^2 exactly), a constant gradient (m_hat and v_hat stay g
and g^2 at every t), beta1 = beta2 = 0, and zero gradients (pure decay).
"""
import numpy as np


def adamw_step_ref(p, g, m, v, *, lr, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01, step=1):
    """One AdamW step of one tensor in fp64.  Returns (p_new, m_new, v_new)."""
    p = np.asarray(p, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** step)
    v_hat = v / (1.0 - beta2 ** step)
    p_new = p - lr * wd * p - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p_new, m, v
