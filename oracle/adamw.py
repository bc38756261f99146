"""Plain float64 oracle of the AdamW step on the non-matrix parameters.

TEST INFRASTRUCTURE ONLY (imported by tests/ and the cpu_baseline leg of
bench.py).  Every step is one NumPy expression in float64, in the order the
method runs; nothing is shared with the HIP library.

Source: "Record: L_ParallelResiduals_UNetSkips_DepthRecur_Muon_ 1.0901"
(PR #1893), table "Architecture and training stack", row Optimizer: Muon runs
on the matrix parameters and AdamW on the embeddings and scalars.  The page
names the optimizer only; it gives neither its equations nor its
hyperparameters.  Reading taken (R13): AdamW as
Loshchilov and Hutter define it, with decoupled weight decay applied to the
pre-update parameter, bias-corrected moments at step t (t counts from 1) and
eps added to the square root of the corrected second moment:

    p  <- (1 - lr*wd) p
    m  <- beta1 m + (1 - beta1) g
    v  <- beta2 v + (1 - beta2) g^2
    p  <- p - lr * (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)

No amsgrad, no maximisation.  Inputs are promoted to float64; callers pass the
same float32 values the GPU library receives.
"""

from __future__ import annotations

import numpy as np


def adamw_update(p, g, m, v, *, lr: float, beta1: float, beta2: float, eps: float, wd: float, step: int):
    """One AdamW step on one tensor; returns (p', m', v') in float64."""
    p = np.asarray(p, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    decayed = (1.0 - lr * wd) * p
    m_new = beta1 * m + (1.0 - beta1) * g
    v_new = beta2 * v + (1.0 - beta2) * (g * g)
    m_hat = m_new / (1.0 - beta1 ** step)
    v_hat = v_new / (1.0 - beta2 ** step)
    p_new = decayed - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p_new, m_new, v_new
