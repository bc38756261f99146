"""Plain float64 oracle of one Muon optimizer step plus the weight EMA.

TEST INFRASTRUCTURE ONLY (imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py).  It is deliberately slow and obvious: every step
of the method is one NumPy expression in float64, in the order the method runs,
with no blocking, fusion, reordering or reduced precision.  It shares no code,
table or constant generator with the HIP library.

Sources (the pages are cited by title and section):

* "Record: L_ParallelResiduals_UNetSkips_DepthRecur_Muon_ 1.0901" (PR #1893),
  table "Architecture and training stack", row Optimizer: Muon runs on the
  matrix parameters with momentum 0.99 and MATRIX_LR 0.022; row EMA: the weight
  EMA uses EMA_DECAY 0.9965.
* "Record: Combined 3-Layer Recurrence + Parallel Residuals + Polar Express +
  Brotli" (PR #1396), table "Techniques Combined": MuonEq-R normalises rows
  before the Newton-Schulz (NS) iteration; the NS iteration takes a
  per-iteration coefficient schedule ("Polar Express", 4 steps); WD is 0.105.
* "Record: SP8192 + Improved Parallel Residuals + Muon 0.97 + ..." (PR #1557),
  section "Techniques": Muon momentum 0.97 with row normalisation, matrix LR
  0.03, EMA 0.997.
* "Record: Improved Parallel Residuals + Systems Optimization" (PR #1584),
  section "Summary": the fused Muon kernel and the batched EMA change systems
  code only, so the optimizer's arithmetic is the plain one written here.

The pages name the method but do not print its equations.  This oracle takes
the plainest reading of "Muon" (the readings are listed below):

  R1 momentum (Nesterov, SGD form):   M' = mu*M + G;   U = G + mu*M'
     (without Nesterov: U = M').
  R2 MuonEq-R row normalisation, over the rows of the stored (out x in) matrix,
     before everything else that follows:  U_i <- U_i / (||U_i||_2 + eps).
  R3 Frobenius scaling:  X0 = R / (||R||_F + eps), so every singular value of
     X0 is at most 1.
  R4 the NS iteration runs on the short side: if rows > cols it works on X0^T
     and transposes back at the end.
  R5 per-iteration coefficient table: row k of the table (a_k, b_k, c_k) drives
     iteration k:  A = X X^T;  B = b_k A + c_k A A;  X <- a_k X + B X.
  R6 shape-scaled learning rate: s = sqrt(max(1, rows/cols)).
  R7 decoupled weight decay applied to the pre-update weight:
     W' = (1 - lr*wd) W - lr*s*O.
  R8 weight EMA after the step, over every parameter:
     E' = d E + (1 - d) P, with P the post-step parameter.
  eps = 1e-7 in R2 and R3.

All floating-point inputs (arrays and scalars) are promoted to float64 before
use; callers pass the same float32 values the GPU library receives.
"""

from __future__ import annotations

import math
from typing import Sequence

import numpy as np

EPS = 1e-7


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def momentum_update(buf, grad, mu: float, nesterov: bool = True):
    """Momentum buffer update and the vector the orthogonaliser sees (R1).

    Page: PR #1893, "Architecture and training stack", Optimizer row (Muon,
    momentum 0.99); PR #1557, "Techniques" (momentum 0.97).
    Returns (M', U) in float64.
    """
    buf = _f64(buf)
    grad = _f64(grad)
    mu = float(mu)
    buf_new = mu * buf + grad
    if nesterov:
        u = grad + mu * buf_new
    else:
        u = buf_new
    return buf_new, u


def row_normalize(u, eps: float = EPS):
    """MuonEq-R: every row of the stored matrix divided by its L2 norm (R2).

    Page: PR #1396, "Techniques Combined", MuonEq-R row ("Row-norm before NS").
    A zero row stays zero (eps keeps the division finite).
    """
    u = _f64(u)
    norms = np.sqrt(np.sum(u * u, axis=1, keepdims=True))
    return u / (norms + eps)


def frobenius_normalize(x, eps: float = EPS):
    """Scale the whole matrix to unit Frobenius norm (R3)."""
    x = _f64(x)
    return x / (math.sqrt(float(np.sum(x * x))) + eps)


def newton_schulz(x, coeffs: Sequence[Sequence[float]]):
    """The quintic NS iteration on a matrix that is already short-side first (R5).

    Page: PR #1396, "Techniques Combined", Polar Express Newton-Schulz row (a
    schedule of per-step coefficients; the number of rows of ``coeffs`` is the
    number of iterations).  Iteration k uses row k.
    """
    x = _f64(x)
    for a, b, c in coeffs:
        a, b, c = float(a), float(b), float(c)
        gram = x @ x.T
        poly = b * gram + c * (gram @ gram)
        x = a * x + poly @ x
    return x


def orthogonalize(u, coeffs: Sequence[Sequence[float]], row_norm: bool, eps: float = EPS):
    """R2 (optional), R3, R4 and R5 on one stored (rows x cols) matrix; returns O."""
    r = row_normalize(u, eps) if row_norm else _f64(u)
    x0 = frobenius_normalize(r, eps)
    rows, cols = x0.shape
    transposed = rows > cols
    x = x0.T if transposed else x0
    x = newton_schulz(x, coeffs)
    return x.T if transposed else x


def shape_scale(rows: int, cols: int) -> float:
    """Shape-scaled learning-rate factor (R6)."""
    return math.sqrt(max(1.0, rows / cols))


def apply_update(w, o, lr: float, wd: float, scale: float):
    """Decoupled weight decay plus the scaled orthogonal update (R7).

    Page: PR #1396, "Techniques Combined", WD=0.105 row; PR #1893, Optimizer row
    (MATRIX_LR 0.022).
    """
    w = _f64(w)
    o = _f64(o)
    lr, wd, scale = float(lr), float(wd), float(scale)
    return (1.0 - lr * wd) * w - lr * scale * o


def muon_step_matrix(w, g, buf, *, lr: float, mu: float, nesterov: bool, wd: float,
                     row_norm: bool, coeffs: Sequence[Sequence[float]]):
    """One Muon step on one matrix.  Returns (W', M', O) in float64."""
    buf_new, u = momentum_update(buf, g, mu, nesterov)
    o = orthogonalize(u, coeffs, row_norm)
    rows, cols = o.shape
    w_new = apply_update(w, o, lr, wd, shape_scale(rows, cols))
    return w_new, buf_new, o


def ema_update(ema, param, decay: float):
    """Weight EMA over one tensor (R8).

    Page: PR #1893, "Architecture and training stack", EMA row (EMA_DECAY
    0.9965, applied to the weights); PR #1557, "Techniques" (EMA 0.997).
    """
    e = _f64(ema)
    p = _f64(param)
    d = float(decay)
    return d * e + (1.0 - d) * p
