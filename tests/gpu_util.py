"""Helpers shared by the GPU parity tests (upload, one library step, metrics)."""

from __future__ import annotations

import sys

import numpy as np

import oracle.muon as om

NS_TOL_BF16 = 2e-2      # relative Frobenius error of O per matrix, bf16 NS
NS_TOL_FP32 = 1e-4      # relative Frobenius error of O per matrix, fp32 NS
NS_TOL_BF16X3 = 1e-3    # relative Frobenius error of O per matrix, compensated bf16 NS
ELEM_TOL = 1e-6         # relative max-norm error of the fp32 elementwise parts


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def rel_frob(got, want) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / den) if den > 0 else float(np.linalg.norm(got))


def rel_max(got, want) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.abs(want).max() if want.size else 0.0
    err = np.abs(got - want).max() if want.size else 0.0
    return float(err / den) if den > 0 else float(err)


def f32(x) -> float:
    """The float32 value of a Python scalar, promoted back (what the library sees)."""
    return float(np.float32(x))


def gpu_step(mats, grads, moms, *, lr, momentum, wd, coeffs, nesterov=True, row_norm=True,
             ns_precision=0, want_o=True, workspace=None, emas=None, ema_decay=0.0):
    """Upload, run one library step, return (W', M', O, E') as host arrays.

    O is None if not requested; emas (host arrays or None entries) are the EMA
    shadows advanced inside the step, E' is None where no shadow was given.
    """
    import torch
    import muon_optimizer_step_amd as ms
    P = [dev(w) for w in mats]
    G = [dev(g) for g in grads]
    M = [dev(m) for m in moms]
    O = [torch.full_like(p, float("nan")) for p in P] if want_o else None
    E = [dev(e) if e is not None else None for e in emas] if emas is not None else None
    ms.muon_step(P, G, M, lr=lr, momentum=momentum, weight_decay=wd, coeffs=coeffs, nesterov=nesterov,
                 row_norm=row_norm, ns_precision=ns_precision, update_outs=O, workspace=workspace,
                 emas=E, ema_decay=ema_decay)
    torch.cuda.synchronize()
    e_out = [host(e) if e is not None else None for e in E] if E is not None else None
    return [host(p) for p in P], [host(m) for m in M], ([host(o) for o in O] if want_o else None), e_out


def check_fused_ema(e_in, w_gpu, e_gpu, decay, label=""):
    """E' of the step against the oracle EMA fed the GPU's W'; returns the worst error."""
    worst = 0.0
    for i, (e0, w, e) in enumerate(zip(e_in, w_gpu, e_gpu)):
        if e0 is None:
            assert e is None
            continue
        err = rel_max(e, om.ema_update(e0, w, f32(decay)))
        assert err <= ELEM_TOL, f"{label} fused EMA tensor {i}: {err:.3e}"
        worst = max(worst, err)
    return worst


def check_layers(w_in, g_in, m_in, w_gpu, m_gpu, o_gpu, *, lr, momentum, wd, coeffs, nesterov, row_norm,
                 ns_tol, label=""):
    """Layered parity for one matrix; returns the O error."""
    mu = f32(momentum)
    m_ref, u_ref = om.momentum_update(m_in, g_in, mu, nesterov)
    e_m = rel_max(m_gpu, m_ref)
    assert e_m <= ELEM_TOL, f"{label} momentum rel err {e_m:.3e}"
    rows, cols = w_in.shape
    # W' from the oracle's apply step fed the GPU's O (the NS error is checked separately)
    w_ref = om.apply_update(w_in, o_gpu, f32(lr), f32(wd), om.shape_scale(rows, cols))
    e_w = rel_max(w_gpu, w_ref)
    assert e_w <= ELEM_TOL, f"{label} weight rel err {e_w:.3e}"
    o_ref = om.orthogonalize(u_ref, [[f32(v) for v in row] for row in coeffs], row_norm)
    e_o = rel_frob(o_gpu, o_ref)
    assert e_o <= ns_tol, f"{label} NS output rel Frobenius err {e_o:.3e} > {ns_tol}"
    return e_o
